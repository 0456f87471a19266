"""lora_linear captured in a HIP graph: every replay equals the eager result, bit for bit.

The graph is replayed several times with eager work of the program and synchronisations in
between (the library records no memset nodes; this checks that replays after the first stay
correct).
"""

import numpy as np
import pytest

from synth import random_case

from .gpu_util import bf16_dev, log, to_device

pytestmark = pytest.mark.gpu


GRAPH_CASES = [
    # seed, M, d_in, d_out, n, r_max, mode (1 decode, 2 prefill), rank-compact pool
    (91, 96, 1024, 768, 12, 16, 1, False),   # small-batch fused decode path
    (92, 96, 1024, 768, 12, 16, 2, False),   # prefill
    (93, 200, 1024, 520, 40, 32, 1, False),  # medium decode path
    (94, 300, 4096, 2056, 50, 64, 1, False),  # stream-K decode path
    (95, 300, 4096, 2056, 50, 64, 1, True),   # stream-K, compact pool
    (96, 200, 1024, 520, 40, 32, 2, True),    # prefill, compact pool
    (97, 48, 1024, 520, 300, 16, 1, False),   # small batch, pool larger than the batch (slot per row)
    (98, 40, 512, 264, 90, 24, 1, True),      # small batch, compact pool larger than the batch
    (99, 64, 1024, 392, 30, 8, 1, False),     # small batch, rank 8 in 16-wide slots
]


@pytest.mark.parametrize("case", GRAPH_CASES,
                         ids=[f"M{c[1]}-{'dec' if c[6] == 1 else 'pre'}{'-compact' if c[7] else ''}"
                              for c in GRAPH_CASES])
def test_graph_replays_match_eager(case):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L
    from synth import compact_pool

    seed, M, d_in, d_out, n, r_max, mode, compact = case
    log(f"graph: {case}")
    ranks = None
    if compact:
        ranks = (8 * np.random.default_rng(seed).integers(1, r_max // 8 + 1, size=n)).astype(np.int32)
    w = random_case(seed, M, d_in, d_out, n, r_max, ranks=ranks, base_frac=0.2)
    dw = to_device(w)
    p = dw.projs[0]
    r = w.r_max
    y = torch.empty((M, p.d_out), dtype=torch.bfloat16, device="cuda")
    ws, nb = L.workspace(M, p.d_in, p.d_out, r, n)
    if compact:
        wb = w.as_bf16().projections[0]
        A_c, B_c, off, rows = compact_pool(wb.A, wb.B, w.ranks)
        A_c, B_c, off = bf16_dev(A_c), bf16_dev(B_c), torch.from_numpy(off).cuda()

    def call():
        if compact:
            L.lora_linear_compact(p.x, p.W, A_c, B_c, dw.scale, dw.ranks, off, rows, dw.ids, M,
                                  p.d_in, p.d_out, r, n, None, y, L.LORA_BF16, mode, ws, nb)
        else:
            L.lora_linear(p.x, p.W, p.A, p.B, dw.scale, dw.ranks, dw.ids, M, p.d_in, p.d_out, r, n,
                          None, y, L.LORA_BF16, mode, ws, nb)

    call()
    torch.cuda.synchronize()
    eager = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        y.fill_(0)
        ws.fill_(0xAB)  # scribble over the workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))


def test_graph_replays_match_eager_multi():
    """lora_linear_multi (two projections of one x, merged stream-K launches) in a graph."""
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    M, d_in, d_out, n, r_max = 300, 4096, 2048, 24, 16
    log(f"graph: lora_linear_multi M={M} {d_in}x{d_out} two projections")
    w0 = random_case(101, M, d_in, d_out, n, r_max, base_frac=0.2)
    w1 = random_case(102, M, d_in, d_out, n, r_max, ids=w0.ids, ranks=w0.ranks)
    d0, d1 = to_device(w0), to_device(w1)
    p0, p1 = d0.projs[0], d1.projs[0]
    ys = [torch.empty((M, d_out), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    nb = L.lora_workspace_bytes_multi(M, d_in, d_out, r_max, n, 2)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def call():
        L.lora_linear_multi(p0.x, [p0.W, p1.W], [p0.A, p1.A], [p0.B, p1.B], d0.scale, d0.ranks,
                            d0.ids, M, d_in, d_out, r_max, n, None, ys, L.LORA_BF16,
                            L.LORA_MODE_DECODE, ws, nb)

    call()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for y in ys:
            y.fill_(0)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), f"replay {rep}"
        call()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16))
