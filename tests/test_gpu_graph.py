"""lora_linear captured in a HIP graph: every replay equals the eager result, bit for bit.

The graph is replayed several times with eager work of the program and synchronisations in
between (the library records no memset nodes; this checks that replays after the first stay
correct).
"""

import numpy as np
import pytest

from synth import random_case

from .gpu_util import log, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [1, 2], ids=["decode", "prefill"])
def test_graph_replays_match_eager(mode):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    log(f"graph: mode {mode}")
    w = random_case(90 + mode, 96, 1024, 768, 12, 16, base_frac=0.2)
    dw = to_device(w)
    p = dw.projs[0]
    M, n, r = w.M, w.n_adapters, w.r_max
    y = torch.empty((M, p.d_out), dtype=torch.bfloat16, device="cuda")
    ws, nb = L.workspace(M, p.d_in, p.d_out, r, n)

    def call():
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
