"""lora_linear_noalloc (the library's own device scratch, no workspace argument) against
lora_linear with a caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, bit for bit equal (the same kernels run); a call too large for the scratch is
rejected; a HIP graph of the call replays to the eager result."""

import numpy as np
import pytest

import oracle
from synth import random_case

from .gpu_util import assert_parity, bf16_host, log, to_device

pytestmark = pytest.mark.gpu


def _both(w, mode):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    dw = to_device(w)
    p = dw.projs[0]
    M, n, r = w.M, w.n_adapters, w.r_max
    y_ws = torch.empty((M, p.d_out), dtype=torch.bfloat16, device="cuda")
    y_na = torch.full((M, p.d_out), 5.0, dtype=torch.bfloat16, device="cuda")
    ws, nb = L.workspace(M, p.d_in, p.d_out, r, n)
    L.lora_linear(p.x, p.W, p.A, p.B, dw.scale, dw.ranks, dw.ids, M, p.d_in, p.d_out, r, n, None,
                  y_ws, L.LORA_BF16, mode, ws, nb)
    L.lora_linear_noalloc(p.x, p.W, p.A, p.B, dw.scale, dw.ranks, dw.ids, M, p.d_in, p.d_out, r, n,
                          None, y_na, L.LORA_BF16, mode)
    torch.cuda.synchronize()
    return y_ws, y_na, dw


def test_noalloc_matches_lora_linear_twice():
    big = random_case(301, 64, 4096, 4096, 32, 16, base_frac=0.1)
    small = random_case(302, 17, 512, 264, 5, 12, base_frac=0.2)
    for w, mode in ((big, 1), (small, 2)):
        log(f"noalloc: M={w.M} {w.projections[0].d_in}x{w.projections[0].d_out} mode {mode}")
        y_ws, y_na, _ = _both(w, mode)
        import torch

        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16))
        p = w.projections[0]
        ref = oracle.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
        assert_parity(bf16_host(y_na), ref, f"noalloc M={w.M}")


def test_noalloc_rejects_calls_beyond_its_scratch():
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    M, d_in, d_out, n = 512, 4096, 11008, 64
    assert L.lora_workspace_bytes(M, d_in, d_out, 16, n) > L.LORA_NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.LoraError) as e:
        L.lora_linear_noalloc(dummy, dummy, dummy, dummy, dummy, None, dummy, M, d_in, d_out, 16, n,
                              None, dummy, L.LORA_BF16, 1)
    assert e.value.status == 5


def test_noalloc_in_a_graph():
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    w = random_case(303, 96, 1024, 768, 12, 16, base_frac=0.2)
    dw = to_device(w)
    p = dw.projs[0]
    M, n, r = w.M, w.n_adapters, w.r_max
    y = torch.empty((M, p.d_out), dtype=torch.bfloat16, device="cuda")

    def call():
        L.lora_linear_noalloc(p.x, p.W, p.A, p.B, dw.scale, dw.ranks, dw.ids, M, p.d_in, p.d_out, r,
                              n, None, y, L.LORA_BF16, 1)

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
    for rep in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        call()
        torch.cuda.synchronize()
