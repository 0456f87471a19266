"""lora_linear_fp8w (base weight as OCP E4M3 fp8 codes with per-column scales, bf16 adapters)
against the CPU oracle's fp8 layer, through the C ABI.

- every non-NaN code decoded by the kernel, bit for bit: a one-hot row of x with unit scales
  turns each output column into one code's value (a single exact product);
- parity over shapes (every decode split plan, ragged columns, odd r_max, per-adapter alpha)
  and on the decode q_proj batch (64 x 4096 x 4096, 32 adapters) at full size, every row;
- rows with id -1 bit-identical to a base-only call; graph replays equal the eager call.
Parity rule as in test_gpu_parity.
"""

import numpy as np
import pytest

import oracle
from synth import fp8_base, make_workload, random_case

from .gpu_util import assert_parity, bf16_host, log, to_device

pytestmark = pytest.mark.gpu


def fp8_call(dw, W8, w_scale, y_f32=False, ids=None, mode=1, segs=None):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    p = dw.projs[0]
    M = dw.M
    y = torch.empty((M, p.d_out), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    ws, nb = L.workspace(M, p.d_in, p.d_out, dw.w.r_max, dw.n)
    L.lora_linear_fp8w(p.x, W8, w_scale, p.A, p.B, dw.scale, dw.ranks, dw.ids if ids is None else ids,
                       M, p.d_in, p.d_out, dw.w.r_max, dw.n, segs, y,
                       L.LORA_F32 if y_f32 else L.LORA_BF16, mode, ws, nb)
    torch.cuda.synchronize()
    return y.cpu().numpy() if y_f32 else bf16_host(y)


def dev_fp8(W8, w_scale):
    import torch

    return torch.from_numpy(np.ascontiguousarray(W8)).cuda(), torch.from_numpy(w_scale).cuda()


def test_every_code_decodes_exactly():
    """x = e_k (one row), unit scales, id -1: y[0, c] = dec(W8[c, k]) with no rounding."""
    import torch

    d_in, d_out, k = 256, 256, 77
    w = random_case(400, 1, d_in, d_out, 2, 8, ids=[-1])
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0  # the two NaN codes
    rng = np.random.default_rng(400)
    W8 = rng.integers(0, 256, size=(d_out, d_in)).astype(np.uint8)
    W8[W8 == 0x7F] = 0
    W8[W8 == 0xFF] = 0
    W8[:, k] = codes
    wx = w.projections[0]
    wx.x[:] = 0
    wx.x[0, k] = 0x3F80  # bf16 1.0
    dw = to_device(w)
    W8d, sd = dev_fp8(W8, np.ones(d_out, np.float32))
    y = fp8_call(dw, W8d, sd, y_f32=True, ids=torch.tensor([-1], dtype=torch.int32, device="cuda"))
    ref = oracle.fp8_e4m3_decode(codes)
    assert np.array_equal(y[0], ref)  # (code 0x80, -0, sums to +0 like the oracle's layer)
    p = w.projections[0]
    assert np.array_equal(y, oracle.lora_linear_fp8w(p.x, W8, np.ones(d_out, np.float32), p.A, p.B,
                                                     w.alpha, w.ranks, w.ids))


CASES = [
    # seed, M, d_in, d_out, n, r_max, base_frac
    (401, 1, 128, 64, 3, 8, 0.0),
    (402, 17, 1024, 264, 5, 16, 0.2),
    (403, 64, 4096, 1032, 33, 16, 0.1),
    (404, 100, 2048, 520, 40, 12, 0.1),     # odd r_max: padded stride below the bucket
    (405, 128, 1088, 776, 300, 32, 0.2),    # pool larger than the batch
    (406, 200, 512, 4104, 9, 64, 0.3),      # 129-256 rows
    (407, 256, 11008, 256, 70, 16, 0.1),    # long K
    (408, 33, 192, 8, 4, 5, 0.25),          # one ragged column tile, a short split
    # up to 128 rows with r_max a rank bucket, the shrink runs as adapter tiles of the fp8
    # GEMM's launch: r_max 64 with adapters numbered by id (64-row tiles) and by first use
    # (32-row tiles)
    (411, 48, 512, 264, 20, 64, 0.1),
    (412, 20, 256, 136, 40, 64, 0.2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}-M{c[1]}-{c[2]}x{c[3]}-r{c[5]}" for c in CASES])
@pytest.mark.parametrize("y_f32", [False, True], ids=["bf16", "f32"])
def test_fp8_random_shapes(case, y_f32):
    seed, M, d_in, d_out, n, r_max, base_frac = case
    log(f"fp8: {case} y_f32={y_f32}")
    w = random_case(seed, M, d_in, d_out, n, r_max, base_frac=base_frac)
    W8, w_scale = fp8_base(seed, d_in, d_out)
    dw = to_device(w)
    y = fp8_call(dw, *dev_fp8(W8, w_scale), y_f32=y_f32)
    p = w.projections[0]
    ref = oracle.lora_linear_fp8w(p.x, W8, w_scale, p.A, p.B, w.alpha, w.ranks, w.ids)
    assert_parity(y, ref, f"fp8 {case}")


def test_fp8_uniform_codes():
    """Every code (subnormals, +-448) drawn uniformly: large, spread-out base values."""
    w = random_case(409, 40, 512, 264, 6, 16, base_frac=0.1)
    W8, w_scale = fp8_base(409, 512, 264, uniform_codes=True)
    dw = to_device(w)
    y = fp8_call(dw, *dev_fp8(W8, w_scale), y_f32=True)
    p = w.projections[0]
    ref = oracle.lora_linear_fp8w(p.x, W8, w_scale, p.A, p.B, w.alpha, w.ranks, w.ids)
    assert_parity(y, ref, "fp8 uniform codes")


def test_fp8_decode_qproj_full_size():
    """The decode q_proj batch (64 x 4096 -> 4096, 32 adapters of rank 16) with its base
    weight stored as fp8: every row, and the delta alone against the oracle's delta."""
    import torch

    w = make_workload(2).as_bf16()
    W8, w_scale = fp8_base(w.seed, 4096, 4096)
    dw = to_device(w)
    W8d, sd = dev_fp8(W8, w_scale)
    log("fp8: decode q_proj 64 x 4096 x 4096")
    y = fp8_call(dw, W8d, sd)
    p = w.projections[0]
    ref = oracle.lora_linear_fp8w(p.x, W8, w_scale, p.A, p.B, w.alpha, w.ranks, w.ids)
    mr, ml = assert_parity(y, ref, "fp8 decode q_proj")
    log(f"  y: max_rel={mr:.2e} mean_rel={ml:.2e}")
    base = np.full(w.M, -1, np.int32)
    yf = fp8_call(dw, W8d, sd, y_f32=True)
    yb = fp8_call(dw, W8d, sd, y_f32=True, ids=torch.from_numpy(base).cuda())
    ref_b = oracle.lora_linear_fp8w(p.x, W8, w_scale, p.A, p.B, w.alpha, w.ranks, base)
    mr, ml = assert_parity(yf - yb, ref - ref_b, "fp8 decode q_proj delta")
    log(f"  delta: max_rel={mr:.2e} mean_rel={ml:.2e}")


@pytest.mark.parametrize("M", [64, 200])
def test_fp8_base_rows_bit_identical(M):
    import torch

    w = random_case(410 + M, M, 1024, 520, 12, 16, base_frac=0.3)
    W8, w_scale = fp8_base(410, 1024, 520)
    dw = to_device(w)
    W8d, sd = dev_fp8(W8, w_scale)
    y = fp8_call(dw, W8d, sd)
    yb = fp8_call(dw, W8d, sd, ids=torch.from_numpy(np.full(M, -1, np.int32)).cuda())
    base = w.ids == -1
    assert base.any() and np.array_equal(y[base], yb[base])
    assert not np.array_equal(y[~base], yb[~base])


def test_fp8_graph_replays_and_checks():
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    w = random_case(420, 96, 1024, 768, 12, 16, base_frac=0.2)
    W8, w_scale = fp8_base(420, 1024, 768)
    dw = to_device(w)
    W8d, sd = dev_fp8(W8, w_scale)
    p = dw.projs[0]
    M, n, r = w.M, w.n_adapters, w.r_max
    y = torch.empty((M, p.d_out), dtype=torch.bfloat16, device="cuda")
    ws, nb = L.workspace(M, p.d_in, p.d_out, r, n)

    def call():
        L.lora_linear_fp8w(p.x, W8d, sd, p.A, p.B, dw.scale, dw.ranks, dw.ids, M, p.d_in, p.d_out,
                           r, n, None, y, L.LORA_BF16, 1, ws, nb)

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
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        call()
        torch.cuda.synchronize()
    # checked mode: a bad id is reported, nothing enqueued
    bad = w.ids.copy()
    bad[5] = n
    with pytest.raises(L.LoraError) as e:
        L.lora_linear_fp8w(p.x, W8d, sd, p.A, p.B, dw.scale, dw.ranks,
                           torch.from_numpy(bad).cuda(), M, p.d_in, p.d_out, r, n, None, y,
                           L.LORA_BF16, 1 | L.LORA_MODE_CHECKED, ws, nb)
    assert e.value.status == 8
    with pytest.raises(L.LoraError) as e:  # prefill is not served by the fp8 base
        L.lora_linear_fp8w(p.x, W8d, sd, p.A, p.B, dw.scale, dw.ranks, dw.ids, M, p.d_in, p.d_out,
                           r, n, None, y, L.LORA_BF16, 2, ws, nb)
    assert e.value.status == 9
