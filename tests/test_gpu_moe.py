"""lora_moe_linear (routed experts, each with its own base weight and per-adapter pairs) against
the CPU oracle's MoE layer, through the C ABI.

- parity over shapes: several K splits and row blocks per expert, ragged column tiles,
  r_max 8 .. 64 (a multiple of 8, true ranks below it), empty slots, tokens without an
  adapter, per-adapter alpha, skewed routing, pools larger than the batch, bf16 and fp32 y;
- the adapter term alone (a call minus the same call with every id -1) against the oracle's,
  so the LoRA delta is held to the rule on its own scale;
- the decode MoE batch at full size (64 tokens, top-4 of 32 experts of 2880 x 2880, 8 adapters
  of rank 16), every row;
- exact properties: empty slots are zero rows, rows without an adapter equal a base-only
  call bit for bit, doubling the routing weights doubles y exactly (fp32 y), graph replays
  equal the eager call; checked mode reports bad expert and adapter ids.
Parity rule as in test_gpu_parity.
"""

import numpy as np
import pytest

import oracle
from synth import make_moe_workload, moe_case

from .gpu_util import assert_parity, bf16_host, log

pytestmark = pytest.mark.gpu


class DevMoe:
    def __init__(self, w, topk_w=True):
        import torch

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

        self.w = w
        self.x, self.W, self.A, self.B = bf(w.x), bf(w.W), bf(w.A), bf(w.B)
        self.ids = torch.from_numpy(w.ids.astype(np.int32)).cuda()
        self.ranks = torch.from_numpy(w.ranks.astype(np.int32)).cuda()
        self.scale = torch.from_numpy((w.alpha.astype(np.float32) / w.ranks.astype(np.float32))
                                      .astype(np.float32)).cuda()
        self.topk = torch.from_numpy(w.topk_ids.astype(np.int32)).cuda()
        self.topk_w = torch.from_numpy(w.topk_w.astype(np.float32)).cuda() if topk_w else None


def moe_call(d, y_f32=False, ids=None, topk_w="default", mode=1, ws=None):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    w = d.w
    y = torch.empty((w.M, w.top_k, w.d_out), dtype=torch.float32 if y_f32 else torch.bfloat16,
                    device="cuda")
    if ws is None:
        ws = L.moe_workspace(w.M, w.top_k, w.n_experts, w.d_in, w.d_out, w.r_max, w.n_adapters)
    L.lora_moe_linear(d.x, d.W, d.A, d.B, d.scale, d.ranks, d.ids if ids is None else ids, d.topk,
                      d.topk_w if topk_w == "default" else topk_w, w.M, w.top_k, w.n_experts,
                      w.d_in, w.d_out, w.r_max, w.n_adapters, y,
                      L.LORA_F32 if y_f32 else L.LORA_BF16, mode, ws[0], ws[1])
    torch.cuda.synchronize()
    return y.cpu().numpy() if y_f32 else bf16_host(y)


def ref_of(w, ids=None, topk_w="default"):
    return oracle.moe_lora_linear(w.x, w.W, w.A, w.B, w.alpha, w.ranks,
                                  w.ids if ids is None else ids, w.topk_ids,
                                  w.topk_w if topk_w == "default" else topk_w)


CASES = [
    # seed, M, top_k, E, d_in, d_out, n, r_max, empty, zipf
    (501, 9, 2, 4, 128, 64, 3, 8, 0.2, 0.0),
    (502, 33, 4, 8, 256, 200, 5, 16, 0.1, 0.0),     # ragged column tile
    (503, 17, 8, 16, 512, 136, 40, 24, 0.1, 0.0),   # r_max 24 (bucket 32), pool > batch
    (504, 100, 2, 3, 192, 64, 7, 64, 0.0, 0.0),     # ~67 pairs per expert: three row blocks
    (505, 5, 1, 1, 1024, 1032, 2, 32, 0.0, 0.0),    # one expert, many K splits
    (506, 64, 4, 32, 768, 512, 8, 16, 0.05, 1.2),   # skewed routing: some experts idle
    (507, 200, 6, 12, 320, 392, 600, 8, 0.1, 0.0),  # 600 adapters: the bitmap spans words
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}-M{c[1]}k{c[2]}E{c[3]}-{c[4]}x{c[5]}-r{c[7]}"
                                             for c in CASES])
@pytest.mark.parametrize("y_f32", [False, True], ids=["bf16", "f32"])
def test_moe_random_shapes(case, y_f32):
    seed, M, top_k, E, d_in, d_out, n, r_max, empty, zipf = case
    log(f"moe: {case} y_f32={y_f32}")
    w = moe_case(seed, M, top_k, E, d_in, d_out, n, r_max, base_frac=0.2, empty_frac=empty,
                 zipf_s=zipf)
    d = DevMoe(w)
    y = moe_call(d, y_f32=y_f32)
    ref = ref_of(w)
    assert_parity(y, ref, f"moe {case}")
    empty_slots = w.topk_ids < 0
    assert not np.any(y[empty_slots]), "empty slots must be zero rows"


@pytest.mark.parametrize("case", CASES[:4] + CASES[5:], ids=[f"s{c[0]}" for c in CASES[:4] + CASES[5:]])
def test_moe_delta_alone(case):
    """The adapter term on its own scale: (call) - (call with every id -1) vs the oracle's."""
    import torch

    seed, M, top_k, E, d_in, d_out, n, r_max, empty, zipf = case
    w = moe_case(seed, M, top_k, E, d_in, d_out, n, r_max, base_frac=0.2, empty_frac=empty,
                 zipf_s=zipf)
    w.ids[0] = -1  # at least one token without an adapter
    d = DevMoe(w)
    base = np.full(M, -1, np.int32)
    yf = moe_call(d, y_f32=True)
    yb = moe_call(d, y_f32=True, ids=torch.from_numpy(base).cuda())
    ref = ref_of(w)
    ref_b = ref_of(w, ids=base)
    mr, ml = assert_parity(yf - yb, ref - ref_b, f"moe delta {case}")
    log(f"  delta: max_rel={mr:.2e} mean_rel={ml:.2e}")
    no_adapter = w.ids < 0
    assert no_adapter.any()
    assert np.array_equal(yf[no_adapter], yb[no_adapter]), "rows without an adapter = base-only call"


def test_moe_decode_full_size():
    """The decode MoE batch: 64 tokens, top-4 of 32 experts of 2880 x 2880, 8 adapters of rank
    16: every (token, slot) row, and the delta alone."""
    import torch

    w = make_moe_workload()
    log(f"moe: {w.name}")
    d = DevMoe(w)
    y = moe_call(d)
    ref = ref_of(w)
    mr, ml = assert_parity(y, ref, "moe decode full size")
    log(f"  y: max_rel={mr:.2e} mean_rel={ml:.2e}")
    base = np.full(w.M, -1, np.int32)
    yf = moe_call(d, y_f32=True)
    yb = moe_call(d, y_f32=True, ids=torch.from_numpy(base).cuda())
    mr, ml = assert_parity(yf - yb, ref - ref_of(w, ids=base), "moe decode delta")
    log(f"  delta: max_rel={mr:.2e} mean_rel={ml:.2e}")


def test_moe_routing_weight_exact():
    """y is the routed row times its weight, applied last: doubling topk_w doubles y exactly
    (fp32 y), and without weights every slot is its expert's unweighted row."""
    import torch

    w = moe_case(510, 40, 4, 8, 256, 264, 6, 16, base_frac=0.2, empty_frac=0.1)
    d = DevMoe(w)
    y1 = moe_call(d, y_f32=True)
    y2 = moe_call(d, y_f32=True, topk_w=2 * d.topk_w)
    assert np.array_equal(y2, 2 * y1)
    y0 = moe_call(d, y_f32=True, topk_w=None)
    assert_parity(y0, ref_of(w, topk_w=None), "moe unweighted")
    nz = w.topk_ids >= 0
    ratio_ok = np.allclose(y1[nz], w.topk_w[nz][:, None] * y0[nz], rtol=1e-6, atol=0)
    assert ratio_ok
    torch.cuda.synchronize()


def test_moe_graph_replays_and_checks():
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    w = moe_case(520, 48, 4, 16, 512, 520, 10, 16, base_frac=0.2, empty_frac=0.05)
    d = DevMoe(w)
    ws = L.moe_workspace(w.M, w.top_k, w.n_experts, w.d_in, w.d_out, w.r_max, w.n_adapters)
    y = torch.empty((w.M, w.top_k, w.d_out), dtype=torch.bfloat16, device="cuda")

    def call(mode=1, ids=None, topk=None):
        L.lora_moe_linear(d.x, d.W, d.A, d.B, d.scale, d.ranks, d.ids if ids is None else ids,
                          d.topk if topk is None else topk, d.topk_w, w.M, w.top_k, w.n_experts,
                          w.d_in, w.d_out, w.r_max, w.n_adapters, y, L.LORA_BF16, mode, ws[0],
                          ws[1])

    call()
    torch.cuda.synchronize()
    eager = y.clone()
    assert_parity(bf16_host(eager), ref_of(w), "moe eager")
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
        ws[0].fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        call()
        torch.cuda.synchronize()
    # checked mode: a bad expert id or adapter id is reported and nothing is enqueued
    bad_topk = w.topk_ids.copy()
    bad_topk[3, 1] = w.n_experts
    y.fill_(0)
    with pytest.raises(L.LoraError) as e:
        call(mode=1 | L.LORA_MODE_CHECKED, topk=torch.from_numpy(bad_topk).cuda())
    assert e.value.status == 8
    bad_ids = w.ids.copy()
    bad_ids[7] = w.n_adapters
    with pytest.raises(L.LoraError) as e:
        call(mode=L.LORA_MODE_CHECKED, ids=torch.from_numpy(bad_ids).cuda())
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert not torch.any(y.view(torch.int16)), "a rejected call enqueues nothing"
    call(mode=1 | L.LORA_MODE_CHECKED)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), eager.view(torch.int16))
    # unchecked: an expert id past the last is an empty slot (zero row), an adapter id past
    # the last adds no adapter term
    call(topk=torch.from_numpy(bad_topk).cuda())
    torch.cuda.synchronize()
    assert not torch.any(y[3, 1].view(torch.int16))
