"""The layer at the largest sizes the ABI accepts: LORA_MAX_ROWS rows and LORA_MAX_ADAPTERS
adapters in one call, in both modes, with the smallest dimensions (d_in = d_out = r_max = 8)
so that the oracle still checks every output element.  Every adapter is touched about 230
times, so prefill tiles hold hundreds of short adapter runs; the segments are checked bit for
bit at that size too."""

import numpy as np
import pytest

import oracle
from synth import random_case

from .gpu_util import assert_parity, gpu_linear, gpu_segments, log, to_device

pytestmark = pytest.mark.gpu

_CASE = {}


def max_case():
    from rank_adapter_gemm_sgmv_amd import lora as L

    if not _CASE:
        w = random_case(77, L.LORA_MAX_ROWS, 8, 8, L.LORA_MAX_ADAPTERS, 8, base_frac=0.1)
        _CASE["w"] = w
        _CASE["dw"] = to_device(w)
        p = w.projections[0]
        _CASE["ref"] = oracle.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
    return _CASE["w"], _CASE["dw"], _CASE["ref"]


@pytest.mark.parametrize("mode", [1, 2], ids=["decode", "prefill"])
def test_max_rows_and_adapters(mode):
    w, dw, ref = max_case()
    log(f"limits: M={w.M} n={w.n_adapters} mode {mode}")
    y = gpu_linear(dw, 0, mode)
    assert_parity(y, ref, f"max sizes, mode {mode}")
    base = w.ids == -1
    assert base.any() and (~base).any()


def test_max_rows_segments():
    w, _, _ = max_case()
    log(f"limits: segments M={w.M} n={w.n_adapters}")
    got, _, _ = gpu_segments(w.ids, w.n_adapters)
    ref = oracle.build_segments(w.ids, w.n_adapters, 16)
    for key in ("perm", "offsets", "seg_adapter", "tiles", "meta"):
        assert np.array_equal(got[key], ref[key]), key
