"""The CPU oracle against the pins of tests/oracle_pins.py and the pages' worked example.

CPU only.  Sources: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to) and
"Serving Many LoRA Adapters From One Base Model" (ai-tldr.dev); see oracle_pins.py.
"""

import os

import numpy as np
import pytest

from synth import make_workload, pool_param_count, random_case

from .oracle_pins import ALL_PINS, Orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(Orc(oracle_lib))


def test_golden_adapter_size():
    """Pool size of a rank-16 q/k/v/o adapter, 32 layers, hidden 4096: the printed line.

    From "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU", section "How much memory
    does one LoRA adapter actually cost?".  The count comes from the stacked-pool shapes
    A[n, d_in, r] and B[n, r, d_out] used by the generator and the library.
    """
    with open(os.path.join(GOLDEN, "lora_bytes.txt")) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    params_line, printed = lines
    cfg = dict(kv.split("=") for kv in params_line.split())
    hidden, layers, rank = int(cfg["hidden"]), int(cfg["layers"]), int(cfg["rank"])
    targets = cfg["targets"].split(",")
    nbytes_per = int(cfg["dtype_bytes"])
    w = random_case(0, 1, 8, 8, 1, 8, storage="bf16")  # shapes only: one adapter per matrix
    per_matrix = pool_param_count(1, hidden, hidden, rank)
    params = per_matrix * len(targets) * layers
    assert params == 16_777_216 and params * nbytes_per == 33_554_432
    assert f"{params / 1e6:.1f}M params, {params * nbytes_per / 2 ** 20:.1f} MiB" == printed
    # the generator's pool arrays hold exactly rank * (d_in + d_out) elements per adapter
    p = w.projections[0]
    assert p.A.size + p.B.size == pool_param_count(1, 8, 8, 8)


def test_mlp_pool_size():
    """Config 5's pool: 1024 adapters of rank 16 on a 4096 <-> 11008 projection."""
    params = pool_param_count(1024, 4096, 11008, 16)
    assert params == 1024 * 16 * (4096 + 11008)
    assert params * 2 / 2 ** 20 == pytest.approx(472.0, abs=0.05)


def test_generated_pool_matches_formula():
    w = make_workload(1)
    p = w.projections[0]
    assert p.A.size + p.B.size == pool_param_count(4, 256, 256, 8)


def test_bad_ids_raise(oracle_lib):
    w = random_case(3, 8, 16, 16, 2, 8, storage="f32")
    p = w.projections[0]
    for bad in (2, -2, 99):
        ids = w.ids.copy()
        ids[3] = bad
        with pytest.raises(ValueError):
            oracle_lib.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, ids)
        with pytest.raises(ValueError):
            oracle_lib.build_segments(ids, 2, 16)
        with pytest.raises(ValueError):
            oracle_lib.lora_shrink(p.x, p.A, ids)


def test_empty_batch(oracle_lib):
    w = random_case(4, 0, 16, 24, 2, 8, storage="f32")
    p = w.projections[0]
    y = oracle_lib.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
    assert y.shape == (0, 24)
    seg = oracle_lib.build_segments(w.ids, 2, 16)
    assert list(seg["meta"]) == [0, 0, 0, 0] and list(seg["offsets"]) == [0, 0, 0]


def test_steps_compose(oracle_lib):
    """shrink then expand on top of the base-only result reproduces the whole layer."""
    w = make_workload(1).as_bf16()
    p = w.projections[0]
    y = oracle_lib.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
    base = oracle_lib.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks,
                                  np.full(w.M, -1, np.int32))
    t = oracle_lib.lora_shrink(p.x, p.A, w.ids)
    y2 = oracle_lib.lora_expand(t, p.B, w.alpha, w.ranks, w.ids, base)
    assert np.array_equal(y, y2)
