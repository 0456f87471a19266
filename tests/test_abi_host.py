"""The C-ABI library on the host: it loads without a GPU, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments before enqueueing anything.

CPU only: no call here reaches a kernel launch.  Fake non-NULL device addresses are used
only where validation fails before any pointer is touched.
"""

import os
import re

import pytest

from rank_adapter_gemm_sgmv_amd import lora as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "lora.h")

FAKE = 1 << 20  # 16/256-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    for name in names:
        assert hasattr(L.library(), name), name


def test_status_strings():
    for code, name in L.STATUS.items():
        assert L.lora_status_string(code).startswith(name)
    assert "unknown" in L.lora_status_string(99)


def test_max_tiles():
    assert L.lora_max_tiles(0, 4) == 0
    assert L.lora_max_tiles(16, 4) == 4 + 1
    assert L.lora_max_tiles(512, 1024) == 512 + 32
    assert L.lora_max_tiles(4096, 8) == 8 + 256


def test_workspace_bytes():
    assert L.lora_workspace_bytes(0, 4096, 4096, 16, 32) == 0
    assert L.lora_workspace_bytes(64, 4096, 4096, 65, 32) == 0  # bad rank
    assert L.lora_workspace_bytes(64, 4096, 4096, 0, 32) == 0
    # any r_max in [1, 64] is sized at its rank bucket
    assert L.lora_workspace_bytes(64, 4096, 4096, 12, 32) == L.lora_workspace_bytes(64, 4096, 4096, 16, 32)
    assert L.lora_workspace_bytes(64, 4096, 4096, 1, 32) == L.lora_workspace_bytes(64, 4096, 4096, 8, 32)
    assert L.lora_workspace_bytes(64, 4095, 4096, 16, 32) == 0  # d_in not a multiple of 8
    b = L.lora_workspace_bytes(64, 4096, 4096, 16, 32)
    assert b > 0 and b % 256 == 0
    # grows with rows, rank and adapters
    assert L.lora_workspace_bytes(128, 4096, 4096, 16, 32) > b
    assert L.lora_workspace_bytes(64, 4096, 4096, 64, 32) > b
    assert L.lora_workspace_bytes(64, 4096, 4096, 16, 4096) > b


def _linear(**over):
    args = dict(x=FAKE, W=FAKE, A=FAKE, B=FAKE, scale=FAKE, ranks=None, ids=FAKE, M=64, d_in=4096,
                d_out=4096, r_max=16, n_adapters=32, segs=None, y=FAKE, y_dtype=L.LORA_BF16,
                mode=L.LORA_MODE_DECODE, ws=FAKE, ws_bytes=0, stream=0)
    args.update(over)
    return L.lora_linear(**args)


@pytest.mark.parametrize("over,code", [
    (dict(M=-1), 2), (dict(M=L.LORA_MAX_ROWS + 1), 2), (dict(d_in=12), 2), (dict(d_out=0), 2),
    (dict(n_adapters=0), 2), (dict(n_adapters=L.LORA_MAX_ADAPTERS + 1), 2),
    (dict(r_max=65), 3), (dict(r_max=128), 3), (dict(r_max=0), 3), (dict(r_max=-8), 3),
    (dict(y_dtype=5), 6), (dict(mode=7), 9), (dict(mode=0x103), 9), (dict(mode=0x200), 9),
    (dict(x=None), 1), (dict(W=None), 1), (dict(ids=None), 1), (dict(ws=None), 1),
    (dict(x=FAKE + 2), 4), (dict(y=FAKE + 8), 4), (dict(ws=FAKE + 16), 4),
    (dict(ws_bytes=1024), 5),
])
def test_linear_rejects(over, code):
    with pytest.raises(L.LoraError) as e:
        _linear(**over)
    assert e.value.status == code


def test_linear_empty_batch_is_noop():
    _linear(M=0, x=None, y=None, ws=None)  # M = 0 returns LORA_OK, nothing enqueued


def test_build_segments_rejects():
    seg = L.lora_segments_t(FAKE, FAKE, FAKE, FAKE, FAKE)
    with pytest.raises(L.LoraError) as e:
        L.lora_build_segments(None, 10, 4, seg, stream=0)
    assert e.value.status == 1
    with pytest.raises(L.LoraError) as e:
        L.lora_build_segments(FAKE, 10, 0, seg, stream=0)
    assert e.value.status == 2
    with pytest.raises(L.LoraError) as e:
        L.lora_build_segments(FAKE, 10, 4, L.lora_segments_t(FAKE, None, FAKE, FAKE, FAKE), stream=0)
    assert e.value.status == 1
    with pytest.raises(L.LoraError) as e:
        L.lora_build_segments(FAKE + 2, 10, 4, seg, stream=0)
    assert e.value.status == 4
    L.lora_build_segments(None, 0, 4, seg, stream=0)  # empty batch: no-op


def test_shrink_expand_reject():
    seg = L.lora_segments_t(FAKE, FAKE, FAKE, FAKE, FAKE)
    with pytest.raises(L.LoraError) as e:
        L.lora_shrink(FAKE, FAKE, None, 64, 4096, 16, 32, seg, FAKE, FAKE, 16, stream=0)
    assert e.value.status == 5
    with pytest.raises(L.LoraError) as e:
        L.lora_shrink(FAKE, FAKE, None, 64, 4096, 65, 32, seg, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.status == 3
    with pytest.raises(L.LoraError) as e:
        L.lora_expand(FAKE, FAKE, None, None, 64, 4096, 16, 32, seg, FAKE, 0, stream=0)
    assert e.value.status == 1
    with pytest.raises(L.LoraError) as e:
        L.lora_expand(FAKE, FAKE, FAKE, None, 64, 4096, 16, 32, seg, FAKE, 3, stream=0)
    assert e.value.status == 6


def _compact(**over):
    ws = L.lora_workspace_bytes(64, 4096, 4096, 64, 32)
    args = dict(x=FAKE, W=FAKE, A=FAKE, B=FAKE, scale=FAKE, ranks=FAKE, rank_offsets=FAKE,
                pool_rows=256, ids=FAKE, M=64, d_in=4096, d_out=4096, r_max=64, n_adapters=32,
                segs=None, y=FAKE, y_dtype=L.LORA_BF16, mode=L.LORA_MODE_DECODE, ws=FAKE,
                ws_bytes=ws, stream=0)
    args.update(over)
    return L.lora_linear_compact(**args)


@pytest.mark.parametrize("over,code", [
    (dict(ranks=None), 1), (dict(rank_offsets=None), 1), (dict(rank_offsets=FAKE + 2), 4),
    (dict(pool_rows=0), 2), (dict(pool_rows=32 * 64 + 1), 2),
    # the checks lora_linear makes come first
    (dict(r_max=0), 3), (dict(ws_bytes=1024), 5), (dict(x=None), 1),
])
def test_linear_compact_rejects(over, code):
    with pytest.raises(L.LoraError) as e:
        _compact(**over)
    assert e.value.status == code


def test_linear_compact_empty_batch_is_noop():
    _compact(M=0, x=None, y=None, ws=None)


def test_shrink_expand_compact_reject():
    seg = L.lora_segments_t(FAKE, FAKE, FAKE, FAKE, FAKE)
    ws = 1 << 30
    with pytest.raises(L.LoraError) as e:  # ranks and offsets are required
        L.lora_shrink_compact(FAKE, FAKE, None, FAKE, 64, 64, 4096, 16, 32, seg, FAKE, FAKE, ws, stream=0)
    assert e.value.status == 1
    with pytest.raises(L.LoraError) as e:
        L.lora_shrink_compact(FAKE, FAKE, FAKE, None, 64, 64, 4096, 16, 32, seg, FAKE, FAKE, ws, stream=0)
    assert e.value.status == 1
    with pytest.raises(L.LoraError) as e:  # pool larger than n * r_max
        L.lora_shrink_compact(FAKE, FAKE, FAKE, FAKE, 32 * 16 + 1, 64, 4096, 16, 32, seg, FAKE, FAKE,
                              ws, stream=0)
    assert e.value.status == 2
    with pytest.raises(L.LoraError) as e:
        L.lora_expand_compact(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 4096, 16, 32, seg, FAKE, 0, stream=0)
    assert e.value.status == 2
    with pytest.raises(L.LoraError) as e:
        L.lora_expand_compact(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 64, 64, 4096, 16, 32, seg, FAKE, 0,
                              stream=0)
    assert e.value.status == 4
    # M = 0: no-op after the argument checks
    L.lora_shrink_compact(None, None, FAKE, FAKE, 64, 0, 4096, 16, 32, seg, None, None, 0, stream=0)
    L.lora_expand_compact(None, None, None, FAKE, FAKE, 64, 0, 4096, 16, 32, seg, None, 0, stream=0)


def test_status_pool():
    assert L.lora_status_string(10).startswith("LORA_ERR_POOL")
    assert L.LORA_MODE_CHECKED == 0x100


def test_noalloc_rejects_before_touching_the_device():
    """lora_linear_noalloc validates like lora_linear (no GPU needed for these), and rejects a
    call whose workspace would exceed its scratch."""
    args = dict(x=FAKE, W=FAKE, A=FAKE, B=FAKE, scale=FAKE, ranks=None, ids=FAKE, M=64, d_in=4096,
                d_out=4096, r_max=16, n_adapters=32, segs=None, y=FAKE, y_dtype=L.LORA_BF16,
                mode=L.LORA_MODE_DECODE, stream=0)
    for over, code in ((dict(M=-1), 2), (dict(r_max=65), 3), (dict(d_in=12), 2),
                       (dict(M=512, d_out=11008), 5)):
        with pytest.raises(L.LoraError) as e:
            L.lora_linear_noalloc(**{**args, **over})
        assert e.value.status == code
    assert L.lora_workspace_bytes(512, 4096, 11008, 16, 32) > L.LORA_NOALLOC_SCRATCH_BYTES
    L.lora_linear_noalloc(**{**args, "M": 0, "x": None, "y": None})  # no-op


@pytest.mark.parametrize("over,code", [
    (dict(d_in=4104), 2), (dict(d_in=64), 2), (dict(M=257), 2), (dict(r_max=65), 3),
    (dict(mode=L.LORA_MODE_PREFILL), 9), (dict(mode=5), 9), (dict(w_scale=None), 1),
    (dict(W8=None), 1), (dict(W8=FAKE + 8), 4), (dict(w_scale=FAKE + 2), 4),
    (dict(ws_bytes=1024), 5), (dict(y_dtype=4), 6),
])
def test_linear_fp8w_rejects(over, code):
    args = dict(x=FAKE, W8=FAKE, w_scale=FAKE, A=FAKE, B=FAKE, scale=FAKE, ranks=None, ids=FAKE,
                M=64, d_in=4096, d_out=4096, r_max=16, n_adapters=32, segs=None, y=FAKE,
                y_dtype=L.LORA_BF16, mode=L.LORA_MODE_DECODE, ws=FAKE,
                ws_bytes=L.lora_workspace_bytes(64, 4096, 4096, 16, 32), stream=0)
    args.update(over)
    with pytest.raises(L.LoraError) as e:
        L.lora_linear_fp8w(**args)
    assert e.value.status == code


def test_moe_workspace_bytes():
    b = L.lora_moe_workspace_bytes(64, 4, 32, 2880, 2880, 16, 8)
    assert b > 0 and b % 256 == 0
    assert L.lora_moe_workspace_bytes(0, 4, 32, 2880, 2880, 16, 8) == 0
    assert L.lora_moe_workspace_bytes(64, 4, 32, 2880, 2880, 12, 8) == 0  # r_max % 8
    assert L.lora_moe_workspace_bytes(2049, 4, 32, 2880, 2880, 16, 8) == 0  # pairs > max
    assert L.lora_moe_workspace_bytes(2048, 4, 32, 2880, 2880, 16, 8) > b
    assert L.lora_moe_workspace_bytes(64, 4, 32, 96, 2880, 16, 8) == 0  # d_in < 128


@pytest.mark.parametrize("over,code", [
    (dict(M=-1), 2), (dict(top_k=0), 2), (dict(top_k=65), 2), (dict(n_experts=0), 2),
    (dict(n_experts=4097), 2), (dict(M=L.LORA_MOE_MAX_PAIRS // 4 + 1), 2), (dict(d_in=96), 2),
    (dict(d_in=2888), 2), (dict(d_out=2884), 2), (dict(n_adapters=0), 2),
    (dict(r_max=12), 3), (dict(r_max=4), 3), (dict(r_max=72), 3),
    (dict(mode=L.LORA_MODE_PREFILL), 9), (dict(mode=6), 9), (dict(y_dtype=3), 6),
    (dict(topk_ids=None), 1), (dict(W=None), 1), (dict(ids=None), 1),
    (dict(topk_w=FAKE + 2), 4), (dict(W=FAKE + 8), 4), (dict(ws=FAKE + 64), 4),
    (dict(ws_bytes=1024), 5),
])
def test_moe_linear_rejects(over, code):
    args = dict(x=FAKE, W=FAKE, A=FAKE, B=FAKE, scale=FAKE, ranks=None, ids=FAKE, topk_ids=FAKE,
                topk_w=FAKE, M=64, top_k=4, n_experts=32, d_in=2880, d_out=2880, r_max=16,
                n_adapters=8, y=FAKE, y_dtype=L.LORA_BF16, mode=L.LORA_MODE_DECODE, ws=FAKE,
                ws_bytes=L.lora_moe_workspace_bytes(64, 4, 32, 2880, 2880, 16, 8), stream=0)
    args.update(over)
    with pytest.raises(L.LoraError) as e:
        L.lora_moe_linear(**args)
    assert e.value.status == code


def test_moe_empty_batch_is_noop():
    L.lora_moe_linear(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, 4, 32, 2880, 2880,
                      16, 8, None, L.LORA_BF16, L.LORA_MODE_DECODE, None, 0, stream=0)


def test_workspace_bytes_multi():
    one = L.lora_workspace_bytes(512, 4096, 11008, 16, 1024)
    assert L.lora_workspace_bytes_multi(512, 4096, 11008, 16, 1024, 0) == 0
    assert L.lora_workspace_bytes_multi(512, 4096, 11008, 16, 1024, L.LORA_MAX_PROJ + 1) == 0
    assert L.lora_workspace_bytes_multi(512, 4096, 11008, 16, 1024, 1) == one
    # the stream-K batch: one shrink area per projection and the merged launch's partial tiles
    two = L.lora_workspace_bytes_multi(512, 4096, 11008, 16, 1024, 2)
    assert two > one and two % 256 == 0
    # batches outside the stream-K range run projection by projection on one workspace
    for M in (64, 200, 2048):
        assert (L.lora_workspace_bytes_multi(M, 4096, 4096, 16, 32, 3) ==
                L.lora_workspace_bytes(M, 4096, 4096, 16, 32))
    assert L.lora_workspace_bytes_multi(64, 4096, 4096, 65, 32, 2) == 0


def _multi(n_proj=2, **over):
    args = dict(x=FAKE, Ws=[FAKE] * n_proj, As=[FAKE] * n_proj, Bs=[FAKE] * n_proj, scale=FAKE,
                ranks=None, ids=FAKE, M=512, d_in=4096, d_out=11008, r_max=16, n_adapters=1024,
                segs=None, ys=[FAKE] * n_proj, y_dtype=L.LORA_BF16, mode=L.LORA_MODE_DECODE,
                ws=FAKE, ws_bytes=L.lora_workspace_bytes(512, 4096, 11008, 16, 1024), stream=0)
    args.update(over)
    return L.lora_linear_multi(**args)


@pytest.mark.parametrize("over,code", [
    (dict(n_proj=0), 2), (dict(n_proj=L.LORA_MAX_PROJ + 1), 2),
    (dict(Ws=None), 1), (dict(ys=None), 1), (dict(As=[FAKE, None]), 1), (dict(ys=[FAKE, FAKE + 8]), 4),
    (dict(r_max=65), 3), (dict(M=-1), 2),
    # enough for one projection's sequence, not for the merged stream-K launch of two
    (dict(), 5),
])
def test_linear_multi_rejects(over, code):
    n_proj = over.pop("n_proj", 2)
    with pytest.raises(L.LoraError) as e:
        _multi(n_proj=n_proj, **over)
    assert e.value.status == code


def test_linear_multi_empty_batch_is_noop():
    _multi(M=0, x=None, ys=[None, None], ws=None)
