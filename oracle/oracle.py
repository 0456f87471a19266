"""ctypes front end of the plain-C oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use this module.
It widens bfloat16 bit patterns to float32 exactly (the bits shifted into the high half of
a float32 word) and passes float32 arrays to oracle.c, which computes the layer of
"Multi-LoRA Serving: Why 100 Adapters Fit on One GPU", section "Why can't you just merge
LoRA weights into the base model?", row by row in float32.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -O3 only vectorises the innermost column loops; every output element still sums its
# terms in ascending index order.  No -march: the same instructions on any x86-64 host.
CFLAGS = ["-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c99",
          "-Wall", "-Wextra"]

_lib = None


class OracleError(ValueError):
    pass


def library_path() -> str:
    return _LIB


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c with gcc into a shared library (when missing or stale)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, src, "-o", tmp], check=True)
        os.replace(tmp, out)
    return out


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def load_library(path: str):
    """Load an oracle build from an explicit path (used by the oracle's own mutation tests)."""
    return _load(path)


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int32
    lib.oracle_build_segments.argtypes = [P, I, I, I, P, P, P, P, P]
    lib.oracle_lora_shrink.argtypes = [P, P, P, I, I, I, I, P, I]
    lib.oracle_lora_expand.argtypes = [P, P, P, P, P, I, I, I, I, P, I]
    lib.oracle_lora_linear.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, I, P, I]
    lib.oracle_lora_linear_fp8w.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, P, I, P, I]
    lib.oracle_lora_linear_fp8w.restype = ctypes.c_int
    lib.oracle_moe_lora_linear.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, I]
    lib.oracle_moe_lora_linear.restype = ctypes.c_int
    lib.oracle_fp8_e4m3_decode_array.argtypes = [P, ctypes.c_int64, P]
    lib.oracle_fp8_e4m3_decode_array.restype = None
    for f in (lib.oracle_build_segments, lib.oracle_lora_shrink, lib.oracle_lora_expand,
              lib.oracle_lora_linear):
        f.restype = ctypes.c_int
    return lib


def _f32(a: np.ndarray) -> np.ndarray:
    """float32 as is; uint16 read as bfloat16 bits and widened exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (np.ascontiguousarray(a).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if a.dtype != np.float32:
        raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {a.dtype}")
    return np.ascontiguousarray(a)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(code: int, what: str) -> None:
    if code == 0:
        return
    if code == 2:
        raise OracleError(f"{what}: adapter id out of range [-1, n_adapters)")
    raise OracleError(f"{what}: oracle error code {code}")


def _threads(n: Optional[int]) -> int:
    """Explicit count, else OMP_NUM_THREADS when set (a shared host's CPU share), else
    every core."""
    if n:
        return int(n)
    env = os.environ.get("OMP_NUM_THREADS", "")
    return int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)


def build_segments(ids, n_adapters: int, tile_rows: int, lib=None) -> dict:
    """Stable grouping of rows by adapter: perm, offsets, seg_adapter, tiles, meta."""
    lib = lib or _load()
    ids = _i32(ids)
    M = int(ids.shape[0])
    max_tiles = min(M, n_adapters) + M // tile_rows
    perm = np.full(M, -7, np.int32)
    offsets = np.full(n_adapters + 1, -7, np.int32)
    seg_adapter = np.full(max(min(M, n_adapters), 1), -7, np.int32)
    tiles = np.full(max(2 * max_tiles, 2), -7, np.int32)
    meta = np.full(4, -7, np.int32)
    _check(lib.oracle_build_segments(_ptr(ids), M, int(n_adapters), int(tile_rows), _ptr(perm),
                                      _ptr(offsets), _ptr(seg_adapter), _ptr(tiles), _ptr(meta)),
           "build_segments")
    n_seg, n_tiles = int(meta[0]), int(meta[3])
    return dict(perm=perm, offsets=offsets, seg_adapter=seg_adapter[:n_seg].copy(),
                tiles=tiles[: 2 * n_tiles].reshape(n_tiles, 2).copy(), meta=meta)


def lora_shrink(x, A, ids, n_threads: Optional[int] = None, lib=None) -> np.ndarray:
    """t[M, r_max] (float32); zero rows for id -1."""
    lib = lib or _load()
    x, A, ids = _f32(x), _f32(A), _i32(ids)
    M, d_in = x.shape
    n, d_in2, r_max = A.shape
    assert d_in2 == d_in and ids.shape == (M,)
    t = np.empty((M, r_max), np.float32)
    _check(lib.oracle_lora_shrink(_ptr(x), _ptr(A), _ptr(ids), M, d_in, r_max, n, _ptr(t),
                                  _threads(n_threads)), "lora_shrink")
    return t


def lora_expand(t, B, alpha, ranks, ids, y, n_threads: Optional[int] = None, lib=None) -> np.ndarray:
    """Returns y + (t B_i) * alpha_i / r_i on rows with an adapter (float32 copy of y)."""
    lib = lib or _load()
    t, B, y = _f32(t), _f32(B), _f32(y).copy()
    alpha, ranks, ids = np.ascontiguousarray(alpha, np.float32), _i32(ranks), _i32(ids)
    M, r_max = t.shape
    n, r2, d_out = B.shape
    assert r2 == r_max and y.shape == (M, d_out) and ids.shape == (M,)
    _check(lib.oracle_lora_expand(_ptr(t), _ptr(B), _ptr(alpha), _ptr(ranks), _ptr(ids), M, d_out,
                                  r_max, n, _ptr(y), _threads(n_threads)), "lora_expand")
    return y


def lora_linear(x, W, A, B, alpha, ranks, ids, rows=None, n_threads: Optional[int] = None,
                lib=None) -> np.ndarray:
    """y = x W + (x A_i) B_i alpha_i / r_i per row, float32.

    rows: optional list of row indices; then only those rows are computed and returned
    as y[len(rows), d_out] in list order.
    """
    lib = lib or _load()
    x, W, A, B = _f32(x), _f32(W), _f32(A), _f32(B)
    alpha, ranks, ids = np.ascontiguousarray(alpha, np.float32), _i32(ranks), _i32(ids)
    M, d_in = x.shape
    d_in2, d_out = W.shape
    n, d_in3, r_max = A.shape
    assert d_in2 == d_in and d_in3 == d_in and B.shape == (n, r_max, d_out)
    assert ids.shape == (M,) and alpha.shape == (n,) and ranks.shape == (n,)
    if rows is None:
        rows_a, n_rows, out_rows = None, 0, M
    else:
        rows_a = _i32(rows)
        n_rows = out_rows = int(rows_a.shape[0])
    y = np.empty((out_rows, d_out), np.float32)
    _check(lib.oracle_lora_linear(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(alpha), _ptr(ranks),
                                  _ptr(ids), M, d_in, d_out, r_max, n,
                                  None if rows_a is None else _ptr(rows_a), n_rows, _ptr(y),
                                  _threads(n_threads)), "lora_linear")
    return y


def fp8_e4m3_decode(codes, lib=None) -> np.ndarray:
    """float32 values of OCP E4M3 fp8 codes (uint8), from the format definition."""
    lib = lib or _load()
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, np.float32)
    lib.oracle_fp8_e4m3_decode_array(_ptr(c), int(c.size), _ptr(out))
    return out


def lora_linear_fp8w(x, W8, w_scale, A, B, alpha, ranks, ids, rows=None,
                     n_threads: Optional[int] = None, lib=None) -> np.ndarray:
    """y = x W_eff + (x A_i) B_i alpha_i / r_i per row, float32, with the base weight given as
    fp8 codes W8[d_out, d_in] (uint8, OCP E4M3) and per-column scales w_scale[d_out]:
    W_eff[k, c] = w_scale[c] * dec(W8[c, k]), the scale applied to the fp32 sum over k."""
    lib = lib or _load()
    x, A, B = _f32(x), _f32(A), _f32(B)
    W8 = np.ascontiguousarray(np.asarray(W8, dtype=np.uint8))
    w_scale = np.ascontiguousarray(w_scale, np.float32)
    alpha, ranks, ids = np.ascontiguousarray(alpha, np.float32), _i32(ranks), _i32(ids)
    M, d_in = x.shape
    d_out, d_in2 = W8.shape
    n, d_in3, r_max = A.shape
    assert d_in2 == d_in and d_in3 == d_in and B.shape == (n, r_max, d_out)
    assert w_scale.shape == (d_out,) and ids.shape == (M,)
    if rows is None:
        rows_a, n_rows, out_rows = None, 0, M
    else:
        rows_a = _i32(rows)
        n_rows = out_rows = int(rows_a.shape[0])
    y = np.empty((out_rows, d_out), np.float32)
    _check(lib.oracle_lora_linear_fp8w(_ptr(x), _ptr(W8), _ptr(w_scale), _ptr(A), _ptr(B),
                                       _ptr(alpha), _ptr(ranks), _ptr(ids), M, d_in, d_out, r_max,
                                       n, None if rows_a is None else _ptr(rows_a), n_rows,
                                       _ptr(y), _threads(n_threads)), "lora_linear_fp8w")
    return y


def moe_lora_linear(x, W, A, B, alpha, ranks, ids, topk_ids, topk_w=None,
                    n_threads: Optional[int] = None, lib=None) -> np.ndarray:
    """MoE-LoRA per (token, slot): y[m, j] = topk_w[m, j] * (x_m W_e + (x_m A[i, e]) B[i, e]
    alpha_i / r_i) with e = topk_ids[m, j] (-1: zero row), i = ids[m] (-1: no adapter term).
    W[E, d_in, d_out], A[n, E, d_in, r_max], B[n, E, r_max, d_out]; returns y[M, top_k, d_out]."""
    lib = lib or _load()
    x, W, A, B = _f32(x), _f32(W), _f32(A), _f32(B)
    alpha, ranks, ids = np.ascontiguousarray(alpha, np.float32), _i32(ranks), _i32(ids)
    topk_ids = _i32(topk_ids)
    M, d_in = x.shape
    E, d_in2, d_out = W.shape
    n, E2, d_in3, r_max = A.shape
    top_k = int(topk_ids.shape[1]) if topk_ids.ndim == 2 else 1
    assert d_in2 == d_in and d_in3 == d_in and E2 == E and B.shape == (n, E, r_max, d_out)
    assert topk_ids.shape == (M, top_k) and ids.shape == (M,)
    tw = None if topk_w is None else np.ascontiguousarray(topk_w, np.float32)
    if tw is not None:
        assert tw.shape == (M, top_k)
    y = np.empty((M, top_k, d_out), np.float32)
    _check(lib.oracle_moe_lora_linear(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(alpha), _ptr(ranks),
                                      _ptr(ids), _ptr(topk_ids), None if tw is None else _ptr(tw),
                                      M, top_k, E, d_in, d_out, r_max, n, _ptr(y),
                                      _threads(n_threads)), "moe_lora_linear")
    return y
