"""Python binding of liblora_mi355x.so (include/lora.h) -- argument marshalling only.

Every function has the name and argument order of its C entry point.  Array arguments are
torch CUDA tensors (or raw device addresses as ints); this module only turns them into
pointers, passes the current torch stream when none is given, and raises LoraError on a
non-zero status.  Every step of the computation runs in the HIP kernels of the library.
There is no fallback: if the library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblora_mi355x.so")

LORA_TILE_ROWS = 16
LORA_MAX_ADAPTERS = 16384
LORA_MAX_ROWS = 1 << 22
LORA_MAX_PROJ = 4
LORA_PREFILL_MIN_ROWS = 768
LORA_NOALLOC_SCRATCH_BYTES = 32 << 20
LORA_MOE_MAX_PAIRS = 8192

LORA_BF16, LORA_F32 = 0, 1
LORA_MODE_AUTO, LORA_MODE_DECODE, LORA_MODE_PREFILL = 0, 1, 2
LORA_MODE_CHECKED = 0x100  # OR-ed into a mode: sync, check ids and adapter tables on the host

STATUS = {
    0: "LORA_OK", 1: "LORA_ERR_NULL", 2: "LORA_ERR_SHAPE", 3: "LORA_ERR_RANK",
    4: "LORA_ERR_ALIGN", 5: "LORA_ERR_WORKSPACE", 6: "LORA_ERR_DTYPE", 7: "LORA_ERR_HIP",
    8: "LORA_ERR_BAD_ID", 9: "LORA_ERR_MODE", 10: "LORA_ERR_POOL",
}

# every symbol include/lora.h declares
EXPORTS = ("lora_max_tiles", "lora_workspace_bytes", "lora_build_segments", "lora_shrink",
           "lora_shrink_compact", "lora_expand", "lora_expand_compact", "lora_linear",
           "lora_linear_profiled", "lora_linear_compact", "lora_linear_compact_profiled",
           "lora_linear_noalloc", "lora_linear_fp8w", "lora_linear_fp8w_profiled",
           "lora_moe_workspace_bytes", "lora_moe_linear", "lora_moe_linear_profiled",
           "lora_workspace_bytes_multi", "lora_linear_multi", "lora_linear_multi_profiled",
           "lora_status_string", "lora_last_hip_error")


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {lora_status_string(status)}"
        if status == 7:
            msg += f" ({lora_last_hip_error()})"
        super().__init__(msg)
        self.status = status


class lora_segments_t(ctypes.Structure):
    _fields_ = [("perm", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("seg_adapter", ctypes.c_void_p), ("tiles", ctypes.c_void_p),
                ("meta", ctypes.c_void_p)]


def _load():
    # torch ships its own HIP runtime with the same soname (libamdhip64.so.7) as the one the
    # library was linked against.  Loading torch first makes the library bind to that
    # already-loaded runtime; loading it first would bring in a second HIP runtime in the
    # same process, and then one of the two sees no device.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m rank_adapter_gemm_sgmv_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.lora_max_tiles.argtypes = [I, I]
    lib.lora_max_tiles.restype = I
    lib.lora_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.lora_workspace_bytes.restype = S
    lib.lora_build_segments.argtypes = [P, I, I, lora_segments_t, P]
    lib.lora_build_segments.restype = ctypes.c_int
    lib.lora_shrink.argtypes = [P, P, P, I, I, I, I, lora_segments_t, P, P, S, P]
    lib.lora_shrink.restype = ctypes.c_int
    lib.lora_shrink_compact.argtypes = [P, P, P, P, I, I, I, I, I, lora_segments_t, P, P, S, P]
    lib.lora_shrink_compact.restype = ctypes.c_int
    lib.lora_expand.argtypes = [P, P, P, P, I, I, I, I, lora_segments_t, P, ctypes.c_int, P]
    lib.lora_expand.restype = ctypes.c_int
    lib.lora_expand_compact.argtypes = [P, P, P, P, P, I, I, I, I, I, lora_segments_t, P,
                                        ctypes.c_int, P]
    lib.lora_expand_compact.restype = ctypes.c_int
    lib.lora_linear.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I,
                                ctypes.POINTER(lora_segments_t), P, ctypes.c_int, ctypes.c_int,
                                P, S, P]
    lib.lora_linear.restype = ctypes.c_int
    lib.lora_linear_fp8w.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I,
                                     ctypes.POINTER(lora_segments_t), P, ctypes.c_int, ctypes.c_int,
                                     P, S, P]
    lib.lora_linear_fp8w.restype = ctypes.c_int
    lib.lora_linear_fp8w_profiled.argtypes = lib.lora_linear_fp8w.argtypes + [
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p), I, ctypes.POINTER(I)]
    lib.lora_linear_fp8w_profiled.restype = ctypes.c_int
    lib.lora_moe_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.lora_moe_workspace_bytes.restype = S
    lib.lora_moe_linear.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P,
                                    ctypes.c_int, ctypes.c_int, P, S, P]
    lib.lora_moe_linear.restype = ctypes.c_int
    lib.lora_moe_linear_profiled.argtypes = lib.lora_moe_linear.argtypes + [
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p), I, ctypes.POINTER(I)]
    lib.lora_moe_linear_profiled.restype = ctypes.c_int
    lib.lora_linear_noalloc.argtypes = lib.lora_linear.argtypes[:16] + [P]
    lib.lora_linear_noalloc.restype = ctypes.c_int
    lib.lora_linear_profiled.argtypes = lib.lora_linear.argtypes + [
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p), I, ctypes.POINTER(I)]
    lib.lora_linear_profiled.restype = ctypes.c_int
    lib.lora_linear_compact.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I,
                                        ctypes.POINTER(lora_segments_t), P, ctypes.c_int,
                                        ctypes.c_int, P, S, P]
    lib.lora_linear_compact.restype = ctypes.c_int
    lib.lora_linear_compact_profiled.argtypes = lib.lora_linear_compact.argtypes + [
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p), I, ctypes.POINTER(I)]
    lib.lora_linear_compact_profiled.restype = ctypes.c_int
    lib.lora_workspace_bytes_multi.argtypes = [I, I, I, I, I, I]
    lib.lora_workspace_bytes_multi.restype = S
    lib.lora_linear_multi.argtypes = [P, I, P, P, P, P, P, P, I, I, I, I, I,
                                      ctypes.POINTER(lora_segments_t), P, ctypes.c_int,
                                      ctypes.c_int, P, S, P]
    lib.lora_linear_multi.restype = ctypes.c_int
    lib.lora_linear_multi_profiled.argtypes = lib.lora_linear_multi.argtypes + [
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p), I, ctypes.POINTER(I)]
    lib.lora_linear_multi_profiled.restype = ctypes.c_int
    lib.lora_status_string.argtypes = [ctypes.c_int]
    lib.lora_status_string.restype = ctypes.c_char_p
    lib.lora_last_hip_error.argtypes = []
    lib.lora_last_hip_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library():
    return _lib


def _ptr(a) -> Optional[int]:
    """Device address of a tensor (or an int address); None stays NULL."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LoraError(status, where)


def _seg_struct(seg) -> lora_segments_t:
    if isinstance(seg, lora_segments_t):
        return seg
    return lora_segments_t(_ptr(seg.perm), _ptr(seg.offsets), _ptr(seg.seg_adapter),
                           _ptr(seg.tiles), _ptr(seg.meta))


# ---- the entry points -------------------------------------------------------------------


def lora_status_string(status: int) -> str:
    return _lib.lora_status_string(int(status)).decode()


def lora_last_hip_error() -> str:
    return _lib.lora_last_hip_error().decode()


def lora_max_tiles(M: int, n_adapters: int) -> int:
    return int(_lib.lora_max_tiles(M, n_adapters))


def lora_workspace_bytes(M: int, d_in: int, d_out: int, r_max: int, n_adapters: int) -> int:
    return int(_lib.lora_workspace_bytes(M, d_in, d_out, r_max, n_adapters))


def lora_build_segments(ids, M: int, n_adapters: int, seg, stream=None) -> None:
    _check(_lib.lora_build_segments(_ptr(ids), M, n_adapters, _seg_struct(seg), _stream(stream)),
           "lora_build_segments")


def lora_shrink(x, A, ranks, M: int, d_in: int, r_max: int, n_adapters: int, seg, t, ws,
                ws_bytes: int, stream=None) -> None:
    _check(_lib.lora_shrink(_ptr(x), _ptr(A), _ptr(ranks), M, d_in, r_max, n_adapters,
                            _seg_struct(seg), _ptr(t), _ptr(ws), ws_bytes, _stream(stream)),
           "lora_shrink")


def lora_shrink_compact(x, A, ranks, rank_offsets, pool_rows: int, M: int, d_in: int, r_max: int,
                        n_adapters: int, seg, t, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.lora_shrink_compact(_ptr(x), _ptr(A), _ptr(ranks), _ptr(rank_offsets), pool_rows,
                                    M, d_in, r_max, n_adapters, _seg_struct(seg), _ptr(t),
                                    _ptr(ws), ws_bytes, _stream(stream)), "lora_shrink_compact")


def lora_expand_compact(t, B, scale, ranks, rank_offsets, pool_rows: int, M: int, d_out: int,
                        r_max: int, n_adapters: int, seg, y, y_dtype: int, stream=None) -> None:
    _check(_lib.lora_expand_compact(_ptr(t), _ptr(B), _ptr(scale), _ptr(ranks), _ptr(rank_offsets),
                                    pool_rows, M, d_out, r_max, n_adapters, _seg_struct(seg),
                                    _ptr(y), y_dtype, _stream(stream)), "lora_expand_compact")


def lora_expand(t, B, scale, ranks, M: int, d_out: int, r_max: int, n_adapters: int, seg, y,
                y_dtype: int, stream=None) -> None:
    _check(_lib.lora_expand(_ptr(t), _ptr(B), _ptr(scale), _ptr(ranks), M, d_out, r_max,
                            n_adapters, _seg_struct(seg), _ptr(y), y_dtype, _stream(stream)),
           "lora_expand")


def lora_linear(x, W, A, B, scale, ranks, ids, M: int, d_in: int, d_out: int, r_max: int,
                n_adapters: int, segs, y, y_dtype: int, mode: int, ws, ws_bytes: int,
                stream=None) -> None:
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    _check(_lib.lora_linear(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks),
                            _ptr(ids), M, d_in, d_out, r_max, n_adapters, seg_p, _ptr(y), y_dtype,
                            mode, _ptr(ws), ws_bytes, _stream(stream)), "lora_linear")


def lora_linear_fp8w(x, W8, w_scale, A, B, scale, ranks, ids, M: int, d_in: int, d_out: int,
                     r_max: int, n_adapters: int, segs, y, y_dtype: int, mode: int, ws,
                     ws_bytes: int, stream=None) -> None:
    """lora_linear with an fp8 (E4M3) base: W8[d_out, d_in] codes (uint8), w_scale[d_out]."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    _check(_lib.lora_linear_fp8w(_ptr(x), _ptr(W8), _ptr(w_scale), _ptr(A), _ptr(B), _ptr(scale),
                                 _ptr(ranks), _ptr(ids), M, d_in, d_out, r_max, n_adapters, seg_p,
                                 _ptr(y), y_dtype, mode, _ptr(ws), ws_bytes, _stream(stream)),
           "lora_linear_fp8w")


def lora_linear_fp8w_profiled(x, W8, w_scale, A, B, scale, ranks, ids, M: int, d_in: int,
                              d_out: int, r_max: int, n_adapters: int, segs, y, y_dtype: int,
                              mode: int, ws, ws_bytes: int, stream=None, max_kernels: int = 16):
    """lora_linear_fp8w with per-kernel HIP event timing; returns [(kernel name, ms), ...]."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    ms = (ctypes.c_float * max_kernels)()
    names = (ctypes.c_char_p * max_kernels)()
    n = ctypes.c_int32(0)
    _check(_lib.lora_linear_fp8w_profiled(
        _ptr(x), _ptr(W8), _ptr(w_scale), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks), _ptr(ids), M,
        d_in, d_out, r_max, n_adapters, seg_p, _ptr(y), y_dtype, mode, _ptr(ws), ws_bytes,
        _stream(stream), ms, names, max_kernels, ctypes.byref(n)), "lora_linear_fp8w_profiled")
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


def lora_moe_workspace_bytes(M: int, top_k: int, n_experts: int, d_in: int, d_out: int,
                             r_max: int, n_adapters: int) -> int:
    return int(_lib.lora_moe_workspace_bytes(M, top_k, n_experts, d_in, d_out, r_max, n_adapters))


def lora_moe_linear(x, W, A, B, scale, ranks, ids, topk_ids, topk_w, M: int, top_k: int,
                    n_experts: int, d_in: int, d_out: int, r_max: int, n_adapters: int, y,
                    y_dtype: int, mode: int, ws, ws_bytes: int, stream=None) -> None:
    """MoE-LoRA: y[M, top_k, d_out] per (token, slot); W[E, d_in, d_out], A[n, E, d_in, r_max],
    B[n, E, r_max, d_out], topk_ids[M, top_k] (-1: empty slot), topk_w[M, top_k] or None."""
    _check(_lib.lora_moe_linear(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks),
                                _ptr(ids), _ptr(topk_ids), _ptr(topk_w), M, top_k, n_experts, d_in,
                                d_out, r_max, n_adapters, _ptr(y), y_dtype, mode, _ptr(ws),
                                ws_bytes, _stream(stream)), "lora_moe_linear")


def lora_moe_linear_profiled(x, W, A, B, scale, ranks, ids, topk_ids, topk_w, M: int, top_k: int,
                             n_experts: int, d_in: int, d_out: int, r_max: int, n_adapters: int,
                             y, y_dtype: int, mode: int, ws, ws_bytes: int, stream=None,
                             max_kernels: int = 16):
    """lora_moe_linear with per-kernel HIP event timing; returns [(kernel name, ms), ...]."""
    ms = (ctypes.c_float * max_kernels)()
    names = (ctypes.c_char_p * max_kernels)()
    n = ctypes.c_int32(0)
    _check(_lib.lora_moe_linear_profiled(
        _ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks), _ptr(ids), _ptr(topk_ids),
        _ptr(topk_w), M, top_k, n_experts, d_in, d_out, r_max, n_adapters, _ptr(y), y_dtype, mode,
        _ptr(ws), ws_bytes, _stream(stream), ms, names, max_kernels, ctypes.byref(n)),
        "lora_moe_linear_profiled")
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


def moe_workspace(M: int, top_k: int, n_experts: int, d_in: int, d_out: int, r_max: int,
                  n_adapters: int, device="cuda"):
    """A uint8 device tensor of lora_moe_workspace_bytes() bytes (256-byte aligned by torch)."""
    import torch

    nbytes = lora_moe_workspace_bytes(M, top_k, n_experts, d_in, d_out, r_max, n_adapters)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device), nbytes


def lora_linear_noalloc(x, W, A, B, scale, ranks, ids, M: int, d_in: int, d_out: int, r_max: int,
                        n_adapters: int, segs, y, y_dtype: int, mode: int, stream=None) -> None:
    """lora_linear on the library's own device scratch (no workspace argument)."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    _check(_lib.lora_linear_noalloc(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks),
                                    _ptr(ids), M, d_in, d_out, r_max, n_adapters, seg_p, _ptr(y),
                                    y_dtype, mode, _stream(stream)), "lora_linear_noalloc")


def lora_linear_profiled(x, W, A, B, scale, ranks, ids, M: int, d_in: int, d_out: int,
                         r_max: int, n_adapters: int, segs, y, y_dtype: int, mode: int, ws,
                         ws_bytes: int, stream=None, max_kernels: int = 16):
    """lora_linear with per-kernel HIP event timing; returns [(kernel name, ms), ...]."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    ms = (ctypes.c_float * max_kernels)()
    names = (ctypes.c_char_p * max_kernels)()
    n = ctypes.c_int32(0)
    _check(_lib.lora_linear_profiled(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks),
                                     _ptr(ids), M, d_in, d_out, r_max, n_adapters, seg_p, _ptr(y),
                                     y_dtype, mode, _ptr(ws), ws_bytes, _stream(stream), ms, names,
                                     max_kernels, ctypes.byref(n)), "lora_linear_profiled")
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


def lora_workspace_bytes_multi(M: int, d_in: int, d_out: int, r_max: int, n_adapters: int,
                               n_proj: int) -> int:
    return int(_lib.lora_workspace_bytes_multi(M, d_in, d_out, r_max, n_adapters, n_proj))


def _ptr_array(ts):
    """Host array of device addresses (None for a missing list)."""
    if ts is None:
        return None
    return (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])


def lora_linear_multi(x, Ws, As, Bs, scale, ranks, ids, M: int, d_in: int, d_out: int,
                      r_max: int, n_adapters: int, segs, ys, y_dtype: int, mode: int, ws,
                      ws_bytes: int, stream=None, n_proj: Optional[int] = None) -> None:
    """lora_linear for len(Ws) projections that share x and the adapter tables (Ws, As, Bs,
    ys: lists of device tensors, one per projection)."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    if n_proj is None:  # the length of the lists (a missing list is passed as NULL)
        n_proj = next((len(v) for v in (Ws, As, Bs, ys) if v is not None), 0)
    n = n_proj
    _check(_lib.lora_linear_multi(_ptr(x), n, _ptr_array(Ws), _ptr_array(As), _ptr_array(Bs),
                                  _ptr(scale), _ptr(ranks), _ptr(ids), M, d_in, d_out, r_max,
                                  n_adapters, seg_p, _ptr_array(ys), y_dtype, mode, _ptr(ws),
                                  ws_bytes, _stream(stream)), "lora_linear_multi")


def lora_linear_multi_profiled(x, Ws, As, Bs, scale, ranks, ids, M: int, d_in: int, d_out: int,
                               r_max: int, n_adapters: int, segs, ys, y_dtype: int, mode: int,
                               ws, ws_bytes: int, stream=None, max_kernels: int = 24):
    """lora_linear_multi with per-kernel HIP event timing; returns [(kernel name, ms), ...]."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    ms = (ctypes.c_float * max_kernels)()
    names = (ctypes.c_char_p * max_kernels)()
    n = ctypes.c_int32(0)
    _check(_lib.lora_linear_multi_profiled(
        _ptr(x), len(Ws), _ptr_array(Ws), _ptr_array(As), _ptr_array(Bs), _ptr(scale), _ptr(ranks),
        _ptr(ids), M, d_in, d_out, r_max, n_adapters, seg_p, _ptr_array(ys), y_dtype, mode,
        _ptr(ws), ws_bytes, _stream(stream), ms, names, max_kernels, ctypes.byref(n)),
        "lora_linear_multi_profiled")
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


def lora_linear_compact(x, W, A, B, scale, ranks, rank_offsets, pool_rows: int, ids, M: int,
                        d_in: int, d_out: int, r_max: int, n_adapters: int, segs, y, y_dtype: int,
                        mode: int, ws, ws_bytes: int, stream=None) -> None:
    """lora_linear on a rank-compact pool (A_i, B_i stored at rank r_i from rank row
    rank_offsets[i] of pool_rows rows)."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    _check(_lib.lora_linear_compact(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks),
                                    _ptr(rank_offsets), pool_rows, _ptr(ids), M, d_in, d_out,
                                    r_max, n_adapters, seg_p, _ptr(y), y_dtype, mode, _ptr(ws),
                                    ws_bytes, _stream(stream)), "lora_linear_compact")


def lora_linear_compact_profiled(x, W, A, B, scale, ranks, rank_offsets, pool_rows: int, ids,
                                 M: int, d_in: int, d_out: int, r_max: int, n_adapters: int,
                                 segs, y, y_dtype: int, mode: int, ws, ws_bytes: int,
                                 stream=None, max_kernels: int = 16):
    """lora_linear_compact with per-kernel HIP event timing; returns [(kernel name, ms)]."""
    seg_p = None if segs is None else ctypes.byref(_seg_struct(segs))
    ms = (ctypes.c_float * max_kernels)()
    names = (ctypes.c_char_p * max_kernels)()
    n = ctypes.c_int32(0)
    _check(_lib.lora_linear_compact_profiled(
        _ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(scale), _ptr(ranks), _ptr(rank_offsets),
        pool_rows, _ptr(ids), M, d_in, d_out, r_max, n_adapters, seg_p, _ptr(y), y_dtype, mode,
        _ptr(ws), ws_bytes, _stream(stream), ms, names, max_kernels, ctypes.byref(n)),
        "lora_linear_compact_profiled")
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


# ---- device buffers (torch is only the allocator here) ----------------------------------


class Segments:
    """Caller-owned device buffers for lora_build_segments (int32 torch tensors)."""

    def __init__(self, M: int, n_adapters: int, device="cuda"):
        import torch

        kw = dict(dtype=torch.int32, device=device)
        self.M, self.n_adapters = M, n_adapters
        self.perm = torch.empty(max(M, 1), **kw)
        self.offsets = torch.empty(n_adapters + 1, **kw)
        self.seg_adapter = torch.empty(max(1, min(M, n_adapters)), **kw)
        self.tiles = torch.empty(max(2, 2 * lora_max_tiles(M, n_adapters)), **kw)
        self.meta = torch.empty(4, **kw)

    def struct(self) -> lora_segments_t:
        return _seg_struct(self)


def workspace(M: int, d_in: int, d_out: int, r_max: int, n_adapters: int, device="cuda"):
    """A uint8 device tensor of lora_workspace_bytes() bytes (256-byte aligned by torch)."""
    import torch

    nbytes = lora_workspace_bytes(M, d_in, d_out, r_max, n_adapters)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device), nbytes
