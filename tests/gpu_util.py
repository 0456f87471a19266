"""Helpers for the GPU parity tests: device copies of a workload, calls through the C ABI,
and the parity rule.

The rule for floating-point outputs: max|y_gpu - y_ref| <= 2e-2 * max|y_ref| and
mean relative error sum|y_gpu - y_ref| / sum|y_ref| <= 5e-3, over the whole output of a call
(every row; max|y_ref| is taken over that whole output).
"""

from __future__ import annotations

import dataclasses
import sys

import numpy as np

from synth import Workload, bf16_bits_to_f32

MAX_REL = 2e-2
MEAN_REL = 5e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(y - ref)
    den = np.abs(ref).max() if ref.size else 0.0
    max_rel = float(d.max() / den) if ref.size and den > 0 else float(d.max() if ref.size else 0.0)
    mean_rel = float(d.sum() / np.abs(ref).sum()) if ref.size and np.abs(ref).sum() > 0 else 0.0
    return max_rel, mean_rel


def assert_parity(y, ref, what: str, max_rel=MAX_REL, mean_rel=MEAN_REL):
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    mr, ml = metrics(y, ref)
    assert mr <= max_rel and ml <= mean_rel, f"{what}: max_rel={mr:.3e} mean_rel={ml:.3e}"
    return mr, ml


def bf16_dev(bits: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_host(t) -> np.ndarray:
    import torch

    return bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


@dataclasses.dataclass
class DevProjection:
    x: object
    W: object
    A: object
    B: object
    d_in: int
    d_out: int


@dataclasses.dataclass
class DevWorkload:
    w: Workload
    ids: object
    ranks: object
    scale: object
    projs: list

    @property
    def M(self):
        return self.w.M

    @property
    def n(self):
        return self.w.n_adapters


def scale_of(w: Workload) -> np.ndarray:
    """scale_i = alpha_i / r_i in float32 (what a caller of the library passes)."""
    return (w.alpha.astype(np.float32) / w.ranks.astype(np.float32)).astype(np.float32)


def to_device(w: Workload) -> DevWorkload:
    import torch

    wb = w.as_bf16()
    projs = [DevProjection(bf16_dev(p.x), bf16_dev(p.W), bf16_dev(p.A), bf16_dev(p.B), p.d_in,
                           p.d_out) for p in wb.projections]
    return DevWorkload(wb, torch.from_numpy(w.ids.astype(np.int32)).cuda(),
                       torch.from_numpy(w.ranks.astype(np.int32)).cuda(),
                       torch.from_numpy(scale_of(w)).cuda(), projs)


def gpu_linear(dw: DevWorkload, pi: int = 0, mode=None, y_f32=False, ids=None, segs=None,
               ranks="default"):
    """One lora_linear call; returns y as float32 numpy."""
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    p = dw.projs[pi]
    M = dw.M
    mode = L.LORA_MODE_AUTO if mode is None else mode
    y = torch.empty((M, p.d_out), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    ws, nbytes = L.workspace(M, p.d_in, p.d_out, dw.w.r_max, dw.n)
    L.lora_linear(p.x, p.W, p.A, p.B, dw.scale, dw.ranks if ranks == "default" else ranks,
                  dw.ids if ids is None else ids, M, p.d_in, p.d_out, dw.w.r_max, dw.n, segs, y,
                  L.LORA_F32 if y_f32 else L.LORA_BF16, mode, ws, nbytes)
    torch.cuda.synchronize()
    return y.cpu().numpy() if y_f32 else bf16_host(y)


def gpu_segments(ids_np: np.ndarray, n: int):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    M = int(ids_np.shape[0])
    seg = L.Segments(M, n)
    ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
    L.lora_build_segments(ids, M, n, seg)
    torch.cuda.synchronize()
    meta = seg.meta.cpu().numpy()
    out = dict(perm=seg.perm.cpu().numpy()[:M], offsets=seg.offsets.cpu().numpy(),
               seg_adapter=seg.seg_adapter.cpu().numpy()[: meta[0]],
               tiles=seg.tiles.cpu().numpy()[: 2 * meta[3]].reshape(-1, 2), meta=meta)
    return out, seg, ids
