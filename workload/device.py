"""Stages a generated Problem in device memory and calls the HIP library on it.

Marshalling only: the arrays are copied to the current HIP device as they are
(bf16 bit patterns viewed as torch.bfloat16, e4m3 codes as uint8), and the
attention itself runs in libattn119.so through exact_attention_119_amd.lib.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from exact_attention_119_amd import lib as L
from .gen import Problem


@dataclasses.dataclass
class DeviceProblem:
    p: Problem
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    dtype: int
    mask: Optional[L.attn_mask]
    fp8: Optional[L.attn_fp8]
    blockmap: Optional[torch.Tensor]  # the block map, or the variable-length workspace
    keep: tuple  # device tensors the mask / fp8 structs point to
    cu_seqlens: Optional[torch.Tensor] = None  # packed variable-length batch
    compact_map: bool = False  # the block map in its compact form (no class and list sections)


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(p: Problem, device="cuda", pv_mode: int = L.ATTN_PV_F16,
              qk_mode: int = L.ATTN_QK_BF16, compact_map: bool = False) -> DeviceProblem:
    """compact_map: allocate and build the block map in its compact form (every call takes
    either form; packed batches always use it)."""
    if p.dtype == "bf16":
        q, k, v = (_dev(x.view(np.int16), device).view(torch.bfloat16) for x in (p.q, p.k, p.v))
        dtype, fp8, keep = L.ATTN_BF16, None, ()
    else:
        q, k, v = (_dev(x, device) for x in (p.q, p.k, p.v))
        qs, ks, vs = (_dev(x, device) for x in (p.q_scale, p.k_scale, p.v_scale))
        dtype, fp8, keep = L.ATTN_FP8_E4M3, L.make_fp8(qs, ks, vs, pv_mode, qk_mode), (qs, ks, vs)
    doc = _dev(p.doc_id, device) if p.doc_id is not None else None
    slopes = _dev(p.alibi_slopes.astype(np.float32), device) if p.alibi_slopes is not None else None
    keep = keep + tuple(x for x in (doc, slopes) if x is not None)
    mask = None
    if p.flags:
        mask = L.make_mask(p.flags, p.window, p.softcap, doc, slopes)
    o = torch.empty((p.B, p.H, p.N, p.d), dtype=torch.bfloat16, device=device)
    lse = torch.empty((p.B, p.H, p.N), dtype=torch.float32, device=device)
    blockmap = None
    if p.cu_seqlens is not None:
        cu = _dev(p.cu_seqlens, device)
        nbytes = L.attn_varlen_workspace_bytes(p.N, mask)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return DeviceProblem(p, q, k, v, o, lse, dtype, mask, fp8, ws, keep, cu, compact_map=True)
    if p.flags & L.POSITIONAL:
        nbytes = (L.attn_blockmap_compact_bytes if compact_map else L.attn_blockmap_bytes)(p.B, p.N, mask)
        blockmap = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return DeviceProblem(p, q, k, v, o, lse, dtype, mask, fp8, blockmap, keep, compact_map=compact_map)


def build_map(dp: DeviceProblem, stream=None) -> None:
    if dp.cu_seqlens is not None:
        L.attn_varlen_prepare(dp.cu_seqlens, dp.p.N, dp.mask, dp.blockmap, stream)
    elif dp.blockmap is not None:
        build = L.attn_blockmap_build_compact if dp.compact_map else L.attn_blockmap_build
        build(dp.p.B, dp.p.N, dp.mask, dp.blockmap, stream)


def needs_map(dp: DeviceProblem) -> bool:
    """Whether the forward pass needs a block map: document masks and packed batches do;
    causal and window masks on the bf16 path derive their block lists in the kernel."""
    return dp.blockmap is not None and (dp.cu_seqlens is not None or bool(dp.p.flags & L.ATTN_DOCUMENT))


def forward(dp: DeviceProblem, rescale_tau: float = 8.0, stream=None, use_map: bool = True) -> None:
    """The forward pass; use_map=False leaves the block map out where the mask allows."""
    if dp.cu_seqlens is not None:
        L.attn_fwd_varlen(dp.q[0], dp.k[0], dp.v[0], dp.o[0], dp.lse[0], scale=dp.p.scale, workspace=dp.blockmap,
                          dtype=dp.dtype, mask=dp.mask, fp8=dp.fp8, rescale_tau=rescale_tau, stream=stream)
        return
    fwd = L.attn_fwd if dp.p.Hkv == dp.p.H else L.attn_fwd_gqa
    fwd(dp.q, dp.k, dp.v, dp.o, dp.lse, scale=dp.p.scale, dtype=dp.dtype, mask=dp.mask,
        blockmap=dp.blockmap if (use_map or needs_map(dp)) else None, fp8=dp.fp8, rescale_tau=rescale_tau,
        stream=stream)


def step(dp: DeviceProblem, rescale_tau: float = 8.0, stream=None, use_map: bool = True) -> None:
    """One pass of the whole path: block map (if the mask needs one), then the forward pass.
    use_map=False builds and passes the map only where the forward pass needs it."""
    if use_map or needs_map(dp):
        build_map(dp, stream)
    forward(dp, rescale_tau, stream, use_map)


def outputs(dp: DeviceProblem):
    """(O as float64 numpy, LSE as float64 numpy) after synchronising."""
    torch.cuda.synchronize()
    return dp.o.float().cpu().numpy().astype(np.float64), dp.lse.cpu().numpy().astype(np.float64)
