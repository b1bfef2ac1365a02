"""ctypes binding of libattn119.so -- argument marshalling only.

The functions carry the C names of include/attn119.h.  Tensors are torch tensors
on the current HIP device (torch supplies device memory and streams); every step
of the computation runs in the library's HIP kernels.  There is no fallback: if
the library is not built, load() raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn119.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_BAD_BLOCKMAP = -3
ATTN_ERR_HIP = -4
ATTN_ERR_BAD_DOC_ID = -5

ATTN_BF16 = 0
ATTN_FP8_E4M3 = 1

ATTN_CAUSAL = 1
ATTN_WINDOW = 2
ATTN_DOCUMENT = 4
ATTN_ALIBI = 8
ATTN_SOFTCAP = 16
POSITIONAL = ATTN_CAUSAL | ATTN_WINDOW | ATTN_DOCUMENT

ATTN_PV_F16 = 0
ATTN_PV_E4M3 = 1

ATTN_QK_BF16 = 0
ATTN_QK_E4M3 = 1
ATTN_PV_FP4 = 2

EXPORTS = ("attn_blockmap_bytes", "attn_blockmap_layout_of", "attn_blockmap_build",
           "attn_blockmap_status", "attn_check_args", "attn_check_args_gqa", "attn_fwd", "attn_fwd_gqa",
           "attn_fwd_kernel_name", "attn_status_str", "attn_varlen_workspace_bytes", "attn_varlen_prepare",
           "attn_fwd_varlen", "attn_fp8_quantize", "attn_bwd", "attn_bwd_gqa", "attn_bwd_gqa_noalloc",
           "attn_fwd_rescale_counts", "attn_varlen_layout_of", "attn_bwd_varlen", "attn_blockmap_compact_bytes",
           "attn_blockmap_compact_layout_of", "attn_blockmap_build_compact")


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class attn_mask(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("window", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("doc_id", ctypes.c_void_p), ("alibi_slopes", ctypes.c_void_p)]


class attn_fp8(ctypes.Structure):
    _fields_ = [("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("pv_mode", ctypes.c_int32), ("qk_mode", ctypes.c_int32)]


class attn_blockmap_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("cls", "counts", "idx", "row_lo", "row_hi", "col_lo", "col_hi", "pairs",
                                               "status", "order", "total")]


_LIB: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the built library (once) and declares its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m exact_attention_119_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.attn_status_str.argtypes = [i32]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_blockmap_bytes.argtypes = [i32, i32, ctypes.POINTER(attn_mask), ctypes.POINTER(sz)]
    lib.attn_blockmap_bytes.restype = i32
    lib.attn_blockmap_layout_of.argtypes = [i32, i32, ctypes.POINTER(attn_blockmap_layout)]
    lib.attn_blockmap_layout_of.restype = i32
    lib.attn_blockmap_build.argtypes = [i32, i32, ctypes.POINTER(attn_mask), vp, sz, vp]
    lib.attn_blockmap_build.restype = i32
    lib.attn_blockmap_compact_bytes.argtypes = [i32, i32, ctypes.POINTER(attn_mask), ctypes.POINTER(sz)]
    lib.attn_blockmap_compact_bytes.restype = i32
    lib.attn_blockmap_compact_layout_of.argtypes = [i32, i32, ctypes.POINTER(attn_blockmap_layout)]
    lib.attn_blockmap_compact_layout_of.restype = i32
    lib.attn_blockmap_build_compact.argtypes = [i32, i32, ctypes.POINTER(attn_mask), vp, sz, vp]
    lib.attn_blockmap_build_compact.restype = i32
    lib.attn_blockmap_status.argtypes = [vp, sz, vp]
    lib.attn_blockmap_status.restype = i32
    lib.attn_check_args.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, ctypes.POINTER(attn_mask),
                                    vp, sz, ctypes.POINTER(attn_fp8), f32]
    lib.attn_check_args.restype = i32
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, ctypes.POINTER(attn_mask), vp, sz,
                             ctypes.POINTER(attn_fp8), f32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_check_args_gqa.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                        ctypes.POINTER(attn_mask), vp, sz, ctypes.POINTER(attn_fp8), f32]
    lib.attn_check_args_gqa.restype = i32
    lib.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, ctypes.POINTER(attn_mask),
                                 vp, sz, ctypes.POINTER(attn_fp8), f32, vp]
    lib.attn_fwd_gqa.restype = i32
    lib.attn_fwd_rescale_counts.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                            ctypes.POINTER(attn_mask), vp, sz, ctypes.POINTER(attn_fp8), f32, vp]
    lib.attn_fwd_rescale_counts.restype = i32
    lib.attn_varlen_workspace_bytes.argtypes = [i32, ctypes.POINTER(attn_mask), ctypes.POINTER(sz)]
    lib.attn_varlen_workspace_bytes.restype = i32
    lib.attn_varlen_layout_of.argtypes = [i32, ctypes.POINTER(attn_blockmap_layout)]
    lib.attn_varlen_layout_of.restype = i32
    lib.attn_varlen_prepare.argtypes = [vp, i32, i32, ctypes.POINTER(attn_mask), vp, sz, vp]
    lib.attn_varlen_prepare.restype = i32
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, ctypes.POINTER(attn_mask),
                                    vp, sz, ctypes.POINTER(attn_fp8), f32, vp]
    lib.attn_fwd_varlen.restype = i32
    lib.attn_fp8_quantize.argtypes = [vp, vp, vp, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_uint32), vp]
    lib.attn_fp8_quantize.restype = i32
    lib.attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                 ctypes.POINTER(attn_mask), vp, sz, vp]
    lib.attn_bwd_gqa.restype = i32
    lib.attn_bwd_gqa_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                         ctypes.POINTER(attn_mask), vp, sz, vp]
    lib.attn_bwd_gqa_noalloc.restype = i32
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, ctypes.POINTER(attn_mask),
                             vp, sz, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                    ctypes.POINTER(attn_mask), vp, sz, vp]
    lib.attn_bwd_varlen.restype = i32
    lib.attn_fwd_kernel_name.argtypes = [i32, i32, ctypes.POINTER(attn_mask), ctypes.POINTER(attn_fp8)]
    lib.attn_fwd_kernel_name.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_str(status: int) -> str:
    return load().attn_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_mask(flags: int = 0, window: int = 0, softcap: float = 0.0, doc_id=None, alibi_slopes=None):
    return attn_mask(int(flags), int(window), float(softcap), _ptr(doc_id), _ptr(alibi_slopes))


def make_fp8(q_scale, k_scale, v_scale, pv_mode: int = ATTN_PV_F16, qk_mode: int = ATTN_QK_BF16):
    return attn_fp8(_ptr(q_scale), _ptr(k_scale), _ptr(v_scale), int(pv_mode), int(qk_mode))


def attn_blockmap_bytes(B: int, N: int, mask: Optional[attn_mask] = None) -> int:
    out = ctypes.c_size_t(0)
    _check(load().attn_blockmap_bytes(B, N, ctypes.byref(mask) if mask else None, ctypes.byref(out)),
           "attn_blockmap_bytes")
    return out.value


def attn_blockmap_layout_of(B: int, N: int) -> dict:
    lay = attn_blockmap_layout()
    _check(load().attn_blockmap_layout_of(B, N, ctypes.byref(lay)), "attn_blockmap_layout_of")
    return {n: getattr(lay, n) for n, _ in attn_blockmap_layout._fields_}


def attn_varlen_layout_of(total: int) -> dict:
    """Offsets of the compact block map inside a packed batch's workspace (cls and idx 0:
    absent; the sequence ids start at `total`)."""
    lay = attn_blockmap_layout()
    _check(load().attn_varlen_layout_of(int(total), ctypes.byref(lay)), "attn_varlen_layout_of")
    return {n: getattr(lay, n) for n, _ in attn_blockmap_layout._fields_}


def attn_blockmap_build(B: int, N: int, mask: Optional[attn_mask], blockmap, stream=None) -> None:
    """Builds the block map into the uint8 device tensor `blockmap`."""
    _check(load().attn_blockmap_build(B, N, ctypes.byref(mask) if mask else None, _ptr(blockmap),
                                      blockmap.numel() * blockmap.element_size(), _stream(stream)),
           "attn_blockmap_build")


def attn_blockmap_compact_bytes(B: int, N: int, mask: Optional[attn_mask] = None) -> int:
    out = ctypes.c_size_t(0)
    _check(load().attn_blockmap_compact_bytes(B, N, ctypes.byref(mask) if mask else None, ctypes.byref(out)),
           "attn_blockmap_compact_bytes")
    return out.value


def attn_blockmap_compact_layout_of(B: int, N: int) -> dict:
    lay = attn_blockmap_layout()
    _check(load().attn_blockmap_compact_layout_of(B, N, ctypes.byref(lay)), "attn_blockmap_compact_layout_of")
    return {n: getattr(lay, n) for n, _ in attn_blockmap_layout._fields_}


def attn_blockmap_build_compact(B: int, N: int, mask: Optional[attn_mask], blockmap, stream=None) -> None:
    """Builds the compact block map (no class and list sections) into `blockmap`."""
    _check(load().attn_blockmap_build_compact(B, N, ctypes.byref(mask) if mask else None, _ptr(blockmap),
                                              blockmap.numel() * blockmap.element_size(), _stream(stream)),
           "attn_blockmap_build_compact")


def attn_blockmap_status(blockmap, stream=None) -> int:
    return load().attn_blockmap_status(_ptr(blockmap), blockmap.numel() * blockmap.element_size(),
                                       _stream(stream))


def attn_check_args(q, k, v, o, lse, B, H, N, d, scale, dtype, mask=None, blockmap=None, blockmap_bytes=0,
                    fp8=None, rescale_tau=8.0) -> int:
    """Host-side validation; pointers may be plain integers (no GPU needed)."""
    return load().attn_check_args(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                  int(dtype), ctypes.byref(mask) if mask else None, _ptr(blockmap),
                                  int(blockmap_bytes), ctypes.byref(fp8) if fp8 else None, float(rescale_tau))


def attn_check_args_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, dtype, mask=None, blockmap=None,
                        blockmap_bytes=0, fp8=None, rescale_tau=8.0) -> int:
    """attn_check_args with H_kv key/value heads shared by groups of H / H_kv query heads."""
    return load().attn_check_args_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, H_kv, N, d,
                                      float(scale), int(dtype), ctypes.byref(mask) if mask else None,
                                      _ptr(blockmap), int(blockmap_bytes), ctypes.byref(fp8) if fp8 else None,
                                      float(rescale_tau))


def attn_fwd_kernel_name(d: int, dtype: int = ATTN_BF16, mask: Optional[attn_mask] = None,
                         fp8: Optional[attn_fp8] = None) -> Optional[str]:
    """The compiled kernel variant attn_fwd selects (host logic only), or None."""
    r = load().attn_fwd_kernel_name(int(d), int(dtype), ctypes.byref(mask) if mask else None,
                                    ctypes.byref(fp8) if fp8 else None)
    return r.decode() if r is not None else None


def attn_fwd(q, k, v, o, lse, *, scale: float, dtype: int = ATTN_BF16, mask: Optional[attn_mask] = None,
             blockmap=None, fp8: Optional[attn_fp8] = None, rescale_tau: float = 8.0, stream=None) -> None:
    """Enqueues the forward pass.  q, k, v, o: [B][H][N][d] device tensors; lse: [B][H][N] fp32."""
    B, H, N, d = (int(x) for x in q.shape)
    mbytes = 0 if blockmap is None else blockmap.numel() * blockmap.element_size()
    _check(load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(dtype),
                           ctypes.byref(mask) if mask else None, _ptr(blockmap), mbytes,
                           ctypes.byref(fp8) if fp8 else None, float(rescale_tau), _stream(stream)),
           "attn_fwd")


def attn_fwd_gqa(q, k, v, o, lse, *, scale: float, dtype: int = ATTN_BF16, mask: Optional[attn_mask] = None,
                 blockmap=None, fp8: Optional[attn_fp8] = None, rescale_tau: float = 8.0, stream=None) -> None:
    """Grouped-query forward pass.  q, o: [B][H][N][d]; k, v: [B][H_kv][N][d]; lse: [B][H][N] fp32."""
    B, H, N, d = (int(x) for x in q.shape)
    H_kv = int(k.shape[1])
    mbytes = 0 if blockmap is None else blockmap.numel() * blockmap.element_size()
    _check(load().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, H_kv, N, d, float(scale),
                               int(dtype), ctypes.byref(mask) if mask else None, _ptr(blockmap), mbytes,
                               ctypes.byref(fp8) if fp8 else None, float(rescale_tau), _stream(stream)),
           "attn_fwd_gqa")


def attn_fwd_rescale_counts(q, k, v, o, lse, counts, *, scale: float, dtype: int = ATTN_BF16,
                            mask: Optional[attn_mask] = None, blockmap=None, fp8: Optional[attn_fp8] = None,
                            rescale_tau: float = 8.0, stream=None) -> None:
    """attn_fwd_gqa that also writes the rescale events of every query row into counts
    (int32 [B][H][N])."""
    B, H, N, d = (int(x) for x in q.shape)
    H_kv = int(k.shape[1])
    mbytes = 0 if blockmap is None else blockmap.numel() * blockmap.element_size()
    _check(load().attn_fwd_rescale_counts(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(counts), B, H, H_kv,
                                          N, d, float(scale), int(dtype), ctypes.byref(mask) if mask else None,
                                          _ptr(blockmap), mbytes, ctypes.byref(fp8) if fp8 else None,
                                          float(rescale_tau), _stream(stream)),
           "attn_fwd_rescale_counts")


def attn_varlen_workspace_bytes(total: int, mask: Optional[attn_mask] = None) -> int:
    n = ctypes.c_size_t()
    _check(load().attn_varlen_workspace_bytes(int(total), ctypes.byref(mask) if mask else None, ctypes.byref(n)),
           "attn_varlen_workspace_bytes")
    return n.value


def attn_varlen_prepare(cu_seqlens, total: int, mask: Optional[attn_mask], workspace, stream=None) -> None:
    """Sequence ids and block map of a packed batch; cu_seqlens: int32 device [nseq + 1]."""
    nseq = int(cu_seqlens.numel()) - 1
    _check(load().attn_varlen_prepare(_ptr(cu_seqlens), nseq, int(total), ctypes.byref(mask) if mask else None,
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)),
           "attn_varlen_prepare")


def attn_fwd_varlen(q, k, v, o, lse, *, scale: float, workspace, dtype: int = ATTN_BF16,
                    mask: Optional[attn_mask] = None, fp8: Optional[attn_fp8] = None, rescale_tau: float = 8.0,
                    stream=None) -> None:
    """Packed variable-length forward pass.  q, o: [H][total][d]; k, v: [H_kv][total][d];
    lse: [H][total]; workspace prepared by attn_varlen_prepare."""
    H, total, d = (int(x) for x in q.shape[-3:])
    H_kv = int(k.shape[-3])
    _check(load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, H_kv, total, d, float(scale),
                                  int(dtype), ctypes.byref(mask) if mask else None, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  ctypes.byref(fp8) if fp8 else None, float(rescale_tau), _stream(stream)),
           "attn_fwd_varlen")


def attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, *, scale: float, workspace,
                    mask: Optional[attn_mask] = None, stream=None) -> None:
    """Packed variable-length backward pass (bf16).  q, o, dout, dq: [H][total][d]; k, v, dk,
    dv: [H_kv][total][d]; lse, delta: [H][total]; workspace prepared by attn_varlen_prepare."""
    H, total, d = (int(x) for x in q.shape[-3:])
    H_kv = int(k.shape[-3])
    _check(load().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(delta), H, H_kv, total, d, float(scale),
                                  ctypes.byref(mask) if mask else None, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "attn_bwd_varlen")


def attn_fp8_quantize(x, codes, scales, rotate_signs=None, stream=None) -> None:
    """Block-quantise bf16 x [B][H][N][d] to e4m3 codes (uint8, same shape) and fp32 scales
    [B][H][ceil(N/128)] on the device; rotate_signs: d/32 sign words (host) or None."""
    B, H, N, d = (int(t) for t in x.shape)
    sg = None
    if rotate_signs is not None:
        words = [int(w) & 0xFFFFFFFF for w in rotate_signs]
        if len(words) != d // 32:
            raise ValueError(f"rotate_signs needs {d // 32} words")
        sg = (ctypes.c_uint32 * len(words))(*words)
    _check(load().attn_fp8_quantize(_ptr(x), _ptr(codes), _ptr(scales), B, H, N, d, sg, _stream(stream)),
           "attn_fp8_quantize")


def attn_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, *, scale: float, mask: Optional[attn_mask] = None,
                 blockmap=None, stream=None) -> None:
    """Backward pass (bf16).  q, o, dout, dq: [B][H][N][d]; k, v, dk, dv: [B][H_kv][N][d];
    lse: the forward call's [B][H][N] fp32; delta: [B][H][N] fp32 scratch."""
    B, H, N, d = (int(x) for x in q.shape)
    H_kv = int(k.shape[1])
    mbytes = 0 if blockmap is None else blockmap.numel() * blockmap.element_size()
    _check(load().attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(delta), B, H, H_kv, N, d, float(scale),
                               ctypes.byref(mask) if mask else None, _ptr(blockmap), mbytes, _stream(stream)),
           "attn_bwd_gqa")


def attn_bwd_gqa_noalloc(q, k, v, o, lse, dout, dq, dk, dv, *, scale: float, mask: Optional[attn_mask] = None,
                         blockmap=None, stream=None) -> None:
    """attn_bwd_gqa without the delta workspace: the row sums live in the library's per-GPU
    scratch array (no allocation; calls overlapping on one GPU race)."""
    B, H, N, d = (int(x) for x in q.shape)
    H_kv = int(k.shape[1])
    mbytes = 0 if blockmap is None else blockmap.numel() * blockmap.element_size()
    _check(load().attn_bwd_gqa_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, H, H_kv, N, d, float(scale),
                                       ctypes.byref(mask) if mask else None, _ptr(blockmap), mbytes,
                                       _stream(stream)),
           "attn_bwd_gqa_noalloc")


def read_blockmap(blockmap, B: int, N: int, compact: bool = False) -> dict:
    """Splits a block map copied back to the host into its sections (numpy); the compact
    form has no "cls" and "idx" (None)."""
    raw = blockmap.detach().cpu().numpy() if hasattr(blockmap, "detach") else np.asarray(blockmap)
    raw = raw.view(np.uint8)
    lay = attn_blockmap_compact_layout_of(B, N) if compact else attn_blockmap_layout_of(B, N)
    nb = (N + 127) // 128
    hdr = raw[:64].view(np.int32)

    def sec(name, dtype, shape):
        if compact and name in ("cls", "idx"):
            return None
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return raw[lay[name]:lay[name] + n].view(dtype).reshape(shape)

    return dict(header=dict(magic=int(hdr.view(np.uint32)[0]), B=int(hdr[1]), N=int(hdr[2]), nqb=int(hdr[3]),
                            nkb=int(hdr[4]), flags=int(hdr.view(np.uint32)[5]), window=int(hdr[6]),
                            order_full_cost=int(hdr[7]), order_partial_cost=int(hdr[8]), compact=int(hdr[9])),
                cls=sec("cls", np.uint8, (B, nb, nb)), counts=sec("counts", np.int32, (B, nb, 2)),
                idx=sec("idx", np.int32, (B, nb, 2, nb)), row_lo=sec("row_lo", np.int32, (B, N)),
                row_hi=sec("row_hi", np.int32, (B, N)), col_lo=sec("col_lo", np.int32, (B, N)),
                col_hi=sec("col_hi", np.int32, (B, N)), pairs=sec("pairs", np.int64, (B, nb)),
                status=sec("status", np.int32, (B, nb)), order=sec("order", np.int32, (B * nb,)))
