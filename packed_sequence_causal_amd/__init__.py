"""Sample packing and document-causal attention on MI355X (gfx950).

Thin ctypes binding over ``libpsc.so`` (C ABI in ``include/psc.h``).  It only
marshals arguments: torch tensors provide device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: without the built library every call raises.
``PSC_LIBRARY`` (environment) names another build of the library to load
instead of the in-tree ``libpsc.so`` (the host-sanitizer test uses it).

Entry points (same names as the C ABI without the ``psc_`` prefix):
  pack_sizes, pack_build                  build_pack / build_unpack on the GPU
  varlen_attn_workspace, varlen_attn_fwd, varlen_attn_bwd
                                          document-causal attention (bf16 or fp32)
  varlen_attn_fwd_noalloc                 the forward with the library's own scratch
  varlen_attn_fwd_rope, varlen_attn_bwd_rope
                                          attention with the rotary embedding fused in
  check_cu_seqlens, cu_seqlens_status     device check of the cu_seqlens precondition
  rope                                    rotary embedding at the packer's indexes
  row_max_seqlen, unpack_data, split_sequence
                                          data steps after the packer
  timing_enable, timing_select, timing_reset, timing_read
                                          per-kernel HIP-event timing
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PACK, UNPACK = 0, 1
F32, BF16 = 0, 1

OK = 0
ERR_INVALID = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_CAPACITY = -4
ERR_HIP = -5

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PSC_LIBRARY") or os.path.join(_HERE, "libpsc.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libpsc_debug.so")
_libs = {}

_c_i64p = ctypes.POINTER(ctypes.c_int64)
_c_sizep = ctypes.POINTER(ctypes.c_size_t)
_vp = ctypes.c_void_p

_SIGNATURES = {
    "psc_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "psc_version": (ctypes.c_int, []),
    "psc_pack_sizes": (ctypes.c_int, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32, _c_i64p, _c_i64p, _c_sizep]),
    "psc_pack_build": (ctypes.c_int, [ctypes.c_int, _vp, _vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int64, _vp, _vp, _vp, _vp, ctypes.c_int64, _vp,
                                      _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "psc_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "psc_timing_select": (ctypes.c_int, [ctypes.c_uint32]),
    "psc_timing_reset": (ctypes.c_int, []),
    "psc_timing_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double), _c_i64p]),
    "psc_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
    "psc_varlen_attn_workspace": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 _c_sizep]),
    "psc_varlen_attn_fwd": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _vp,
                                           ctypes.c_int64, _vp, _vp, ctypes.c_size_t, _vp]),
    "psc_varlen_attn_fwd_noalloc": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.c_int64, _vp, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_float, _vp, ctypes.c_int64, _vp, _vp]),
    "psc_varlen_attn_bwd": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp]),
    "psc_varlen_attn_fwd_rope": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_float,
                                                ctypes.c_float, _vp, ctypes.c_int64, _vp, _vp, ctypes.c_size_t, _vp]),
    "psc_varlen_attn_bwd_rope": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_float,
                                                ctypes.c_float, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "psc_check_cu_seqlens": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int64, _vp, _vp]),
    "psc_cu_seqlens_status": (ctypes.c_int, [ctypes.c_int32]),
    "psc_debug_checks": (ctypes.c_int, []),
    "psc_row_max_seqlen": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, ctypes.c_int64, _vp, _vp]),
    "psc_unpack_data": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_int64, _vp, _vp,
                                       ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]),
    "psc_split_sequence": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp,
                                          _vp]),
    "psc_rope": (ctypes.c_int, [ctypes.c_int, _vp, ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_int64,
                                ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_float, ctypes.c_int,
                                _vp]),
}


class PscError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


def lib(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpsc.so, or the library at `path` (raises if it was not built)."""
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing; build it with __graft_entry__.build() "
                               "or python -m packed_sequence_causal_amd.build --debug")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _libs[path] = L
    return _libs[path]


def debug_lib() -> ctypes.CDLL:
    """libpsc_debug.so: the same library built with device checks of
    cu_seqlens before every attention launch."""
    return lib(DEBUG_LIB_PATH)


def strerror(status: int) -> str:
    return lib().psc_strerror(status).decode()


def _check(status: int, where: str):
    if status != OK:
        raise PscError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which the binding allocates: the caller's stream when one is
    given, so torch's caching allocator never hands a block the kernels still
    use on `stream` to work on another stream."""
    import contextlib

    import torch

    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _expect(t, name, shape, dtype, device):
    """Raise ValueError unless t is a contiguous tensor of this shape and dtype
    on `device` (the C ABI only sees a pointer and writes the full extent)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}; got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device} (contiguous={t.is_contiguous()})")


# ------------------------------------------------------------------ packing

def pack_sizes(mode: int, n_docs: int, n_tokens: int, micro_bsz: int, seq_len: int):
    """(n_rows, max_segments, workspace_bytes) for pack_build."""
    rows, segs, ws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib().psc_pack_sizes(mode, n_docs, n_tokens, micro_bsz, seq_len, ctypes.byref(rows),
                                ctypes.byref(segs), ctypes.byref(ws)), "psc_pack_sizes")
    return rows.value, segs.value, ws.value


def pack_build(tokens, doc_offsets, micro_bsz: int, seq_len: int, mode: int = PACK, out: Optional[dict] = None,
               workspace=None, stream=None) -> dict:
    """Pack documents on the GPU.

    tokens: int32 [n_tokens] device tensor; doc_offsets: int64 [n_docs + 1].
    Returns device tensors input_ids, labels, indexes [n_rows, PL],
    cu_seqlens [max_segments + 1] (valid up to stats[0]), row_seg_ptr
    [n_rows + 1], row_valid_len [n_rows], stats [4] (n_seg, max_seqlen,
    rows_filled, 0).  Pass ``out`` (a previous result) and ``workspace`` to
    reuse buffers.
    """
    import torch

    n_docs = doc_offsets.numel() - 1
    n_tokens = tokens.numel()
    rows, segs, ws = pack_sizes(mode, n_docs, n_tokens, micro_bsz, seq_len)
    dev = tokens.device
    PL = micro_bsz * seq_len
    with _on(stream):
        if out is None:
            i32 = dict(dtype=torch.int32, device=dev)
            out = {
                "input_ids": torch.empty(rows, PL, **i32),
                "labels": torch.empty(rows, PL, **i32),
                "indexes": torch.empty(rows, PL, **i32),
                "cu_seqlens": torch.empty(segs + 1, **i32),
                "row_seg_ptr": torch.empty(rows + 1, **i32),
                "row_valid_len": torch.empty(max(rows, 1), **i32),
                "stats": torch.empty(4, **i32),
            }
        workspace = _workspace(workspace, ws, dev)
    _check(lib().psc_pack_build(mode, _ptr(tokens), _ptr(doc_offsets), n_docs, n_tokens, micro_bsz, seq_len,
                                rows, _ptr(out["input_ids"]), _ptr(out["labels"]), _ptr(out["indexes"]),
                                _ptr(out["cu_seqlens"]), out["cu_seqlens"].numel() - 1,
                                _ptr(out["row_seg_ptr"]), _ptr(out["row_valid_len"]), _ptr(out["stats"]),
                                _ptr(workspace), workspace.numel(), _stream(stream)), "psc_pack_build")
    out["_workspace"] = workspace
    return out


# ---------------------------------------------------------------- attention

def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tok_stride(t, name):
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [T, heads, D] with unit dim stride and head stride D")
    return t.stride(0)


def varlen_attn_workspace(pass_: int, dtype: int, total_tokens: int, n_segments: int, max_seqlen: int,
                          hq: int, hkv: int, head_dim: int, library=None) -> int:
    """Workspace bytes of pass 0 (forward), 1 (backward), 2 (rotary forward)
    or 3 (rotary backward); `library` as in the calls (the debug library's
    are longer)."""
    b = ctypes.c_size_t()
    _check((library or lib()).psc_varlen_attn_workspace(pass_, dtype, total_tokens, n_segments, max_seqlen, hq, hkv, head_dim,
                                           ctypes.byref(b)), "psc_varlen_attn_workspace")
    return b.value


def _workspace(workspace, need: int, device):
    """The caller's workspace, checked, or a new one of `need` bytes (on the
    current stream: call inside the stream context)."""
    import torch

    if workspace is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if (workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous()
            or workspace.device != device):
        raise ValueError(f"workspace must be a contiguous 1-D uint8 tensor on {device}")
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes; this call needs {need}")
    return workspace


def _check_inputs(q, k, v, cu_seqlens, nseg):
    import torch

    T, hq, D = q.shape
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or t.shape[0] != T or t.shape[2] != D or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be [T, hkv, D] with q's T, D, dtype and device")
    if v.shape[1] != k.shape[1]:
        raise ValueError("k and v must have the same number of heads")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor on q's device")
    if cu_seqlens.numel() < nseg + 1:
        raise ValueError("cu_seqlens must hold n_segments + 1 entries")


def varlen_attn_fwd(q, k, v, cu_seqlens, max_seqlen: int, n_segments: Optional[int] = None,
                    softmax_scale: Optional[float] = None, out=None, lse=None, workspace=None, stream=None,
                    library=None):
    """Forward pass.  q [T,hq,D], k/v [T,hkv,D] (views allowed), cu_seqlens
    int32 [n_segments + 1].  Returns (out [T,hq,D], lse float32 [hq,T])."""
    import torch

    T, hq, D = q.shape
    hkv = k.shape[1]
    dt = _dtype_code(q)
    nseg = cu_seqlens.numel() - 1 if n_segments is None else n_segments
    _check_inputs(q, k, v, cu_seqlens, nseg)
    L = library or lib()
    b = ctypes.c_size_t()
    _check(L.psc_varlen_attn_workspace(0, dt, T, nseg, max_seqlen, hq, hkv, D, ctypes.byref(b)),
           "psc_varlen_attn_workspace")
    ws = b.value
    with _on(stream):
        if out is None:
            out = torch.empty(T, hq, D, dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty(hq, T, dtype=torch.float32, device=q.device)
        workspace = _workspace(workspace, ws, q.device)
    if out.dim() != 3 or tuple(out.shape) != (T, hq, D) or out.dtype != q.dtype or out.device != q.device:
        raise ValueError(f"out must be a {q.dtype} [T, hq, D] = {(T, hq, D)} tensor on {q.device}")
    _expect(lse, "lse", (hq, T), torch.float32, q.device)
    _check(L.psc_varlen_attn_fwd(dt, _ptr(q), _ptr(k), _ptr(v), _tok_stride(q, "q"), _tok_stride(k, "k"),
                                     _tok_stride(v, "v"), _ptr(cu_seqlens), nseg, max_seqlen, T, hq, hkv, D,
                                     float(softmax_scale or 0.0), _ptr(out), _tok_stride(out, "out"), _ptr(lse),
                                     _ptr(workspace), workspace.numel(), _stream(stream)), "psc_varlen_attn_fwd")
    return out, lse


def varlen_attn_fwd_noalloc(q, k, v, cu_seqlens, max_seqlen: int, n_segments: Optional[int] = None,
                            softmax_scale: Optional[float] = None, out=None, lse=None, stream=None):
    """varlen_attn_fwd through psc_varlen_attn_fwd_noalloc: the library keeps
    the schedule in its own per-GPU scratch, so a caller that passes out and
    lse makes the call allocate nothing (calls overlapping on one GPU race)."""
    import torch

    T, hq, D = q.shape
    hkv = k.shape[1]
    dt = _dtype_code(q)
    nseg = cu_seqlens.numel() - 1 if n_segments is None else n_segments
    _check_inputs(q, k, v, cu_seqlens, nseg)
    with _on(stream):
        if out is None:
            out = torch.empty(T, hq, D, dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty(hq, T, dtype=torch.float32, device=q.device)
    if out.dim() != 3 or tuple(out.shape) != (T, hq, D) or out.dtype != q.dtype or out.device != q.device:
        raise ValueError(f"out must be a {q.dtype} [T, hq, D] = {(T, hq, D)} tensor on {q.device}")
    _expect(lse, "lse", (hq, T), torch.float32, q.device)
    _check(lib().psc_varlen_attn_fwd_noalloc(dt, _ptr(q), _ptr(k), _ptr(v), _tok_stride(q, "q"),
                                             _tok_stride(k, "k"), _tok_stride(v, "v"), _ptr(cu_seqlens), nseg,
                                             max_seqlen, T, hq, hkv, D, float(softmax_scale or 0.0), _ptr(out),
                                             _tok_stride(out, "out"), _ptr(lse), _stream(stream)),
           "psc_varlen_attn_fwd_noalloc")
    return out, lse


def varlen_attn_bwd(q, k, v, out, dout, lse, cu_seqlens, max_seqlen: int, n_segments: Optional[int] = None,
                    softmax_scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None,
                    stream=None, grad_dtype: Optional[int] = None, library=None):
    """Backward pass.  Returns (dq [T,hq,D], dk [T,hkv,D], dv [T,hkv,D]) in
    float32, or bf16 with grad_dtype=BF16 (bf16 inputs only)."""
    import torch

    T, hq, D = q.shape
    hkv = k.shape[1]
    dt = _dtype_code(q)
    gdt = F32 if grad_dtype is None else grad_dtype
    nseg = cu_seqlens.numel() - 1 if n_segments is None else n_segments
    _check_inputs(q, k, v, cu_seqlens, nseg)
    for name, t in (("out", out), ("dout", dout)):
        if t.dim() != 3 or tuple(t.shape) != (T, hq, D) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be a {q.dtype} [T, hq, D] = {(T, hq, D)} tensor on {q.device}")
    _expect(lse, "lse", (hq, T), torch.float32, q.device)
    gtype = torch.bfloat16 if gdt == BF16 else torch.float32
    L = library or lib()
    b = ctypes.c_size_t()
    _check(L.psc_varlen_attn_workspace(1, dt, T, nseg, max_seqlen, hq, hkv, D, ctypes.byref(b)),
           "psc_varlen_attn_workspace")
    ws = b.value
    with _on(stream):
        g = dict(dtype=gtype, device=q.device)
        dq = torch.empty(T, hq, D, **g) if dq is None else dq
        dk = torch.empty(T, hkv, D, **g) if dk is None else dk
        dv = torch.empty(T, hkv, D, **g) if dv is None else dv
        workspace = _workspace(workspace, ws, q.device)
    _expect(dq, "dq", (T, hq, D), gtype, q.device)
    _expect(dk, "dk", (T, hkv, D), gtype, q.device)
    _expect(dv, "dv", (T, hkv, D), gtype, q.device)
    _check(L.psc_varlen_attn_bwd(dt, gdt, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                     _tok_stride(q, "q"), _tok_stride(k, "k"), _tok_stride(v, "v"),
                                     _tok_stride(out, "out"), _tok_stride(dout, "dout"), _ptr(cu_seqlens), nseg,
                                     max_seqlen, T, hq, hkv, D, float(softmax_scale or 0.0), _ptr(dq), _ptr(dk),
                                     _ptr(dv), _ptr(workspace), workspace.numel(), _stream(stream)),
           "psc_varlen_attn_bwd")
    return dq, dk, dv


def _positions(positions, T, device):
    import torch

    if positions.dtype != torch.int32 or positions.device != device or not positions.is_contiguous() \
            or positions.numel() != T:
        raise ValueError("positions must be a contiguous int32 tensor with one entry per token on q's device")


def varlen_attn_fwd_rope(q, k, v, cu_seqlens, max_seqlen: int, positions, rope_base: float = 10000.0,
                         n_segments: Optional[int] = None, softmax_scale: Optional[float] = None, out=None, lse=None,
                         workspace=None, stream=None):
    """Attention of q, k rotated by positions (the packer's indexes), with the
    rotation fused in.  q and k are rotated IN PLACE (they then hold the
    rotated q~, k~ for varlen_attn_bwd_rope).  Returns (out, lse)."""
    import torch

    T, hq, D = q.shape
    hkv = k.shape[1]
    dt = _dtype_code(q)
    nseg = cu_seqlens.numel() - 1 if n_segments is None else n_segments
    _check_inputs(q, k, v, cu_seqlens, nseg)
    _positions(positions, T, q.device)
    ws = varlen_attn_workspace(2, dt, T, nseg, max_seqlen, hq, hkv, D)
    with _on(stream):
        if out is None:
            out = torch.empty(T, hq, D, dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty(hq, T, dtype=torch.float32, device=q.device)
        workspace = _workspace(workspace, ws, q.device)
    if out.dim() != 3 or tuple(out.shape) != (T, hq, D) or out.dtype != q.dtype or out.device != q.device:
        raise ValueError(f"out must be a {q.dtype} [T, hq, D] = {(T, hq, D)} tensor on {q.device}")
    _expect(lse, "lse", (hq, T), torch.float32, q.device)
    _check(lib().psc_varlen_attn_fwd_rope(dt, _ptr(q), _ptr(k), _ptr(v), _tok_stride(q, "q"), _tok_stride(k, "k"),
                                          _tok_stride(v, "v"), _ptr(cu_seqlens), nseg, max_seqlen, T, hq, hkv, D,
                                          _ptr(positions), float(rope_base), float(softmax_scale or 0.0), _ptr(out),
                                          _tok_stride(out, "out"), _ptr(lse), _ptr(workspace), workspace.numel(),
                                          _stream(stream)), "psc_varlen_attn_fwd_rope")
    return out, lse


def varlen_attn_bwd_rope(q_rot, k_rot, v, out, dout, lse, cu_seqlens, max_seqlen: int, positions,
                         rope_base: float = 10000.0, n_segments: Optional[int] = None,
                         softmax_scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None,
                         stream=None, grad_dtype: Optional[int] = None):
    """Gradients with respect to the unrotated q, k (and v), from the rotated
    q~, k~ that varlen_attn_fwd_rope left; the turn back is fused into the
    dQ and dK kernels.  Returns (dq, dk, dv)."""
    import torch

    T, hq, D = q_rot.shape
    hkv = k_rot.shape[1]
    dt = _dtype_code(q_rot)
    gdt = F32 if grad_dtype is None else grad_dtype
    nseg = cu_seqlens.numel() - 1 if n_segments is None else n_segments
    _check_inputs(q_rot, k_rot, v, cu_seqlens, nseg)
    _positions(positions, T, q_rot.device)
    for name, t in (("out", out), ("dout", dout)):
        if t.dim() != 3 or tuple(t.shape) != (T, hq, D) or t.dtype != q_rot.dtype or t.device != q_rot.device:
            raise ValueError(f"{name} must be a {q_rot.dtype} [T, hq, D] = {(T, hq, D)} tensor on {q_rot.device}")
    _expect(lse, "lse", (hq, T), torch.float32, q_rot.device)
    gtype = torch.bfloat16 if gdt == BF16 else torch.float32
    ws = varlen_attn_workspace(3, dt, T, nseg, max_seqlen, hq, hkv, D)
    with _on(stream):
        g = dict(dtype=gtype, device=q_rot.device)
        dq = torch.empty(T, hq, D, **g) if dq is None else dq
        dk = torch.empty(T, hkv, D, **g) if dk is None else dk
        dv = torch.empty(T, hkv, D, **g) if dv is None else dv
        workspace = _workspace(workspace, ws, q_rot.device)
    _expect(dq, "dq", (T, hq, D), gtype, q_rot.device)
    _expect(dk, "dk", (T, hkv, D), gtype, q_rot.device)
    _expect(dv, "dv", (T, hkv, D), gtype, q_rot.device)
    _check(lib().psc_varlen_attn_bwd_rope(dt, gdt, _ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(out), _ptr(dout),
                                          _ptr(lse), _tok_stride(q_rot, "q"), _tok_stride(k_rot, "k"),
                                          _tok_stride(v, "v"), _tok_stride(out, "out"), _tok_stride(dout, "dout"),
                                          _ptr(cu_seqlens), nseg, max_seqlen, T, hq, hkv, D, _ptr(positions),
                                          float(rope_base), float(softmax_scale or 0.0), _ptr(dq), _ptr(dk), _ptr(dv),
                                          _ptr(workspace), workspace.numel(), _stream(stream)),
           "psc_varlen_attn_bwd_rope")
    return dq, dk, dv


def check_cu_seqlens(cu_seqlens, total_tokens: int, n_segments: Optional[int] = None, flags=None, stream=None,
                     library=None):
    """Enqueue the device check of cu_seqlens (0 = c_0 < ... < c_n = T);
    returns the int32 [1] flags tensor it writes (0 when the array is valid,
    else the OR of CU_BAD_START, CU_BAD_END, CU_NOT_INCREASING)."""
    import torch

    nseg = cu_seqlens.numel() - 1 if n_segments is None else n_segments
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < nseg + 1:
        raise ValueError("cu_seqlens must be a contiguous int32 tensor with n_segments + 1 entries")
    with _on(stream):
        flags = torch.empty(1, dtype=torch.int32, device=cu_seqlens.device) if flags is None else flags
    _expect(flags, "flags", (1,), torch.int32, cu_seqlens.device)
    _check((library or lib()).psc_check_cu_seqlens(_ptr(cu_seqlens), nseg, total_tokens, _ptr(flags),
                                                  _stream(stream)), "psc_check_cu_seqlens")
    return flags


CU_BAD_START, CU_BAD_END, CU_NOT_INCREASING = 1, 2, 4


def cu_seqlens_status(flags: int) -> int:
    """OK for a flags word of 0 from check_cu_seqlens, ERR_INVALID otherwise."""
    return lib().psc_cu_seqlens_status(int(flags))


# ---------------------------------------------------------- instrumentation

def row_max_seqlen(packed: dict, out=None, stream=None):
    """packed_data_normalizer's max_seqlen of every row of pack_build's output
    (int32 [n_rows])."""
    import torch

    n_rows = packed["row_seg_ptr"].numel() - 1
    if out is None:
        out = torch.empty(n_rows, dtype=torch.int32, device=packed["cu_seqlens"].device)
    _check(lib().psc_row_max_seqlen(_ptr(packed["cu_seqlens"]), packed["cu_seqlens"].numel(),
                                    _ptr(packed["row_seg_ptr"]), n_rows, _ptr(out), _stream(stream)),
           "psc_row_max_seqlen")
    return out


def unpack_data(packed: dict, micro_bsz: int, seq_len: int, out_ids=None, out_labels=None, stream=None):
    """unpack_data of pack_build's output: (input_ids, labels) int32
    [n_rows * micro_bsz, seq_len], one document per row."""
    import torch

    ids = packed["input_ids"]
    n_rows, PL = ids.shape
    rvl = packed.get("row_valid_len")
    if rvl is None:
        raise ValueError("unpack_data needs the packer's row_valid_len")
    i32 = dict(dtype=torch.int32, device=ids.device)
    out_ids = torch.empty(n_rows * micro_bsz, seq_len, **i32) if out_ids is None else out_ids
    out_labels = torch.empty(n_rows * micro_bsz, seq_len, **i32) if out_labels is None else out_labels
    _check(lib().psc_unpack_data(_ptr(ids), _ptr(packed["labels"]), n_rows, PL, _ptr(packed["cu_seqlens"]),
                                 packed["cu_seqlens"].numel(), _ptr(packed["row_seg_ptr"]), _ptr(rvl), micro_bsz,
                                 seq_len, _ptr(out_ids), _ptr(out_labels), _stream(stream)), "psc_unpack_data")
    return out_ids, out_labels


def split_sequence(x, tp: int, rank: int, out=None, stream=None):
    """split_data_sequence_parallel of an int32 [rows, length] tensor: rank
    `rank` of `tp` gets [rows, length / tp]."""
    import torch

    if x.dim() != 2 or not x.is_contiguous() or x.dtype != torch.int32:
        raise ValueError("x must be a contiguous int32 [rows, length] tensor")
    rows, length = x.shape
    if tp < 1 or length % tp:
        raise ValueError("length must be a multiple of tp")
    out = torch.empty(rows, length // tp, dtype=torch.int32, device=x.device) if out is None else out
    _check(lib().psc_split_sequence(_ptr(x), rows, length, tp, rank, _ptr(out), _stream(stream)),
           "psc_split_sequence")
    return out


def rope(q, k, positions, base: float = 10000.0, inverse: bool = False, stream=None):
    """Rotate q [T,hq,D] and k [T,hkv,D] (or None) in place by positions int32
    [T] (the packer's indexes); inverse=True applies the backward rotation.
    Returns (q, k)."""
    T, hq, D = q.shape
    hkv = 0 if k is None else k.shape[1]
    if k is not None and (k.shape[0] != T or k.shape[2] != D or k.dtype != q.dtype):
        raise ValueError("q and k must agree in tokens, head dim and dtype")
    if positions.numel() != T:
        raise ValueError("positions must have one entry per token")
    _check(lib().psc_rope(_dtype_code(q), _ptr(q), _tok_stride(q, "q"), hq, _ptr(k),
                          0 if k is None else _tok_stride(k, "k"), hkv, T, D, _ptr(positions), float(base),
                          1 if inverse else 0, _stream(stream)), "psc_rope")
    return q, k


KERNELS = {"pack": 0, "attn_schedule": 1, "attn_fwd": 2, "attn_bwd_pre": 3, "attn_bwd_dkdv": 4, "attn_bwd_dq": 5,
           "rope": 6, "data_steps": 7}


def timing_enable(on: bool = True):
    _check(lib().psc_timing_enable(1 if on else 0), "psc_timing_enable")


def timing_select(kernels=None):
    """Time only the named kernels (names as in KERNELS) while timing is on;
    None times every kernel."""
    mask = 0xFFFFFFFF if kernels is None else sum(1 << KERNELS[k] for k in kernels)
    _check(lib().psc_timing_select(mask), "psc_timing_select")


def timing_reset():
    _check(lib().psc_timing_reset(), "psc_timing_reset")


def timing_read() -> dict:
    """{kernel name: (total_ms, launches)} since the last reset; waits for the
    recorded events."""
    out = {}
    for name, kid in KERNELS.items():
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(lib().psc_timing_read(kid, ctypes.byref(ms), ctypes.byref(n)), "psc_timing_read")
        out[name] = (ms.value, n.value)
    return out
