"""Exact blockwise (ring) softmax attention on MI355X -- Python binding of libra.

Every step of the computation runs in libra's gfx950 HIP kernels; this module only
marshals torch tensors (device memory) and the current HIP stream into the C ABI
declared in ``include/ra.h``.  There is no fallback: if ``libra.so`` is missing or a
call fails, an exception is raised.

Calls (names as in the C ABI, without the ``ra_`` prefix):

* ``attn_fwd(q, k, v, causal=..., num_chunks=..., start_chunk=..., q_offset=...,
  kv_offset=..., scale=...) -> (o, lse)``
* ``lse_merge(o_parts, lse_parts) -> (o, lse)``
* ``ulysses_permute(src, P, rank, dir) -> dst``
* ``attn_bwd(q, k, v, o, dout, lse, ...) -> (dq, dk, dv)``
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "attn_fwd", "lse_merge", "ulysses_permute", "attn_bwd", "attn_bwd_workspace_size",
    "attn_fwd_validate", "lse_merge_validate", "ulysses_permute_validate", "attn_bwd_validate",
    "status_string", "version", "lib", "LIB_PATH", "RaError", "STATUS",
    "attn_fwd_varlen", "attn_fwd_varlen_validate", "attn_bwd_varlen", "attn_bwd_varlen_validate",
    "attn_bwd_accum", "attn_bwd_accum_validate", "ring_attn_bwd_chunked",
    "fp8_quantize", "fp8_quantize_validate", "attn_fwd_fp8", "attn_fwd_fp8_validate",
    "ring_attn_fp8_chunked", "ulysses_permute_multi", "ulysses_permute_multi_validate",
    "attn_bwd_noalloc", "noalloc_scratch_bytes", "fp8_quantize_multi",
    "fp8_quantize_multi_validate",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")

STATUS = {
    0: "RA_OK", -1: "RA_ERR_NULL", -2: "RA_ERR_DTYPE", -3: "RA_ERR_SHAPE", -4: "RA_ERR_STRIDE",
    -5: "RA_ERR_ALIGN", -6: "RA_ERR_RANGE", -7: "RA_ERR_UNSUPPORTED", -8: "RA_ERR_HIP",
    -9: "RA_ERR_WORKSPACE", -10: "RA_ERR_SCRATCH",
}
RA_F32, RA_BF16, RA_FP8_E4M3 = 0, 1, 2
MAX_MERGE_PARTS = 64


class RaError(RuntimeError):
    """A libra call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.name = STATUS.get(status, str(status))


class RaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class RaAttnParams(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("causal", ctypes.c_int32),
                ("num_chunks", ctypes.c_int32), ("start_chunk", ctypes.c_int32),
                ("q_offset", ctypes.c_int64), ("kv_offset", ctypes.c_int64),
                ("scale", ctypes.c_float), ("sched", ctypes.c_void_p)]


# One zero-initialised uint64 work counter per (device, stream) for the bf16 forward's
# tile order (ra_attn_params.sched): calls on one stream never overlap, and every call
# leaves the counter as it found it.
_SCHED = {}


def _sched_counter(t: torch.Tensor) -> int:
    key = (t.device.index, torch.cuda.current_stream(t.device).cuda_stream)
    c = _SCHED.get(key)
    if c is None:
        c = torch.zeros(1, dtype=torch.int64, device=t.device)
        _SCHED[key] = c
    return c.data_ptr()


_LIB = None
_P = ctypes.POINTER


def lib() -> ctypes.CDLL:
    """The loaded libra.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libra.so not found at {LIB_PATH}; build it with "
                               "`python -m long_context_exact_tiled_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        T, PP = _P(RaTensor), _P(RaAttnParams)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sigs = {
            "ra_attn_fwd": [T, T, T, PP, T, T, vp],
            "ra_attn_fwd_validate": [T, T, T, PP, T, T],
            "ra_attn_fwd_varlen": [T, T, T, vp, i32, PP, T, T, vp],
            "ra_attn_fwd_varlen_validate": [T, T, T, vp, i32, PP, T, T],
            "ra_lse_merge": [i32, T, T, T, T, vp],
            "ra_lse_merge_validate": [i32, T, T, T, T],
            "ra_ulysses_permute": [T, T, i32, i32, i32, vp],
            "ra_ulysses_permute_validate": [T, T, i32, i32, i32],
            "ra_ulysses_permute_n": [i32, T, T, i32, i32, i32, vp],
            "ra_ulysses_permute_n_validate": [i32, T, T, i32, i32, i32],
            "ra_attn_bwd": [T, T, T, T, T, T, PP, T, T, T, vp, sz, vp],
            "ra_attn_bwd_validate": [T, T, T, T, T, T, PP, T, T, T],
            "ra_attn_bwd_noalloc": [T, T, T, T, T, T, PP, T, T, T, vp],
            "ra_noalloc_scratch_bytes": [],
            "ra_attn_bwd_varlen": [T, T, T, T, T, T, vp, i32, PP, T, T, T, vp, sz, vp],
            "ra_attn_bwd_varlen_validate": [T, T, T, T, T, T, vp, i32, PP, T, T, T],
            "ra_attn_bwd_workspace_size": [T, T, PP],
            "ra_attn_bwd_accum": [T, T, T, T, T, T, PP, T, T, T, vp, sz, vp],
            "ra_attn_bwd_accum_validate": [T, T, T, T, T, T, PP, T, T, T],
            "ra_fp8_quantize": [T, T, T, i32, vp, sz, vp],
            "ra_fp8_quantize_validate": [T, T, T, i32],
            "ra_fp8_quantize_workspace_size": [T],
            "ra_fp8_quantize_n": [i32, T, T, T, vp, vp, sz, vp],
            "ra_fp8_quantize_n_validate": [i32, T, T, T, vp],
            "ra_fp8_quantize_n_workspace_size": [i32, T],
            "ra_attn_fwd_fp8": [T, T, T, T, T, T, PP, T, T, vp],
            "ra_attn_fwd_fp8_validate": [T, T, T, T, T, T, PP, T, T],
            "ra_status_string": [ctypes.c_int],
            "ra_version": [],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.ra_attn_bwd_workspace_size.restype = ctypes.c_size_t
        L.ra_fp8_quantize_workspace_size.restype = ctypes.c_size_t
        L.ra_fp8_quantize_n_workspace_size.restype = ctypes.c_size_t
        L.ra_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.ra_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().ra_status_string(int(status)).decode()


def version() -> int:
    return int(lib().ra_version())


def _check(status: int):
    if status != 0:
        raise RaError(status, status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RA_F32
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return RA_FP8_E4M3
    raise RaError(-2, f"RA_ERR_DTYPE: unsupported torch dtype {t.dtype}")


def desc(t: torch.Tensor) -> RaTensor:
    """ra_tensor view of a torch tensor (no copy)."""
    if t.dim() > 4 or t.dim() < 1:
        raise RaError(-3, "RA_ERR_SHAPE: tensors must have 1..4 dimensions")
    d = RaTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale) -> RaAttnParams:
    p = RaAttnParams()
    p.struct_size = ctypes.sizeof(RaAttnParams)
    p.causal = int(bool(causal))
    p.num_chunks = int(num_chunks)
    p.start_chunk = int(start_chunk)
    p.q_offset = int(q_offset)
    p.kv_offset = int(kv_offset)
    p.scale = 0.0 if scale is None else float(scale)
    return p


def _stream(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise RaError(-1, "RA_ERR_NULL: tensors must live in GPU memory")
    return torch.cuda.current_stream(t.device).cuda_stream


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             num_chunks: int = 1, start_chunk: int = 0, q_offset: int = 0, kv_offset: int = 0,
             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None,
             out_dtype: Optional[torch.dtype] = None,
             sched: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact attention of q [B,Hq,Sq,D] over k, v [B,Hkv,Skv,D] split into ``num_chunks``
    chunks visited from ``start_chunk`` in ring order.  Returns (o, lse).  ``sched``
    passes this stream's work counter (tile order only; results are the same)."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    p.sched = _sched_counter(q) if sched and q.is_cuda else None
    dq, dk, dv, do, dl = desc(q), desc(k), desc(v), desc(out), desc(lse)
    _check(lib().ra_attn_fwd(dq, dk, dv, ctypes.byref(p), do, dl, _stream(q)))
    return out, lse


def attn_fwd_validate(q, k, v, out, lse, *, causal=False, num_chunks=1, start_chunk=0,
                      q_offset=0, kv_offset=0, scale=None) -> int:
    """Host-side argument check of attn_fwd (no device access); returns the status."""
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    return int(lib().ra_attn_fwd_validate(desc(q), desc(k), desc(v), ctypes.byref(p),
                                          desc(out), desc(lse)))


def fp8_quantize(x: torch.Tensor, *, transpose: bool = False, out=None, descale=None,
                 workspace: Optional[torch.Tensor] = None):
    """bf16 [B,H,S,D] -> (e4m3 codes, fp32 descale [B,H]) with one scale per (batch, head);
    transpose=True gives codes [B,H,D,S_pad] (S_pad = S rounded up to 16), the V^T layout
    attn_fwd_fp8 reads."""
    B, H, S, D = x.shape
    if out is None:
        shape = (B, H, D, (S + 15) // 16 * 16) if transpose else (B, H, S, D)
        out = torch.empty(shape, dtype=torch.float8_e4m3fn, device=x.device)
    if descale is None:
        descale = torch.empty(B, H, dtype=torch.float32, device=x.device)
    if workspace is None:
        need = int(lib().ra_fp8_quantize_workspace_size(desc(x)))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib().ra_fp8_quantize(desc(x), desc(out), desc(descale), int(bool(transpose)),
                                 workspace.data_ptr(), workspace.numel(), _stream(x)))
    return out, descale


def _quant_outs(xs, transposes):
    outs, descs = [], []
    for x, t in zip(xs, transposes):
        B, H, S, D = x.shape
        shape = (B, H, D, (S + 15) // 16 * 16) if t else (B, H, S, D)
        outs.append(torch.empty(shape, dtype=torch.float8_e4m3fn, device=x.device))
        descs.append(torch.empty(B, H, dtype=torch.float32, device=x.device))
    return outs, descs


def fp8_quantize_multi(xs: Sequence[torch.Tensor], transposes: Sequence[bool], *, outs=None,
                       descales=None, workspace: Optional[torch.Tensor] = None):
    """fp8_quantize of several tensors (q, k, v of a layer, each with its own transpose
    flag) in two launches.  Returns (codes list, descale list)."""
    xs, transposes = list(xs), [int(bool(t)) for t in transposes]
    if not xs or len(transposes) != len(xs):
        raise RaError(-6, "RA_ERR_RANGE: xs and transposes must be non-empty and of equal length")
    if outs is None or descales is None:
        o2, d2 = _quant_outs(xs, transposes)
        outs = o2 if outs is None else list(outs)
        descales = d2 if descales is None else list(descales)
    n = len(xs)
    sa = (RaTensor * n)(*[desc(t) for t in xs])
    oa = (RaTensor * n)(*[desc(t) for t in outs])
    da = (RaTensor * n)(*[desc(t) for t in descales])
    ta = (ctypes.c_int32 * n)(*transposes)
    if workspace is None:
        need = int(lib().ra_fp8_quantize_n_workspace_size(n, sa))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=xs[0].device)
    _check(lib().ra_fp8_quantize_n(n, sa, oa, da, ctypes.cast(ta, ctypes.c_void_p),
                                   workspace.data_ptr(), workspace.numel(), _stream(xs[0])))
    return list(outs), list(descales)


def fp8_quantize_multi_validate(xs, outs, descales, transposes) -> int:
    n = len(xs)
    m = max(n, 1)
    sa = (RaTensor * m)(*[desc(t) for t in xs])
    oa = (RaTensor * m)(*[desc(t) for t in outs])
    da = (RaTensor * m)(*[desc(t) for t in descales])
    ta = (ctypes.c_int32 * m)(*[int(bool(t)) for t in transposes])
    return int(lib().ra_fp8_quantize_n_validate(n, sa, oa, da, ctypes.cast(ta, ctypes.c_void_p)))


def fp8_quantize_validate(x, out, descale, *, transpose=False) -> int:
    """Host-side argument check of fp8_quantize (no device access); returns the status."""
    return int(lib().ra_fp8_quantize_validate(desc(x), desc(out), desc(descale),
                                              int(bool(transpose))))


def attn_fwd_fp8(q, k, vt, q_descale, k_descale, v_descale, *, causal: bool = False,
                 num_chunks: int = 1, start_chunk: int = 0, q_offset: int = 0,
                 kv_offset: int = 0, scale: Optional[float] = None, out=None, lse=None,
                 out_dtype: torch.dtype = torch.bfloat16, sched: bool = True):
    """attn_fwd over e4m3 codes (q, k [B,H,S,D]; vt [B,Hkv,D,S_pad]) with fp32 descales
    per (batch, head).  Returns (o, lse).  ``sched`` as for attn_fwd."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    p.sched = _sched_counter(q) if sched and q.is_cuda else None
    _check(lib().ra_attn_fwd_fp8(desc(q), desc(k), desc(vt), desc(q_descale), desc(k_descale),
                                 desc(v_descale), ctypes.byref(p), desc(out), desc(lse),
                                 _stream(q)))
    return out, lse


def attn_fwd_fp8_validate(q, k, vt, q_descale, k_descale, v_descale, out, lse, *,
                          causal=False, num_chunks=1, start_chunk=0, q_offset=0, kv_offset=0,
                          scale=None) -> int:
    """Host-side argument check of attn_fwd_fp8 (no device access); returns the status."""
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    return int(lib().ra_attn_fwd_fp8_validate(desc(q), desc(k), desc(vt), desc(q_descale),
                                              desc(k_descale), desc(v_descale),
                                              ctypes.byref(p), desc(out), desc(lse)))


def _cu_arg(cu_seqlens: torch.Tensor):
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise RaError(-2, "RA_ERR_DTYPE: cu_seqlens must be a contiguous 1-D int32 tensor")
    if cu_seqlens.numel() < 2:
        raise RaError(-6, "RA_ERR_RANGE: cu_seqlens needs at least two entries")
    return ctypes.c_void_p(cu_seqlens.data_ptr()), int(cu_seqlens.numel() - 1)


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                    *, causal: bool = False, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None,
                    sched: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention over packed documents: q [B,Hq,T,D], k, v [B,Hkv,T,D]; document d holds
    tokens cu_seqlens[d] .. cu_seqlens[d+1]-1 (a device int32 tensor) and each query sees
    only its own document's keys.  Returns (o, lse).  ``sched`` as for attn_fwd."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    cu, n = _cu_arg(cu_seqlens)
    p = _params(causal, 1, 0, 0, 0, scale)
    p.sched = _sched_counter(q) if sched and q.is_cuda else None
    _check(lib().ra_attn_fwd_varlen(desc(q), desc(k), desc(v), cu, n, ctypes.byref(p),
                                    desc(out), desc(lse), _stream(q)))
    return out, lse


def attn_fwd_varlen_validate(q, k, v, cu_seqlens, out, lse, *, causal=False, scale=None) -> int:
    """Host-side argument check of attn_fwd_varlen (no device access); returns the status."""
    cu, n = _cu_arg(cu_seqlens)
    p = _params(causal, 1, 0, 0, 0, scale)
    return int(lib().ra_attn_fwd_varlen_validate(desc(q), desc(k), desc(v), cu, n,
                                                 ctypes.byref(p), desc(out), desc(lse)))


def _parts_arrays(o_parts, lse_parts):
    n = len(o_parts)
    oa = (RaTensor * max(n, 1))(*[desc(t) for t in o_parts])
    la = (RaTensor * max(len(lse_parts), 1))(*[desc(t) for t in lse_parts])
    return n, oa, la


def lse_merge(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor], *,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
              out_dtype: Optional[torch.dtype] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge partial (o_i, lse_i) over disjoint key sets.  Returns (o, lse)."""
    if len(o_parts) != len(lse_parts):
        raise RaError(-3, "RA_ERR_SHAPE: o_parts and lse_parts differ in length")
    ref = o_parts[0]
    if out is None:
        out = torch.empty(ref.shape, dtype=out_dtype or ref.dtype, device=ref.device)
    if lse is None:
        lse = torch.empty(ref.shape[:3], dtype=torch.float32, device=ref.device)
    n, oa, la = _parts_arrays(o_parts, lse_parts)
    _check(lib().ra_lse_merge(n, oa, la, desc(out), desc(lse), _stream(ref)))
    return out, lse


def lse_merge_validate(o_parts, lse_parts, out, lse) -> int:
    n, oa, la = _parts_arrays(o_parts, lse_parts)
    return int(lib().ra_lse_merge_validate(n, oa, la, desc(out), desc(lse)))


def _permute_out_shape(src: torch.Tensor, P: int, rank: int, dir: int):
    if dir == 0:
        P_, Sl, H, D = src.shape
        shape = (H // P, P * Sl, D)
        return shape if rank >= 0 else (P,) + shape
    raise ValueError("dir=1 needs an explicit `out` of shape [P, S/P, H, D]")


def ulysses_permute(src: torch.Tensor, P: int, rank: int, dir: int = 0, *,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sequence shards [P,S/P,H,D] -> head shard [H/P,S,D] (dir 0) or back (dir 1)."""
    if out is None:
        out = torch.empty(_permute_out_shape(src, P, rank, dir), dtype=src.dtype,
                          device=src.device)
    _check(lib().ra_ulysses_permute(desc(src), desc(out), int(P), int(rank), int(dir),
                                    _stream(src)))
    return out


def ulysses_permute_multi(srcs: Sequence[torch.Tensor], P: int, rank: int, dir: int = 0, *,
                          outs: Optional[Sequence[torch.Tensor]] = None):
    """ulysses_permute of several tensors (e.g. q, k, v of a layer) in one launch.
    Returns the list of destinations."""
    srcs = list(srcs)
    if outs is None:
        outs = [torch.empty(_permute_out_shape(s, P, rank, dir), dtype=s.dtype, device=s.device)
                for s in srcs]
    outs = list(outs)
    if len(outs) != len(srcs) or not srcs:
        raise RaError(-6, "RA_ERR_RANGE: srcs and outs must be non-empty and of equal length")
    sa = (RaTensor * len(srcs))(*[desc(t) for t in srcs])
    oa = (RaTensor * len(outs))(*[desc(t) for t in outs])
    _check(lib().ra_ulysses_permute_n(len(srcs), sa, oa, int(P), int(rank), int(dir),
                                      _stream(srcs[0])))
    return outs


def ulysses_permute_multi_validate(srcs, outs, P, rank, dir) -> int:
    sa = (RaTensor * max(len(srcs), 1))(*[desc(t) for t in srcs])
    oa = (RaTensor * max(len(outs), 1))(*[desc(t) for t in outs])
    return int(lib().ra_ulysses_permute_n_validate(len(srcs), sa, oa, int(P), int(rank),
                                                   int(dir)))


def ulysses_permute_validate(src, out, P, rank, dir) -> int:
    return int(lib().ra_ulysses_permute_validate(desc(src), desc(out), int(P), int(rank),
                                                 int(dir)))


def attn_bwd_workspace_size(q: torch.Tensor, k: torch.Tensor, *, causal=False, num_chunks=1,
                            start_chunk=0, q_offset=0, kv_offset=0, scale=None) -> int:
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    return int(lib().ra_attn_bwd_workspace_size(desc(q), desc(k), ctypes.byref(p)))


def attn_bwd(q, k, v, o, dout, lse, *, causal=False, num_chunks=1, start_chunk=0, q_offset=0,
             kv_offset=0, scale=None, dq=None, dk=None, dv=None,
             workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(dout * o), recomputing P from the saved lse."""
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib().ra_attn_bwd_workspace_size(desc(q), desc(k), ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().ra_attn_bwd(desc(q), desc(k), desc(v), desc(o), desc(dout), desc(lse),
                             ctypes.byref(p), desc(dq), desc(dk), desc(dv),
                             workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, dout, lse, *, causal=False, num_chunks=1, start_chunk=0,
                     q_offset=0, kv_offset=0, scale=None, dq=None, dk=None, dv=None):
    """attn_bwd whose workspace is the library's fixed per-GPU scratch (no allocation by
    the library; calls that overlap on one GPU race).  Runs on q's device."""
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    with torch.cuda.device(q.device):
        _check(lib().ra_attn_bwd_noalloc(desc(q), desc(k), desc(v), desc(o), desc(dout),
                                         desc(lse), ctypes.byref(p), desc(dq), desc(dk),
                                         desc(dv), _stream(q)))
    return dq, dk, dv


def noalloc_scratch_bytes() -> int:
    return int(lib().ra_noalloc_scratch_bytes())


def attn_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, *, causal=False, scale=None, dq=None,
                    dk=None, dv=None, workspace: Optional[torch.Tensor] = None):
    """Gradients of attn_fwd_varlen (packed documents, cu_seqlens a device int32 tensor)."""
    p = _params(causal, 1, 0, 0, 0, scale)
    cu, n = _cu_arg(cu_seqlens)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib().ra_attn_bwd_workspace_size(desc(q), desc(k), ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().ra_attn_bwd_varlen(desc(q), desc(k), desc(v), desc(o), desc(dout), desc(lse),
                                    cu, n, ctypes.byref(p), desc(dq), desc(dk), desc(dv),
                                    workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dq, dk, dv


def attn_bwd_varlen_validate(q, k, v, o, dout, lse, cu_seqlens, dq, dk, dv, *, causal=False,
                             scale=None) -> int:
    """Host-side argument check of attn_bwd_varlen (no device access); returns the status."""
    p = _params(causal, 1, 0, 0, 0, scale)
    cu, n = _cu_arg(cu_seqlens)
    return int(lib().ra_attn_bwd_varlen_validate(desc(q), desc(k), desc(v), desc(o), desc(dout),
                                                 desc(lse), cu, n, ctypes.byref(p), desc(dq),
                                                 desc(dk), desc(dv)))


def attn_bwd_accum(q, k, v, o, dout, lse, dq_acc, dk_acc, dv_acc, *, causal=False, q_offset=0,
                   kv_offset=0, scale=None, workspace: Optional[torch.Tensor] = None):
    """One ring-backward step: adds this block's gradients against the key/value chunk
    (k, v at global position kv_offset) to the fp32 accumulators, in place."""
    p = _params(causal, 1, 0, q_offset, kv_offset, scale)
    need = int(lib().ra_attn_bwd_workspace_size(desc(q), desc(k), ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().ra_attn_bwd_accum(desc(q), desc(k), desc(v), desc(o), desc(dout), desc(lse),
                                   ctypes.byref(p), desc(dq_acc), desc(dk_acc), desc(dv_acc),
                                   workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dq_acc, dk_acc, dv_acc


def attn_bwd_accum_validate(q, k, v, o, dout, lse, dq_acc, dk_acc, dv_acc, *, causal=False,
                            num_chunks=1, start_chunk=0, q_offset=0, kv_offset=0,
                            scale=None) -> int:
    """Host-side argument check of attn_bwd_accum (no device access); returns the status."""
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    return int(lib().ra_attn_bwd_accum_validate(desc(q), desc(k), desc(v), desc(o), desc(dout),
                                                desc(lse), ctypes.byref(p), desc(dq_acc),
                                                desc(dk_acc), desc(dv_acc)))


def attn_bwd_validate(q, k, v, o, dout, lse, dq, dk, dv, *, causal=False, num_chunks=1,
                      start_chunk=0, q_offset=0, kv_offset=0, scale=None) -> int:
    p = _params(causal, num_chunks, start_chunk, q_offset, kv_offset, scale)
    return int(lib().ra_attn_bwd_validate(desc(q), desc(k), desc(v), desc(o), desc(dout),
                                          desc(lse), ctypes.byref(p), desc(dq), desc(dk),
                                          desc(dv)))


def ring_visible_chunks(Sq: int, Skv: int, *, num_chunks: int, start_chunk: int = 0,
                        causal: bool = False, q_offset: int = 0, kv_offset: int = 0):
    """Chunks in ring order (start + t) mod P that hold at least one key visible to the
    last query row; the rest are skipped (their partial would be (0, -inf))."""
    L = Skv // num_chunks
    order = [(start_chunk + t) % num_chunks for t in range(num_chunks)]
    if not causal:
        return order
    last_q = q_offset + Sq - 1
    return [c for c in order if kv_offset + c * L <= last_q]


def ring_attn_chunked(q, k, v, *, num_chunks: int, start_chunk: int = 0, causal: bool = False,
                      q_offset: int = 0, kv_offset: int = 0, scale: Optional[float] = None,
                      out_dtype: Optional[torch.dtype] = None):
    """One ring rank's share computed chunk by chunk, as a ring would deliver the chunks:
    one attn_fwd per visible chunk into fp32 partials, then one lse_merge."""
    Skv = k.shape[2]
    L = Skv // num_chunks
    chunks = ring_visible_chunks(q.shape[2], Skv, num_chunks=num_chunks,
                                 start_chunk=start_chunk, causal=causal, q_offset=q_offset,
                                 kv_offset=kv_offset)
    if not chunks:
        chunks = [start_chunk]  # every row empty: one call yields o = 0, lse = -inf
    o_parts, lse_parts = [], []
    for c in chunks:
        o_c, l_c = attn_fwd(q, k[:, :, c * L:(c + 1) * L], v[:, :, c * L:(c + 1) * L],
                            causal=causal, q_offset=q_offset, kv_offset=kv_offset + c * L,
                            scale=scale, out_dtype=torch.float32)
        o_parts.append(o_c)
        lse_parts.append(l_c)
    return lse_merge(o_parts, lse_parts, out_dtype=out_dtype or q.dtype)


def ring_attn_fp8_chunked(q, k, vt, q_descale, k_descale, v_descale, *, num_chunks: int,
                          start_chunk: int = 0, causal: bool = False, q_offset: int = 0,
                          kv_offset: int = 0, scale: Optional[float] = None,
                          out_dtype: torch.dtype = torch.bfloat16):
    """ring_attn_chunked over e4m3 codes: one attn_fwd_fp8 per visible chunk into fp32
    partials, then one lse_merge.  Chunks of vt [B,Hkv,D,S_pad] are column slices, so
    Skv / num_chunks must be a multiple of 16."""
    Skv = k.shape[2]
    L = Skv // num_chunks
    chunks = ring_visible_chunks(q.shape[2], Skv, num_chunks=num_chunks,
                                 start_chunk=start_chunk, causal=causal, q_offset=q_offset,
                                 kv_offset=kv_offset)
    if not chunks:
        chunks = [start_chunk]  # every row empty: one call yields o = 0, lse = -inf
    o_parts, lse_parts = [], []
    for c in chunks:
        sl = slice(c * L, (c + 1) * L)
        o_c, l_c = attn_fwd_fp8(q, k[:, :, sl], vt[:, :, :, sl], q_descale, k_descale, v_descale,
                                causal=causal, q_offset=q_offset, kv_offset=kv_offset + c * L,
                                scale=scale, out_dtype=torch.float32)
        o_parts.append(o_c)
        lse_parts.append(l_c)
    return lse_merge(o_parts, lse_parts, out_dtype=out_dtype)


def ring_attn_bwd_chunked(q, k, v, o, dout, lse, *, num_chunks: int, start_chunk: int = 0,
                          causal: bool = False, q_offset: int = 0, kv_offset: int = 0,
                          scale: Optional[float] = None, dq_acc=None, dk_acc=None, dv_acc=None,
                          workspace: Optional[torch.Tensor] = None):
    """One ring rank's backward chunk by chunk: one attn_bwd_accum per visible chunk in
    ring order into fp32 accumulators (zeroed here when not given).  o and lse are the
    rank's merged forward result; dk_acc/dv_acc cover every chunk [B, Hkv, Skv, D]."""
    Skv = k.shape[2]
    L = Skv // num_chunks
    if dq_acc is None:
        dq_acc = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    if dk_acc is None:
        dk_acc = torch.zeros(k.shape, dtype=torch.float32, device=k.device)
    if dv_acc is None:
        dv_acc = torch.zeros(v.shape, dtype=torch.float32, device=v.device)
    if workspace is None:
        p = _params(causal, 1, 0, q_offset, kv_offset, scale)
        need = int(lib().ra_attn_bwd_workspace_size(desc(q), desc(k), ctypes.byref(p)))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    for c in ring_visible_chunks(q.shape[2], Skv, num_chunks=num_chunks,
                                 start_chunk=start_chunk, causal=causal, q_offset=q_offset,
                                 kv_offset=kv_offset):
        sl = slice(c * L, (c + 1) * L)
        attn_bwd_accum(q, k[:, :, sl], v[:, :, sl], o, dout, lse, dq_acc, dk_acc[:, :, sl],
                       dv_acc[:, :, sl], causal=causal, q_offset=q_offset,
                       kv_offset=kv_offset + c * L, scale=scale, workspace=workspace)
    return dq_acc, dk_acc, dv_acc
