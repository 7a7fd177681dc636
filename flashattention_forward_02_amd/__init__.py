"""FlashAttention forward (and its gradients) for AMD MI355X (gfx950): Python face of libfa.so.

Every function here marshals torch tensors (device memory, the current HIP stream) into a
call of the C ABI declared in include/fa.h; all arithmetic runs in the library's HIP kernels.
Outputs are allocated with torch on the inputs' device (the library itself never allocates).

    O = fwd(q, k, v)                                  # q [B,H,Nq,d], k/v [B,H,Nk,d]
    O = fwd(q, k, v, causal=True)                     # row i sees keys j <= i + Nk - Nq
    O = fwd(q, k_g, v_g)                              # grouped K/V heads: k_g, v_g [B,H_kv,Nk,d]
    part = fwd_split(q, k, v, num_splits=16)          # (m, l, o) partial states per key range
    O = merge_states(*part, order=[...])              # fold them in the given order
    O, lse = fwd_lse(q, k, v)                         # plus each row's log-sum-exp
    dq, dk, dv = bwd(q, k, v, O, dO, lse)             # gradients, P recomputed from lse
    plse, po = fwd_split_lse(q, k, v, num_splits=16)  # partial states in the (lse, o / l) form
    O, lse = merge_lse(plse, po, order=[...])         # combined with weights exp(lse_s - lse)
"""
from __future__ import annotations

import math

from . import _native
from ._native import FaError, FA_F32, FA_BF16, FA_F16  # noqa: F401

__all__ = ["fwd", "fwd_lse", "bwd", "fwd_split", "merge_states", "fwd_split_lse", "merge_lse", "FaError", "lib_path"]

lib_path = _native.LIB_PATH


_TORCH = None
_DTYPES = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def _dtype_code(dt):
    global _DTYPES
    if _DTYPES is None:
        torch = _torch()
        _DTYPES = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.float16: FA_F16}
    code = _DTYPES.get(dt)
    if code is None:
        raise TypeError(f"unsupported dtype {dt} (float32, bfloat16, float16)")
    return code


def _stream_ptr(device):
    """The raw handle of the current HIP stream of `device` (a torch.device or a device index)."""
    torch = _torch()
    index = device if isinstance(device, int) else device.index
    if index is None:
        index = torch.cuda.current_device()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:      # the handle without building a Stream object (about 1.8 us less per call)
        return raw(index)
    return torch.cuda.current_stream(index).cuda_stream


def _check_qkv(q, k, v):
    # cheap attribute tests first; the messages name the offending tensor
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        for name, t in (("q", q), ("k", k), ("v", v)):
            if not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor")
    qs, ks, vs = q.shape, k.shape, v.shape
    if len(qs) != 4 or len(ks) != 4 or len(vs) != 4:
        for name, t in (("q", q), ("k", k), ("v", v)):
            if t.dim() != 4:
                raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        for name, t in (("q", q), ("k", k), ("v", v)):
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
    if ks != vs or qs[0] != ks[0] or qs[3] != ks[3] or ks[1] < 1 or qs[1] % ks[1]:
        raise ValueError(f"shape mismatch: q {tuple(qs)}, k {tuple(ks)}, v {tuple(vs)} "
                         "(k and v: [B, H_kv, Nk, d] with H a multiple of H_kv)")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if not (q.get_device() == k.get_device() == v.get_device()):
        raise ValueError("q, k and v must be on one device")


def fwd(q, k, v, scale=None, out_dtype=None, return_stats=False, out=None, causal=False):
    """O = softmax(scale * q k^T) v per (b, h); scale defaults to 1/sqrt(d). See fa_fwd / fa_fwd_ext in include/fa.h.

    k and v may have fewer heads than q (grouped K/V heads: query head h reads K/V head h // (H // H_kv)).
    ``causal``: row i sees keys j <= i + Nk - Nq only (needs Nq <= Nk).
    With ``return_stats`` also returns m (row max of the scaled scores) and l (sum of exp(s - m)), fp32 [B,H,Nq].
    """
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    elif out.shape != (B, H, Nq, d) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, Nq, d] tensor of out_dtype")
    m = l = None
    if return_stats:
        m = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
        l = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    mp = m.data_ptr() if m is not None else None
    lp = l.data_ptr() if l is not None else None
    H_kv = k.shape[1]
    if H_kv == H and not causal:
        _native.check(_native.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), mp, lp,
                                     B, H, Nq, Nk, d, float(scale), _dtype_code(q.dtype), _dtype_code(out_dtype),
                                     _stream_ptr(q.get_device())))
    else:
        _native.check(_native.fa_fwd_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), mp, lp,
                                         B, H, H_kv, Nq, Nk, d, float(scale), int(bool(causal)), _dtype_code(q.dtype),
                                         _dtype_code(out_dtype), _stream_ptr(q.get_device())))
    return (out, m, l) if return_stats else out


def fwd_split(q, k, v, num_splits, scale=None, workspace=None, causal=False):
    """Split-KV partial states (part_m [S,B,H,Nq], part_l, part_o [S,B,H,Nq,d], fp32). See fa_fwd_split(_ext).

    Grouped K/V heads and ``causal`` as in ``fwd``; under the mask a key range a row cannot see gives it the
    empty state (-inf, 0, 0).
    """
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        part_m = torch.empty((num_splits, B, H, Nq), dtype=torch.float32, device=q.device)
        part_l = torch.empty_like(part_m)
        part_o = torch.empty((num_splits, B, H, Nq, d), dtype=torch.float32, device=q.device)
    else:
        part_m, part_l, part_o = workspace
    H_kv = k.shape[1]
    if H_kv == H and not causal:
        _native.check(_native.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), part_m.data_ptr(),
                                           part_l.data_ptr(), part_o.data_ptr(), num_splits, B, H, Nq, Nk, d,
                                           float(scale), _dtype_code(q.dtype), _stream_ptr(q.get_device())))
    else:
        _native.check(_native.fa_fwd_split_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), part_m.data_ptr(),
                                               part_l.data_ptr(), part_o.data_ptr(), num_splits, B, H, H_kv, Nq, Nk,
                                               d, float(scale), int(bool(causal)), _dtype_code(q.dtype),
                                               _stream_ptr(q.get_device())))
    return part_m, part_l, part_o


def merge_states(part_m, part_l, part_o, order=None, out_dtype=None, return_stats=False, out=None):
    """Fold partial states in ``order`` (default 0..S-1) into O [B,H,Nq,d]. See fa_merge_states."""
    torch = _torch()
    S, B, H, Nq, d = part_o.shape
    for t in (part_m, part_l, part_o):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("partial states must be contiguous float32")
    if part_m.shape != (S, B, H, Nq) or part_l.shape != (S, B, H, Nq):
        raise ValueError("part_m / part_l must be [S, B, H, Nq]")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=part_o.device)
    m = l = None
    if return_stats:
        m = torch.empty((B, H, Nq), dtype=torch.float32, device=part_o.device)
        l = torch.empty((B, H, Nq), dtype=torch.float32, device=part_o.device)
    _native.check(_native.fa_merge_states(part_m.data_ptr(), part_l.data_ptr(), part_o.data_ptr(),
                                          None if order is None else list(order), S, B, H, Nq, d, out.data_ptr(),
                                          _dtype_code(out_dtype), m.data_ptr() if m is not None else None,
                                          l.data_ptr() if l is not None else None, _stream_ptr(part_o.get_device())))
    return (out, m, l) if return_stats else out


def fwd_lse(q, k, v, scale=None, out_dtype=None, causal=False, out=None):
    """(O, lse): fwd plus each row's log-sum-exp m + ln(l) of the scaled scores, fp32 [B,H,Nq]. See fa_fwd_lse."""
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    elif out.shape != (B, H, Nq, d) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, Nq, d] tensor of out_dtype")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _native.check(_native.fa_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                     B, H, k.shape[1], Nq, Nk, d, float(scale), int(bool(causal)),
                                     _dtype_code(q.dtype), _dtype_code(out_dtype), _stream_ptr(q.get_device())))
    return out, lse


def bwd(q, k, v, o, dout, lse, scale=None, causal=False, return_delta=False, out=None):
    """(dq, dk, dv), fp32, of O = softmax(scale q k^T) v given dL/dO. See fa_bwd.

    ``o`` and ``lse`` come from ``fwd_lse`` on the same inputs; ``dout`` has q's dtype (bf16 or fp16).
    dk and dv have k's shape (with grouped K/V heads they sum over the query heads of a group).
    With ``return_delta`` also returns D = rowsum(dout * o), fp32 [B,H,Nq]. ``out`` = (dq, dk, dv, delta)
    supplies the four output buffers (contiguous float32 of those shapes) instead of allocating them.
    """
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t, dt in (("o", o, None), ("dout", dout, q.dtype)):
        if t.shape != q.shape or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous [B, H, Nq, d] tensor on q's device")
        if dt is not None and t.dtype != dt:
            raise TypeError(f"{name} must have q's dtype")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    if out is None:
        dq = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
        dv = torch.empty(k.shape, dtype=torch.float32, device=q.device)
        delta = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv, delta = out
        for t, shp in ((dq, (B, H, Nq, d)), (dk, tuple(k.shape)), (dv, tuple(k.shape)), (delta, (B, H, Nq))):
            if tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError("out must be contiguous float32 (dq, dk, dv, delta) of the documented shapes")
    _native.check(_native.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                 B, H, k.shape[1], Nq, Nk, d, float(scale), int(bool(causal)), _dtype_code(q.dtype),
                                 _dtype_code(o.dtype), _stream_ptr(q.get_device())))
    return (dq, dk, dv, delta) if return_delta else (dq, dk, dv)


def fwd_split_lse(q, k, v, num_splits, scale=None, workspace=None, causal=False):
    """Split-KV partial states in the (lse, o) form: part_lse [S,B,H,Nq], part_o [S,B,H,Nq,d] (o already divided
    by the range's own l), fp32. See fa_fwd_split_lse. Grouped heads and ``causal`` as in ``fwd``."""
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        part_lse = torch.empty((num_splits, B, H, Nq), dtype=torch.float32, device=q.device)
        part_o = torch.empty((num_splits, B, H, Nq, d), dtype=torch.float32, device=q.device)
    else:
        part_lse, part_o = workspace
    _native.check(_native.fa_fwd_split_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), part_lse.data_ptr(),
                                           part_o.data_ptr(), num_splits, B, H, k.shape[1], Nq, Nk, d, float(scale),
                                           int(bool(causal)), _dtype_code(q.dtype), _stream_ptr(q.get_device())))
    return part_lse, part_o


def merge_lse(part_lse, part_o, order=None, out_dtype=None, out=None, return_lse=True):
    """Combine (lse, o) partial states in ``order``: returns (O [B,H,Nq,d], lse [B,H,Nq]). See fa_merge_lse."""
    torch = _torch()
    S, B, H, Nq, d = part_o.shape
    for t in (part_lse, part_o):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("partial states must be contiguous float32")
    if part_lse.shape != (S, B, H, Nq):
        raise ValueError("part_lse must be [S, B, H, Nq]")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=part_o.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=part_o.device) if return_lse else None
    _native.check(_native.fa_merge_lse(part_lse.data_ptr(), part_o.data_ptr(), None if order is None else list(order),
                                       S, B, H, Nq, d, out.data_ptr(), _dtype_code(out_dtype),
                                       lse.data_ptr() if lse is not None else None, _stream_ptr(part_o.get_device())))
    return (out, lse) if return_lse else out


def probe_mfma_bf16(nblocks=2048, iters=1024, out=None):
    """Launch the matrix-core probe of fa_probe.h on the current stream; returns (flops, out).

    ``out`` (optional) is a float32 device tensor of at least nblocks * 256 elements.
    """
    torch = _torch()
    if out is None:
        out = torch.empty(nblocks * 256, dtype=torch.float32, device="cuda")
    _native.check(_native.fa_probe_mfma_bf16(out.data_ptr(), out.numel(), nblocks, iters, _stream_ptr(out.get_device())))
    return float(nblocks) * 4 * iters * 8 * 32768, out


def probe_mfma_f32(nblocks=2048, iters=1024, out=None):
    """Launch the fp32 matrix-core probe of fa_probe.h on the current stream; returns (flops, out)."""
    torch = _torch()
    if out is None:
        out = torch.empty(nblocks * 256, dtype=torch.float32, device="cuda")
    _native.check(_native.fa_probe_mfma_f32(out.data_ptr(), out.numel(), nblocks, iters, _stream_ptr(out.get_device())))
    return float(nblocks) * 4 * iters * 8 * 2048, out


def probe_hbm_read(buf, nblocks=1024, out=None):
    """Launch the streaming-read probe of fa_probe.h over every byte of the device tensor ``buf``; returns the
    number of bytes read. ``out`` (optional) is an int32 device tensor of at least nblocks * 256 elements."""
    torch = _torch()
    if out is None:
        out = torch.empty(nblocks * 256, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _native.check(_native.fa_probe_hbm_read(buf.data_ptr(), nbytes, out.data_ptr(), out.numel(), nblocks,
                                            _stream_ptr(buf.get_device())))
    return nbytes
