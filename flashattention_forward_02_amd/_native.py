"""ctypes view of libfa.so: one Python function per C entry point of include/fa.h, same names.

Argument marshalling only. Raises ImportError when the library has not been built; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32, FA_BF16, FA_F16 = 0, 1, 2
FA_OK, FA_EINVAL, FA_EUNSUPPORTED, FA_EHIP = 0, 1, 2, 3
FA_MAX_SPLITS = 256
EXPORTS = ("fa_fwd", "fa_fwd_split", "fa_fwd_ext", "fa_fwd_split_ext", "fa_fwd_lse", "fa_bwd", "fa_merge_states",
           "fa_fwd_split_lse", "fa_merge_lse", "fa_status_string", "fa_last_error", "fa_abi_version",
           "fa_probe_mfma_bf16", "fa_probe_hbm_read", "fa_bwd_noalloc", "fa_probe_mfma_f32")
FA_NOALLOC_MAX_ROWS = 4194304

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfa.so (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m flashattention_forward_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.fa_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
        L.fa_fwd.restype = I
        L.fa_fwd_split.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, P]
        L.fa_fwd_split.restype = I
        L.fa_fwd_ext.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P]
        L.fa_fwd_ext.restype = I
        L.fa_fwd_split_ext.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P]
        L.fa_fwd_split_ext.restype = I
        L.fa_fwd_lse.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P]
        L.fa_fwd_lse.restype = I
        L.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P]
        L.fa_bwd.restype = I
        L.fa_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P]
        L.fa_bwd_noalloc.restype = I
        L.fa_merge_states.argtypes = [P, P, P, P, I, I, I, I, I, P, I, P, P, P]
        L.fa_merge_states.restype = I
        L.fa_fwd_split_lse.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P]
        L.fa_fwd_split_lse.restype = I
        L.fa_merge_lse.argtypes = [P, P, P, I, I, I, I, I, P, I, P, P]
        L.fa_merge_lse.restype = I
        L.fa_status_string.argtypes = [I]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_last_error.argtypes = []
        L.fa_last_error.restype = ctypes.c_char_p
        L.fa_abi_version.argtypes = []
        L.fa_abi_version.restype = I
        LL = ctypes.c_longlong
        L.fa_probe_mfma_bf16.argtypes = [P, LL, I, I, P]
        L.fa_probe_mfma_bf16.restype = I
        L.fa_probe_mfma_f32.argtypes = [P, LL, I, I, P]
        L.fa_probe_mfma_f32.restype = I
        L.fa_probe_hbm_read.argtypes = [P, LL, P, LL, I, P]
        L.fa_probe_hbm_read.restype = I
        _lib = L
    return _lib


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{lib().fa_status_string(status).decode()}: {detail}")


def check(status: int) -> None:
    if status != FA_OK:
        raise FaError(status, lib().fa_last_error().decode())


def fa_fwd(q, k, v, o, m_out, l_out, B, H, Nq, Nk, d, scale, in_dtype, out_dtype, stream):
    return lib().fa_fwd(q, k, v, o, m_out, l_out, B, H, Nq, Nk, d, scale, in_dtype, out_dtype, stream)


def fa_fwd_split(q, k, v, part_m, part_l, part_o, num_splits, B, H, Nq, Nk, d, scale, in_dtype, stream):
    return lib().fa_fwd_split(q, k, v, part_m, part_l, part_o, num_splits, B, H, Nq, Nk, d, scale, in_dtype, stream)


def fa_fwd_ext(q, k, v, o, m_out, l_out, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype, out_dtype, stream):
    return lib().fa_fwd_ext(q, k, v, o, m_out, l_out, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype, out_dtype, stream)


def fa_fwd_split_ext(q, k, v, part_m, part_l, part_o, num_splits, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype,
                     stream):
    return lib().fa_fwd_split_ext(q, k, v, part_m, part_l, part_o, num_splits, B, H, H_kv, Nq, Nk, d, scale, causal,
                                  in_dtype, stream)


def fa_fwd_lse(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype, out_dtype, stream):
    return lib().fa_fwd_lse(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype, out_dtype, stream)


def fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype, o_dtype,
           stream):
    return lib().fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype,
                        o_dtype, stream)


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype, o_dtype,
                   stream):
    return lib().fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype,
                                o_dtype, stream)


def fa_merge_states(part_m, part_l, part_o, order, num_splits, B, H, Nq, d, o, out_dtype, m_out, l_out, stream):
    if order is not None:
        order = (ctypes.c_int * num_splits)(*[int(x) for x in order])
    return lib().fa_merge_states(part_m, part_l, part_o, order, num_splits, B, H, Nq, d, o, out_dtype, m_out, l_out,
                                 stream)


def fa_fwd_split_lse(q, k, v, part_lse, part_o, num_splits, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype, stream):
    return lib().fa_fwd_split_lse(q, k, v, part_lse, part_o, num_splits, B, H, H_kv, Nq, Nk, d, scale, causal,
                                  in_dtype, stream)


def fa_merge_lse(part_lse, part_o, order, num_splits, B, H, Nq, d, o, out_dtype, lse_out, stream):
    if order is not None:
        order = (ctypes.c_int * num_splits)(*[int(x) for x in order])
    return lib().fa_merge_lse(part_lse, part_o, order, num_splits, B, H, Nq, d, o, out_dtype, lse_out, stream)


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


def fa_last_error() -> str:
    return lib().fa_last_error().decode()


def fa_abi_version() -> int:
    return lib().fa_abi_version()


def fa_probe_mfma_bf16(out, out_elems, nblocks, iters, stream):
    return lib().fa_probe_mfma_bf16(out, out_elems, nblocks, iters, stream)


def fa_probe_mfma_f32(out, out_elems, nblocks, iters, stream):
    return lib().fa_probe_mfma_f32(out, out_elems, nblocks, iters, stream)


def fa_probe_hbm_read(src, nbytes, out, out_elems, nblocks, stream):
    return lib().fa_probe_hbm_read(src, nbytes, out, out_elems, nblocks, stream)
