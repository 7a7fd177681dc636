"""Seeded synthetic inputs for the FlashAttention forward workloads.

This module is shared by the tests, the bench and the oracle's pins. It holds
random-number draws and storage-format conversion only (float32 draws rounded
to bf16/fp16 bit patterns); none of attention's arithmetic lives here.

Workloads (shapes follow the source pages; all draws are i.i.d. N(0, 1)):

* ``single_head_fp32``   B=H=1, N=256, d=64, fp32 (the first row of the accuracy
  table in "FlashAttention 简化版：Tiling + Online Softmax", §4.1).
* ``one_query_long_keys`` one query of d=64 against 4096 keys, drawn exactly as
  demo 1 of "CS349E 第 11 讲 01_online_softmax.py" draws them (q, then K, then V
  from ``numpy.random.default_rng(0)``), cast to fp32; plus a batched form of
  4096 queries sharing K, V whose row 0 is that query.
* ``headline_bf16``      B=4, H=16, N=4096, d=64, bf16 (the N=4096, d=64 shape the
  pages use for their memory arithmetic).
* ``long_seq_bf16``      B=1, H=32, N=16384, d=128, bf16, K drawn x3.
* ``decode_bf16``        B=16, H=32, Nq=1, Nk=32768, d=128, bf16, 16 KV splits.

Large tensors are drawn per (b, h, tensor) from ``default_rng([seed, b, h, t])``
so any single head can be regenerated on its own. The decode workload (8.6 GB
of K/V) is drawn on the device with torch's seeded generator instead; the
sampled heads the oracle needs are copied back to the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to IEEE half (numpy's cast rounds to nearest even); return uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


@dataclass
class Tensor:
    """A host tensor in one of the three storage formats.

    ``data`` is float32 for ``dtype == "f32"`` and the uint16 bit patterns for
    ``"bf16"`` / ``"f16"``.
    """
    data: np.ndarray
    dtype: str

    @property
    def shape(self):
        return self.data.shape

    def as_f64(self) -> np.ndarray:
        """The exact values, widened to float64."""
        if self.dtype == "f32":
            return self.data.astype(np.float64)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        if self.dtype == "f16":
            return f16_bits_to_f32(self.data).astype(np.float64)
        raise ValueError(self.dtype)

    def to_torch(self, device):
        """Copy to a torch tensor of the matching dtype (bit-exact)."""
        import torch
        if self.dtype == "f32":
            t = torch.from_numpy(np.ascontiguousarray(self.data))
        else:
            t = torch.from_numpy(np.ascontiguousarray(self.data).view(np.int16))
            t = t.view(torch.bfloat16 if self.dtype == "bf16" else torch.float16)
        return t.to(device)


def encode(x_f32: np.ndarray, dtype: str) -> Tensor:
    x_f32 = np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "f32":
        return Tensor(x_f32, "f32")
    if dtype == "bf16":
        return Tensor(bf16_bits_from_f32(x_f32), "bf16")
    if dtype == "f16":
        return Tensor(f16_bits_from_f32(x_f32), "f16")
    raise ValueError(dtype)


def fp32_inverse_sqrt(d: int) -> float:
    """The float32 value of 1/sqrt(d) that both sides are handed as the scale."""
    return float(np.float32(1.0 / math.sqrt(d)))


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------

def head_draw(seed: int, b: int, h: int, t: int, n: int, d: int, mult: float = 1.0) -> np.ndarray:
    """float32 [n, d] N(0,1) draws for tensor t (0=Q, 1=K, 2=V) of head (b, h), times ``mult`` in float32."""
    x = np.random.default_rng([seed, b, h, t]).standard_normal((n, d), dtype=np.float32)
    if mult != 1.0:
        x = x * np.float32(mult)
    return x


def per_head_tensor(seed: int, B: int, H: int, N: int, d: int, t: int, dtype: str, mult: float = 1.0) -> Tensor:
    """[B, H, N, d] tensor assembled from independent per-head draws."""
    out = None
    for b in range(B):
        for h in range(H):
            enc = encode(head_draw(seed, b, h, t, N, d, mult), dtype)
            if out is None:
                out = np.empty((B, H, N, d), dtype=enc.data.dtype)
            out[b, h] = enc.data
    return Tensor(out, dtype)


@dataclass
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    seed: int
    k_mult: float = 1.0
    num_splits: int = 0
    extra: dict = field(default_factory=dict)
    H_kv: int = 0            # K/V heads (0: same as H)
    causal: bool = False     # row i sees keys j <= i + Nk - Nq

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def scale(self) -> float:
        return fp32_inverse_sqrt(self.d)

    @property
    def visible_pairs(self) -> float:
        """(query, key) pairs that enter the softmax: Nq * Nk, or under the causal mask
        sum_i (i + Nk - Nq + 1) = Nq (Nk - Nq + 1) + Nq (Nq - 1) / 2."""
        if not self.causal:
            return float(self.Nq) * self.Nk
        return float(self.Nq) * (self.Nk - self.Nq + 1) + self.Nq * (self.Nq - 1) / 2.0

    @property
    def flops(self) -> float:
        """4*d flops (the two matrix products QK^T and PV) per visible (query, key) pair, per (b, h)."""
        return 4.0 * self.B * self.H * self.d * self.visible_pairs


SINGLE_HEAD_FP32 = Workload("single_head_fp32 B=1 H=1 N=256 d=64", 1, 1, 256, 256, 64, "f32", 42)
ONE_QUERY_LONG_KEYS = Workload("one_query_long_keys Nq=1 Nk=4096 d=64", 1, 1, 1, 4096, 64, "f32", 0,
                               extra={"block": 256})
BATCHED_QUERIES_LONG_KEYS = Workload("batched_queries Nq=4096 Nk=4096 d=64", 1, 1, 4096, 4096, 64, "f32", 0)
HEADLINE_BF16 = Workload("headline B=4 H=16 N=4096 d=64 bf16", 4, 16, 4096, 4096, 64, "bf16", 3)
LONG_SEQ_BF16 = Workload("long_seq B=1 H=32 N=16384 d=128 bf16 Kx3", 1, 32, 16384, 16384, 128, "bf16", 4,
                         k_mult=3.0)
CAUSAL_BF16 = Workload("causal B=4 H=16 N=4096 d=64 bf16", 4, 16, 4096, 4096, 64, "bf16", 3, causal=True)
# The headline shape in fp16 (the same draws rounded to fp16).
HEADLINE_F16 = Workload("headline_f16 B=4 H=16 N=4096 d=64 fp16", 4, 16, 4096, 4096, 64, "f16", 3)
# The backward pass on the headline inputs; dL/dO is tensor 3 of the same per-head draws.
BWD_BF16 = Workload("backward B=4 H=16 N=4096 d=64 bf16 (dO: tensor 3)", 4, 16, 4096, 4096, 64, "bf16", 3)
# The backward pass on the causal workload (same draws, the causal mask).
BWD_CAUSAL_BF16 = Workload("backward causal B=4 H=16 N=4096 d=64 bf16 (dO: tensor 3)", 4, 16, 4096, 4096, 64, "bf16",
                           3, causal=True)
# The backward pass at d = 128 on the headline batch shape (per-head draws of seed 3 at d = 128).
BWD_D128_BF16 = Workload("backward B=4 H=16 N=4096 d=128 bf16 (dO: tensor 3)", 4, 16, 4096, 4096, 128, "bf16", 3)
GQA_DECODE_BF16 = Workload("gqa_decode B=16 H=32 H_kv=8 Nq=1 Nk=32768 d=128 bf16", 16, 32, 1, 32768, 128, "bf16", 6,
                           num_splits=16, H_kv=8)
DECODE_BF16 = Workload("split_kv_decode B=16 H=32 Nq=1 Nk=32768 d=128 bf16", 16, 32, 1, 32768, 128, "bf16", 5,
                       num_splits=16)


def single_head_fp32(seed: int = 42, N: int = 256, d: int = 64):
    """Q, K, V [1, 1, N, d] float32 from default_rng(seed), drawn in the order Q, K, V."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, N, d), dtype=np.float32)
    k = rng.standard_normal((1, 1, N, d), dtype=np.float32)
    v = rng.standard_normal((1, 1, N, d), dtype=np.float32)
    return Tensor(q, "f32"), Tensor(k, "f32"), Tensor(v, "f32")


def one_query_long_keys_f64(seed: int = 0, S: int = 4096, d: int = 64):
    """The float64 draws of demo 1 of the lecture-11 script: q [d], then K [S, d], then V [S, d]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(d)
    K = rng.standard_normal((S, d))
    V = rng.standard_normal((S, d))
    return q, K, V, rng


def one_query_long_keys(seed: int = 0, S: int = 4096, d: int = 64, batched: bool = False):
    """fp32 [1,1,Nq,d] Q and [1,1,S,d] K, V. Batched: 4096 further query rows are drawn after V and row 0 is q."""
    q, K, V, rng = one_query_long_keys_f64(seed, S, d)
    if batched:
        Q = rng.standard_normal((S, d))
        Q[0] = q
    else:
        Q = q[None, :]
    f = lambda a: Tensor(np.ascontiguousarray(a, dtype=np.float32)[None, None], "f32")
    return f(Q), f(K), f(V)


def workload_inputs(w: Workload):
    """Host Q, K, V for a per-head-drawn workload (headline, long sequence, or any ad-hoc shape)."""
    q = per_head_tensor(w.seed, w.B, w.H, w.Nq, w.d, 0, w.dtype)
    k = per_head_tensor(w.seed, w.B, w.kv_heads, w.Nk, w.d, 1, w.dtype, w.k_mult)
    v = per_head_tensor(w.seed, w.B, w.kv_heads, w.Nk, w.d, 2, w.dtype)
    return q, k, v


def grad_output(w: Workload):
    """Host dL/dO [B, H, Nq, d] for a per-head-drawn workload (tensor index 3 of the same seed)."""
    return per_head_tensor(w.seed, w.B, w.H, w.Nq, w.d, 3, w.dtype)


def small_case(seed: int, B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, k_mult: float = 1.0):
    """An ad-hoc small workload drawn per head (used for ragged and edge-case parity tests)."""
    return workload_inputs(Workload(f"small-{seed}", B, H, Nq, Nk, d, dtype, seed, k_mult))


def device_draw(shape, seed: int, dtype: str, device, mult: float = 1.0):
    """N(0,1) float32 draws from torch's seeded generator on ``device``, times ``mult``, rounded to ``dtype``.

    Used where host generation would take minutes (the 8.6 GB decode K/V). torch's
    float32 -> bf16/fp16 casts round to nearest even.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return x.to(tdt) if tdt != torch.float32 else x


def decode_inputs_device(w: Workload, device):
    """Q [B,H,Nq,d], K, V [B,H_kv,Nk,d] for a split-KV decode workload, drawn on the device
    (seeds 1000*seed + 0, 1, 2)."""
    q = device_draw((w.B, w.H, w.Nq, w.d), w.seed * 1000 + 0, w.dtype, device)
    k = device_draw((w.B, w.kv_heads, w.Nk, w.d), w.seed * 1000 + 1, w.dtype, device, w.k_mult)
    v = device_draw((w.B, w.kv_heads, w.Nk, w.d), w.seed * 1000 + 2, w.dtype, device)
    return q, k, v


def merge_order(seed: int, num_splits: int) -> np.ndarray:
    """The shuffled merge order: default_rng(seed).permutation(num_splits)."""
    return np.random.default_rng(seed).permutation(num_splits).astype(np.int32)


def torch_to_f64(t) -> np.ndarray:
    """Exact float64 copy of a (host or device) torch tensor of dtype f32/bf16/f16."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()
