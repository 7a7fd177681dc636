"""Pins of the fp64 backward oracle against things other than itself (CPU only).

The gradients of O = softmax(scale Q K^T) V follow from the definition
([FA-Simplified §1.1]) by the chain rule; [FA-Fill Exercise 5] fixes how the backward pass
recomputes P from the stored statistics and gives dV = P^T dO; [CS349E-L11] notes that
FlashAttention-2 keeps the log-sum-exp L = m + ln(l) as the one stored statistic.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, B, H, H_kv, Nq, Nk, d):
    r = _rng(seed)
    return (r.standard_normal((B, H, Nq, d)), r.standard_normal((B, H_kv, Nk, d)),
            r.standard_normal((B, H_kv, Nk, d)), r.standard_normal((B, H, Nq, d)))


@pytest.mark.parametrize("H,H_kv,Nq,Nk,causal", [(1, 1, 4, 6, False), (2, 1, 5, 5, True), (2, 2, 3, 7, True)])
def test_backward_matches_finite_differences(H, H_kv, Nq, Nk, causal):
    """Central differences of sum(O * dO), the forward definition, in every input element."""
    d, scale = 3, 0.7
    q, k, v, do = _inputs(11 + Nq, 1, H, H_kv, Nq, Nk, d)
    dq, dk, dv, _, _ = oracle.attention_backward_fp64(q, k, v, do, scale, causal=causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            up = oracle.attention_loss_fp64(q, k, v, do, scale, causal)
            x[idx] = old - h
            dn = oracle.attention_loss_fp64(q, k, v, do, scale, causal)
            x[idx] = old
            assert abs((up - dn) / (2 * h) - g[idx]) < 1e-7, (idx, (up - dn) / (2 * h), g[idx])


@pytest.mark.parametrize("B,H,H_kv,Nq,Nk,d,causal", [(1, 2, 2, 33, 40, 16, False), (2, 4, 2, 37, 37, 8, True),
                                                     (1, 3, 1, 20, 50, 32, True)])
def test_backward_matches_torch_autograd_fp64(B, H, H_kv, Nq, Nk, d, causal):
    q, k, v, do = _inputs(5 + Nk, B, H, H_kv, Nq, Nk, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    dq, dk, dv, _, _ = oracle.attention_backward_fp64(q, k, v, do, scale, causal=causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kr = tk.repeat_interleave(H // H_kv, dim=1)
    vr = tv.repeat_interleave(H // H_kv, dim=1)
    s = scale * (tq @ kr.transpose(-1, -2))
    if causal:  # row i sees keys j <= i + (Nk - Nq), written out here with torch ops
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        s = s.masked_fill(j > i + (Nk - Nq), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vr
    o.backward(torch.tensor(do))
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_backward_closed_forms():
    B, H, H_kv, Nq, d = 1, 4, 2, 9, 6
    # one key: softmax is identically 1, so dQ = dK = 0 and dV sums dO over the rows of its group
    q, k, v, do = _inputs(3, B, H, H_kv, Nq, 1, d)
    dq, dk, dv, lse, _ = oracle.attention_backward_fp64(q, k, v, do, 0.4)
    assert np.all(dq == 0) and np.all(dk == 0)
    for hk in range(H_kv):
        want = do[0, 2 * hk:2 * hk + 2].sum(axis=(0, 1))
        assert np.allclose(dv[0, hk, 0], want, atol=1e-13)
    assert np.allclose(lse, 0.4 * np.einsum("bhqd,bhd->bhq", q, np.repeat(k[:, :, 0], 2, axis=1)), atol=1e-13)
    # zero scale: uniform weights 1/Nk; dQ = dK = 0 exactly, dV_j = (1/Nk) sum of dO over the group
    Nk = 7
    q, k, v, do = _inputs(4, B, H, H_kv, Nq, Nk, d)
    dq, dk, dv, lse, _ = oracle.attention_backward_fp64(q, k, v, do, 0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    for hk in range(H_kv):
        want = do[0, 2 * hk:2 * hk + 2].sum(axis=(0, 1)) / Nk
        assert np.allclose(dv[0, hk], want[None, :], atol=1e-13)
    assert np.allclose(lse, math.log(Nk), atol=1e-14)
    # constant V rows: O does not depend on P, so dQ = dK = 0
    v[:] = v[:, :, :1]
    dq, dk, _, _, _ = oracle.attention_backward_fp64(q, k, v, do, 0.5)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_dk_sums_to_zero_and_delta_identity(causal):
    """Shifting every key by one vector shifts a row's scores by a constant, so sum_j dK_j = 0;
    and D_i = sum_j P_ij dP_ij equals sum_c dO_ic O_ic because O = P V."""
    q, k, v, do = _inputs(21, 2, 4, 2, 30, 30, 16)
    dq, dk, dv, lse, delta = oracle.attention_backward_fp64(q, k, v, do, 0.25, causal=causal)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
    o = oracle.attention_fp64(q, k, v, 0.25, causal=causal)
    assert np.max(np.abs(delta - (do * o).sum(axis=-1))) < 1e-12


def test_lse_matches_library_logsumexp():
    q, k, v, do = _inputs(8, 1, 2, 2, 40, 70, 32)
    _, _, _, lse, _ = oracle.attention_backward_fp64(q, k, v, do, 0.3, causal=True)
    s = 0.3 * np.einsum("bhqd,bhkd->bhqk", q, k)
    mask = np.arange(70)[None, :] > np.arange(40)[:, None] + 30
    s = np.where(mask, -np.inf, s)
    assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=-1))) < 1e-12


def test_exercise5_blocked_dv_from_statistics():
    """[FA-Fill Exercise 5]: torch seed 42, Q, K, V [64, 32] and dO drawn in that order, 1/sqrt(d),
    blocks of 16; dV rebuilt block by block from the global (m, l) matches autograd (the page
    asserts 1e-4 in float32; in float64 it is exact to rounding)."""
    torch.manual_seed(42)
    N, d = 64, 32
    Q = torch.randn(N, d)
    K = torch.randn(N, d)
    V = torch.randn(N, d, requires_grad=True)
    S = Q @ K.T / math.sqrt(d)
    O = torch.softmax(S, dim=-1) @ V
    dO = torch.randn_like(O)
    O.backward(dO)
    dv_page = V.grad.numpy().astype(np.float64)
    q, k, v, do = (x.detach().numpy().astype(np.float64) for x in (Q, K, V, dO))
    scale = 1 / math.sqrt(d)
    _, m, l = oracle.attention_fp64(q[None], k[None], v[None], scale, return_stats=True)
    blocked = oracle.dv_from_statistics_blocked(q, k, do, m[0], l[0], scale, block=16)
    assert np.max(np.abs(blocked - dv_page)) < 1e-4                      # the exercise's own bar
    _, _, dv, _, _ = oracle.attention_backward_fp64(q[None, None], k[None, None], v[None, None],
                                                    do[None, None], scale)
    assert np.max(np.abs(blocked - dv[0, 0])) < 1e-13
