"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names the passage or the mathematical fact it checks. Sources:
[FA-Simplified] "FlashAttention 简化版：Tiling + Online Softmax";
[FA-Fill] "Flash Attention 代码填空 (Level 2-3)";
[CS349E-L11] "CS349E 第 11 讲 01_online_softmax.py";
[FA-Scratch] "从零手写 FlashAttention（PyTorch实现 + 原理推导）".
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _rng(seed):
    return np.random.default_rng(seed)


# --- P1: brute force on tiny inputs ------------------------------------------------------------

@pytest.mark.parametrize("Nq,Nk,d,scale", [(1, 1, 1, 0.5), (3, 5, 4, 0.5), (7, 16, 8, 1 / math.sqrt(8)),
                                           (12, 12, 10, 1.0), (5, 3, 6, 2.5)])
def test_brute_force_matches_definition(Nq, Nk, d, scale):
    r = _rng(100 + Nq * 31 + Nk)
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    ref = oracle.brute_force_attention(q, k, v, scale)
    got = oracle.attention_fp64(q[None], k[None], v[None], scale)[0]
    assert np.max(np.abs(got - ref)) < 1e-14


def test_scratch_page_example_unscaled_chunked():
    """[FA-Scratch §1, §5, §6]: [1,12,10] tensors, no scale, 4 query chunks x 3 key chunks agree with standard attention."""
    r = _rng(2160643)
    q, k, v = (r.standard_normal((1, 12, 10)) for _ in range(3))
    ref = oracle.brute_force_attention(q[0], k[0], v[0], 1.0)
    tiled = oracle.online_attention(q, k, v, 1.0, Br=3, Bc=4)[0]
    full = oracle.attention_fp64(q, k, v, 1.0)[0]
    assert np.allclose(tiled, ref, rtol=1e-5, atol=1e-8)  # the page's allclose
    assert np.max(np.abs(tiled - ref)) < 1e-14 and np.max(np.abs(full - ref)) < 1e-14


# --- library routines ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 37, 45, 16), (1, 2, 64, 200, 64), (1, 1, 5, 1, 128)])
def test_attention_matches_torch_sdpa_fp64(shape):
    B, H, Nq, Nk, d = shape
    r = _rng(7 + Nq)
    q, k, v = r.standard_normal((B, H, Nq, d)), r.standard_normal((B, H, Nk, d)), r.standard_normal((B, H, Nk, d))
    scale = float(np.float32(1 / math.sqrt(d)))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
    got = oracle.attention_fp64(q, k, v, scale, row_block=16)
    assert np.max(np.abs(got - ref)) < 1e-13


def test_stats_match_logsumexp():
    """m is the row max of the scaled scores and m + log l the row logsumexp (scipy)."""
    r = _rng(9)
    q, k, v = r.standard_normal((1, 2, 30, 8)), r.standard_normal((1, 2, 50, 8)), r.standard_normal((1, 2, 50, 8))
    _, m, l = oracle.attention_fp64(q, k, v, 0.3, return_stats=True)
    s = 0.3 * np.einsum("bhqd,bhkd->bhqk", q, k)
    assert np.max(np.abs(m - s.max(-1))) < 1e-14
    assert np.max(np.abs(m + np.log(l) - scipy.special.logsumexp(s, axis=-1))) < 1e-13


# --- P4: online softmax = safe softmax ----------------------------------------------------------

def test_online_and_safe_softmax_match_library():
    """[FA-Fill Exercise 2]: 4 x 8 inputs times 10; both forms equal the library softmax."""
    x = _rng(42).standard_normal((4, 8)) * 10
    ref = scipy.special.softmax(x, axis=-1)
    assert np.max(np.abs(oracle.safe_softmax(x) - ref)) < 1e-15
    assert np.max(np.abs(oracle.online_softmax(x) - ref)) < 1e-14


def test_safe_softmax_survives_where_naive_overflows():
    """[FA-Simplified §2.1]: exp(x) overflows for large x; subtracting the max keeps every exp in (0, 1]."""
    x = _rng(1).standard_normal((3, 9)) + 1000.0
    assert not np.all(np.isfinite(oracle.naive_softmax(x)))
    ref = scipy.special.softmax(x - 1000.0, axis=-1)
    assert np.max(np.abs(oracle.safe_softmax(x) - ref)) < 1e-14
    assert np.max(np.abs(oracle.online_softmax(x) - ref)) < 1e-14


# --- P5/P6: closed forms --------------------------------------------------------------------------

def test_rows_sum_to_one_and_identity_values():
    """V = I (Nk <= d) makes O the probability matrix itself: rows sum to 1 and equal the library softmax."""
    r = _rng(5)
    Nk, d = 24, 32
    q, k = r.standard_normal((1, 40, d)), r.standard_normal((1, Nk, d))
    V = np.zeros((1, Nk, d))
    V[0, :, :Nk] = np.eye(Nk)
    P = oracle.attention_fp64(q, k, V, 0.2)[0][:, :Nk]
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-14
    assert np.max(np.abs(P - scipy.special.softmax(0.2 * q[0] @ k[0].T, axis=1))) < 1e-15


def test_closed_forms():
    r = _rng(6)
    d = 16
    q = r.standard_normal((1, 9, d))
    k = r.standard_normal((1, 13, d))
    v = r.standard_normal((1, 13, d))
    # one key: O = V[0]
    assert np.max(np.abs(oracle.attention_fp64(q, k[:, :1], v[:, :1], 0.25)[0] - v[0, 0])) < 1e-15
    # constant V rows: O = that row
    c = r.standard_normal(d)
    vc = np.broadcast_to(c, v.shape).copy()
    assert np.max(np.abs(oracle.attention_fp64(q, k, vc, 0.25)[0] - c)) < 1e-14
    # zero scale or zero query: uniform weights, O = column mean of V
    assert np.max(np.abs(oracle.attention_fp64(q, k, v, 0.0)[0] - v[0].mean(axis=0))) < 1e-14
    assert np.max(np.abs(oracle.attention_fp64(np.zeros_like(q), k, v, 0.7)[0] - v[0].mean(axis=0))) < 1e-14
    # two keys: O = sigma(s0 - s1) v0 + sigma(s1 - s0) v1
    s = 0.25 * q[0] @ k[0, :2].T
    w0 = 1.0 / (1.0 + np.exp(-(s[:, 0] - s[:, 1])))
    ref = w0[:, None] * v[0, 0] + (1.0 - w0)[:, None] * v[0, 1]
    assert np.max(np.abs(oracle.attention_fp64(q, k[:, :2], v[:, :2], 0.25)[0] - ref)) < 1e-14


# --- P7: invariances ------------------------------------------------------------------------------

def test_shift_and_permutation_invariance():
    """A per-row constant added to the scores (K + u, scale*q.u ~ 100, where exp would reach e^100) and a joint
    permutation of K and V rows leave O unchanged ([FA-Simplified §2.1]; [FA-Fill Exercise 2])."""
    r = _rng(8)
    d, Nq, Nk = 32, 20, 70
    q, k, v = r.standard_normal((1, Nq, d)), r.standard_normal((1, Nk, d)), r.standard_normal((1, Nk, d))
    scale = 0.125
    u = q[0].mean(axis=0)
    u = u * (100.0 / (scale * float(q[0].mean(axis=0) @ u)))
    base = oracle.attention_fp64(q, k, v, scale)
    shifted = oracle.attention_fp64(q, k + u, v, scale)
    # rows whose shift is large still agree: the max subtraction absorbs it
    assert np.max(np.abs(shifted - base)) < 1e-11
    perm = r.permutation(Nk)
    assert np.max(np.abs(oracle.attention_fp64(q, k[:, perm], v[:, perm], scale) - base)) < 1e-14


# --- P2: one pass = three passes (lecture-11 demo 1) ------------------------------------------------

def test_one_pass_equals_three_pass_demo1():
    """[CS349E-L11] demo 1: S = 4096 keys, d = 64, blocks of 256, default_rng(0); differences at the 1e-16 level."""
    q, K, V, _ = si.one_query_long_keys_f64(0, 4096, 64)
    scale = 1 / math.sqrt(64)
    ref = oracle.attention_fp64(q[None, :], K, V, scale)[0]
    one = oracle.online_attention_row(q, K, V, 256)
    two = oracle.two_pass_attention_row(q, K, V, 256)
    assert np.max(np.abs(one - ref)) < 1e-15
    assert np.max(np.abs(two - ref)) < 1e-15
    # the running state block by block: the maximum never decreases; after the first block the
    # empty start state has weight 0, so (m, l) are that block's own maximum and sum
    hist = []
    oracle.online_attention_row(q, K[:1024], V[:1024], 256, history=hist)
    assert len(hist) == 4
    s0 = (K[:256] @ q) / 8.0
    assert hist[0][0] == s0.max()
    assert abs(hist[0][1] - np.exp(s0 - s0.max()).sum()) < 1e-12
    ms = [h[0] for h in hist]
    assert all(b >= a for a, b in zip(ms, ms[1:]))
    s_all = (K[:1024] @ q) / 8.0
    assert ms[-1] == s_all.max()
    assert abs(hist[-1][1] - np.exp(s_all - s_all.max()).sum()) < 1e-12


@pytest.mark.parametrize("Br,Bc", [(64, 64), (1, 256), (48, 80), (256, 7)])
def test_tiled_forward_is_tile_independent(Br, Bc):
    """[FA-Simplified §3.1]: the tiled loops do the same arithmetic as standard attention; ragged tails included."""
    q, k, v = (t.as_f64() for t in si.small_case(11, 2, 2, 130, 301, 32, "f32"))
    ref = oracle.attention_fp64(q, k, v, 0.17)
    got, m, l = oracle.online_attention(q, k, v, 0.17, Br, Bc, return_stats=True)
    _, m_ref, l_ref = oracle.attention_fp64(q, k, v, 0.17, return_stats=True)
    assert np.max(np.abs(got - ref)) < 1e-14
    assert np.max(np.abs(m - m_ref)) < 1e-14          # BLAS may sum the dot products in another order
    assert np.max(np.abs(l - l_ref) / l_ref) < 1e-13


# --- P8: Algorithm-1 order ----------------------------------------------------------------------------

def test_fa1_order_matches_delayed_normalisation():
    """[FA-Fill Exercise 4] (N = 256, d = 64, block 32) against the delayed form of [FA-Simplified §2.3]."""
    r = _rng(42)
    q, k, v = r.standard_normal((256, 64)), r.standard_normal((256, 64)), r.standard_normal((256, 64))
    scale = 1 / math.sqrt(64)
    a = oracle.fa1_order_attention(q, k, v, scale, 32)
    b = oracle.online_attention(q[None], k[None], v[None], scale, 32, 32)[0]
    assert np.max(np.abs(a - b)) < 1e-14
    assert np.max(np.abs(a - oracle.attention_fp64(q[None], k[None], v[None], scale)[0])) < 1e-14


# --- P3: merge order independence (lecture-11 demo 2) --------------------------------------------------

def test_merge_orders_demo2():
    """[CS349E-L11] demo 2: S = 3000, d = 32, x * 3, 11 random cuts, default_rng(1); every order agrees at 1e-16."""
    rng = np.random.default_rng(1)
    S, d = 3000, 32
    x = rng.standard_normal(S) * 3
    V = rng.standard_normal((S, d))
    ref = scipy.special.softmax(x) @ V                     # library softmax, not the oracle
    m0, l0, o0 = oracle.partial_state(x[None, :], V)
    assert np.max(np.abs(o0[0] / l0[0] - ref)) < 1e-13
    one_shot = o0[0] / l0[0]
    cuts = np.sort(rng.choice(np.arange(1, S), size=11, replace=False))
    segs = np.split(np.arange(S), cuts)
    assert len(segs) == 12
    states = [oracle.partial_state(x[None, s], V[s]) for s in segs]
    perm = rng.permutation(len(states))
    for merged in (oracle.merge_sequential(states), oracle.merge_tree(states),
                   oracle.merge_sequential(states, order=perm)):
        assert np.max(np.abs(oracle.finish_state(merged)[0] - one_shot)) < 1e-14   # a few ulp of |O| ~ 0.5
        assert merged[0][0] == m0[0]


def test_merge_empty_states_are_identity():
    """A state with no keys (m = -inf, l = 0, o = 0) merges as the identity and never produces NaN."""
    r = _rng(3)
    a = oracle.partial_state(r.standard_normal((2, 5)), r.standard_normal((5, 4)))
    empty = oracle.partial_state(np.zeros((2, 0)), np.zeros((0, 4)))
    for merged in (oracle.merge_states(a, empty), oracle.merge_states(empty, a)):
        for x, y in zip(merged, a):
            assert np.array_equal(x, y)
    both = oracle.merge_states(empty, empty)
    assert np.all(both[0] == -np.inf) and np.all(both[1] == 0) and not np.any(np.isnan(both[2]))
    # a row with no key at all finishes as O = 0 (the value the (lse, o) form gives it), not 0 / 0;
    # the other rows finish as o / l
    mixed = (np.array([both[0][0], a[0][1]]), np.array([0.0, a[1][1]]), np.stack([both[2][0], a[2][1]]))
    fin = oracle.finish_state(mixed)
    assert np.all(fin[0] == 0.0) and np.allclose(fin[1], a[2][1] / a[1][1], rtol=1e-15, atol=0)


@pytest.mark.parametrize("Nk,S", [(100, 7), (64, 64), (5000, 16), (33, 1)])
def test_split_states_merge_to_full_attention(Nk, S):
    r = _rng(Nk + S)
    q, k, v = r.standard_normal((3, 16)), r.standard_normal((Nk, 16)), r.standard_normal((Nk, 16))
    bounds = oracle.split_bounds(Nk, S)
    assert bounds[0][0] == 0 and bounds[-1][1] == Nk
    assert all(b0 < b1 for b0, b1 in bounds) and all(bounds[i][1] == bounds[i + 1][0] for i in range(S - 1))
    states = oracle.split_partial_states(q, k, v, 0.25, S)
    order = r.permutation(S)
    ref = oracle.attention_fp64(q[None], k[None], v[None], 0.25)[0]
    assert np.max(np.abs(oracle.finish_state(oracle.merge_sequential(states, order)) - ref)) < 1e-14


# --- P9: low-precision P (lecture-11 demo 4) --------------------------------------------------------

def test_rounding_matches_library_casts():
    r = _rng(12)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        (r.random(10000) * 1e-30).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0, 65504.0],
                                 dtype=np.float32)])           # exact ties: round to even
    ref_bf = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x), ref_bf)
    ref_h = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_f16(x), ref_h)


def _demo4():
    rng = np.random.default_rng(2)
    S, d = 8192, 64
    q = rng.standard_normal(d)
    K = rng.standard_normal((S, d))
    V = rng.standard_normal((S, d))
    s = K @ q / np.sqrt(d)
    p = np.exp(s - s.max())
    ref = (p / p.sum()) @ V
    return p, V, ref


def test_low_precision_p_error_magnitudes_demo4():
    """[CS349E-L11] demo 4: P rounded to BF16 gives ~1e-3 relative error, FP16 ~1e-4, FP32 far less;
    accumulating l itself in FP16/BF16 is orders of magnitude worse."""
    p, V, ref = _demo4()

    def rel(pq):
        out = (pq @ V) / p.sum()
        return np.abs(out - ref).max() / np.abs(ref).max()

    e32 = rel(p.astype(np.float32).astype(np.float64))
    ebf = rel(oracle.round_to_bf16(p))
    eh = rel(oracle.round_to_f16(p))
    assert 10 ** -3.5 < ebf < 10 ** -2.5
    assert 10 ** -4.5 < eh < 10 ** -3.5
    assert e32 < 1e-6 and eh < ebf
    l16 = np.float16(0.0)
    for x in p.astype(np.float16):
        l16 = np.float16(l16 + x)
    lbf = 0.0
    for x in oracle.round_to_bf16(p):
        lbf = float(oracle.round_to_bf16(np.float32(lbf + x)).reshape(-1)[0])
    for lv in (float(l16), lbf):
        assert abs(lv - p.sum()) / p.sum() > 30 * eh


# --- printed figures -----------------------------------------------------------------------------------

def _fig(fid):
    figs = json.load(open(GOLDEN))["figures"]
    return next(f for f in figs if f["id"] == fid)["value"]


def test_pages_memory_figures():
    """The closed-form memory figures the pages print (tests/golden/pages_figures.json, each cited there)."""
    assert 4096 * 4096 * 4 == _fig("S_bytes_fp32_N4096")
    assert 2 * 4096 * 4096 * 4 == _fig("SP_bytes_fp32_N4096")
    assert 16384 * 16384 * 4 == _fig("S_bytes_fp32_N16384")
    assert round(64 * 64 * 4 / 1e6, 3) == _fig("tile_bytes_fp32_64x64_MB")
    assert 4096 ** 2 // (64 * 64) == _fig("matrix_ratio_N4096_64x64")
    assert 4096 * 64 * 4 / 1024 ** 2 == _fig("mem_Q_MB")
    assert 2 * 4096 * 4096 * 4 / 1024 ** 2 == _fig("mem_intermediate_MB")
    assert 4096 * 4096 * 2 / 1024 ** 2 == _fig("score_matrix_fp16_per_head_MiB")
    assert abs(math.log(65504.0) - _fig("fp16_exp_overflow_at")) < 0.005
    with np.errstate(over="ignore"):
        assert np.isinf(np.float16(np.exp(np.float16(12.0))))


def test_pages_operation_count_figures():
    """[CS349E-L11] demo 3: non-matmul work relative to 4 N^2 d matmul flops, priced 16x (25% and 16%)."""
    N, d, Bc = 4096, 128, 128
    Tc = N // Bc
    matmul = 4 * N * N * d
    softmax_ops = 4 * N * N
    fa1 = softmax_ops + Tc * N * d * 4
    fa2 = softmax_ops + Tc * N * d + N * d
    assert round(16 * fa1 / matmul, 2) == _fig("nonmatmul_time_share_fa1")
    assert round(16 * fa2 / matmul, 2) == _fig("nonmatmul_time_share_fa2")


def test_pages_oracle_magnitudes():
    """The 1e-16 / 1e-3 / 1e-4 magnitudes recomputed with the oracle on the demos' own draws."""
    q, K, V, _ = si.one_query_long_keys_f64(0, 4096, 64)
    diff = np.max(np.abs(oracle.online_attention_row(q, K, V, 256)
                         - oracle.attention_fp64(q[None, :], K, V, 1 / 8)[0]))
    assert diff < 10 * _fig("one_pass_vs_three_pass_maxdiff")
    p, V4, ref = _demo4()
    ebf = np.abs((oracle.round_to_bf16(p) @ V4) / p.sum() - ref).max() / np.abs(ref).max()
    assert _fig("pv_rel_err_bf16") / 10 ** 0.5 < ebf < _fig("pv_rel_err_bf16") * 10 ** 0.5


# --- P10: the causal mask and grouped K/V heads ([FA-Simplified §7]) ----------------------------

def _causal_brute(q, k, v, scale):
    """Literal loops: query row i of Nq attends keys j = 0 .. i + (Nk - Nq), nothing else."""
    Nq, Nk = len(q), len(k)
    out = []
    for i in range(Nq):
        keys = range(0, i + (Nk - Nq) + 1)
        s = [float(scale) * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j])) for j in keys]
        mx = max(s)
        p = [math.exp(x - mx) for x in s]
        l = math.fsum(p)
        out.append([math.fsum(p[n] * float(v[j][c]) for n, j in enumerate(keys)) / l for c in range(len(v[0]))])
    return np.array(out)


@pytest.mark.parametrize("Nq,Nk,d", [(1, 1, 2), (5, 5, 3), (3, 7, 4), (1, 4, 2), (6, 6, 5), (4, 9, 3)])
def test_causal_brute_force(Nq, Nk, d):
    r = _rng(700 + Nq * 13 + Nk)
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    got = oracle.attention_fp64(q[None], k[None], v[None], 0.6, causal=True)[0]
    assert np.max(np.abs(got - _causal_brute(q, k, v, 0.6))) < 1e-14


def test_causal_square_matches_torch_sdpa():
    """Nq = Nk: the usual decoder mask; torch's float64 attention with is_causal=True (its mask keeps j <= i)."""
    r = _rng(710)
    q, k, v = (r.standard_normal((2, 3, 37, 8)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.3).numpy()
    assert np.max(np.abs(oracle.attention_fp64(q, k, v, 0.3, causal=True) - ref)) < 1e-13


def test_causal_rows_are_prefix_attention():
    """Row i equals unmasked attention over the first i + Nk - Nq + 1 keys; the first row of a square problem
    is v[0]; the last row of any problem is the unmasked result."""
    r = _rng(711)
    Nq, Nk, d = 19, 45, 6
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    got = oracle.attention_fp64(q[None], k[None], v[None], 0.4, causal=True)[0]
    for i in range(Nq):
        n = i + Nk - Nq + 1
        ref = oracle.attention_fp64(q[None, i:i + 1], k[None, :n], v[None, :n], 0.4)[0, 0]
        assert np.max(np.abs(got[i] - ref)) < 1e-14
    full = oracle.attention_fp64(q[None], k[None], v[None], 0.4)[0]
    assert np.max(np.abs(got[-1] - full[-1])) < 1e-14
    sq = oracle.attention_fp64(q[None, :, :], k[None, :Nq], v[None, :Nq], 0.4, causal=True)[0]
    assert np.max(np.abs(sq[0] - v[0])) == 0.0


def test_causal_queries_are_the_last_positions():
    """Nq < Nk: the result equals the last Nq rows of the square causal problem whose last queries are these
    (the reading: the queries are the final positions of the key sequence)."""
    r = _rng(712)
    Nq, Nk, d = 7, 30, 5
    qfull, k, v = r.standard_normal((Nk, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    square = oracle.attention_fp64(qfull[None], k[None], v[None], 0.5, causal=True)[0]
    tail = oracle.attention_fp64(qfull[None, Nk - Nq:], k[None], v[None], 0.5, causal=True)[0]
    assert np.max(np.abs(square[Nk - Nq:] - tail)) < 1e-14


def test_causal_needs_nq_le_nk():
    q = np.zeros((1, 5, 2))
    with pytest.raises(ValueError):
        oracle.attention_fp64(q, q[:, :3], q[:, :3], 1.0, causal=True)


def test_gqa_head_map():
    """Consecutive query heads share a K/V head: H = 8 over H_kv = 2 reads 0,0,0,0,1,1,1,1; MQA reads head 0."""
    assert [oracle.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head_of(h, 6, 1) for h in range(6)] == [0] * 6
    assert [oracle.kv_head_of(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


@pytest.mark.parametrize("H,H_kv,causal", [(8, 2, False), (6, 1, False), (4, 4, False), (8, 2, True), (6, 3, True)])
def test_gqa_matches_torch_sdpa(H, H_kv, causal):
    """torch's float64 attention with enable_gqa=True (K/V heads repeated to the query heads, in order)."""
    r = _rng(720 + H * 7 + H_kv)
    q = r.standard_normal((2, H, 23, 8))
    k, v = r.standard_normal((2, H_kv, 23, 8)), r.standard_normal((2, H_kv, 23, 8))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=0.35,
        enable_gqa=True).numpy()
    assert np.max(np.abs(oracle.attention_fp64(q, k, v, 0.35, causal=causal) - ref)) < 1e-13


def test_gqa_equals_mha_on_repeated_heads():
    r = _rng(730)
    q = r.standard_normal((1, 6, 11, 4))
    k, v = r.standard_normal((1, 2, 15, 4)), r.standard_normal((1, 2, 15, 4))
    rep = oracle.attention_fp64(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.5, causal=True)
    assert np.max(np.abs(oracle.attention_fp64(q, k, v, 0.5, causal=True) - rep)) == 0.0


def test_causal_split_states_merge_to_causal_attention():
    """Split states under the mask (some rows see none of a split's keys) merge, in any order, to the masked result."""
    r = _rng(740)
    Nq, Nk, d = 9, 40, 5
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    states = oracle.split_partial_states(q, k, v, 0.45, 8, causal=True)
    m0 = states[-1][0]
    assert np.sum(np.isneginf(m0)) > 0 and np.all(states[-1][1][np.isneginf(m0)] == 0)
    ref = oracle.attention_fp64(q[None], k[None], v[None], 0.45, causal=True)[0]
    for order in (None, list(range(7, -1, -1)), [3, 0, 6, 1, 7, 2, 5, 4]):
        got = oracle.finish_state(oracle.merge_sequential(states, order))
        assert np.max(np.abs(got - ref)) < 1e-14


# --- the (lse, o) partial-state form ([CS349E-L11], the note after demo 2) -----------------------

def test_lse_form_merge_demo2():
    """The demo's own segmentation recipe (default_rng(1), S=3000, d=32, x*3, 12 random segments): the
    (lse, o / l) states merged in three orders equal the one-shot output, and the merged lse equals
    scipy's logsumexp of the row (the page calls the two encodings equivalent)."""
    rng = np.random.default_rng(1)
    S, d = 3000, 32
    x = rng.standard_normal(S) * 3
    V = rng.standard_normal((S, d))
    cuts = np.sort(rng.choice(np.arange(1, S), size=11, replace=False))
    bounds = list(zip(np.concatenate([[0], cuts]), np.concatenate([cuts, [S]])))
    states = [oracle.partial_state_lse(x[None, a:b], V[a:b]) for a, b in bounds]
    ref = scipy.special.softmax(x) @ V
    for order in (None, rng.permutation(len(states)), list(range(len(states)))[::-1]):
        lse, out = oracle.merge_lse(states, order)
        assert np.max(np.abs(out[0] - ref)) < 1e-14
        assert abs(lse[0] - scipy.special.logsumexp(x)) < 1e-12


@pytest.mark.parametrize("Nq,Nk,S,causal", [(7, 50, 4, False), (30, 30, 5, True), (9, 40, 8, True)])
def test_lse_form_split_matches_attention(Nq, Nk, S, causal):
    r = _rng(40 + Nk)
    q, k, v = r.standard_normal((Nq, 16)), r.standard_normal((Nk, 16)), r.standard_normal((Nk, 16))
    states = oracle.split_partial_states_lse(q, k, v, 0.3, S, causal=causal)
    lse, out = oracle.merge_lse(states, _rng(5).permutation(S))
    ref = oracle.attention_fp64(q[None], k[None], v[None], 0.3, causal=causal)[0]
    assert np.max(np.abs(out - ref)) < 1e-13
    s = 0.3 * q @ k.T
    if causal:
        s = np.where(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq), s, -np.inf)
    assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=1))) < 1e-12
    if causal:  # some parts hold no visible key for the first rows: (-inf, 0)
        assert any(np.any(np.isneginf(st[0])) for st in states)


def test_lse_form_empty_and_single_states():
    r = _rng(9)
    V = r.standard_normal((6, 4))
    s = r.standard_normal((3, 6))
    one = oracle.partial_state_lse(s, V)
    empty = oracle.partial_state_lse(s[:, :0], V[:0])
    assert np.all(np.isneginf(empty[0])) and np.all(empty[1] == 0)
    for states in ([one], [empty, one], [one, empty, empty]):
        lse, out = oracle.merge_lse(states)
        assert np.array_equal(lse, one[0]) or np.max(np.abs(lse - one[0])) < 1e-15
        assert np.max(np.abs(out - one[1])) < 1e-15
    lse, out = oracle.merge_lse([empty, empty])
    assert np.all(np.isneginf(lse)) and np.all(out == 0)
