"""Plain, slow, float64 attention and online-softmax reference (test infrastructure only).

See the package docstring for the source tags ([FA-Simplified], [FA-Fill],
[CS349E-L11], [FA-Scratch]) and what pins each function.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# The definition: three passes over each score row
# ---------------------------------------------------------------------------

def scores_fp64(q, k, scale) -> np.ndarray:
    """s[i, j] = scale * sum_c q[i, c] * k[j, c], in float64.

    [FA-Simplified §1.1] and [FA-Fill Exercise 1]: S = Q K^T / sqrt(d); the scale
    is applied before the maximum is taken. ``scale`` is taken as given (callers
    pass the float32 value the GPU receives); [FA-Scratch §1] is the case scale = 1.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    return float(scale) * (q @ k.T)


def attention_rows_fp64(q, k, v, scale, last_key=None):
    """Full attention for one head: q [Nq, d], k [Nk, d], v [Nk, dv] -> (O [Nq, dv], m [Nq], l [Nq]).

    The three passes of the stored-row form ([CS349E-L11] ``attn_row_3pass``;
    [FA-Simplified §2.1]): m = max_j s_j; p_j = exp(s_j - m), l = sum_j p_j;
    O = (sum_j p_j v_j) / l. ``m`` is the row maximum of the scaled scores and
    ``l`` the sum of exp(s_j - m) (the statistics [FA-Fill Exercise 5] keeps for
    the backward pass).

    ``last_key`` (optional, one int per query row) restricts row i to the keys
    j <= last_key[i]: the scores of the other keys are -inf, so they take no part
    in m, p, l or O (the causal mask of [FA-Simplified §7]; see ``causal_last_key``).
    Every row must keep at least one key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] < 1:
        raise ValueError("softmax over an empty key set is undefined (Nk must be >= 1)")
    s = scores_fp64(q, k, scale)                 # pass 0: the whole score row is stored
    if last_key is not None:
        last_key = np.asarray(last_key).reshape(-1)
        if last_key.shape[0] != q.shape[0] or np.any(last_key < 0):
            raise ValueError("last_key needs one index >= 0 per query row")
        s = np.where(np.arange(k.shape[0])[None, :] <= last_key[:, None], s, NEG_INF)
    m = s.max(axis=1)                            # pass 1: row maximum
    p = np.exp(s - m[:, None])                   # pass 2: exponentials and their sum (exp(-inf) = 0)
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]                     # pass 3: normalise and weight V
    return o, m, l


def causal_last_key(rows, Nq: int, Nk: int) -> np.ndarray:
    """Last key each query row may see under the causal mask: row i sees keys j <= i + (Nk - Nq).

    [FA-Simplified §7] names the causal mask of decoder models (GPT) as the first
    extension and gives no formula. For Nq = Nk this is the usual rule j <= i. For
    Nq < Nk the queries are read as the last Nq positions of the Nk-long sequence
    (a decoder attending to its cached keys), so the last query sees every key.
    Nq > Nk would leave the first rows without keys and is rejected.
    """
    if Nq > Nk:
        raise ValueError("the causal mask needs Nq <= Nk (every query row keeps at least one key)")
    return np.asarray(rows, dtype=np.int64) + (Nk - Nq)


def kv_head_of(h: int, H: int, H_kv: int) -> int:
    """K/V head read by query head h when H query heads share H_kv K/V heads.

    [FA-Simplified §7] names multi-query / grouped-query attention (MQA / GQA) as an
    extension that cuts K/V memory, without a layout. Reading taken: consecutive
    query heads form the groups, H / H_kv heads each, so head h reads K/V head
    h // (H / H_kv); H_kv = H is ordinary multi-head attention and H_kv = 1 is MQA.
    """
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"H={H} is not a multiple of H_kv={H_kv}")
    return h // (H // H_kv)


def attention_fp64(q, k, v, scale, row_block: int = 512, return_stats: bool = False, causal: bool = False):
    """O = softmax(scale * Q K^T) V for [B, H, Nq, d] queries and [B, H_kv, Nk, d] keys and values.

    The result every kernel must reproduce ([FA-Simplified §3.1]: tiling does the
    same arithmetic as standard attention, only its rounding order differs;
    [FA-Simplified §4.1]). Rows are processed in blocks of ``row_block`` queries
    so no buffer exceeds [row_block, Nk] float64; that is a memory bound on this
    reference only and changes no arithmetic.

    K and V may have fewer heads than Q (axis -3): query head h then reads K/V head
    ``kv_head_of(h, H, H_kv)``. With ``causal`` row i sees the keys up to
    ``causal_last_key(i, Nq, Nk)``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim == 2:
        q, k, v = q[None], k[None], v[None]
        squeeze = True
    else:
        squeeze = False
    lead, H, H_kv = q.shape[:-3], q.shape[-3], k.shape[-3]
    assert k.shape[:-3] == lead and v.shape[:-3] == lead, "Q, K, V leading dims differ"
    assert v.shape[-3] == H_kv, "K and V head counts differ"
    Nq, Nk = q.shape[-2], k.shape[-2]
    qf = q.reshape((-1, H, Nq, q.shape[-1]))
    kf = k.reshape((-1, H_kv, Nk, k.shape[-1]))
    vf = v.reshape((-1, H_kv, Nk, v.shape[-1]))
    out = np.empty((qf.shape[0], H, Nq, vf.shape[-1]))
    ms = np.empty((qf.shape[0], H, Nq))
    ls = np.empty((qf.shape[0], H, Nq))
    for b in range(qf.shape[0]):
        for h in range(H):
            hk = kv_head_of(h, H, H_kv)
            for r0 in range(0, Nq, row_block):
                rows = np.arange(r0, min(Nq, r0 + row_block))
                last = causal_last_key(rows, Nq, Nk) if causal else None
                o, m, l = attention_rows_fp64(qf[b, h, rows], kf[b, hk], vf[b, hk], scale, last)
                out[b, h, rows] = o
                ms[b, h, rows] = m
                ls[b, h, rows] = l
    out = out.reshape(lead + (H, Nq, vf.shape[-1]))
    ms = ms.reshape(lead + (H, Nq))
    ls = ls.reshape(lead + (H, Nq))
    if squeeze:
        out, ms, ls = out[0], ms[0], ls[0]
    if return_stats:
        return out, ms, ls
    return out


# ---------------------------------------------------------------------------
# Softmax forms
# ---------------------------------------------------------------------------

def naive_softmax(x) -> np.ndarray:
    """exp(x_i) / sum_j exp(x_j) without the shift: overflows for large x ([FA-Fill Exercise 2])."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        return e / e.sum(axis=-1, keepdims=True)


def safe_softmax(x) -> np.ndarray:
    """Two-pass stable softmax: subtract the row maximum, exponentiate, divide by the sum.

    [FA-Simplified §2.1]; [FA-Fill Exercise 2]; [FA-Scratch §3].
    """
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def online_softmax(x) -> np.ndarray:
    """Element-at-a-time online softmax over the last axis, in plain Python floats.

    [FA-Fill Exercise 2]: while scanning a row keep the running maximum m and the
    running sum l of exp(x - m); when x_j raises the maximum, the old sum is
    scaled by exp(m_old - m_new) before exp(x_j - m_new) is added. A second scan
    writes exp(x_j - m) / l. For small inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty_like(flat)
    for r, row in enumerate(flat):
        m, l = NEG_INF, 0.0
        for xj in row:
            xj = float(xj)
            m_next = max(m, xj)
            l = l * math.exp(m - m_next) + math.exp(xj - m_next)
            m = m_next
        for j, xj in enumerate(row):
            out[r, j] = math.exp(float(xj) - m) / l
    return out.reshape(x.shape)


# ---------------------------------------------------------------------------
# The one-pass (m, l, acc) recurrence
# ---------------------------------------------------------------------------

def _key_blocks(n: int, block: int):
    """Key ranges [start, stop) of consecutive blocks of ``block`` keys (the last one may be shorter)."""
    return [(b0, min(n, b0 + block)) for b0 in range(0, n, block)]


def online_attention_row(q, K, V, block: int, scale=None, history=None) -> np.ndarray:
    """One query against all keys in a single pass over blocks of ``block`` keys.

    [FA-Simplified §2.3] (the recurrence of [CS349E-L11] demo 1): the row's state starts
    as the empty state (m, l, acc) = (-inf, 0, 0), and each block is folded into it. A
    block contributes its own partial state (its maximum, its sum of exponentials, its
    weighted sum of V rows), and folding it in is the merge rule of ``merge_states``:
    the side whose maximum is lower is scaled by exp(m_side - m_new), which is exactly
    the correction factor exp(m_old - m_new) the page applies to l and acc when a block
    raises the maximum (and 0 for the empty start state). The answer is acc / l.
    When ``history`` is a list, the running (m, l) after each block is appended.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[0])
    state = (np.array([NEG_INF]), np.zeros(1), np.zeros((1, V.shape[1])))
    for b0, b1 in _key_blocks(K.shape[0], block):
        s_block = float(scale) * (K[b0:b1] @ q)
        state = merge_states(state, partial_state(s_block[None, :], V[b0:b1]))
        if history is not None:
            history.append((float(state[0][0]), float(state[1][0])))
    return finish_state(state)[0]


def two_pass_attention_row(q, K, V, block: int, scale=None) -> np.ndarray:
    """Two scans over key blocks ([CS349E-L11] demo 1's two-pass variant): statistics, then weights.

    Scan one reduces the blocks' scores to the row's (m, l) without storing them across
    blocks: every block gives (max, sum exp(s - max)), and the row's statistics are
    m = max over blocks, l = sum over blocks of l_b exp(m_b - m). Scan two recomputes each
    block's scores and adds exp(s - m) / l times that block's V rows.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[0])
    blocks = _key_blocks(K.shape[0], block)
    stats = np.empty((len(blocks), 2))
    for i, (b0, b1) in enumerate(blocks):
        s_block = float(scale) * (K[b0:b1] @ q)
        stats[i, 0] = s_block.max()
        stats[i, 1] = np.exp(s_block - stats[i, 0]).sum()
    m = stats[:, 0].max()
    l = float(np.sum(stats[:, 1] * np.exp(stats[:, 0] - m)))
    out = np.zeros(V.shape[1])
    for b0, b1 in blocks:
        w = np.exp(float(scale) * (K[b0:b1] @ q) - m) / l
        out += w @ V[b0:b1]
    return out


def online_attention(q, k, v, scale, Br: int, Bc: int, return_stats: bool = False):
    """Tiled forward, Q tiles outside and K/V tiles inside, normalised once at the end.

    [FA-Simplified §2.3 and §3.1]; [FA-Scratch §4-§5]. For each Q tile of Br rows
    the state (m, l, O) is reset to (-inf, 0, 0); for each K/V tile of Bc keys:
    S = scale Q_i K_j^T; m' = max(m, rowmax S); c = exp(m - m');
    P = exp(S - m'); l = c l + rowsum P; O = c O + P V_j; m = m'. After the last
    tile O / l is written. Tails shorter than Br or Bc are processed as shorter
    tiles. Works on [..., N, d] inputs, one head at a time.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    Nq, Nk = q.shape[-2], k.shape[-2]
    qf = q.reshape(-1, Nq, q.shape[-1])
    kf = k.reshape(-1, Nk, k.shape[-1])
    vf = v.reshape(-1, Nk, v.shape[-1])
    out = np.empty((qf.shape[0], Nq, vf.shape[-1]))
    ms = np.empty((qf.shape[0], Nq))
    ls = np.empty((qf.shape[0], Nq))
    for h in range(qf.shape[0]):
        for i0 in range(0, Nq, Br):
            Qi = qf[h, i0:i0 + Br]
            m = np.full(Qi.shape[0], NEG_INF)
            l = np.zeros(Qi.shape[0])
            O = np.zeros((Qi.shape[0], vf.shape[-1]))
            for j0 in range(0, Nk, Bc):
                S = float(scale) * (Qi @ kf[h, j0:j0 + Bc].T)
                m_next = np.maximum(m, S.max(axis=1))
                c = np.exp(m - m_next)
                P = np.exp(S - m_next[:, None])
                l = c * l + P.sum(axis=1)
                O = c[:, None] * O + P @ vf[h, j0:j0 + Bc]
                m = m_next
            out[h, i0:i0 + Br] = O / l[:, None]
            ms[h, i0:i0 + Br] = m
            ls[h, i0:i0 + Br] = l
    out = out.reshape(lead + (Nq, vf.shape[-1]))
    if return_stats:
        return out, ms.reshape(lead + (Nq,)), ls.reshape(lead + (Nq,))
    return out


def fa1_order_attention(q, k, v, scale, block: int) -> np.ndarray:
    """K/V blocks in the outer loop, with O kept normalised after every block ([FA-Fill Exercise 4]).

    The query blocks of the exercise's inner loop are independent of one another, so all
    query rows are updated together here. Per K/V block j, for every row: the new maximum
    m' = max(m, rowmax S_j); the mass carried over from earlier blocks, l exp(m - m'); the new
    total l' = carried + rowsum exp(S_j - m'); and O, which always holds the normalised
    output of the keys seen so far, becomes the l'-weighted mix of the old O (weight
    carried / l') and of this block's exp(S_j - m') V_j / l'. Nothing is divided at the end.
    Single head: q [Nq, d], k, v [Nk, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq = q.shape[0]
    O = np.zeros((Nq, v.shape[1]))
    l = np.zeros(Nq)
    m = np.full(Nq, NEG_INF)
    for b0, b1 in _key_blocks(k.shape[0], block):
        S = float(scale) * (q @ k[b0:b1].T)
        m_new = np.maximum(m, S.max(axis=1))
        E = np.exp(S - m_new[:, None])
        carried = l * np.exp(m - m_new)
        total = carried + E.sum(axis=1)
        O = (carried / total)[:, None] * O + (E @ v[b0:b1]) / total[:, None]
        m, l = m_new, total
    return O


# ---------------------------------------------------------------------------
# Partial states and their merge (split-KV)
# ---------------------------------------------------------------------------

def partial_state(s, V):
    """(m, l, o) of one segment of score rows: m = max s, l = sum exp(s - m), o = sum exp(s - m) v (unnormalised).

    [CS349E-L11] demo 2 builds these per segment and finishes a state as o / l,
    which fixes o as the unnormalised weighted sum. ``s`` is [rows, n], V [n, dv].
    An empty segment (n = 0) is the identity state (-inf, 0, 0).
    """
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    V = np.asarray(V, dtype=np.float64)
    if s.shape[1] == 0:
        return (np.full(s.shape[0], NEG_INF), np.zeros(s.shape[0]), np.zeros((s.shape[0], V.shape[1])))
    m = s.max(axis=1)
    live = np.isfinite(m)        # a row whose scores are all -inf (masked) keeps the identity state
    p = np.zeros_like(s)
    p[live] = np.exp(s[live] - m[live, None])
    return m, p.sum(axis=1), p @ V


def _weight(m_part, m_total):
    """exp(m_part - m_total), with 0 for an empty part (m_part = -inf) so that -inf - (-inf) never occurs."""
    m_part = np.asarray(m_part, dtype=np.float64)
    w = np.zeros_like(m_part)
    live = np.isfinite(m_part)
    w[live] = np.exp(m_part[live] - np.asarray(m_total, dtype=np.float64)[live])
    return w


def merge_states(a, b):
    """Combine two partial states of disjoint key sets into the state of their union.

    The merge [CS349E-L11] demo 2 uses but does not print, derived from the
    recurrence of [FA-Scratch §4] and the two-block identity of [FA-Simplified §2.2]:
    m = max(m_a, m_b); l = l_a e^(m_a-m) + l_b e^(m_b-m); o = o_a e^(m_a-m) + o_b e^(m_b-m).
    A part whose m is -inf (no keys) contributes weight 0.
    """
    ma, la, oa = a
    mb, lb, ob = b
    m = np.maximum(ma, mb)
    wa, wb = _weight(ma, m), _weight(mb, m)
    return m, la * wa + lb * wb, oa * wa[..., None] + ob * wb[..., None]


def merge_sequential(states, order=None):
    """Fold states left to right, in ``order`` (a permutation of their indices) when given ([CS349E-L11] demo 2)."""
    idx = list(range(len(states))) if order is None else [int(i) for i in order]
    acc = states[idx[0]]
    for i in idx[1:]:
        acc = merge_states(acc, states[i])
    return acc


def merge_tree(states):
    """Pairwise (tree) merge, as a parallel reduction would do it ([CS349E-L11] demo 2)."""
    level = list(states)
    while len(level) > 1:
        nxt = []
        for i in range(0, len(level), 2):
            nxt.append(merge_states(level[i], level[i + 1]) if i + 1 < len(level) else level[i])
        level = nxt
    return level[0]


def finish_state(state):
    """o / l: the attention output of a (merged) state ([CS349E-L11] demo 2).

    A row whose state is empty (l = 0: none of its parts held a key the row may see) has no
    softmax to finish; it gets O = 0, the value the (lse, o) form gives such a row.
    """
    m, l, o = state
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    out = np.zeros_like(o)
    live = l > 0
    out[live] = o[live] / l[live][..., None]
    return out


def split_bounds(Nk: int, num_splits: int):
    """Key ranges of a split-KV partition: split c covers [floor(c Nk / S), floor((c+1) Nk / S)).

    The pages split a key row into contiguous segments ([CS349E-L11] demo 2,
    flash-decoding); this balanced rule is the partition the library documents.
    """
    return [((c * Nk) // num_splits, ((c + 1) * Nk) // num_splits) for c in range(num_splits)]


def split_partial_states(q, k, v, scale, num_splits: int, causal: bool = False):
    """Per-split (m, l, o) for one head: q [Nq, d], k, v [Nk, d] -> list of states over ``split_bounds``.

    With ``causal`` the scores of keys past ``causal_last_key`` are -inf first; a split
    holding no key a row may see gives that row the identity state (-inf, 0, 0).
    """
    s = scores_fp64(q, k, scale)
    if causal:
        last = causal_last_key(np.arange(s.shape[0]), s.shape[0], s.shape[1])
        s = np.where(np.arange(s.shape[1])[None, :] <= last[:, None], s, NEG_INF)
    v = np.asarray(v, dtype=np.float64)
    return [partial_state(s[:, a:b], v[a:b]) for a, b in split_bounds(k.shape[0], num_splits)]


# ---------------------------------------------------------------------------
# The (lse, o) form of a partial state (flash-decoding)
# ---------------------------------------------------------------------------

def partial_state_lse(s, V):
    """(lse, o_n) of one segment of score rows: lse = m + ln(l), o_n = o / l.

    [CS349E-L11], the note after demo 2: flash-decoding stores per segment the output already
    divided by the segment's own l and lse_s = m_s + log l_s (one value fewer than (m, l, o)).
    ``s`` is [rows, n], V [n, dv]. A row with no keys (empty segment, or all scores -inf) gets
    (-inf, 0).
    """
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    V = np.asarray(V, dtype=np.float64)
    rows, dv = s.shape[0], V.shape[1]
    lse = np.full(rows, NEG_INF)
    on = np.zeros((rows, dv))
    if s.shape[1] == 0:
        return lse, on
    m = s.max(axis=1)
    live = np.isfinite(m)
    p = np.exp(s[live] - m[live, None])
    l = p.sum(axis=1)
    lse[live] = m[live] + np.log(l)
    on[live] = (p @ V) / l[:, None]
    return lse, on


def merge_lse(states, order=None):
    """Combine (lse_s, o_s) states: lse = ln(sum_s exp(lse_s)), O = sum_s exp(lse_s - lse) o_s.

    [CS349E-L11] (note after demo 2): the parts are weighted by exp(lse_s - lse). The log-sum-exp is
    taken as max_s lse_s + ln(sum_s exp(lse_s - max)); both sums run in ``order`` (a permutation of
    the state indices; default ascending). Empty parts (lse_s = -inf) weigh 0; a row whose parts
    are all empty gets O = 0 and lse = -inf.
    """
    idx = list(range(len(states))) if order is None else [int(i) for i in order]
    L = np.stack([np.asarray(states[i][0], dtype=np.float64) for i in idx])        # [S, rows]
    O = np.stack([np.asarray(states[i][1], dtype=np.float64) for i in idx])        # [S, rows, dv]
    mx = L.max(axis=0)
    live = np.isfinite(mx)
    w = np.zeros_like(L)
    fin = np.isfinite(L) & live[None, :]
    w[fin] = np.exp(L[fin] - np.broadcast_to(mx, L.shape)[fin])
    lse = np.full(mx.shape, NEG_INF)
    lse[live] = mx[live] + np.log(w[:, live].sum(axis=0))
    wt = np.zeros_like(L)
    wt[fin] = np.exp(L[fin] - np.broadcast_to(lse, L.shape)[fin])
    out = (wt[..., None] * O).sum(axis=0)
    return lse, out


def split_partial_states_lse(q, k, v, scale, num_splits: int, causal: bool = False):
    """Per-split (lse, o / l) for one head over ``split_bounds`` (the causal mask as in ``split_partial_states``)."""
    s = scores_fp64(q, k, scale)
    if causal:
        last = causal_last_key(np.arange(s.shape[0]), s.shape[0], s.shape[1])
        s = np.where(np.arange(s.shape[1])[None, :] <= last[:, None], s, NEG_INF)
    v = np.asarray(v, dtype=np.float64)
    return [partial_state_lse(s[:, a:b], v[a:b]) for a, b in split_bounds(k.shape[0], num_splits)]


# ---------------------------------------------------------------------------
# Brute force for tiny inputs
# ---------------------------------------------------------------------------

def brute_force_attention(q, k, v, scale):
    """Literal loops over Python floats with math.exp and math.fsum; for tiny single-head inputs only.

    The standard-attention definition of [FA-Simplified §1.1] evaluated element
    by element: s_ij = scale sum_c q_ic k_jc; p_ij = exp(s_ij - max_j s_ij);
    O_i = sum_j p_ij v_j / sum_j p_ij.
    """
    q = [[float(x) for x in row] for row in np.asarray(q)]
    k = [[float(x) for x in row] for row in np.asarray(k)]
    v = [[float(x) for x in row] for row in np.asarray(v)]
    out = []
    for qi in q:
        s = [float(scale) * math.fsum(a * b for a, b in zip(qi, kj)) for kj in k]
        mx = max(s)
        p = [math.exp(x - mx) for x in s]
        l = math.fsum(p)
        out.append([math.fsum(p[j] * v[j][c] for j in range(len(k))) / l for c in range(len(v[0]))])
    return np.array(out)


# ---------------------------------------------------------------------------
# Low-precision rounding of P (the precision demo)
# ---------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return them widened to float64.

    [CS349E-L11] demo 4 casts P to BF16 before P.V while m, l and the
    accumulator stay in FP32. Rounding is done on the float32 bit pattern: add
    0x7FFF plus the lowest kept bit, then clear the low 16 bits.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return (r.astype(np.uint32)).view(np.float32).astype(np.float64)


def round_to_f16(x) -> np.ndarray:
    """Round float32 values to the nearest IEEE half (ties to even), widened to float64 ([CS349E-L11] demo 4)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)
