"""GPU parity of the (lse, o) split-KV state form (fa_fwd_split_lse, fa_merge_lse) against the oracle.

"CS349E 第 11 讲 01_online_softmax.py" (the note after demo 2): flash-decoding stores per key range the
output already divided by the range's own l and lse_s = m_s + ln(l_s), and combines ranges with
weights exp(lse_s - lse). oracle.partial_state_lse / merge_lse are pinned in tests/test_oracle_pins.py.
"""
import sys

import numpy as np
import pytest
import scipy.special

import oracle
import seeded_inputs as si
from tests._parity import assert_close, stat_bound

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import flashattention_forward_02_amd as fa

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def masked_scores(q, k, scale, causal):
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if causal:
        Nq, Nk = s.shape[-2:]
        s = np.where(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq), s, -np.inf)
    return s


# (B, H, H_kv, Nq, Nk, d, S, causal): the few-row path (Nq <= 16) and the tiled kernels, ragged
# ranges, grouped heads, the mask (ranges a row cannot see give (-inf, 0))
CASES = [
    (1, 2, 2, 1, 1000, 64, 7, False),
    (2, 4, 2, 3, 777, 128, 16, True),
    (1, 2, 1, 40, 300, 64, 5, True),
    (1, 1, 1, 200, 200, 128, 3, False),
    (2, 2, 2, 100, 129, 64, 2, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s)))
def test_lse_states_and_merge(dtype, shape):
    B, H, H_kv, Nq, Nk, d, S, causal = shape
    say(f"lse states dtype={dtype} shape={shape}")
    q = si.per_head_tensor(900 + Nk, B, H, Nq, d, 0, dtype)
    k = si.per_head_tensor(900 + Nk, B, H_kv, Nk, d, 1, dtype)
    v = si.per_head_tensor(900 + Nk, B, H_kv, Nk, d, 2, dtype)
    scale = si.fp32_inverse_sqrt(d)
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    plse, po = fa.fwd_split_lse(qd, kd, vd, S, scale=scale, causal=causal)
    torch.cuda.synchronize()
    plse, po = si.torch_to_f64(plse), si.torch_to_f64(po)
    qf, kf, vf = q.as_f64(), k.as_f64(), v.as_f64()
    g = H // H_kv
    for b in range(B):
        for h in range(H):
            states = oracle.split_partial_states_lse(qf[b, h], kf[b, h // g], vf[b, h // g], scale, S, causal=causal)
            for c, (lse_ref, on_ref) in enumerate(states):
                empty = np.isneginf(lse_ref)
                assert np.array_equal(np.isneginf(plse[c, b, h]), empty), f"part {c}: empty rows differ"
                assert np.all(po[c, b, h][empty] == 0)
                lo, hi = oracle.split_bounds(Nk, S)[c]
                bound = stat_bound(qf[b, h], kf[b, h // g, lo:hi], scale)
                live = ~empty
                assert np.all(np.abs(plse[c, b, h][live] - lse_ref[live]) <= bound[live] * 2)
                assert_close(po[c, b, h][live], on_ref[live], dtype, f"part {c}")
    ref = oracle.attention_fp64(qf, kf, vf, scale, causal=causal)
    lse_ref = scipy.special.logsumexp(masked_scores(qf, np.repeat(kf, g, axis=1), scale, causal), axis=-1)
    bound = stat_bound(qf, np.repeat(kf, g, axis=1), scale)
    for order in (None, si.merge_order(5, S), list(range(S))[::-1]):
        o, lse = fa.merge_lse(*[torch.from_numpy(x.astype(np.float32)).to(DEV) for x in (plse, po)], order=order)
        torch.cuda.synchronize()
        assert_close(si.torch_to_f64(o), ref, dtype, f"merged order={order}")
        assert np.all(np.abs(si.torch_to_f64(lse) - lse_ref) <= 2 * bound + 1e-6)


def test_merge_lse_all_empty_row_and_bf16_output():
    """A row whose ranges are all empty gets O = 0 and lse = -inf; a bf16 output is the rounded fp32 one."""
    S, B, H, Nq, d = 3, 1, 1, 4, 64
    plse = torch.full((S, B, H, Nq), float("-inf"), device=DEV)
    po = torch.zeros((S, B, H, Nq, d), device=DEV)
    plse[1, 0, 0, 1:] = torch.tensor([0.5, -2.0, 3.0], device=DEV)
    po[1, 0, 0, 1:] = torch.randn(3, d, device=DEV)
    o, lse = fa.merge_lse(plse, po)
    ob = fa.merge_lse(plse, po, out_dtype=torch.bfloat16, return_lse=False)
    torch.cuda.synchronize()
    assert torch.all(o[0, 0, 0] == 0) and torch.isneginf(lse[0, 0, 0])
    assert torch.equal(o[0, 0, 1:], po[1, 0, 0, 1:]) and torch.equal(lse[0, 0, 1:], plse[1, 0, 0, 1:])
    assert torch.equal(ob, o.to(torch.bfloat16))


def test_decode_bf16_full_size_lse_form():
    """The split-KV decode workload (B=16, H=32, Nq=1, Nk=32768, d=128 bf16, 16 ranges, merged in the shuffled
    order default_rng(5).permutation(16)) in the (lse, o) form: every row against the oracle."""
    w = si.DECODE_BF16
    say("lse decode full size")
    q, k, v = si.decode_inputs_device(w, DEV)
    order = si.merge_order(w.seed, w.num_splits)
    plse, po = fa.fwd_split_lse(q, k, v, w.num_splits, scale=w.scale)
    o, lse = fa.merge_lse(plse, po, order=order)
    torch.cuda.synchronize()
    qf, kf, vf = (si.torch_to_f64(x) for x in (q, k, v))
    ref = oracle.attention_fp64(qf, kf, vf, w.scale)
    assert_close(si.torch_to_f64(o), ref, "bf16", "decode lse form")
    s = w.scale * np.einsum("bhqd,bhkd->bhqk", qf, kf)
    bound = stat_bound(qf, kf, w.scale)
    assert np.all(np.abs(si.torch_to_f64(lse) - scipy.special.logsumexp(s, axis=-1)) <= 2 * bound + 1e-6)
