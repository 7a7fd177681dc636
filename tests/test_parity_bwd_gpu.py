"""GPU parity of the row log-sum-exp (fa_fwd_lse) and the backward pass (fa_bwd) against the oracle.

"Flash Attention 代码填空 (Level 2-3)" Exercise 5 defines the backward pass as recomputation of P
from the forward statistics with dV = P^T dO; dQ and dK follow from the definition (see
oracle/backward.py, pinned in tests/test_oracle_backward_pins.py). Every case goes through the C
ABI via the package binding and is compared element by element with
oracle.attention_backward_fp64 on the same bf16 / fp16 values, at the tolerances of
tests/_parity.py (BWD_TOL).
"""
import sys

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests._parity import assert_grad_close, stat_bound

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import flashattention_forward_02_amd as fa

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def case(seed, B, H, H_kv, Nq, Nk, d, dtype):
    """Q and dO with H heads, K and V with H_kv heads: independent seeded per-head draws (dO is tensor 3)."""
    q = si.per_head_tensor(seed, B, H, Nq, d, 0, dtype)
    k = si.per_head_tensor(seed, B, H_kv, Nk, d, 1, dtype)
    v = si.per_head_tensor(seed, B, H_kv, Nk, d, 2, dtype)
    do = si.per_head_tensor(seed, B, H, Nq, d, 3, dtype)
    return q, k, v, do


def zero_bounds(q, k, v, do, group, scale):
    """Elementwise bounds for dQ and dK where their reference is zero (one key): dS_ij = P_ij (dP_ij - D_i)
    is then the difference of two fp32 d-term dot products of the same values (dO_i . v_j via the matrix
    core and dO_i . O_i with O_i = v_j), so |dS_ij| <= 2 d 2^-24 sum_c |dO_ic v_jc|, and
    |dQ_i| <= scale sum_j |dS_ij| |K_j|, |dK_j| <= scale sum_i |dS_ij| |Q_i| (summed over the group)."""
    qa, ka, va, da = (np.abs(t.as_f64()) for t in (q, k, v, do))
    d = qa.shape[-1]
    kr, vr = np.repeat(ka, group, axis=1), np.repeat(va, group, axis=1)
    E = 2 * d * 2.0 ** -24 * (da @ np.swapaxes(vr, -1, -2))          # [B, H, Nq, Nk]
    bq = scale * (E @ kr) + 1e-12
    bk_full = scale * (np.swapaxes(E, -1, -2) @ qa)                    # [B, H, Nk, d]
    B, H = qa.shape[:2]
    bk = bk_full.reshape(B, H // group, group, *bk_full.shape[2:]).sum(axis=2) + 1e-12
    return {"dq": bq, "dk": bk}


def run_gpu(q, k, v, do, scale, causal, o_dtype=None):
    qd, kd, vd, dod = (t.to_torch(DEV) for t in (q, k, v, do))
    o, lse = fa.fwd_lse(qd, kd, vd, scale=scale, causal=causal, out_dtype=o_dtype)
    dq, dk, dv, delta = fa.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal, return_delta=True)
    torch.cuda.synchronize()
    return tuple(si.torch_to_f64(t) for t in (o, lse, dq, dk, dv, delta))


# (B, H, H_kv, Nq, Nk, d, causal): one key and one row, ragged tails, one tile and several, Nq < Nk,
# grouped heads (dK, dV summed over the group), the causal mask
CASES = [
    (1, 1, 1, 1, 1, 64, False),
    (1, 2, 2, 5, 7, 64, False),
    (1, 1, 1, 130, 1, 64, False),
    (2, 3, 3, 300, 300, 64, False),
    (1, 2, 1, 300, 333, 64, True),
    (1, 1, 1, 513, 1000, 128, True),
    (2, 2, 2, 64, 129, 128, False),
    (1, 4, 2, 200, 200, 128, True),
    (1, 2, 2, 7, 7, 128, True),
    (1, 8, 1, 70, 260, 64, False),
    # whole tiles: 1, 2 and 3 query or key tiles (the ping-pong kernels' steps rotate three buffers)
    (1, 2, 2, 64, 64, 64, False),
    (1, 2, 2, 128, 192, 64, True),
    (1, 1, 1, 192, 128, 64, False),
    # d = 128: 1, 2 and 3 blocks of 128 keys (dK dV, two buffers) and of 64-row steps, grouped heads
    (1, 2, 2, 64, 128, 128, False),
    (1, 2, 1, 128, 256, 128, True),
    (1, 1, 1, 192, 384, 128, False),
    (1, 4, 1, 130, 260, 128, False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s)))
def test_backward_parity(dtype, shape):
    B, H, H_kv, Nq, Nk, d, causal = shape
    say(f"bwd dtype={dtype} shape={shape}")
    q, k, v, do = case(7000 + Nq + 3 * Nk + H, B, H, H_kv, Nq, Nk, d, dtype)
    scale = si.fp32_inverse_sqrt(d)
    o, lse, dq, dk, dv, delta = run_gpu(q, k, v, do, scale, causal)
    rdq, rdk, rdv, rlse, rdelta = oracle.attention_backward_fp64(q.as_f64(), k.as_f64(), v.as_f64(), do.as_f64(),
                                                                 scale, causal=causal)
    kf = np.repeat(k.as_f64(), H // H_kv, axis=1)
    bound = stat_bound(q.as_f64(), kf, scale)
    assert np.all(np.abs(lse - rlse) <= bound), f"lse off by {np.max(np.abs(lse - rlse)):.3e}"
    # D from the GPU's own O: exact to fp32 rounding of that sum
    assert np.allclose(delta, (do.as_f64() * o).sum(axis=-1), rtol=1e-5, atol=1e-5)
    zb = zero_bounds(q, k, v, do, H // H_kv, scale)
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        ma, rl = assert_grad_close(got, ref, dtype, f"{name} {dtype} {shape}", zero_bound=zb.get(name))
        say(f"  {name}: max_abs={ma:.3e} (max|ref| {np.max(np.abs(ref)):.2e}) rel_l2={rl:.3e}")


def test_backward_bf16_output_and_determinism():
    """o given in bf16 (the forward's out_dtype) is accepted; two calls give identical bits."""
    B, H, H_kv, Nq, Nk, d = 1, 2, 2, 200, 260, 64
    q, k, v, do = case(7777, B, H, H_kv, Nq, Nk, d, "bf16")
    scale = si.fp32_inverse_sqrt(d)
    a = run_gpu(q, k, v, do, scale, False, o_dtype=torch.bfloat16)
    b = run_gpu(q, k, v, do, scale, False, o_dtype=torch.bfloat16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    rdq, rdk, rdv, _, _ = oracle.attention_backward_fp64(q.as_f64(), k.as_f64(), v.as_f64(), do.as_f64(), scale)
    for name, got, ref in (("dq", a[2], rdq), ("dk", a[3], rdk), ("dv", a[4], rdv)):
        assert_grad_close(got, ref, "bf16", name)


def test_backward_no_query_rows():
    """Nq = 0: dK = dV = 0 (only the key-side kernel runs)."""
    d = 64
    k = torch.randn(1, 2, 100, d, device=DEV).to(torch.bfloat16)
    v = torch.randn(1, 2, 100, d, device=DEV).to(torch.bfloat16)
    q = torch.empty(1, 2, 0, d, device=DEV, dtype=torch.bfloat16)
    o = torch.empty(1, 2, 0, d, device=DEV)
    lse = torch.empty(1, 2, 0, device=DEV)
    dq, dk, dv = fa.bwd(q, k, v, o, q.clone(), lse)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_headline_shape_sampled_heads():
    """The forward headline shape B=4, H=16, N=4096, d=64 bf16 (seed 3, dO = tensor 3): every head runs on
    the GPU; the oracle checks two heads in full."""
    w = si.HEADLINE_BF16
    q, k, v = si.workload_inputs(w)
    do = si.per_head_tensor(w.seed, w.B, w.H, w.Nq, w.d, 3, w.dtype)
    say("bwd headline shape")
    o, lse, dq, dk, dv, delta = run_gpu(q, k, v, do, w.scale, False)
    for (b, h) in ((0, 0), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv, rlse, _ = oracle.attention_backward_fp64(q.as_f64()[sl], k.as_f64()[sl], v.as_f64()[sl],
                                                                do.as_f64()[sl], w.scale)
        for name, got, ref in (("dq", dq[sl], rdq), ("dk", dk[sl], rdk), ("dv", dv[sl], rdv)):
            ma, rl = assert_grad_close(got, ref, "bf16", f"headline {name} head {(b, h)}")
            say(f"  head {(b, h)} {name}: max_abs={ma:.3e} rel_l2={rl:.3e}")


def test_backward_d128_workload_sampled_heads():
    """The d = 128 backward workload (B=4, H=16, N=4096, d=128 bf16; seed 3, dO = tensor 3), the launch
    bench.py times: every head runs on the GPU; the oracle checks two heads in full."""
    w = si.BWD_D128_BF16
    q, k, v = si.workload_inputs(w)
    do = si.grad_output(w)
    say("bwd d=128 workload")
    o, lse, dq, dk, dv, delta = run_gpu(q, k, v, do, w.scale, False)
    for (b, h) in ((0, 7), (3, 12)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv, rlse, _ = oracle.attention_backward_fp64(q.as_f64()[sl], k.as_f64()[sl], v.as_f64()[sl],
                                                                do.as_f64()[sl], w.scale)
        for name, got, ref in (("dq", dq[sl], rdq), ("dk", dk[sl], rdk), ("dv", dv[sl], rdv)):
            ma, rl = assert_grad_close(got, ref, "bf16", f"d128 workload {name} head {(b, h)}")
            say(f"  head {(b, h)} {name}: max_abs={ma:.3e} rel_l2={rl:.3e}")


def test_backward_causal_workload_sampled_heads():
    """The causal backward workload (B=4, H=16, N=4096, d=64 bf16, the causal mask; seed 3, dO = tensor 3),
    the launch bench.py times: every head runs on the GPU (longest-first block order, all 16 key and
    query tiles of each head); the oracle checks two heads in full."""
    w = si.BWD_CAUSAL_BF16
    q, k, v = si.workload_inputs(w)
    do = si.grad_output(w)
    say("bwd causal workload")
    o, lse, dq, dk, dv, delta = run_gpu(q, k, v, do, w.scale, True)
    for (b, h) in ((1, 4), (2, 11)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv, rlse, _ = oracle.attention_backward_fp64(q.as_f64()[sl], k.as_f64()[sl], v.as_f64()[sl],
                                                                do.as_f64()[sl], w.scale, causal=True)
        for name, got, ref in (("dq", dq[sl], rdq), ("dk", dk[sl], rdk), ("dv", dv[sl], rdv)):
            ma, rl = assert_grad_close(got, ref, "bf16", f"causal workload {name} head {(b, h)}")
            say(f"  head {(b, h)} {name}: max_abs={ma:.3e} rel_l2={rl:.3e}")
