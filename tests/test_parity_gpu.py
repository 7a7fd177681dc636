"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Tolerances live in tests/_parity.py. Small cases span several tiles and ragged tails; the
workload-size cases compare sampled rows that the oracle computes one head at a time.
"""
import sys

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests._parity import assert_close, assert_stats, errors, stat_bound

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import flashattention_forward_02_amd as fa
    from flashattention_forward_02_amd import _native as n

DEV = "cuda:0"
TORCH_DT = {"f32": None, "bf16": None, "f16": None}


def _tdt(dtype):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_case(q, k, v, dtype, scale, out_dtype="f32", stats=True):
    """Run fa_fwd on host Tensors; return O, m, l as float64 numpy (m, l are None when ``stats`` is False:
    the call then asks for O only, which the matrix-core kernel serves with its sum-checked softmax)."""
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    res = fa.fwd(qd, kd, vd, scale=scale, out_dtype=_tdt(out_dtype), return_stats=stats)
    torch.cuda.synchronize()
    if not stats:
        return si.torch_to_f64(res), None, None
    o, m, l = res
    return si.torch_to_f64(o), si.torch_to_f64(m), si.torch_to_f64(l)


# ---------------------------------------------------------------------------------------------
# small shapes: several tiles, ragged tails, every dtype and head dim
# ---------------------------------------------------------------------------------------------

SMALL = [
    # (B, H, Nq, Nk, d)
    (1, 1, 1, 1, 64),
    (1, 1, 5, 7, 64),
    (2, 3, 300, 333, 64),
    (1, 2, 257, 64, 64),
    (1, 1, 513, 1000, 128),
    (2, 1, 64, 129, 128),
    (1, 1, 17, 4097, 64),
    (1, 2, 16, 300, 128),
]


# fp32 launches of at most 256 rows (d = 64) or 1024 (d = 128) run one workgroup per row, larger
# ones the tiled kernels: both sides of each limit, with and without the mask and the statistics.
F32_LIMITS = [(1, 1, 512, 600, 64), (1, 1, 513, 600, 64), (1, 4, 256, 300, 128), (1, 4, 257, 300, 128),
              (2, 2, 128, 129, 64), (2, 2, 129, 129, 64), (1, 3, 100, 1000, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", F32_LIMITS, ids=lambda s: "x".join(map(str, s)))
def test_fp32_kernel_choice_limits(shape, causal):
    B, H, Nq, Nk, d = shape
    say(f"fp32 kernel choice shape={shape} causal={causal}")
    q, k, v = si.small_case(5000 + Nq + Nk + d, B, H, Nq, Nk, d, "f32")
    scale = si.fp32_inverse_sqrt(d)
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    o, m, l = fa.fwd(qd, kd, vd, scale=scale, out_dtype=torch.float32, return_stats=True, causal=causal)
    torch.cuda.synchronize()
    ref, m_ref, l_ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), scale, return_stats=True,
                                              causal=causal)
    assert_close(si.torch_to_f64(o), ref, "f32", f"fp32 {shape} causal={causal}")
    assert_stats(si.torch_to_f64(m), si.torch_to_f64(l), m_ref, l_ref, stat_bound(q.as_f64(), k.as_f64(), scale),
                 f"fp32 {shape} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(dtype, shape):
    B, H, Nq, Nk, d = shape
    say(f"small case dtype={dtype} shape={shape}")
    q, k, v = si.small_case(1000 + Nq + Nk, B, H, Nq, Nk, d, dtype)
    scale = si.fp32_inverse_sqrt(d)
    o, m, l = run_case(q, k, v, dtype, scale)
    ref, m_ref, l_ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), scale, return_stats=True)
    assert_close(o, ref, dtype, f"{dtype} {shape}")
    assert_stats(m, l, m_ref, l_ref, stat_bound(q.as_f64(), k.as_f64(), scale), f"{dtype} {shape}")


# Key-tile counts 1, 2 and 3 (full and ragged), with and without the causal mask and the row
# statistics (without them the tiled kernel takes its sum-checked path): the d = 64 tiled kernel
# synchronises once per 64-key tile, the d = 128 one twice, and the first and last tiles and the
# prologue differ between the two wave groups.
TILE_COUNTS = [(100, nk, False) for nk in (1, 33, 64, 65, 128, 129, 192)] + \
    [(17, 17, True), (64, 64, True), (65, 65, True), (100, 129, True), (130, 130, True), (64, 192, True)]


@pytest.mark.parametrize("stats", [False, True], ids=["fast", "stats"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", TILE_COUNTS, ids=lambda c: f"{c[0]}x{c[1]}{'c' if c[2] else ''}")
def test_key_tile_counts(case, d, stats):
    Nq, Nk, causal = case
    say(f"key tile counts Nq={Nq} Nk={Nk} d={d} causal={causal} stats={stats}")
    q, k, v = si.small_case(3000 + Nq + Nk + d, 1, 2, Nq, Nk, d, "bf16")
    scale = si.fp32_inverse_sqrt(d)
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    res = fa.fwd(qd, kd, vd, scale=scale, out_dtype=torch.float32, return_stats=stats, causal=causal)
    torch.cuda.synchronize()
    ref, m_ref, l_ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), scale, return_stats=True,
                                              causal=causal)
    if stats:
        o, m, l = (si.torch_to_f64(x) for x in res)
        assert_stats(m, l, m_ref, l_ref, stat_bound(q.as_f64(), k.as_f64(), scale), f"tiles {case} d={d}")
    else:
        o = si.torch_to_f64(res)
    assert_close(o, ref, "bf16", f"tiles {case} d={d} stats={stats}")


# No kernel uses atomics or an order that depends on timing, so repeated calls give identical bits.
DETERMINISM = [("bf16", (2, 4, 700, 900, 64), False), ("bf16", (1, 3, 300, 500, 128), True), ("f32", (1, 1, 256, 300, 64), False),
               ("f32", (1, 2, 300, 400, 64), True), ("f32", (1, 2, 600, 300, 128), False), ("bf16", (2, 4, 1, 5000, 128), False)]


@pytest.mark.parametrize("case", DETERMINISM, ids=lambda c: f"{c[0]}-{'x'.join(map(str, c[1]))}{'c' if c[2] else ''}")
def test_forward_is_bitwise_repeatable(case):
    dtype, (B, H, Nq, Nk, d), causal = case
    say(f"determinism dtype={dtype} shape={(B, H, Nq, Nk, d)} causal={causal}")
    q, k, v = si.small_case(6000 + Nq + Nk + d, B, H, Nq, Nk, d, dtype)
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    runs = []
    for _ in range(3):
        o, m, l = fa.fwd(qd, kd, vd, out_dtype=torch.float32, return_stats=True, causal=causal)
        o_only = fa.fwd(qd, kd, vd, out_dtype=torch.float32, causal=causal)
        ps = fa.fwd_split_lse(qd, kd, vd, 7, causal=causal)
        om = fa.merge_lse(*ps, order=list(range(7))[::-1], return_lse=False)
        torch.cuda.synchronize()
        runs.append([t.cpu().numpy() for t in (o, m, l, o_only, om)])
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            assert np.array_equal(x, y, equal_nan=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_low_precision_output_dtype(dtype):
    q, k, v = si.small_case(77, 2, 2, 300, 500, 64, dtype)
    scale = si.fp32_inverse_sqrt(64)
    o, _, _ = run_case(q, k, v, dtype, scale, out_dtype=dtype)
    ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), scale)
    assert_close(o, ref, dtype, f"{dtype} out")


# ---------------------------------------------------------------------------------------------
# degenerate cases the method has
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_scale_gives_column_mean(dtype):
    q, k, v = si.small_case(5, 1, 2, 300, 130, 64, dtype)
    o, m, l = run_case(q, k, v, dtype, 0.0)
    ref = np.broadcast_to(v.as_f64().mean(axis=2, keepdims=True), o.shape)
    assert_close(o, ref, dtype, "scale=0")
    assert np.all(m == 0.0) and np.allclose(l, 130.0, rtol=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_key_returns_v(dtype):
    q, k, v = si.small_case(6, 1, 1, 300, 1, 128, dtype)
    o, _, l = run_case(q, k, v, dtype, 0.3)
    assert np.array_equal(o, np.broadcast_to(v.as_f64(), o.shape)) or errors(o, np.broadcast_to(v.as_f64(), o.shape))[0] < 1e-6
    assert np.allclose(l, 1.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_score_shift(dtype):
    """Scores near 100 (exp would overflow without the running max) stay finite and correct.

    An fp32 score of magnitude |s| is itself only known to |s| * 2^-24 before the max is
    subtracted, so at |s| ~ 100 the fp32 bar is scaled by the score size: max_abs and rel_l2
    within 2^-20 * max|s| (16 half-ulps of the largest score). bf16 keeps its usual bar.
    """
    q, k, v = si.small_case(8, 1, 1, 260, 300, 64, dtype)
    qf = q.as_f64()
    u = qf[0, 0].mean(axis=0)
    u = u * (100.0 / (0.125 * float(u @ u)))
    k2 = si.encode((k.as_f64() + u).astype(np.float32), dtype)
    o, _, _ = run_case(q, k2, v, dtype, 0.125)
    ref, m_ref, _ = oracle.attention_fp64(qf, k2.as_f64(), v.as_f64(), 0.125, return_stats=True)
    assert np.all(np.isfinite(o)) and float(np.max(m_ref)) > 50.0
    if dtype == "f32":
        bar = 2.0 ** -20 * float(np.max(np.abs(m_ref)))
        max_abs, rel_l2 = errors(o, ref)
        assert max_abs <= bar and rel_l2 <= bar, (max_abs, rel_l2, bar)
    else:
        assert_close(o, ref, dtype, "shifted")


def test_empty_work_is_noop():
    q = torch.zeros((1, 2, 0, 64), device=DEV, dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 5, 64), device=DEV, dtype=torch.bfloat16)
    o = fa.fwd(q, k, k)
    assert o.shape == (1, 2, 0, 64)
    q = torch.zeros((0, 2, 4, 64), device=DEV, dtype=torch.bfloat16)
    k = torch.zeros((0, 2, 5, 64), device=DEV, dtype=torch.bfloat16)
    assert fa.fwd(q, k, k).shape == (0, 2, 4, 64)


def test_device_pointer_validation():
    x = torch.zeros(4 * 64 + 8, device=DEV, dtype=torch.bfloat16)
    st = n.fa_fwd(x.data_ptr() + 2, x.data_ptr(), x.data_ptr(), x.data_ptr(), None, None, 1, 1, 4, 4, 64, 0.125,
                  n.FA_BF16, n.FA_F32, None)
    assert st == n.FA_EINVAL and "aligned" in n.fa_last_error()


def test_raw_c_abi_call_on_current_stream():
    """Call fa_fwd with raw pointers (no Python wrapper logic) on a side stream."""
    q, k, v = si.small_case(21, 1, 2, 100, 200, 64, "bf16")
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    o = torch.empty((1, 2, 100, 64), device=DEV, dtype=torch.float32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        st = n.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), None, None, 1, 2, 100, 200, 64,
                      0.125, n.FA_BF16, n.FA_F32, s.cuda_stream)
    assert st == n.FA_OK, n.fa_last_error()
    s.synchronize()
    ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), 0.125)
    assert_close(si.torch_to_f64(o), ref, "bf16", "raw abi")


def test_no_device_allocation_and_no_nxn_buffer():
    """The library allocates nothing: free device memory is unchanged across a large call, which an
    N x N fp32 score buffer (4 GiB at B*H=64, N=4096) would not leave unchanged."""
    w = si.HEADLINE_BF16
    g = torch.Generator(device=DEV)
    g.manual_seed(1)
    q = torch.randn((w.B, w.H, w.Nq, w.d), device=DEV, generator=g).to(torch.bfloat16)
    k = torch.randn((w.B, w.H, w.Nk, w.d), device=DEV, generator=g).to(torch.bfloat16)
    v = torch.randn((w.B, w.H, w.Nk, w.d), device=DEV, generator=g).to(torch.bfloat16)
    o = torch.empty((w.B, w.H, w.Nq, w.d), device=DEV, dtype=torch.float32)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    fa.fwd(q, k, v, out=o)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert abs(free1 - free0) < 64 * 2 ** 20, (free0, free1)


@pytest.mark.parametrize("path", ["fp32_fwd", "split_merge", "lse_bwd"])
def test_no_device_allocation_other_paths(path):
    """The fp32 forward, the split-KV states with their merge, and the forward-with-lse plus backward
    allocate nothing either: with every output and workspace allocated up front, free device memory
    and torch's allocation count are unchanged across the calls."""
    g = torch.Generator(device=DEV)
    g.manual_seed(2)
    if path == "fp32_fwd":
        q = torch.randn((1, 1, 4096, 64), device=DEV, generator=g)
        k = torch.randn((1, 1, 4096, 64), device=DEV, generator=g)
        v = torch.randn((1, 1, 4096, 64), device=DEV, generator=g)
        o = torch.empty_like(q)
        run = lambda: fa.fwd(q, k, v, out=o)
    elif path == "split_merge":
        B, H, Nk, d, S = 4, 8, 8192, 128, 16
        q = torch.randn((B, H, 1, d), device=DEV, generator=g).to(torch.bfloat16)
        k = torch.randn((B, H, Nk, d), device=DEV, generator=g).to(torch.bfloat16)
        v = torch.randn((B, H, Nk, d), device=DEV, generator=g).to(torch.bfloat16)
        pm = torch.empty((S, B, H, 1), device=DEV)
        pl = torch.empty_like(pm)
        po = torch.empty((S, B, H, 1, d), device=DEV)
        o = torch.empty((B, H, 1, d), device=DEV)
        order = list(range(S))[::-1]

        def run():
            fa.fwd_split(q, k, v, S, workspace=(pm, pl, po))
            fa.merge_states(pm, pl, po, order=order, out=o)
    else:
        B, H, N, d = 2, 4, 1024, 64
        q, k, v, dout = (torch.randn((B, H, N, d), device=DEV, generator=g).to(torch.bfloat16) for _ in range(4))
        o, lse = fa.fwd_lse(q, k, v)
        grads = (torch.empty((B, H, N, d), device=DEV), torch.empty((B, H, N, d), device=DEV),
                 torch.empty((B, H, N, d), device=DEV), torch.empty((B, H, N), device=DEV))
        run = lambda: fa.bwd(q, k, v, o, dout, lse, out=grads)
    run()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    run()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0, path
    assert abs(free1 - free0) < 64 * 2 ** 20, (path, free0, free1)


# ---------------------------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------------------------

def test_single_head_fp32_256x64():
    say("single_head_fp32")
    q, k, v = si.single_head_fp32()
    o, m, l = run_case(q, k, v, "f32", 0.125)
    ref, m_ref, l_ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), 0.125, return_stats=True)
    assert_close(o, ref, "f32", "single head fp32")
    assert_stats(m, l, m_ref, l_ref, stat_bound(q.as_f64(), k.as_f64(), 0.125))


def test_fp32_key_range_past_2gib():
    """fp32 at d = 64 with 8388645 keys: K and V each span more than 2^31 bytes (past what a 32-bit
    byte count covers), and 300 query rows take the matrix-core kernel. Three rows against the
    oracle; Q, K, V drawn on the device (seeds 7001, 7002, 7003)."""
    B, H, Nq, Nk, d = 1, 1, 300, 8388645, 64
    say("fp32 key range past 2 GiB: drawing 4.3 GB of K and V on the device")
    q = si.device_draw((B, H, Nq, d), 7001, "f32", DEV)
    k = si.device_draw((B, H, Nk, d), 7002, "f32", DEV)
    v = si.device_draw((B, H, Nk, d), 7003, "f32", DEV)
    o, m, l = fa.fwd(q, k, v, scale=0.125, out_dtype=torch.float32, return_stats=True)
    torch.cuda.synchronize()
    say("fp32 key range past 2 GiB: oracle on 3 rows")
    rows = np.array([0, 151, 299])
    qh = si.torch_to_f64(q[0, 0])[rows]
    kh, vh = si.torch_to_f64(k[0, 0]), si.torch_to_f64(v[0, 0])
    del k, v
    ref, m_ref, l_ref = oracle.attention_rows_fp64(qh, kh, vh, 0.125)
    assert_close(si.torch_to_f64(o[0, 0])[rows], ref, "f32", "fp32 key range past 2 GiB")
    assert_stats(si.torch_to_f64(m[0, 0])[rows], si.torch_to_f64(l[0, 0])[rows], m_ref, l_ref,
                 stat_bound(qh, kh, 0.125), "fp32 key range past 2 GiB")


@pytest.mark.parametrize("batched", [False, True])
def test_one_query_long_keys_fp32(batched):
    say(f"one_query_long_keys batched={batched}")
    q, k, v = si.one_query_long_keys(batched=batched)
    o, m, l = run_case(q, k, v, "f32", 0.125)
    ref, m_ref, l_ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), 0.125, return_stats=True)
    assert_close(o, ref, "f32", f"one query batched={batched}")
    assert_stats(m, l, m_ref, l_ref, stat_bound(q.as_f64(), k.as_f64(), 0.125))
    if batched:
        q1, k1, v1 = si.one_query_long_keys(batched=False)
        o1, _, _ = run_case(q1, k1, v1, "f32", 0.125)
        assert np.max(np.abs(o[0, 0, 0] - o1[0, 0, 0])) < 1e-6


def _sampled_rows(w, o, m, l, q, k, v, heads, rows_per_head, seed):
    r = np.random.default_rng(seed)
    qf, kf, vf = q.as_f64() if hasattr(q, "as_f64") else q, k, v
    got, ref, gm, gl, rm, rl, bd = [], [], [], [], [], [], []
    for (b, h) in heads:
        rows = np.sort(r.choice(w.Nq, size=min(rows_per_head, w.Nq), replace=False))
        kh = kf(b, h) if callable(kf) else kf[b, h]
        vh = vf(b, h) if callable(vf) else vf[b, h]
        qh = qf(b, h) if callable(qf) else qf[b, h]
        o_ref, m_ref, l_ref = oracle.attention_rows_fp64(qh[rows], kh, vh, w.scale)
        got.append(o[b, h, rows]); ref.append(o_ref)
        gm.append(m[b, h, rows]); gl.append(l[b, h, rows]); rm.append(m_ref); rl.append(l_ref)
        bd.append(stat_bound(qh[rows], kh, w.scale))
    return (np.concatenate(got), np.concatenate(ref), np.concatenate(gm), np.concatenate(gl), np.concatenate(rm),
            np.concatenate(rl), np.concatenate(bd))


def test_headline_bf16_full_size():
    """B=4, H=16, N=4096, d=64 bf16 at full size (the benchmarked launch), sampled rows from 8 heads."""
    w = si.HEADLINE_BF16
    say("headline: generating inputs")
    q, k, v = si.workload_inputs(w)
    say("headline: running fa_fwd")
    o, m, l = run_case(q, k, v, "bf16", w.scale)
    qf, kf, vf = q.as_f64(), k.as_f64(), v.as_f64()
    heads = [(0, 0), (0, 15), (1, 3), (2, 8), (3, 15), (3, 0), (1, 11), (2, 2)]
    got, ref, gm, gl, rm, rl, bd = _sampled_rows(w, o, m, l, qf, kf, vf, heads, 256, 3)
    say(f"headline: errors {errors(got, ref)}")
    assert_close(got, ref, "bf16", "headline sampled rows")
    assert_stats(gm, gl, rm, rl, bd, "headline")
    assert np.all(np.isfinite(o))


def test_long_seq_bf16_full_size():
    """B=1, H=32, N=16384, d=128 bf16 with K x3 at full size; sampled rows from 6 heads."""
    w = si.LONG_SEQ_BF16
    say("long_seq: generating inputs")
    q, k, v = si.workload_inputs(w)
    say("long_seq: running fa_fwd")
    o, m, l = run_case(q, k, v, "bf16", w.scale)
    heads = [(0, 0), (0, 7), (0, 13), (0, 20), (0, 26), (0, 31)]
    qb = lambda b, h: si.bf16_bits_to_f32(q.data[b, h]).astype(np.float64)
    kb = lambda b, h: si.bf16_bits_to_f32(k.data[b, h]).astype(np.float64)
    vb = lambda b, h: si.bf16_bits_to_f32(v.data[b, h]).astype(np.float64)
    got, ref, gm, gl, rm, rl, bd = _sampled_rows(w, o, m, l, qb, kb, vb, heads, 128, 4)
    say(f"long_seq: errors {errors(got, ref)}")
    assert_close(got, ref, "bf16", "long seq sampled rows")
    assert_stats(gm, gl, rm, rl, bd, "long seq")
    assert np.all(np.isfinite(o))


# ---------------------------------------------------------------------------------------------
# split-KV partial states and their merge
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("shape", [(2, 3, 1, 1000, 128, 16), (1, 2, 3, 777, 64, 5), (1, 1, 40, 900, 64, 7),
                                   (1, 2, 300, 700, 128, 3)], ids=lambda s: "x".join(map(str, s)))
def test_split_states_and_merge_orders(dtype, shape):
    B, H, Nq, Nk, d, S = shape
    say(f"split dtype={dtype} shape={shape}")
    q, k, v = si.small_case(300 + Nk, B, H, Nq, Nk, d, dtype)
    scale = si.fp32_inverse_sqrt(d)
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    pm, pl, po = fa.fwd_split(qd, kd, vd, S, scale=scale)
    torch.cuda.synchronize()
    pm, pl, po = si.torch_to_f64(pm), si.torch_to_f64(pl), si.torch_to_f64(po)
    qf, kf, vf = q.as_f64(), k.as_f64(), v.as_f64()
    for b in range(B):
        for h in range(H):
            states = oracle.split_partial_states(qf[b, h], kf[b, h], vf[b, h], scale, S)
            for c, (m_ref, l_ref, o_ref) in enumerate(states):
                # each part: its m, and its normalised output o / l, equal the part's own attention
                lo, hi = oracle.split_bounds(Nk, S)[c]
                bound = stat_bound(qf[b, h], kf[b, h, lo:hi], scale)
                assert np.all(np.abs(pm[c, b, h] - m_ref) <= bound)
                # l and o are relative to the kernel's m; rebase to the oracle's m before comparing
                w_ = np.exp(pm[c, b, h] - m_ref)
                assert np.all(np.abs(pl[c, b, h] * w_ / l_ref - 1) <= 2 * bound)
                assert_close(po[c, b, h] / pl[c, b, h][:, None], o_ref / l_ref[:, None], dtype, f"part {c}")
    ref = oracle.attention_fp64(qf, kf, vf, scale)
    outs = []
    perm = si.merge_order(5, S)
    for order in (None, perm, list(range(S))[::-1]):
        o, m, l = fa.merge_states(*[torch.from_numpy(x.astype(np.float32)).to(DEV) for x in (pm, pl, po)],
                                  order=order, return_stats=True)
        torch.cuda.synchronize()
        o = si.torch_to_f64(o)
        assert_close(o, ref, dtype, f"merged order={order}")
        outs.append(o)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-5


@pytest.mark.parametrize("d", [64, 128])
def test_merge_of_all_empty_parts_gives_zero(d):
    """A row whose parts hold no key (every part m = -inf, l = 0, o = 0) merges to O = 0, m = -inf, l = 0
    (no 0 / 0); the other rows of the same call are o / l of their parts."""
    S, rows = 3, 5
    r = np.random.default_rng(d)
    pm = r.standard_normal((S, 1, 1, rows)).astype(np.float32)
    pl = (1.0 + r.random((S, 1, 1, rows))).astype(np.float32)
    po = r.standard_normal((S, 1, 1, rows, d)).astype(np.float32)
    pm[:, 0, 0, 2] = -np.inf
    pl[:, 0, 0, 2] = 0.0
    po[:, 0, 0, 2] = 0.0
    o, m, l = fa.merge_states(*[torch.from_numpy(x).to(DEV) for x in (pm, pl, po)], return_stats=True)
    torch.cuda.synchronize()
    o, m, l = si.torch_to_f64(o), si.torch_to_f64(m), si.torch_to_f64(l)
    assert np.all(o[0, 0, 2] == 0.0) and m[0, 0, 2] == -np.inf and l[0, 0, 2] == 0.0
    states = [(pm[c, 0, 0].astype(np.float64), pl[c, 0, 0].astype(np.float64), po[c, 0, 0].astype(np.float64))
              for c in range(S)]
    ref = oracle.finish_state(oracle.merge_sequential(states))
    assert np.max(np.abs(o[0, 0] - ref)) < 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S,rows", [(9, 17), (200, 37), (256, 5), (1, 3)], ids=str)
@pytest.mark.parametrize("lse_form", [False, True], ids=["mlo", "lse"])
def test_merge_many_parts(d, S, rows, lse_form):
    """Up to FA_MAX_SPLITS parts, a part count that is not a multiple of the 8 read at a time, more parts
    than threads per row, row counts that leave a workgroup partly empty, and empty parts (m or lse = -inf)
    scattered in: the merge against the oracle's sequential fold (or its (lse, o) combination) in the
    same shuffled order."""
    r = np.random.default_rng(1000 * S + rows + d)
    order = list(r.permutation(S))
    empty = r.random((S, rows)) < 0.2
    empty[order[0], 0] = True                # the first part of the fold is empty for row 0
    m = (3.0 * r.standard_normal((S, 1, 1, rows))).astype(np.float32)
    l = (0.5 + r.random((S, 1, 1, rows))).astype(np.float32)
    o = r.standard_normal((S, 1, 1, rows, d)).astype(np.float32)
    m[:, 0, 0][empty] = -np.inf
    l[:, 0, 0][empty] = 0.0
    o[:, 0, 0][empty] = 0.0
    say(f"merge many parts d={d} S={S} rows={rows} lse={lse_form}")
    if lse_form:
        out, lse = fa.merge_lse(*[torch.from_numpy(x).to(DEV) for x in (m, o)], order=order)
        torch.cuda.synchronize()
        ref_lse, ref_o = oracle.merge_lse([(m[c, 0, 0].astype(np.float64), o[c, 0, 0].astype(np.float64))
                                           for c in range(S)], order=order)
        got_lse = si.torch_to_f64(lse)[0, 0]
        live = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), live)
        assert np.max(np.abs(got_lse[live] - ref_lse[live])) < 1e-5
    else:
        out, mm, ll = fa.merge_states(*[torch.from_numpy(x).to(DEV) for x in (m, l, o)], order=order,
                                      return_stats=True)
        torch.cuda.synchronize()
        states = [(m[c, 0, 0].astype(np.float64), l[c, 0, 0].astype(np.float64), o[c, 0, 0].astype(np.float64))
                  for c in range(S)]
        ref_m, ref_l, ref_acc = oracle.merge_sequential(states, order=order)
        ref_o = oracle.finish_state((ref_m, ref_l, ref_acc))
        got_m, got_l = si.torch_to_f64(mm)[0, 0], si.torch_to_f64(ll)[0, 0]
        live = np.isfinite(ref_m)
        assert np.array_equal(np.isfinite(got_m), live)
        assert np.array_equal(got_m[live], ref_m[live].astype(np.float32).astype(np.float64))   # max is exact
        assert np.max(np.abs(got_l[live] / ref_l[live] - 1)) < 1e-5
    got_o = si.torch_to_f64(out)[0, 0]
    assert np.max(np.abs(got_o - ref_o)) < 2e-5


def test_decode_bf16_full_size_split16_shuffled_merge():
    """B=16, H=32, one query, Nk=32768, d=128 bf16; 16 splits merged in default_rng(5).permutation(16) order;
    64 whole heads against the oracle."""
    w = si.DECODE_BF16
    say("decode: generating inputs on the device")
    q, k, v = si.decode_inputs_device(w, DEV)
    say("decode: split + merge")
    order = si.merge_order(w.seed, w.num_splits)
    pm, pl, po = fa.fwd_split(q, k, v, w.num_splits, scale=w.scale)
    o, m, l = fa.merge_states(pm, pl, po, order=order, return_stats=True)
    o_seq = fa.merge_states(pm, pl, po)
    torch.cuda.synchronize()
    o, m, l, o_seq = (si.torch_to_f64(x) for x in (o, m, l, o_seq))
    assert np.all(np.isfinite(o))
    assert np.max(np.abs(o - o_seq)) < 1e-5
    # 64 of the 512 heads: every batch entry four times, heads drawn without replacement per entry
    rng = np.random.default_rng(55)
    heads = [(b, int(h)) for b in range(w.B) for h in rng.choice(w.H, 4, replace=False)]
    got, ref, gm, gl, rm, rl, bd = [], [], [], [], [], [], []
    for b, h in heads:
        qh, kh, vh = (si.torch_to_f64(x[b, h]) for x in (q, k, v))
        o_ref, m_ref, l_ref = oracle.attention_rows_fp64(qh, kh, vh, w.scale)
        got.append(o[b, h]); ref.append(o_ref); gm.append(m[b, h]); gl.append(l[b, h]); rm.append(m_ref); rl.append(l_ref)
        bd.append(stat_bound(qh, kh, w.scale))
    got, ref = np.concatenate(got), np.concatenate(ref)
    say(f"decode: errors {errors(got, ref)}")
    assert_close(got, ref, "bf16", "decode sampled heads")
    assert_stats(np.concatenate(gm), np.concatenate(gl), np.concatenate(rm), np.concatenate(rl), np.concatenate(bd),
                 "decode")
    # fa_fwd (one launch, no split) agrees with split + merge
    o_full = si.torch_to_f64(fa.fwd(q, k, v, scale=w.scale))
    assert np.max(np.abs(o_full - o)) < 1e-4


# ---------------------------------------------------------------------------------------------
# the rescale threshold: 0 is the pages' recurrence literally; the default defers rescaling
# ---------------------------------------------------------------------------------------------

_THRESHOLD_SCRIPT = r"""
import sys, numpy as np, torch
sys.path.insert(0, %(root)r)
import flashattention_forward_02_amd as fa, oracle, seeded_inputs as si
from tests._parity import assert_close, assert_stats, stat_bound
for (B, H, Nq, Nk, d, kmul) in [(1, 2, 300, 1000, 64, 1.0), (1, 1, 256, 2000, 128, 3.0)]:
    q, k, v = si.small_case(900 + Nk, B, H, Nq, Nk, d, "bf16", k_mult=kmul)
    sc = si.fp32_inverse_sqrt(d)
    o, m, l = fa.fwd(q.to_torch("cuda"), k.to_torch("cuda"), v.to_torch("cuda"), scale=sc, return_stats=True)
    torch.cuda.synchronize()
    ref, mr, lr = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), sc, return_stats=True)
    assert_close(si.torch_to_f64(o), ref, "bf16", "threshold run")
    assert_stats(si.torch_to_f64(m), si.torch_to_f64(l), mr, lr, stat_bound(q.as_f64(), k.as_f64(), sc))
    np.save(%(out)r + "_%%d.npy" %% d, si.torch_to_f64(o))
print("ok", flush=True)
"""


@pytest.mark.parametrize("threshold", ["0", "8"])
def test_rescale_threshold_exact_and_deferred(threshold, tmp_path):
    """Both the literal recurrence (threshold 0: rescale whenever the max grows) and the deferred one
    match the oracle, in a fresh process that sets FA_RESCALE_THRESHOLD."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = str(tmp_path / f"o_{threshold}")
    env = dict(os.environ, FA_RESCALE_THRESHOLD=threshold)
    r = subprocess.run([sys.executable, "-c", _THRESHOLD_SCRIPT % {"root": root, "out": out}], env=env,
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


# ---------------------------------------------------------------------------------------------
# calls without row statistics (the sum-checked softmax of the matrix-core kernel)
# ---------------------------------------------------------------------------------------------

def run_nostats(q, k, v, scale, out_dtype="f32"):
    o = fa.fwd(q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV), scale=scale, out_dtype=_tdt(out_dtype))
    torch.cuda.synchronize()
    return si.torch_to_f64(o)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(2, 3, 300, 333, 64), (1, 1, 513, 1000, 128), (1, 2, 257, 64, 64),
                                   (1, 1, 40, 17, 64), (2, 1, 64, 129, 128)], ids=lambda s: "x".join(map(str, s)))
def test_no_stats_path(dtype, shape):
    B, H, Nq, Nk, d = shape
    q, k, v = si.small_case(4000 + Nq + Nk, B, H, Nq, Nk, d, dtype)
    scale = si.fp32_inverse_sqrt(d)
    o = run_nostats(q, k, v, scale)
    ref = oracle.attention_fp64(q.as_f64(), k.as_f64(), v.as_f64(), scale)
    assert_close(o, ref, dtype, f"no-stats {dtype} {shape}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kmul,shift", [(1.0, 0.0), (3.0, 0.0), (1.0, 100.0), (8.0, 0.0)])
def test_no_stats_path_score_ranges(kmul, shift, d):
    """Keys x3 and x8 (wide score ranges, so the reference moves on later tiles) and scores shifted
    to about 100 (exponents far from 0 in every tile), at both head dims."""
    q, k, v = si.small_case(77 + d, 1, 2, 300, 2000, d, "bf16", k_mult=kmul)
    qf = q.as_f64()
    sc = si.fp32_inverse_sqrt(d)
    if shift:
        u = qf[0, 0].mean(axis=0)
        u = u * (shift / (sc * float(u @ u)))
        k = si.encode((k.as_f64() + u).astype(np.float32), "bf16")
    o = run_nostats(q, k, v, sc)
    ref = oracle.attention_fp64(qf, k.as_f64(), v.as_f64(), sc)
    assert_close(o, ref, "bf16", f"no-stats d={d} kmul={kmul} shift={shift}")


def test_no_stats_increasing_scores_across_tiles():
    """Scores that grow tile after tile (keys scaled up along the sequence) force the reference to move
    many times; a late key far above every earlier one exercises the overflow guard."""
    q, k, v = si.small_case(78, 1, 1, 256, 1024, 64, "bf16")
    kf = k.as_f64()
    ramp = np.linspace(0.1, 6.0, 1024)[None, None, :, None]
    k2 = si.encode((kf * ramp).astype(np.float32), "bf16")
    o = run_nostats(q, k2, v, 0.125)
    ref = oracle.attention_fp64(q.as_f64(), k2.as_f64(), v.as_f64(), 0.125)
    assert_close(o, ref, "bf16", "ramp")


def test_no_stats_zero_scale():
    q, k, v = si.small_case(5, 1, 2, 300, 130, 64, "bf16")
    o = run_nostats(q, k, v, 0.0)
    ref = np.broadcast_to(v.as_f64().mean(axis=2, keepdims=True), o.shape)
    assert_close(o, ref, "bf16", "no-stats scale=0")


def test_headline_bf16_full_size_no_stats():
    """The benchmarked launch exactly (no statistics requested): 6 whole heads (all 4096 rows), one from
    each batch entry and both ends of the head range, plus sampled rows from 8 more heads."""
    w = si.HEADLINE_BF16
    q, k, v = si.workload_inputs(w)
    o, _, _ = run_case(q, k, v, "bf16", w.scale, stats=False)
    qf, kf, vf = q.as_f64(), k.as_f64(), v.as_f64()
    rng = np.random.default_rng(33)
    got, ref = [], []
    for (b, h) in [(0, 0), (1, 15), (2, 7), (3, 8), (3, 15), (0, 10)]:
        got.append(o[b, h])
        ref.append(oracle.attention_rows_fp64(qf[b, h], kf[b, h], vf[b, h], w.scale)[0])
    for (b, h) in [(0, 1), (1, 7), (2, 14), (3, 3), (0, 9), (1, 0), (2, 5), (3, 12)]:
        rows = np.sort(rng.choice(w.Nq, size=256, replace=False))
        got.append(o[b, h, rows])
        ref.append(oracle.attention_rows_fp64(qf[b, h, rows], kf[b, h], vf[b, h], w.scale)[0])
    say(f"headline no-stats errors {errors(np.concatenate(got), np.concatenate(ref))}")
    assert_close(np.concatenate(got), np.concatenate(ref), "bf16", "headline no-stats")
    assert np.all(np.isfinite(o))


def test_long_seq_bf16_full_size_no_stats_whole_heads():
    """B=1, H=32, N=16384, d=128 bf16, K x3, O only (the benchmarked launch, sum-checked softmax): two whole
    heads (all 16384 rows each) against the oracle, and every output finite."""
    w = si.LONG_SEQ_BF16
    say("long_seq no-stats: generating inputs")
    q, k, v = si.workload_inputs(w)
    say("long_seq no-stats: running fa_fwd")
    o, _, _ = run_case(q, k, v, "bf16", w.scale, stats=False)
    assert np.all(np.isfinite(o))
    got, ref = [], []
    for h in (5, 30):
        qh, kh, vh = (si.bf16_bits_to_f32(x.data[0, h]).astype(np.float64) for x in (q, k, v))
        ref.append(oracle.attention_fp64(qh[None], kh[None], vh[None], w.scale)[0])
        got.append(o[0, h])
        say(f"long_seq no-stats: head {h} errors {errors(got[-1], ref[-1])}")
    assert_close(np.concatenate(got), np.concatenate(ref), "bf16", "long seq no-stats whole heads")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kmul,shift,ramp", [(1.0, 0.0, False), (8.0, 0.0, False), (1.0, 100.0, False),
                                             (1.0, 0.0, True)])
def test_lse_sum_checked_score_ranges(kmul, shift, ramp, causal):
    """fa_fwd_lse takes the sum-checked softmax (lse = m_ref ln 2 + ln l for whatever reference the
    row ended with): O and the log-sum-exp against the oracle's m + ln(l) on wide score ranges,
    scores shifted to about 100, and scores growing tile after tile."""
    q, k, v = si.small_case(79, 1, 2, 300, 1000, 64, "bf16", k_mult=kmul)
    qf, kf = q.as_f64(), k.as_f64()
    if shift:
        u = qf[0, 0].mean(axis=0)
        u = u * (shift / (0.125 * float(u @ u)))
        kf = kf + u
    if ramp:
        kf = kf * np.linspace(0.1, 6.0, kf.shape[2])[None, None, :, None]
    k = si.encode(kf.astype(np.float32), "bf16")
    qd, kd, vd = q.to_torch(DEV), k.to_torch(DEV), v.to_torch(DEV)
    o, lse = fa.fwd_lse(qd, kd, vd, scale=0.125, causal=causal)
    torch.cuda.synchronize()
    o, lse = si.torch_to_f64(o), si.torch_to_f64(lse)
    ref, m_ref, l_ref = oracle.attention_fp64(qf, k.as_f64(), v.as_f64(), 0.125, return_stats=True, causal=causal)
    what = f"lse kmul={kmul} shift={shift} ramp={ramp} causal={causal}"
    assert_close(o, ref, "bf16", what)
    # lse = m + ln(l): the bounds of m and of l's relative error (tests/_parity.py) add up
    bound = 2 * stat_bound(qf, k.as_f64(), 0.125)
    dl = np.abs(lse - (m_ref + np.log(l_ref)))
    assert np.all(dl <= bound), f"{what}: lse off by {np.max(dl):.3e} (bound {np.min(bound):.1e}..)"
