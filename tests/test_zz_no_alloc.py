"""fa_bwd_noalloc, the backward entry point that allocates nothing (D in the library's built-in buffer),
against fa_bwd (D in a caller workspace) through the C ABI.

Two calls in a row on the same GPU, the second on a smaller input than the first (so the built-in
buffer still holds the first call's larger D when the second runs): both must give exactly fa_bwd's
gradients -- the same kernels on the same inputs -- and meet the oracle bar of tests/_parity.py.
The first call on a device is its set-up (the HIP runtime loads the library's built-in buffer on
that device when its address is first looked up); every later call must leave device memory
untouched.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests._parity import assert_grad_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import flashattention_forward_02_amd as fa
    from flashattention_forward_02_amd import _native as n
    from tests import test_parity_bwd_gpu as bw

DEV = "cuda:0"
DT = {"bf16": 1, "f16": 2}


def _raw_bwd(noalloc, qd, kd, vd, o, dod, lse, shape, dtype, scale, causal, check_memory=False):
    B, H, H_kv, Nq, Nk, d = shape
    dq = torch.full((B, H, Nq, d), float("nan"), device=DEV)
    dk = torch.full((B, H_kv, Nk, d), float("nan"), device=DEV)
    dv = torch.full((B, H_kv, Nk, d), float("nan"), device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), dod.data_ptr(), lse.data_ptr())
    tail = (B, H, H_kv, Nq, Nk, d, scale, int(causal), DT[dtype], 0, stream)
    torch.cuda.synchronize()
    if noalloc:
        free0 = torch.cuda.mem_get_info()[0]
        alloc0 = torch.cuda.memory_allocated()
        st = n.fa_bwd_noalloc(*args, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *tail)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == alloc0
        if check_memory:
            assert torch.cuda.mem_get_info()[0] == free0, "fa_bwd_noalloc changed free device memory"
    else:
        delta = torch.empty((B, H, Nq), device=DEV)
        st = n.fa_bwd(*args, delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *tail)
        torch.cuda.synchronize()
    assert st == n.FA_OK, n.fa_last_error()
    return dq, dk, dv


# (seed, dtype, B, H, H_kv, Nq, Nk, d, causal): the first call is the larger one
CALLS = [
    (611, "bf16", 2, 4, 2, 700, 900, 64, False),
    (612, "f16", 1, 2, 1, 300, 333, 128, True),
]


def test_noalloc_matches_fa_bwd_on_two_calls_in_a_row():
    assert CALLS[0][2] * CALLS[0][3] * CALLS[0][5] > CALLS[1][2] * CALLS[1][3] * CALLS[1][5]
    for i, (seed, dtype, B, H, H_kv, Nq, Nk, d, causal) in enumerate(CALLS + CALLS[:1]):
        print(f"no-alloc call seed={seed} {dtype} B={B} H={H} H_kv={H_kv} Nq={Nq} Nk={Nk} d={d} causal={causal}",
              flush=True)
        q, k, v, do = bw.case(seed, B, H, H_kv, Nq, Nk, d, dtype)
        scale = si.fp32_inverse_sqrt(d)
        qd, kd, vd, dod = (t.to_torch(DEV) for t in (q, k, v, do))
        o, lse = fa.fwd_lse(qd, kd, vd, scale=scale, causal=causal)
        shape = (B, H, H_kv, Nq, Nk, d)
        ref_gpu = _raw_bwd(False, qd, kd, vd, o, dod, lse, shape, dtype, scale, causal)
        got = _raw_bwd(True, qd, kd, vd, o, dod, lse, shape, dtype, scale, causal, check_memory=i > 0)
        for name, g, r in zip(("dq", "dk", "dv"), got, ref_gpu):
            assert torch.equal(g, r), f"{name}: fa_bwd_noalloc differs from fa_bwd"
        rdq, rdk, rdv = oracle.attention_backward_fp64(q.as_f64(), k.as_f64(), v.as_f64(), do.as_f64(), scale,
                                                       causal=causal)[:3]
        zb = bw.zero_bounds(q, k, v, do, H // H_kv, scale)
        for name, g, r in zip(("dq", "dk", "dv"), got, (rdq, rdk, rdv)):
            assert_grad_close(si.torch_to_f64(g), r, dtype, f"noalloc {name}", zero_bound=zb.get(name))


def test_noalloc_rejects_more_rows_than_its_buffer():
    x = torch.zeros(64, device=DEV, dtype=torch.bfloat16)
    f = torch.zeros(64, device=DEV)
    rows = n.FA_NOALLOC_MAX_ROWS + 1
    st = n.fa_bwd_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), f.data_ptr(), x.data_ptr(), f.data_ptr(),
                          f.data_ptr(), f.data_ptr(), f.data_ptr(), 1, 1, 1, rows, 1, 64, 0.125, 0, 1, 0, None)
    assert st == n.FA_EINVAL and "built-in D buffer" in n.fa_last_error()
