"""The measurement probes of include/fa_probe.h on the GPU (through the C ABI via the package binding).

The streaming-read probe must read every 16-byte word of its buffer exactly once: its per-thread XOR
checksums are recomputed on the host from the assignment (workgroup b takes the b-th of nblocks
contiguous chunks, thread t the words of its chunk at offsets t, t + 256, ...). The matrix-core probes (bf16 and
fp32) must produce finite checksums that are identical in every workgroup (each computes the same
products); the fp32 one is also compared with its closed form.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import flashattention_forward_02_amd as fa

DEV = "cuda:0"


@pytest.mark.parametrize("n16,nblocks", [(64 * 256 * 4 * 3 + 37, 64), (1000, 8), (256, 1), (256 * 8 * 5 + 3, 2)])
def test_read_probe_reads_every_chunk_once(n16, nblocks):
    g = torch.Generator(device=DEV)
    g.manual_seed(n16)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (n16 * 4,), generator=g, device=DEV, dtype=torch.int32)
    out = torch.full((nblocks * 256,), -1, device=DEV, dtype=torch.int32)
    nbytes = fa.probe_hbm_read(buf, nblocks=nblocks, out=out)
    torch.cuda.synchronize()
    assert nbytes == n16 * 16
    chunks = buf.cpu().numpy().view(np.uint32).reshape(n16, 4)
    per_chunk = np.bitwise_xor.reduce(chunks, axis=1)
    expect = np.zeros(nblocks * 256, dtype=np.uint32)
    for b in range(nblocks):
        beg, end = n16 * b // nblocks, n16 * (b + 1) // nblocks
        idx = np.arange(beg, end)
        np.bitwise_xor.at(expect, b * 256 + (idx - beg) % 256, per_chunk[beg:end])
    assert np.array_equal(out.cpu().numpy().view(np.uint32), expect)


def test_mfma_probe_is_deterministic_and_finite():
    flops, out = fa.probe_mfma_bf16(nblocks=32, iters=64)
    torch.cuda.synchronize()
    assert flops == 32 * 4 * 64 * 8 * 32768
    x = out.view(32, 256).cpu().numpy()
    assert np.all(np.isfinite(x)) and np.any(x != 0)
    assert np.array_equal(x, np.broadcast_to(x[0], x.shape))


def test_mfma_f32_probe_is_deterministic_and_matches_its_closed_form():
    nblocks, iters = 16, 40
    flops, out = fa.probe_mfma_f32(nblocks=nblocks, iters=iters)
    torch.cuda.synchronize()
    assert flops == nblocks * 4 * iters * 8 * 2048
    x = out.view(nblocks, 256).cpu().numpy()
    assert np.array_equal(x, np.broadcast_to(x[0], x.shape))
    # every accumulator element (i, j) of a 16x16x4 chain gains sum_k A[i][k] B[k][j] per MFMA, with lane
    # l holding A[l % 16][l / 16] = (l % 16) / 2048 and B[l / 16][l % 16] = (l / 16) / 1024; lane l's
    # four results are rows 4 (l / 16) + r of column l % 16, summed over the 8 chains
    A = np.array([[(i % 16) / 2048.0 for k in range(4)] for i in range(16)])
    Bm = np.array([[k / 1024.0 for j in range(16)] for k in range(4)])
    C = A @ Bm * iters
    want = np.array([8 * sum(C[4 * (l // 16) + r, l % 16] for r in range(4)) for l in range(64)])
    assert np.allclose(x[0].reshape(4, 64)[0], want, rtol=1e-5)
