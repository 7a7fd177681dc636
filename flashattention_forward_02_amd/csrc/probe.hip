// Measurement probes: the empirical ceilings the attention kernels are compared against.
//
//  * probe_mfma_kernel: back-to-back 32x32x16 bf16 MFMAs on register operands, eight independent
//    accumulators per wave so the matrix core never waits on a result. Its rate is the
//    matrix-core throughput this chip sustains at the clock it runs at under that load.
//  * probe_mfma_f32_kernel: the same with 16x16x4 fp32 MFMAs (the fp32 matrix-core rate).
//  * probe_read_kernel: a streaming 16-byte-per-lane read of a large buffer (each byte once), the
//    HBM read bandwidth a memory-bound kernel can reach.
//
// Neither touches memory outside the buffers the host checked; both write one value per thread
// so the work cannot be removed.

#include "fa_internal.h"
#include "mfma_common.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;   // 4 waves
constexpr int kProbeChains = 8;      // independent accumulators per wave

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  // small operands (|x| <= 2^-8): the accumulators stay finite for any iteration count used here
  const float av = (float)(lane & 7) * (1.f / 2048.f), bv = (float)((lane >> 3) & 7) * (1.f / 2048.f);
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(av + (float)i * (1.f / 4096.f));
    b[i] = (__bf16)(bv - (float)i * (1.f / 4096.f));
  }
  f32x16_t acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_f32_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  // small operands (|x| <= 2^-7): the accumulators stay finite for any iteration count used here
  const float a = (float)(lane & 15) * (1.f / 2048.f), b = (float)(lane >> 4) * (1.f / 1024.f);
  f32x4_t acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                                    unsigned* __restrict__ out) {
  // Workgroup b reads the contiguous words [b n16 / nb, (b + 1) n16 / nb) with nontemporal 16-byte
  // loads, eight in flight per lane (of the patterns measured, contiguous per-workgroup chunks of
  // 1-4 MB read this way streamed fastest); the tail loop takes what is left of the chunk.
  const size_t nb = gridDim.x;
  const size_t end = n16 * (blockIdx.x + 1) / nb;
  size_t i = n16 * blockIdx.x / nb + threadIdx.x;
  unsigned x = 0u;
  for (; i + 7 * kProbeThreads < end; i += 8 * kProbeThreads) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * kProbeThreads]);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += kProbeThreads) {
    const u32x4_t v = __builtin_nontemporal_load(&src[i]);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = x;
}
}  // namespace

hipError_t launch_probe_mfma(float* out, int nblocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)nblocks), dim3(kProbeThreads), 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_mfma_f32(float* out, int nblocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_f32_kernel, dim3((unsigned)nblocks), dim3(kProbeThreads), 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t bytes, unsigned* out, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)nblocks), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4_t*>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace fa
