// Merge of split-KV partial states into the attention output.
//
// For each query row the partial states (m_s, l_s, o_s) are folded one after another in the
// caller's order with the pairwise rule used by "CS349E 第 11 讲 01_online_softmax.py" demo 2
// (derived from the recurrence of "从零手写 FlashAttention" §4):
//   m = max(m_a, m_b);  l = l_a e^(m_a - m) + l_b e^(m_b - m);  o = o_a e^(m_a - m) + o_b e^(m_b - m)
// A state with m = -inf holds no keys and gets weight 0, so -inf - (-inf) is never evaluated.
// The answer is o / l. One thread handles 4 columns of one row; the partial-state reads are
// coalesced 16-byte loads.

#include "fa_internal.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float weight(float m_part, float m_total) {
  return (m_part == -INFINITY) ? 0.f : expf(m_part - m_total);
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int C4 = D / 4;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = idx / C4;
  const int c = (int)(idx % C4) * 4;
  if (row >= a.rows) return;

  float m = -INFINITY, l = 0.f;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < a.S; ++k) {
    const size_t p = (size_t)a.order[k] * a.rows + row;
    const float ms = a.part_m[p];
    const float ls = a.part_l[p];
    const f32x4_t os = *reinterpret_cast<const f32x4_t*>(a.part_o + p * D + c);
    const float mn = fmaxf(m, ms);
    const float wa = weight(m, mn), wb = weight(ms, mn);
    l = l * wa + ls * wb;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = o[i] * wa + os[i] * wb;
    m = mn;
  }
  const float inv = 1.f / l;
  const size_t e = (size_t)row * D + c;
  if (a.out_dtype == kF32) {
    f32x4_t x = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.o) + e) = x;
  } else if (a.out_dtype == kBF16) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
    bf16x4_t x = {(__bf16)(o[0] * inv), (__bf16)(o[1] * inv), (__bf16)(o[2] * inv), (__bf16)(o[3] * inv)};
    *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(a.o) + e) = x;
  } else {
    typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
    f16x4_t x = {(_Float16)(o[0] * inv), (_Float16)(o[1] * inv), (_Float16)(o[2] * inv), (_Float16)(o[3] * inv)};
    *reinterpret_cast<f16x4_t*>(static_cast<_Float16*>(a.o) + e) = x;
  }
  if (c == 0) {
    if (a.m_out) a.m_out[row] = m;
    if (a.l_out) a.l_out[row] = l;
  }
}

template <int D>
hipError_t launch_typed(const MergeArgs& a, hipStream_t s) {
  const long long threads = (long long)a.rows * (D / 4);
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  MergeArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<D>), dim3((unsigned)blocks), dim3(256), kargs,
                         0, s);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_typed<64>(a, s);
  if (d == 128) return launch_typed<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
