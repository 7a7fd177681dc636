// Merge of split-KV partial states into the attention output.
//
// For each query row the partial states (m_s, l_s, o_s) are folded one after another in the
// caller's order with the pairwise rule used by "CS349E 第 11 讲 01_online_softmax.py" demo 2
// (derived from the recurrence of "从零手写 FlashAttention" §4):
//   m = max(m_a, m_b);  l = l_a e^(m_a - m) + l_b e^(m_b - m);  o = o_a e^(m_a - m) + o_b e^(m_b - m)
// A state with m = -inf holds no keys and gets weight 0, so -inf - (-inf) is never evaluated.
// The answer is o / l; a row whose states are all empty (l = 0) gets O = 0, as in the (lse, o) form. One thread handles 4 columns of one row; the partial-state reads are
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
  const float inv = l > 0.f ? 1.f / l : 0.f;
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

// Store 4 consecutive fp32 output values in the output type.
__device__ __forceinline__ void store_o4(void* o, size_t e, int out_dtype, const f32x4_t& x) {
  if (out_dtype == kF32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(o) + e) = x;
  } else if (out_dtype == kBF16) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
    bf16x4_t y = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(o) + e) = y;
  } else {
    typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
    f16x4_t y = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    *reinterpret_cast<f16x4_t*>(static_cast<_Float16*>(o) + e) = y;
  }
}

// The (lse, o) form of "CS349E 第 11 讲 01_online_softmax.py" demo 2's note on flash-decoding: each
// part stores its output already divided by its own l and lse_s = m_s + ln(l_s); the parts are
// combined with weights exp(lse_s - lse), lse = ln(sum_s exp(lse_s)) (taken as max + ln of the sum
// of exp(lse_s - max)). Parts with lse_s = -inf (no keys) weigh 0; a row whose parts are all
// empty gets O = 0 and lse = -inf. Sums run in the caller's order.
template <int D>
__global__ __launch_bounds__(256) void merge_lse_kernel(MergeArgs a) {
  constexpr int C4 = D / 4;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = idx / C4;
  const int c = (int)(idx % C4) * 4;
  if (row >= a.rows) return;
  float mx = -INFINITY;
  for (int k = 0; k < a.S; ++k) mx = fmaxf(mx, a.part_m[(size_t)a.order[k] * a.rows + row]);
  float sum = 0.f;
  if (mx != -INFINITY) {
    for (int k = 0; k < a.S; ++k) {
      const float ls = a.part_m[(size_t)a.order[k] * a.rows + row];
      if (ls != -INFINITY) sum += expf(ls - mx);
    }
  }
  const float lse = (mx == -INFINITY) ? -INFINITY : mx + logf(sum);
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
    for (int k = 0; k < a.S; ++k) {
      const size_t p = (size_t)a.order[k] * a.rows + row;
      const float ls = a.part_m[p];
      if (ls == -INFINITY) continue;
      const float w = expf(ls - lse);
      const f32x4_t os = *reinterpret_cast<const f32x4_t*>(a.part_o + p * D + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __builtin_fmaf(w, os[i], o[i]);
    }
  }
  store_o4(a.o, (size_t)row * D + c, a.out_dtype, o);
  if (c == 0 && a.lse_out) a.lse_out[row] = lse;
}

template <int D>
hipError_t launch_typed(const MergeArgs& a, hipStream_t s) {
  const long long threads = (long long)a.rows * (D / 4);
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  MergeArgs args = a;
  void* kargs[] = {&args};
  const void* k = a.lse_format ? reinterpret_cast<const void*>(&merge_lse_kernel<D>)
                               : reinterpret_cast<const void*>(&merge_kernel<D>);
  return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), kargs, 0, s);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_typed<64>(a, s);
  if (d == 128) return launch_typed<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
