// Merge of split-KV partial states into the attention output.
//
// For each query row the partial states (m_s, l_s, o_s) are folded one after another in the
// caller's order with the pairwise rule used by "CS349E 第 11 讲 01_online_softmax.py" demo 2
// (derived from the recurrence of "从零手写 FlashAttention" §4):
//   m = max(m_a, m_b);  l = l_a e^(m_a - m) + l_b e^(m_b - m);  o = o_a e^(m_a - m) + o_b e^(m_b - m)
// A state with m = -inf holds no keys and gets weight 0, so -inf - (-inf) is never evaluated.
// The answer is o / l; a row whose states are all empty (l = 0) gets O = 0, as in the (lse, o) form.
//
// Layout: one thread per 4 columns of a row (C4 = d / 4 threads per row) and 64 threads per
// workgroup (4 rows at d = 64, 2 at d = 128), so a few hundred rows still fill the chip. The
// arithmetic is a sequential fold over the parts, but the loads are not: the workgroup stages the
// order and its rows' per-part scalars (m and l, or lse, in part-index order) in LDS in one round
// of loads, then reads the parts' o vectors 16 at a time in fold order, so a row costs about
// 1 + S / 16 memory round trips instead of one per part and scalar.

#include "fa_internal.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float weight(float m_part, float m_total) {
  return (m_part == -INFINITY) ? 0.f : expf(m_part - m_total);
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

template <int D>
struct MergeCfg {
  static constexpr int C4 = D / 4;        // threads per row
  static constexpr int NT = 64;           // threads per workgroup
  static constexpr int RPB = NT / C4;     // rows per workgroup
  static constexpr int U = 16;            // partial o vectors in flight per thread
};

// Dynamic LDS of a merge workgroup: order[S], then per row NV * S scalars.
template <int D>
inline size_t merge_lds_bytes(int S, int nv) {
  return ((size_t)S + (size_t)MergeCfg<D>::RPB * nv * S) * sizeof(float);
}

// Stages order[] and the workgroup's rows' per-part scalars (x0, and x1 when NV = 2) in LDS, the
// scalars in part-index order (none of these loads waits for another); s0 / s1 point at this
// thread's row. Returns false for the threads of rows past the end (after the workgroup barrier).
template <int D, int NV>
__device__ __forceinline__ bool stage_scalars(const MergeArgs& a, float* sh, long long row0, const float* x0,
                                              const float* x1, float*& s0, float*& s1) {
  typedef MergeCfg<D> C;
  const int S = a.S;
  int* sh_order = reinterpret_cast<int*>(sh);
  // item i: order[i] (i < S), and the scalars of part i / RPB of row row0 + i % RPB (consecutive
  // threads read consecutive rows); both loads of an item are issued before either is written
#pragma unroll 2
  for (int i = threadIdx.x; i < S * C::RPB; i += C::NT) {
    const int part = i / C::RPB, lr = i % C::RPB;
    const bool has_order = i < S, has_row = row0 + lr < a.rows;
    const size_t p = (size_t)part * a.rows + row0 + lr;
    int ord = 0;
    float v0 = 0.f, v1 = 0.f;
    if (has_order) ord = a.order[i];
    if (has_row) {
      v0 = x0[p];
      if constexpr (NV == 2) v1 = x1[p];
    }
    if (has_order) sh_order[i] = ord;
    if (has_row) {
      float* dst = sh + S + (size_t)lr * NV * S + part;
      dst[0] = v0;
      if constexpr (NV == 2) dst[S] = v1;
    }
  }
  __syncthreads();
  const int lr = threadIdx.x / C::C4;
  s0 = sh + S + (size_t)lr * NV * S;
  s1 = s0 + S;
  return row0 + lr < a.rows;
}

// The row's o vectors of parts k0 .. k0 + U - 1 (in fold order; positions past S repeat part S - 1).
template <int D>
__device__ __forceinline__ void load_parts(const MergeArgs& a, const int* sh_order, int k0, long long row, int c,
                                           f32x4_t (&os)[MergeCfg<D>::U]) {
#pragma unroll
  for (int u = 0; u < MergeCfg<D>::U; ++u) {
    const int k = min(k0 + u, a.S - 1);
    const size_t p = (size_t)sh_order[k] * a.rows + row;
    os[u] = *reinterpret_cast<const f32x4_t*>(a.part_o + p * D + c);
  }
}

template <int D>
__global__ __launch_bounds__(MergeCfg<D>::NT) void merge_kernel(MergeArgs a) {
  typedef MergeCfg<D> C;
  extern __shared__ float sh[];
  const int c4 = threadIdx.x % C::C4;
  const int c = c4 * 4;
  const long long row0 = (long long)blockIdx.x * C::RPB;
  const long long row = row0 + threadIdx.x / C::C4;
  float *sm, *sl;
  if (!stage_scalars<D, 2>(a, sh, row0, a.part_m, a.part_l, sm, sl)) return;
  const int* sh_order = reinterpret_cast<const int*>(sh);

  float m = -INFINITY, l = 0.f;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.S; k0 += C::U) {
    f32x4_t os[C::U];
    load_parts<D>(a, sh_order, k0, row, c, os);
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      if (k0 + u >= a.S) break;
      const int part = sh_order[k0 + u];
      const float ms = sm[part], ls = sl[part];
      const float mn = fmaxf(m, ms);
      const float wa = weight(m, mn), wb = weight(ms, mn);
      l = l * wa + ls * wb;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = o[i] * wa + os[u][i] * wb;
      m = mn;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const f32x4_t x = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  store_o4(a.o, (size_t)row * D + c, a.out_dtype, x);
  if (c == 0) {
    if (a.m_out) a.m_out[row] = m;
    if (a.l_out) a.l_out[row] = l;
  }
}

// The (lse, o) form of "CS349E 第 11 讲 01_online_softmax.py" demo 2's note on flash-decoding: each
// part stores its output already divided by its own l and lse_s = m_s + ln(l_s); the parts are
// combined with weights exp(lse_s - lse), lse = ln(sum_s exp(lse_s)) (taken as max + ln of the sum
// of exp(lse_s - max)). Parts with lse_s = -inf (no keys) weigh 0; a row whose parts are all
// empty gets O = 0 and lse = -inf. Sums run in the caller's order.
template <int D>
__global__ __launch_bounds__(MergeCfg<D>::NT) void merge_lse_kernel(MergeArgs a) {
  typedef MergeCfg<D> C;
  extern __shared__ float sh[];
  const int c4 = threadIdx.x % C::C4;
  const int c = c4 * 4;
  const long long row0 = (long long)blockIdx.x * C::RPB;
  const long long row = row0 + threadIdx.x / C::C4;
  float *sl, *unused;
  if (!stage_scalars<D, 1>(a, sh, row0, a.part_m, nullptr, sl, unused)) return;
  const int* sh_order = reinterpret_cast<const int*>(sh);

  float mx = -INFINITY;
  for (int k = 0; k < a.S; ++k) mx = fmaxf(mx, sl[sh_order[k]]);
  float sum = 0.f;
  if (mx != -INFINITY) {
    for (int k = 0; k < a.S; ++k) {
      const float ls = sl[sh_order[k]];
      if (ls != -INFINITY) sum += expf(ls - mx);
    }
  }
  const float lse = (mx == -INFINITY) ? -INFINITY : mx + logf(sum);
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
    for (int k0 = 0; k0 < a.S; k0 += C::U) {
      f32x4_t os[C::U];
      load_parts<D>(a, sh_order, k0, row, c, os);
#pragma unroll
      for (int u = 0; u < C::U; ++u) {
        if (k0 + u >= a.S) break;
        const float ls = sl[sh_order[k0 + u]];
        if (ls == -INFINITY) continue;
        const float w = expf(ls - lse);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __builtin_fmaf(w, os[u][i], o[i]);
      }
    }
  }
  store_o4(a.o, (size_t)row * D + c, a.out_dtype, o);
  if (c == 0 && a.lse_out) a.lse_out[row] = lse;
}

template <int D>
hipError_t launch_typed(const MergeArgs& a, hipStream_t s) {
  const long long blocks = ((long long)a.rows + MergeCfg<D>::RPB - 1) / MergeCfg<D>::RPB;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  MergeArgs args = a;
  void* kargs[] = {&args};
  const void* k = a.lse_format ? reinterpret_cast<const void*>(&merge_lse_kernel<D>)
                               : reinterpret_cast<const void*>(&merge_kernel<D>);
  const size_t lds = merge_lds_bytes<D>(a.S, a.lse_format ? 1 : 2);
  return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(MergeCfg<D>::NT), kargs, lds, s);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_typed<64>(a, s);
  if (d == 128) return launch_typed<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
