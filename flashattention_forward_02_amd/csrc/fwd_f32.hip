// Tiled FlashAttention forward for fp32 inputs (VALU, full fp32 arithmetic).
//
// Same recurrence as the matrix-core kernel ("FlashAttention 简化版：Tiling + Online Softmax",
// §2.3 and §3.1), written for accuracy rather than speed: scores are s = scale * (q . k) in
// fp32, the running max is taken on s, and exp is the accurate expf, so the result tracks the
// float64 definition to a few fp32 ulps.
//
// The output accumulator and l are summed with compensation (Kahan): their sums nearly cancel
// (|O| is small next to sum |p v| when many keys share the weight), and plain fp32 accumulation
// over thousands of keys would lose ~sqrt(Nk) ulps of O.
//
// Layout: D/32 adjacent lanes share one query row, each owning 32 of its columns of q and of
// the output accumulator; a dot product is 32 FMAs per lane plus a butterfly over those lanes.
// Key/value tiles of 32 rows are staged in LDS (every lane of a wave reads the same K/V row at
// the same time, so the reads are broadcasts).

#include "fa_internal.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kThreads = 256;
constexpr int kBCF = 32;  // keys per tile

// sum += x with the rounding error carried in comp (Kahan).
__device__ __forceinline__ void kahan_add(float& sum, float& comp, float x) {
  const float y = x - comp;
  const float t = sum + y;
  comp = (t - sum) - y;
  sum = t;
}

// sum += p * v, the product rounded once into the compensated sum.
__device__ __forceinline__ void kahan_fma(float& sum, float& comp, float p, float v) {
  const float y = __builtin_fmaf(p, v, -comp);
  const float t = sum + y;
  comp = (t - sum) - y;
  sum = t;
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a, int n_qtiles) {
  constexpr int LPR = D / 32;               // lanes per query row
  constexpr int ROWS = kThreads / LPR;      // query rows per workgroup
  constexpr int LOADS = kBCF * D / 4 / kThreads;
  static_assert(LOADS * 4 * kThreads == kBCF * D, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) float ks[kBCF * D];
  __shared__ __attribute__((aligned(16))) float vs[kBCF * D];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = wg % n_qtiles;
  int rest = wg / n_qtiles;
  const int split = rest % a.num_splits;
  rest /= a.num_splits;
  const int h = rest % a.H;
  const int b = rest / a.H;
  const size_t head = (size_t)b * a.H + h;
  const size_t kvh = kv_head_index(b, h, a.H, a.H_kv);
  const float* __restrict__ Q = static_cast<const float*>(a.q) + head * (size_t)a.Nq * D;
  const float* __restrict__ K = static_cast<const float*>(a.k) + kvh * (size_t)a.Nk * D;
  const float* __restrict__ V = static_cast<const float*>(a.v) + kvh * (size_t)a.Nk * D;
  const int kbeg = split_begin(split, a.Nk, a.num_splits);
  int kend = split_begin(split + 1, a.Nk, a.num_splits);

  const int tid = threadIdx.x;
  const int row = qt * ROWS + tid / LPR;
  const int col0 = (tid % LPR) * 32;
  const bool live = row < a.Nq;
  // Causal mask: this row sees keys < row_end; the workgroup stops after the last key any of
  // its rows sees (key tiles wholly past it are skipped).
  int row_end = kend;
  if (a.causal) {
    row_end = min(kend, row + a.causal_off + 1);
    kend = min(kend, min(a.Nq, (qt + 1) * ROWS) - 1 + a.causal_off + 1);
  }

  float q[32], acc[32], comp[32];
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    if (live) x = *reinterpret_cast<const f32x4_t*>(Q + (size_t)row * D + col0 + c);
    q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[c + i] = comp[c + i] = 0.f;
  }
  float m = -INFINITY, l = 0.f, lcomp = 0.f;

  for (int key0 = kbeg; key0 < kend; key0 += kBCF) {
    const int nvalid = min(kBCF, kend - key0);
    __syncthreads();  // the previous tile is consumed
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = (tid + i * kThreads) * 4;
      const int r = e / D;
      f32x4_t kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (r < nvalid) {
        kx = *reinterpret_cast<const f32x4_t*>(K + (size_t)(key0 + r) * D + (e % D));
        vx = *reinterpret_cast<const f32x4_t*>(V + (size_t)(key0 + r) * D + (e % D));
      }
      *reinterpret_cast<f32x4_t*>(&ks[e]) = kx;
      *reinterpret_cast<f32x4_t*>(&vs[e]) = vx;
    }
    __syncthreads();

    float s[kBCF];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBCF; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const f32x4_t kx = *reinterpret_cast<const f32x4_t*>(&ks[j * D + col0 + c]);
        dot = __builtin_fmaf(q[c], kx[0], dot);
        dot = __builtin_fmaf(q[c + 1], kx[1], dot);
        dot = __builtin_fmaf(q[c + 2], kx[2], dot);
        dot = __builtin_fmaf(q[c + 3], kx[3], dot);
      }
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) dot += __shfl_xor(dot, off);
      s[j] = (key0 + j < row_end) ? a.scale * dot : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      acc[c] *= alpha;
      comp[c] *= alpha;
    }
    l *= alpha;
    lcomp *= alpha;
#pragma unroll
    for (int j = 0; j < kBCF; ++j) {
      const float p = (key0 + j < row_end) ? expf(s[j] - mnew) : 0.f;
      kahan_add(l, lcomp, p);
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const f32x4_t vx = *reinterpret_cast<const f32x4_t*>(&vs[j * D + col0 + c]);
#pragma unroll
        for (int i = 0; i < 4; ++i) kahan_fma(acc[c + i], comp[c + i], p, vx[i]);
      }
    }
    m = mnew;
  }

  if (!live) return;
  if (a.split_mode == 0) {
    const float inv = 1.f / l;
    float* O = static_cast<float*>(a.o) + (head * (size_t)a.Nq + row) * D + col0;
#pragma unroll
    for (int c = 0; c < 32; c += 4) {
      f32x4_t x = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
      *reinterpret_cast<f32x4_t*>(O + c) = x;
    }
    if (col0 == 0) {
      if (a.m_out) a.m_out[head * a.Nq + row] = m;
      if (a.l_out) a.l_out[head * a.Nq + row] = l;
      if (a.lse_out) a.lse_out[head * a.Nq + row] = m + logf(l);
    }
  } else {
    const size_t prow = ((size_t)split * a.B * a.H + head) * a.Nq + row;
    float* P = a.part_o + prow * D + col0;
    // (lse, o / l) form: a row with no key in this range keeps (-inf, 0)
    const float w = (a.split_mode == 2) ? (l > 0.f ? 1.f / l : 0.f) : 1.f;
#pragma unroll
    for (int c = 0; c < 32; c += 4) {
      f32x4_t x = {acc[c] * w, acc[c + 1] * w, acc[c + 2] * w, acc[c + 3] * w};
      *reinterpret_cast<f32x4_t*>(P + c) = x;
    }
    if (col0 == 0) {
      if (a.split_mode == 2) {
        a.part_m[prow] = (m == -INFINITY) ? -INFINITY : m + logf(l);
      } else {
        a.part_m[prow] = m;
        a.part_l[prow] = l;
      }
    }
  }
}

template <int D>
hipError_t launch_typed(const FwdArgs& a, hipStream_t s) {
  constexpr int ROWS = kThreads / (D / 32);
  const int n_qtiles = (a.Nq + ROWS - 1) / ROWS;
  const long long nwg = (long long)n_qtiles * a.num_splits * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  int nq = n_qtiles;
  void* kargs[] = {&args, &nq};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_f32_kernel<D>), dim3((unsigned)nwg), dim3(kThreads),
                         kargs, 0, s);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_typed<64>(a, s);
  if (d == 128) return launch_typed<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
