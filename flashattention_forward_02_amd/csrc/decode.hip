// Split-KV / few-query forward: one workgroup per (key range, query row, head).
//
// The flash-decoding decomposition of "CS349E 第 11 讲 01_online_softmax.py" (demo 2
// observations): different compute units take different key segments of the same query and
// each produces the partial state (m, l, o) of its segment, o unnormalised. With one query
// row there is nothing to share between rows, so this path streams K and V once with
// coalesced 16-byte loads and does the arithmetic on the VALU; it is bound by HBM bandwidth.
//
// Inside a workgroup the 256 lanes form 16 groups of 16; a group takes U keys at a time (group g
// owns keys kbeg + g*U + 16*U*i + u), lane t of the group owns columns [t*D/16, (t+1)*D/16) of q,
// of the K and V rows and of its accumulator. A score is D/16 FMAs per lane plus a butterfly over
// the group; each group runs the online-softmax recurrence of "FlashAttention 简化版：Tiling +
// Online Softmax" §2.3 over its keys, and the 16 group states are merged at the end with the merge
// rule of the decoding demo.
//
// These kernels take bf16 / fp16 inputs and use base-2 scores, exp(s - m) = 2^(raw*c - m*c) with
// c = scale*log2(e); fp32 rows go to the fp32 kernels.
//
// decode_rows_kernel (R rows sharing each K/V load) has four times the softmax work per byte of
// decode_kernel, so it keeps its exponentials relative to a reference that moves to the running
// maximum only when the maximum passes it by more than tau (as the tiled kernel does): most keys
// then cost one FMA and one exponential per row, and the rescaling of l and the accumulator is a
// rare, wave-uniform branch; at the end l and the accumulator are re-expressed relative to the
// true maximum, so the partial states are the same (m, l, o) as the plain recurrence gives, up to
// rounding. With one key per group step it also loads each step's K and V words one step ahead.
//
// K and V are streamed with nontemporal loads: 1415 -> 1258 us on B=16, H=32, Nk=32768, d=128 split
// 16 ways (6.07 -> 6.83 TB/s of K and V), 369 -> 342 us with 8 K/V heads. decode_rows_kernel always
// uses them (its workgroups that share a K/V head read it at the same pace: 16 rows of a head, 314 ->
// 286 us); decode_kernel only when each K/V head has one row (its causal rows read a shared K/V at
// different times, and the hint made them slower).

#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = kThreads / 16;

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

// Load N consecutive bf16 / fp16 elements and widen them to fp32.
template <typename T, int N, bool NT = false>
__device__ __forceinline__ void load_row(const T* __restrict__ p, float (&out)[N]) {
  static_assert(N == 4 || N == 8, "");
  unsigned w[N / 2];
  if constexpr (N == 8) {
    const u32x4_t x = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)) : *reinterpret_cast<const u32x4_t*>(p);
    w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
  } else {
    const u32x2_t x = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)) : *reinterpret_cast<const u32x2_t*>(p);
    w[0] = x[0]; w[1] = x[1];
  }
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    if constexpr (std::is_same<T, __bf16>::value) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    } else {
      out[2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] & 0xffffu));
      out[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] >> 16));
    }
  }
}

// 16 bytes of a K or V row, nontemporal (streamed).
template <typename T>
__device__ __forceinline__ u32x4_t stream_u32x4(const T* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

template <typename T>
__device__ __forceinline__ void store_out(void* base, size_t elem, int out_dtype, float x) {
  if (out_dtype == kF32) static_cast<float*>(base)[elem] = x;
  else if (out_dtype == kBF16) static_cast<__bf16*>(base)[elem] = (__bf16)x;
  else static_cast<_Float16*>(base)[elem] = (_Float16)x;
}

template <int D, typename T, int U, bool NT>
__global__ __launch_bounds__(kThreads) void decode_kernel(FwdArgs a) {
  constexpr int NG = kGroups;
  constexpr int DL = D / 16;  // columns per lane
  __shared__ float sh_m[NG], sh_l[NG];
  __shared__ float sh_o[NG][D];

  const int S = a.num_splits;
  const int split = blockIdx.x % S;
  const int rest = blockIdx.x / S;
  const int row = rest % a.Nq;
  const size_t head = rest / a.Nq;
  const size_t kvh = kv_head_index((int)(head / a.H), (int)(head % a.H), a.H, a.H_kv);
  const int kbeg = split_begin(split, a.Nk, S);
  // Under the causal mask this row sees keys up to row + causal_off; the range may be empty.
  const int kend = a.causal ? min(split_begin(split + 1, a.Nk, S), row + a.causal_off + 1)
                            : split_begin(split + 1, a.Nk, S);

  const int tid = threadIdx.x;
  const int g = tid >> 4;
  const int t = tid & 15;
  const T* __restrict__ Qr = static_cast<const T*>(a.q) + (head * a.Nq + row) * (size_t)D + t * DL;
  const T* __restrict__ K = static_cast<const T*>(a.k) + kvh * (size_t)a.Nk * D + t * DL;
  const T* __restrict__ V = static_cast<const T*>(a.v) + kvh * (size_t)a.Nk * D + t * DL;

  float q[DL];
  load_row<T, DL>(Qr, q);
  const float c2 = a.scale_log2e;

  float m = -INFINITY, l = 0.f, acc[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) acc[c] = 0.f;

  for (int base = kbeg + g * U; base < kend; base += NG * U) {
    float kx[U][DL], vx[U][DL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u;
      if (key < kend) {
        load_row<T, DL, NT>(K + (size_t)key * D, kx[u]);
        load_row<T, DL, NT>(V + (size_t)key * D, vx[u]);
      } else {
#pragma unroll
        for (int c = 0; c < DL; ++c) kx[u][c] = vx[u][c] = 0.f;
      }
    }
    float s[U];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) dot = __builtin_fmaf(q[c], kx[u][c], dot);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) dot += __shfl_xor(dot, off);
      const bool ok = base + u < kend;
      s[u] = ok ? dot : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c2);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < DL; ++c) acc[c] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u], c2, -mnew * c2));
      if (s[u] == -INFINITY) p = 0.f;
      l += p;
#pragma unroll
      for (int c = 0; c < DL; ++c) acc[c] = __builtin_fmaf(p, vx[u][c], acc[c]);
    }
    m = mnew;
  }

  // ---- merge the 16 group states ----
  if (t == 0) {
    sh_m[g] = m;
    sh_l[g] = l;
  }
#pragma unroll
  for (int c = 0; c < DL; ++c) sh_o[g][t * DL + c] = acc[c];
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < NG; ++i) M = fmaxf(M, sh_m[i]);
  float w[NG];
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const float mi = sh_m[i];
    w[i] = (mi == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mi - M) * c2);
    L = __builtin_fmaf(w[i], sh_l[i], L);
  }
  // An empty range (possible only under the mask, in split mode) leaves M = -inf, L = 0, o = 0.
  const float m_nat = (M == -INFINITY) ? M : a.scale * M;
  const size_t qrow = head * a.Nq + row;
  for (int c = tid; c < D; c += kThreads) {
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) o = __builtin_fmaf(w[i], sh_o[i][c], o);
    if (a.split_mode == 0) {
      store_out<T>(a.o, qrow * D + c, a.out_dtype, o / L);
    } else {
      const size_t prow = (size_t)split * a.B * a.H * a.Nq + qrow;
      // (lse, o / l) form: an empty range keeps (-inf, 0)
      a.part_o[prow * D + c] = (a.split_mode == 2) ? (L > 0.f ? o / L : 0.f) : o;
    }
  }
  if (tid == 0) {
    if (a.split_mode == 0) {
      if (a.m_out) a.m_out[qrow] = m_nat;
      if (a.l_out) a.l_out[qrow] = L;
      if (a.lse_out) a.lse_out[qrow] = m_nat + logf(L);
    } else {
      const size_t prow = (size_t)split * a.B * a.H * a.Nq + qrow;
      if (a.split_mode == 2) {
        a.part_m[prow] = (M == -INFINITY) ? -INFINITY : m_nat + logf(L);
      } else {
        a.part_m[prow] = m_nat;
        a.part_l[prow] = L;
      }
    }
  }
}

// R query rows of one head per workgroup (bf16 / fp16), so the rows share every K and V load:
// the same lane layout and per-group recurrence as decode_kernel, with R scores per key and R
// (m, l, o) states per group. Grouped K/V heads without the mask (or with one query row, which
// sees every key) are run through it as one head of G * Nq rows per K/V head: query head
// h = hk * G + g, row i is row g * Nq + i of K/V head hk, and [B, H, Nq] is [B, H_kv, G * Nq] in
// memory, so the G query heads of a K/V head read K and V once instead of G times.
template <int D, typename T, int U, int R>
__global__ __launch_bounds__(kThreads) void decode_rows_kernel(FwdArgs a) {
  constexpr int DL = D / 16;  // columns per lane
  __shared__ float sh_m[R][kGroups], sh_l[R][kGroups];
  __shared__ float sh_o[R][kGroups][D];

  const int S = a.num_splits;
  const int n_blocks = (a.Nq + R - 1) / R;
  const int split = blockIdx.x % S;
  const int rest = blockIdx.x / S;
  const int row0 = (rest % n_blocks) * R;
  const size_t head = rest / n_blocks;     // heads share K/V (the caller's view is one-to-one)
  const int kbeg = split_begin(split, a.Nk, S);
  const int kend = split_begin(split + 1, a.Nk, S);

  const int tid = threadIdx.x;
  const int g = tid >> 4;
  const int t = tid & 15;
  const T* __restrict__ K = static_cast<const T*>(a.k) + head * (size_t)a.Nk * D + t * DL;
  const T* __restrict__ V = static_cast<const T*>(a.v) + head * (size_t)a.Nk * D + t * DL;

  float q[R][DL];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int row = min(row0 + j, a.Nq - 1);   // rows past Nq compute row Nq - 1 and are not stored
    load_row<T, DL>(static_cast<const T*>(a.q) + (head * a.Nq + row) * (size_t)D + t * DL, q[j]);
  }
  const float c2 = a.scale_log2e;

  // m: the running maximum of the raw scores; ref: the exponent reference (base-2 units), moved
  // to the maximum only when the maximum passes it by more than tau, as in the tiled kernel
  const float tau = a.rescale_threshold;
  float m[R], ref[R], l[R], acc[R][DL];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    m[j] = -INFINITY;
    ref[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int c = 0; c < DL; ++c) acc[j][c] = 0.f;
  }

  // one key per group step (U = 1, d = 128): its K and V words are loaded one step ahead
  u32x4_t kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
  if constexpr (U == 1 && DL == 8) {
    const int key = kbeg + g;
    if (key < kend) {
      kn = stream_u32x4(K + (size_t)key * D);
      vn = stream_u32x4(V + (size_t)key * D);
    }
  }
  for (int base = kbeg + g * U; base < kend; base += kGroups * U) {
    float kx[U][DL], vx[U][DL];
    if constexpr (U == 1 && DL == 8) {
      const u32x4_t kc = kn, vc = vn;
      const int nk = base + kGroups;
      if (nk < kend) {
        kn = stream_u32x4(K + (size_t)nk * D);
        vn = stream_u32x4(V + (size_t)nk * D);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (std::is_same<T, __bf16>::value) {
          kx[0][2 * i] = __uint_as_float(kc[i] << 16);
          kx[0][2 * i + 1] = __uint_as_float(kc[i] & 0xffff0000u);
          vx[0][2 * i] = __uint_as_float(vc[i] << 16);
          vx[0][2 * i + 1] = __uint_as_float(vc[i] & 0xffff0000u);
        } else {
          kx[0][2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(kc[i] & 0xffffu));
          kx[0][2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(kc[i] >> 16));
          vx[0][2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(vc[i] & 0xffffu));
          vx[0][2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(vc[i] >> 16));
        }
      }
    } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u;
      if (key < kend) {
        load_row<T, DL, true>(K + (size_t)key * D, kx[u]);
        load_row<T, DL, true>(V + (size_t)key * D, vx[u]);
      } else {
#pragma unroll
        for (int c = 0; c < DL; ++c) kx[u][c] = vx[u][c] = 0.f;
      }
    }
    }
    float sc[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d[R];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < DL; ++c) dot = __builtin_fmaf(q[j][c], kx[u][c], dot);
        d[j] = dot;
      }
      if constexpr (R == 4) {
        // Reduce the four partial sums over the 16 lanes while spreading them out: after the
        // exchanges with lanes 8 and 4 apart each lane holds one row's sum over its 4-lane
        // quarter (row 2 b3 + b2, b3 / b2 = lane bits 3 / 2), then a butterfly over the quarter
        // completes it, and four reads from the quarters hand every lane all four sums.
        const bool b3 = (t >> 3) & 1, b2 = (t >> 2) & 1;
        const float s0 = b3 ? d[0] : d[2], s1 = b3 ? d[1] : d[3];
        const float k0 = b3 ? d[2] : d[0], k1 = b3 ? d[3] : d[1];
        const float e0 = k0 + __shfl_xor(s0, 8), e1 = k1 + __shfl_xor(s1, 8);
        float f = (b2 ? e1 : e0) + __shfl_xor(b2 ? e0 : e1, 4);
        f += __shfl_xor(f, 2);
        f += __shfl_xor(f, 1);
        const int gl = tid & ~15;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float dot = __shfl(f, gl + ((j >> 1) << 3) + ((j & 1) << 2));
          sc[u][j] = base + u < kend ? dot : -INFINITY;
        }
      } else {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          float dot = d[j];
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) dot += __shfl_xor(dot, off);
          sc[u][j] = base + u < kend ? dot : -INFINITY;
        }
      }
    }
    bool move = false;
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
      for (int u = 0; u < U; ++u) m[j] = fmaxf(m[j], sc[u][j]);
      const float mc = (m[j] == -INFINITY) ? -INFINITY : m[j] * c2;
      move |= mc > ref[j] + tau;
    }
    if (__ballot(move)) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float mc = (m[j] == -INFINITY) ? -INFINITY : m[j] * c2;
        const float nref = (mc > ref[j] + tau) ? mc : ref[j];
        const float alpha = (ref[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ref[j] - nref);
        l[j] *= alpha;
#pragma unroll
        for (int c = 0; c < DL; ++c) acc[j][c] *= alpha;
        ref[j] = nref;
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][j], c2, -ref[j]));
        if (sc[u][j] == -INFINITY) p = 0.f;
        l[j] += p;
#pragma unroll
        for (int c = 0; c < DL; ++c) acc[j][c] = __builtin_fmaf(p, vx[u][c], acc[j][c]);
      }
    }
  }
  // l and acc relative to the true maximum
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const float mc = (m[j] == -INFINITY) ? -INFINITY : m[j] * c2;
    const float f = (ref[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ref[j] - mc);
    l[j] *= f;
#pragma unroll
    for (int c = 0; c < DL; ++c) acc[j][c] *= f;
  }

  // ---- merge the 16 group states of each row (as in decode_kernel) ----
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (t == 0) {
      sh_m[j][g] = m[j];
      sh_l[j][g] = l[j];
    }
#pragma unroll
    for (int c = 0; c < DL; ++c) sh_o[j][g][t * DL + c] = acc[j][c];
  }
  __syncthreads();
  for (int j = 0; j < R; ++j) {
    const int row = row0 + j;
    if (row >= a.Nq) break;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kGroups; ++i) M = fmaxf(M, sh_m[j][i]);
    float w[kGroups];
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const float mi = sh_m[j][i];
      w[i] = (mi == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mi - M) * c2);
      L = __builtin_fmaf(w[i], sh_l[j][i], L);
    }
    const float m_nat = (M == -INFINITY) ? M : a.scale * M;
    const size_t qrow = head * a.Nq + row;
    for (int c = tid; c < D; c += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int i = 0; i < kGroups; ++i) o = __builtin_fmaf(w[i], sh_o[j][i][c], o);
      if (a.split_mode == 0) {
        store_out<T>(a.o, qrow * D + c, a.out_dtype, o / L);
      } else {
        const size_t prow = (size_t)split * a.B * a.H * a.Nq + qrow;
        a.part_o[prow * D + c] = (a.split_mode == 2) ? (L > 0.f ? o / L : 0.f) : o;
      }
    }
    if (tid == 0) {
      if (a.split_mode == 0) {
        if (a.m_out) a.m_out[qrow] = m_nat;
        if (a.l_out) a.l_out[qrow] = L;
        if (a.lse_out) a.lse_out[qrow] = m_nat + logf(L);
      } else {
        const size_t prow = (size_t)split * a.B * a.H * a.Nq + qrow;
        if (a.split_mode == 2) {
          a.part_m[prow] = (M == -INFINITY) ? -INFINITY : m_nat + logf(L);
        } else {
          a.part_m[prow] = m_nat;
          a.part_l[prow] = L;
        }
      }
    }
  }
}

template <int D, typename T>
hipError_t launch_typed(const FwdArgs& a, hipStream_t s) {
  constexpr int U = (D == 64) ? 8 : 4;
  // Rows that share K and V go to decode_rows_kernel: without the mask (or with one row, which
  // sees every key) the G * Nq rows of each K/V head, viewed as one head.
  if (!a.causal || a.Nq == 1) {
    FwdArgs v = a;
    v.H = a.H_kv;
    v.Nq = (a.H / a.H_kv) * a.Nq;
    v.causal = 0;
    if (v.Nq >= 2) {
      const bool r4 = v.Nq >= 3;
      const int R = r4 ? 4 : 2;
      const long long nwg = (long long)a.num_splits * ((v.Nq + R - 1) / R) * v.H * v.B;
      if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
      void* kargs[] = {&v};
      // one or two keys per group step: the R-row states take the registers, and more waves
      // in flight keep more loads in flight (d = 128, R = 4: 1 key 0.386 ms, 2 keys 0.389,
      // 4 keys 0.50, 8 keys 0.67 on the grouped decode workload)
      constexpr int UR = (D == 128) ? 1 : 2;
      const void* k = r4 ? reinterpret_cast<const void*>(&decode_rows_kernel<D, T, UR, 4>)
                         : reinterpret_cast<const void*>(&decode_rows_kernel<D, T, UR, 2>);
      return hipLaunchKernel(k, dim3((unsigned)nwg), dim3(kThreads), kargs, 0, s);
    }
  }
  const long long nwg = (long long)a.num_splits * a.Nq * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  void* kargs[] = {&args};
  // nontemporal K / V loads when each K/V head is read by one workgroup per range; the rows of a
  // causal launch share theirs at different times, and the hint made them slower (441 vs 317 us at
  // B=4, H=8, Nq=4, Nk=8192)
  const bool nt = a.Nq == 1 && a.H == a.H_kv;
  const void* k = nt ? reinterpret_cast<const void*>(&decode_kernel<D, T, U, true>)
                     : reinterpret_cast<const void*>(&decode_kernel<D, T, U, false>);
  return hipLaunchKernel(k, dim3((unsigned)nwg), dim3(kThreads), kargs, 0, s);
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a, int d, int in_dtype, hipStream_t s) {
  if (in_dtype == kBF16) {
    if (d == 64) return launch_typed<64, __bf16>(a, s);
    if (d == 128) return launch_typed<128, __bf16>(a, s);
  } else if (in_dtype == kF16) {
    if (d == 64) return launch_typed<64, _Float16>(a, s);
    if (d == 128) return launch_typed<128, _Float16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
