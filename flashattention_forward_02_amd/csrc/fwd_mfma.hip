// Tiled FlashAttention forward for bf16 / fp16 inputs on the gfx950 matrix cores.
//
// What is computed ("FlashAttention 简化版：Tiling + Online Softmax", §2.3 and §3.1): one
// workgroup owns a tile of query rows of one (b, h) and streams that head's keys past it in
// tiles of BC keys. Per query row it keeps a running maximum, the running sum l and the fp32
// output accumulator; each key tile computes the scores, adds exp(s - m) to l and exp(s - m) V
// to the accumulator, and when the maximum grows, first scales l and the accumulator by
// exp(m_old - m_new). The accumulator is divided by l once at the end.
//
// How it maps onto CDNA4:
//  * Transposed products. S^T = K Q^T and O^T = V^T P^T, each as 32x32x16 MFMAs. In the
//    32x32 accumulator layout a lane owns one column and 16 rows; with queries as columns a
//    lane holds 16 scores of ONE query (rows = keys) and 16 output dims of that same query.
//    The row max / row sum are in-lane except one exchange with the other half-wave
//    (v_permlane32_swap), and the rescale factor is a per-lane scalar.
//  * P never leaves registers. The S^T accumulator of one 32-key block splits into two
//    8-value halves that are exactly the B operands of two 16-key PV MFMAs, under a fixed
//    permutation of the keys inside the 16-key step. The V^T A operand is read with the same
//    permutation by ds_read_b64_tr_b16 (gfx950's transposing LDS read), so V stays row-major
//    in LDS and is transposed on the way into registers.
//  * K/V tiles go from HBM straight into LDS (global_load_lds_dwordx4: no staging registers,
//    no LDS write instructions), double-buffered: the loads of tile j+1 are issued before the
//    MFMAs of tile j; one wait + barrier per tile. Both tiles are XOR-swizzled in 16-byte
//    chunks so the MFMA operand reads spread over the LDS banks (K: chunk ^ (row % 8) for the
//    row-per-lane 16-byte reads; V: chunk ^ 2*(row % 4) for the 4-row x 32-byte pattern of one
//    transposing read). The swizzle is applied on the global side: the lane that fills LDS
//    chunk (row, c) fetches global chunk (row, c ^ f(row)).
//  * Scores are handled in base 2: with c = scale * log2(e), exp(s - m) = 2^(raw*c - m*c),
//    one FMA and one v_exp_f32 per score. The true running max is kept on the raw dot
//    products (scale >= 0, so max commutes with the scale) and m_out = scale * max.
//  * Deferred rescaling. The exponent reference m_ref of a row moves only when the tile
//    maximum exceeds it by more than `rescale_threshold` (base-2 units); then l and the
//    accumulator are scaled by 2^(m_ref_old - m_ref_new) exactly as in §2.3. In between,
//    p = 2^(raw*c - m_ref) stays below 2^threshold, and since O = acc / l does not depend on
//    the reference (the identity of §2.2), the result is the same up to rounding. With a
//    threshold of 0 this is the pages' recurrence literally (rescale whenever the max grows).
//    At the end l (and, for split states, o) are re-expressed relative to the true maximum.
//    The rescale is a wave-uniform branch, so tiles where no row of a wave needs it skip the
//    D multiplies per row entirely.
//  * P is rounded to the input type (round to nearest even) only as the PV operand; l sums
//    the fp32 values ("CS349E 第 11 讲 01_online_softmax.py", demo 4).
//  * Four waves per workgroup, 64 query rows per wave (two 32-column MFMA blocks share every
//    K/V operand read from LDS), 256 query rows per workgroup. Only the last key tile of a
//    range can be partial; it runs a separate instantiation of the tile body that masks.

#include "fa_internal.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
  typedef bf16x8_t v8;
  static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<_Float16> {
  typedef f16x8_t v8;
  static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kWaves = 4;
constexpr int kNB = 2;                       // 32-query MFMA column blocks per wave
constexpr int kBC = 64;                      // keys per tile
constexpr int kBR = kWaves * kNB * 32;       // query rows per workgroup
constexpr int kThreads = kWaves * 64;

// Max / sum of a value and its counterpart in the other half of the wave (lane l and l ^ 32).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Store 4 consecutive fp32 values of one output row in the output type.
__device__ __forceinline__ void store4(void* base, size_t elem, int out_dtype, float x0, float x1, float x2,
                                       float x3) {
  if (out_dtype == kF32) {
    f32x4_t v = {x0, x1, x2, x3};
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(base) + elem) = v;
  } else if (out_dtype == kBF16) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
    bf16x4_t v = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
    *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(base) + elem) = v;
  } else {
    typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
    f16x4_t v = {(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
    *reinterpret_cast<f16x4_t*>(static_cast<_Float16*>(base) + elem) = v;
  }
}

template <int D, typename T>
struct Tile {
  typedef typename Mma<T>::v8 v8;
  static constexpr int KS = D / 16;                 // 16-wide k steps of S^T = K Q^T
  static constexpr int DB = D / 32;                 // 32-row blocks of O^T
  static constexpr int CH = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int ELEMS = kBC * D;             // elements per K (or V) tile
  static constexpr int CPW = ELEMS / 8 / kWaves;    // 16-byte chunks each wave moves per tensor
  static constexpr int LPW = CPW / 64;              // direct-to-LDS loads per wave per tensor
  static_assert(LPW >= 1 && LPW * 64 * kWaves * 8 == ELEMS, "tile / wave mismatch");
};

// Per-wave state of the online softmax for its 2 x 32 query rows (one value per lane each).
struct RowState {
  float mraw[kNB];   // true running max of the raw dot products
  float m2ref[kNB];  // exponent reference, base-2 units
  float lsum[kNB];   // sum of 2^(raw*c - m2ref)
};

// One key tile: S^T MFMAs, online-softmax update, PV MFMAs. TAIL masks keys >= valid.
template <int D, typename T, bool TAIL>
__device__ __forceinline__ void tile_step(const T* __restrict__ lk, const T* __restrict__ lv,
                                          const typename Tile<D, T>::v8 (&qf)[kNB][Tile<D, T>::KS],
                                          f32x16_t (&acc)[kNB][Tile<D, T>::DB], RowState& st, bool first,
                                          int valid, float c2, float tau, int lane) {
  typedef Tile<D, T> C;
  typedef typename C::v8 v8;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // ---- S^T = K Q^T : rows = 64 keys (two 32-blocks), columns = this wave's queries ----
  f32x16_t s[kNB][2];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][kb][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = kb * 32 + l32;
      const int ch = ks * 2 + hf;
      const v8 kf = *reinterpret_cast<const v8*>(&lk[r * D + ((ch ^ (r & 7)) << 3)]);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) s[nb][kb] = Mma<T>::mma(kf, qf[nb][ks], s[nb][kb]);
    }
  }

  if constexpr (TAIL) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= valid) {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) s[nb][kb][r] = -INFINITY;
        }
      }
  }

  // ---- online softmax ----
  v8 pf[kNB][4];  // PV B operands, one per 16-key step
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    float mx = s[nb][0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][kb][r]);
    mx = xhalf_max(mx);
    st.mraw[nb] = fmaxf(st.mraw[nb], mx);
    const float mx2 = mx * c2;
    const bool need = first || (mx2 > st.m2ref[nb] + tau);
    if (__ballot(need)) {  // wave-uniform: some row of this wave moves its reference
      const float ref = need ? mx2 : st.m2ref[nb];
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(st.m2ref[nb] - ref);
        st.lsum[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nb][db][r] *= alpha;
      }
      st.m2ref[nb] = ref;
    }
    const float nref = -st.m2ref[nb];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = half * 8 + u;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][kb][r], c2, nref));
          if constexpr (TAIL) {
            if (s[nb][kb][r] == -INFINITY) p = 0.f;
          }
          rs += p;
          pf[nb][kb * 2 + half][u] = (T)p;
        }
    st.lsum[nb] += xhalf_sum(rs);
  }

  // ---- O^T += V^T P^T : 16 keys per step, V^T read transposed from row-major LDS ----
  const int tj = lane & 15;
  const int ti = tj >> 2;
  const int tq = tj & 3;
  const int tgb = (lane >> 4) & 1;
#pragma unroll
  for (int g = 0; g < kBC / 16; ++g) {
    const int row1 = 16 * g + 4 * hf + ti;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int col = db * 32 + tgb * 16 + tq * 4;
      const int off1 = row1 * D + (((col >> 3) ^ (ti << 1)) << 3) + (col & 7);
      const int off2 = off1 + 8 * D;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&lv[off1]);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&lv[off2]);
      const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
      const u32x4_t packed = {lo2[0], lo2[1], hi2[0], hi2[1]};
      const v8 vf = __builtin_bit_cast(v8, packed);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[nb][db] = Mma<T>::mma(vf, pf[nb][g], acc[nb][db]);
    }
  }
}

// HBM -> LDS of one K/V tile (keys key0 .. key0 + 63), swizzled as described at the top. Rows
// past `kend` repeat the last key of the range; their scores are masked by the tail tile.
template <int D, typename T>
__device__ __forceinline__ void load_kv_tile(const T* __restrict__ K, const T* __restrict__ V, T* lk, T* lv, int key0,
                                             int kend, int wave, int lane) {
  typedef Tile<D, T> C;
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int base = wave * C::CPW + i * 64;  // first LDS chunk of this load (wave-uniform)
    const int ci = base + lane;
    const int r = ci / C::CH, cpos = ci % C::CH;
    const int key = min(key0 + r, kend - 1);
    const T* gk = K + (size_t)key * D + ((cpos ^ (r & 7)) << 3);
    const T* gv = V + (size_t)key * D + ((cpos ^ ((r & 3) << 1)) << 3);
    __builtin_amdgcn_global_load_lds(gk, (lds_void_t*)&lk[base * 8], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gv, (lds_void_t*)&lv[base * 8], 16, 0, 0);
  }
}

// Workgroups per CU the register budget is sized for: two 4-wave workgroups (2 waves per SIMD,
// 256 registers each) at d = 64, one at d = 128 (512 registers, the accumulator alone is 128).
template <int D> struct Occupancy { static constexpr int kMinBlocks = (D <= 64) ? 2 : 1; };

template <int D, typename T, int MINB = Occupancy<D>::kMinBlocks>
__global__ __launch_bounds__(kThreads, MINB) void fwd_mfma_kernel(FwdArgs a, int n_qtiles) {
  typedef Tile<D, T> C;
  typedef typename C::v8 v8;

  __shared__ __attribute__((aligned(16))) T lds_k[2][C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v[2][C::ELEMS];

  // ---- work item: (query tile, split, h, b) ----
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = wg % n_qtiles;
  int rest = wg / n_qtiles;
  const int split = rest % a.num_splits;
  rest /= a.num_splits;
  const int h = rest % a.H;
  const int b = rest / a.H;
  const size_t head = (size_t)b * a.H + h;
  const T* __restrict__ Q = static_cast<const T*>(a.q) + head * (size_t)a.Nq * D;
  const T* __restrict__ K = static_cast<const T*>(a.k) + head * (size_t)a.Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + head * (size_t)a.Nk * D;
  const int kbeg = split_begin(split, a.Nk, a.num_splits);
  const int kend = split_begin(split + 1, a.Nk, a.num_splits);
  const int nkeys = kend - kbeg;
  const int ntiles = (nkeys + kBC - 1) / kBC;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int qrow0 = qt * kBR + wave * (kNB * 32);

  // ---- Q^T fragments: B operand of S^T = K Q^T, lane = query column, 8 dims per lane ----
  v8 qf[kNB][C::KS];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int row = qrow0 + nb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (row < a.Nq) raw = *reinterpret_cast<const u32x4_t*>(Q + (size_t)row * D + ks * 16 + hf * 8);
      qf[nb][ks] = __builtin_bit_cast(v8, raw);
    }
  }

  auto load_tile = [&](int t, int buf) {
    load_kv_tile<D, T>(K, V, lds_k[buf], lds_v[buf], kbeg + t * kBC, kend, wave, lane);
  };

  const float c2 = a.scale_log2e;
  const float tau = a.rescale_threshold;
  RowState st;
  f32x16_t acc[kNB][C::DB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    st.mraw[nb] = -INFINITY;
    st.m2ref[nb] = 0.f;
    st.lsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][db][r] = 0.f;
  }

  if (ntiles > 0) load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Full tiles, then (outside the loop, so the loop body has one version) the partial last tile.
  const int nfull = nkeys / kBC;
  for (int t = 0; t < nfull; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1, buf ^ 1);
    tile_step<D, T, false>(lds_k[buf], lds_v[buf], qf, acc, st, t == 0, kBC, c2, tau, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (nfull < ntiles) {
    const int buf = nfull & 1;
    tile_step<D, T, true>(lds_k[buf], lds_v[buf], qf, acc, st, nfull == 0, nkeys - nfull * kBC, c2, tau, lane);
  }

  // ---- epilogue: re-express l (and o) relative to the true maximum; O = acc / l ----
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int row = qrow0 + nb * 32 + l32;
    if (row >= a.Nq) continue;
    const float to_true = __builtin_amdgcn_exp2f(st.m2ref[nb] - st.mraw[nb] * c2);
    const float l_true = st.lsum[nb] * to_true;
    if (a.split_mode == 0) {
      const float inv = 1.f / st.lsum[nb];
      const size_t obase = (head * (size_t)a.Nq + row) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dd = db * 32 + 8 * g4 + 4 * hf;
          store4(a.o, obase + dd, a.out_dtype, acc[nb][db][4 * g4] * inv, acc[nb][db][4 * g4 + 1] * inv,
                 acc[nb][db][4 * g4 + 2] * inv, acc[nb][db][4 * g4 + 3] * inv);
        }
      if (hf == 0) {
        if (a.m_out) a.m_out[head * a.Nq + row] = a.scale * st.mraw[nb];
        if (a.l_out) a.l_out[head * a.Nq + row] = l_true;
      }
    } else {
      const size_t prow = ((size_t)split * a.B * a.H + head) * a.Nq + row;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dd = db * 32 + 8 * g4 + 4 * hf;
          store4(a.part_o, prow * D + dd, kF32, acc[nb][db][4 * g4] * to_true, acc[nb][db][4 * g4 + 1] * to_true,
                 acc[nb][db][4 * g4 + 2] * to_true, acc[nb][db][4 * g4 + 3] * to_true);
        }
      if (hf == 0) {
        a.part_m[prow] = a.scale * st.mraw[nb];
        a.part_l[prow] = l_true;
      }
    }
  }
}

template <int D, typename T>
hipError_t launch_typed(const FwdArgs& a, hipStream_t s) {
  const int n_qtiles = (a.Nq + kBR - 1) / kBR;
  const long long nwg = (long long)n_qtiles * a.num_splits * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  int nq = n_qtiles;
  void* kargs[] = {&args, &nq};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_mfma_kernel<D, T>), dim3((unsigned)nwg), dim3(kThreads),
                         kargs, 0, s);
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, int d, int in_dtype, hipStream_t s) {
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
