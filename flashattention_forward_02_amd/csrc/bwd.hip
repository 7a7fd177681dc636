// FlashAttention backward pass for bf16 / fp16 inputs on the gfx950 matrix cores.
//
// What is computed. "Flash Attention 代码填空 (Level 2-3)", Exercise 5: the backward pass keeps
// no score matrix; it recomputes P block by block from the forward pass's row statistics and
// accumulates dV_j = sum_i P_ij^T dO_i. "CS349E 第 11 讲 01_online_softmax.py" notes that only the
// log-sum-exp L = m + ln(l) of each row needs to be kept, so P_ij = exp(S_ij - L_i). dQ and dK
// follow from O = softmax(S) V, S = scale Q K^T by the chain rule:
//     dP = dO V^T,  dS_ij = P_ij (dP_ij - D_i),  D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic,
//     dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// With grouped K/V heads dK and dV of a K/V head sum over the query heads that read it; under
// the causal mask the masked P_ij are 0.
//
// How it maps onto CDNA4. Three kernels, no atomics, every output written by one workgroup:
//  * bwd_delta: D_i = sum_c dO_ic O_ic, one row per D/8 lanes (at d = 64 the dQ kernel computes
//    D itself).
//  * bwd_dq: a workgroup owns 128 query rows of one (b, h) (32 per wave) and streams the head's
//    K and V past them in 64-key tiles, exactly like the forward kernel: S^T = K Q^T and
//    dP^T = V dO^T on 32x32x16 MFMAs with Q and dO held as B operands in registers, then in
//    registers P^T and dS^T, and dQ^T += K^T dS^T with K^T read from LDS by transposing reads.
//  * dK, dV: a workgroup owns keys of one (b, h_kv) and streams the query rows of every query
//    head of the group past them in 64-row tiles: S = Q K^T and dP = dO V^T with K and V held as
//    B operands, P and dS in registers, dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T as
//    A operands. Under the causal mask earlier key tiles are seen by more query rows, so the key
//    tile varies slowest in block order, heaviest (first) first; without it the XCD remap keeps a
//    head's tiles on one L2. The row values are prepared in LDS once per tile by the waves that
//    load them (after the load lands, before the barrier that publishes the tile): lse scaled by
//    log2(e), so P = 2^(s c - L log2 e) takes one FMA per element, and +inf for rows past Nq, so
//    their P is 0 without a mask; D negated, as the initial value of the dP accumulator.
//  In both, the 32x32 accumulator of S (or S^T) splits into 8-value halves that are the B
//  operands of the next 16-step MFMAs under the same fixed row permutation the forward kernel
//  uses for P; the transposing reads follow it. P and dS are rounded to the input type (round to
//  nearest even) only as MFMA operands; everything else is fp32.
//  Tiles go from HBM straight into LDS (global_load_lds), a quarter per wave, with the 16-byte-
//  chunk swizzle swz_rt, under which both the row reads and the transposing reads of a tile are
//  free of bank conflicts.
//  At d = 64 both gradient kernels run as ping-pong kernels (bwd_dq_pp, bwd_dkdv_pp): 8 waves
//  in two groups in opposite matrix-core / softmax phases, as in the forward kernel, 256 rows
//  (keys) per workgroup, three rotating tile buffers. At d = 128 the dQ kernel is the 4-wave one
//  (two workgroups per compute unit) and dK, dV come from bwd_dkdv16 (16 keys per wave on
//  16x16x32 MFMAs, so that two waves fit a SIMD; ping-pong as at d = 64).

#include "fa_internal.h"
#include "mfma_common.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kTile = 64;                        // keys (dQ) or query rows (dK, dV) per streamed tile
constexpr int kOwn = kBwdWaves * 32;             // query rows (dQ) or keys (dK, dV) per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <int D, typename T>
struct BCfg {
  typedef typename Mma<T>::v8 v8;
  static constexpr int KS = D / 16;              // 16-wide k steps over the head dimension
  static constexpr int DB = D / 32;              // 32-dim blocks of the gradient accumulators
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int ELEMS = kTile * D;        // elements per tile
  static constexpr int LPW = ELEMS / 8 / 64 / kBwdWaves;  // 1 KB loads per wave and tile
  static_assert(LPW >= 1 && LPW * 64 * kBwdWaves * 8 == ELEMS, "tile / wave mismatch");
};

// 4-byte-per-lane global -> LDS copy: lane i's 4 bytes land at lds + 4 * i.
__device__ __forceinline__ void global_to_lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 4, 0, 0);
}

// HBM -> LDS of a 64-row tile, a quarter per wave. LDS chunk c of tile row r holds global chunk
// c ^ swz_rt<D>(r); rows at or past `nrows` repeat row nrows - 1 (their results are masked or never
// stored).
template <int D, typename T>
__device__ __forceinline__ void load_tile(const T* __restrict__ X, T* lx, int row0, int nrows, int wave, int lane) {
  typedef BCfg<D, T> C;
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int base = (wave * C::LPW + i) * 64;   // first LDS chunk of this load (wave-uniform)
    const int ci = base + lane;
    const int r = ci / C::CH, cpos = ci % C::CH;
    const int row = min(row0 + r, nrows - 1);
    global_to_lds16(X + (size_t)row * D + ((cpos ^ swz_rt<D>(r)) << 3), &lx[base * 8]);
  }
}

// 64 row values (lse or D) of rows row0.. into LDS; rows at or past nrows repeat the last one.
__device__ __forceinline__ void load_rowvec(const float* __restrict__ x, float* lx, int row0, int nrows, int lane) {
  global_to_lds4(x + min(row0 + lane, nrows - 1), lx);
}

// Eight fp32 values rounded to T: one B operand of a 16-step (values i = 0..7 are registers
// 8 (g % 2) + i of the accumulator block g / 2, the row order the transposing reads follow).
template <typename T>
__device__ __forceinline__ typename Mma<T>::v8 pack8(const float (&x)[8]) {
  typename Mma<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)x[i];
  return r;
}

// Row index (within a 32-row block) of register r of lane half hf in a 32x32 accumulator.
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// This lane's byte offsets of its operand reads within a swizzled tile (LDS chunk c of row r holds
// global chunk c ^ swz_rt<D>(r)):
//  * row read: the 16 bytes of row l32, global chunk 2 ks + hf (an A or B operand row fragment);
//  * transposing read: the A operand X^T[dims of 32-block db][rows of 16-step g] of a row-major
//    tile X, in the row order of the P operands built by pack8 (the forward kernel's V^T read):
//    two 8-byte ds_read_tr16_b64 at rows 16 g + 4 hf + (lane % 16) / 4 and 8 rows further, column
//    32 db + 16 ((lane / 16) % 2) + 4 (lane % 4).
// The swizzle of a row depends only on row % 16, so a row read at row + 32 qb and a transposing
// read at rows + 16 g are these offsets plus a constant (64 qb D or 32 g D bytes), which the reads
// take as an immediate. Kernels pass the offsets through an empty asm once per step, so the
// compiler cannot hoist one register per (buffer, read) out of the loop.
template <int D, typename T>
struct LdsOff {
  unsigned row[D / 16];                  // row read of row l32, chunk 2 ks + hf
  unsigned tr1[D / 32], tr2[D / 32];     // the two 8-byte transposing reads of step g = 0, block db
  __device__ __forceinline__ LdsOff(int lane) {
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) row[ks] = (unsigned)((l32 * D + (((ks * 2 + hf) ^ swz_rt<D>(l32)) << 3)) * sizeof(T));
    const int tj = lane & 15, ti = tj >> 2, tq = tj & 3, tgb = (lane >> 4) & 1;
    const int row1 = 4 * hf + ti;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + tgb * 16 + tq * 4;
      tr1[db] = (unsigned)((row1 * D + (((col >> 3) ^ swz_rt<D>(row1)) << 3) + (col & 7)) * sizeof(T));
      tr2[db] = (unsigned)(((row1 + 8) * D + (((col >> 3) ^ swz_rt<D>(row1 + 8)) << 3) + (col & 7)) * sizeof(T));
    }
  }
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(row[i]));
#pragma unroll
    for (int i = 0; i < D / 32; ++i) asm volatile("" : "+v"(tr1[i]), "+v"(tr2[i]));
  }
};
// Row read of row 32 qb + l32, chunk 2 ks + hf
template <int D, typename T>
__device__ __forceinline__ typename Mma<T>::v8 row_frag_o(const T* lx, const LdsOff<D, T>& o, int qb, int ks) {
  const char* p = reinterpret_cast<const char*>(lx) + o.row[ks] + qb * 32 * D * (int)sizeof(T);
  return *reinterpret_cast<const typename Mma<T>::v8*>(p);
}
// Transposing read of 16-row step g, 32-dim block db
template <int D, typename T>
__device__ __forceinline__ typename Mma<T>::v8 tr_frag_o(const T* lx, const LdsOff<D, T>& o, int g, int db) {
  const char* base = reinterpret_cast<const char*>(lx) + g * 16 * D * (int)sizeof(T);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + o.tr1[db]));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + o.tr2[db]));
  const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
  const u32x4_t packed = {lo2[0], lo2[1], hi2[0], hi2[1]};
  return __builtin_bit_cast(typename Mma<T>::v8, packed);
}

// ---------------------------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic
// ---------------------------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a, long long rows) {
  constexpr int LPR = D / 8;                     // lanes per row, 8 elements each
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int c0 = (threadIdx.x % LPR) * 8;
  float s = 0.f;
  if (row < rows) {
    const size_t e = (size_t)row * D + c0;
    const typename Mma<T>::v8 g = *reinterpret_cast<const typename Mma<T>::v8*>(static_cast<const T*>(a.dout) + e);
    if (a.o_dtype == kF32) {
      const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.o) + e);
      const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.o) + e + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) s = __builtin_fmaf((float)g[i], o0[i], s);
#pragma unroll
      for (int i = 0; i < 4; ++i) s = __builtin_fmaf((float)g[4 + i], o1[i], s);
    } else {
      const typename Mma<T>::v8 o = *reinterpret_cast<const typename Mma<T>::v8*>(static_cast<const T*>(a.o) + e);
#pragma unroll
      for (int i = 0; i < 8; ++i) s = __builtin_fmaf((float)g[i], (float)o[i], s);
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
  if (row < rows && c0 == 0) a.delta[row] = s;
}

// ---------------------------------------------------------------------------------------------
// dQ: 128 query rows of one (b, h) per workgroup, K/V streamed in 64-key tiles
// ---------------------------------------------------------------------------------------------
template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(BwdArgs a, int n_qtiles) {
  typedef BCfg<D, T> C;
  typedef typename C::v8 v8;
  // Two separate buffers per tensor (not one array of two): a load into one is then seen not to
  // alias reads of the other, and reads of the current tile do not wait for the next tile's loads.
  __shared__ __attribute__((aligned(16))) T lds_k0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_k1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v1[C::ELEMS];

  // Under the causal mask later query tiles see more keys: the query tile varies slowest in block
  // order, heaviest first (compute units that finish early take the light tiles). Otherwise the
  // XCD remap keeps a head's tiles on one L2.
  int qt, rest;
  if constexpr (CAUSAL) {
    const int units = gridDim.x / n_qtiles;
    qt = n_qtiles - 1 - (int)blockIdx.x / units;
    rest = (int)blockIdx.x % units;
  } else {
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    qt = wg % n_qtiles;
    rest = wg / n_qtiles;
  }
  const int h = rest % a.H;
  const int b = rest / a.H;
  const size_t head = (size_t)b * a.H + h;
  const size_t kvh = kv_head_index(b, h, a.H, a.H_kv);
  const T* __restrict__ Q = static_cast<const T*>(a.q) + head * (size_t)a.Nq * D;
  const T* __restrict__ dO = static_cast<const T*>(a.dout) + head * (size_t)a.Nq * D;
  const T* __restrict__ K = static_cast<const T*>(a.k) + kvh * (size_t)a.Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + kvh * (size_t)a.Nk * D;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int row = qt * kOwn + wave * 32 + l32;   // this lane's query row (column of S^T)
  const int rowc = min(row, a.Nq - 1);

  // Key range of the workgroup: under the mask it ends after the last key its last row sees.
  int kend = a.Nk;
  if constexpr (CAUSAL) kend = min(kend, min(a.Nq, (qt + 1) * kOwn) + a.causal_off);
  const int T_ = (kend + kTile - 1) / kTile;

  v8 qf[C::KS], dof[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = *reinterpret_cast<const v8*>(Q + (size_t)rowc * D + ks * 16 + hf * 8);
    dof[ks] = *reinterpret_cast<const v8*>(dO + (size_t)rowc * D + ks * 16 + hf * 8);
  }
  const float L2 = a.lse[head * a.Nq + rowc] * kLog2e;
  const float Dr = a.delta[head * a.Nq + rowc];
  const float c2 = a.scale_log2e;
  const int last_key = CAUSAL ? row + a.causal_off : a.Nk - 1;   // keys past it are masked
  // the smallest last_key of the wave's rows (its first row's)
  const int wave_last_key = CAUSAL ? min(qt * kOwn + wave * 32 + a.causal_off, a.Nk - 1) : a.Nk - 1;

  f32x16_t acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  load_tile<D, T>(K, lds_k0, 0, a.Nk, wave, lane);
  load_tile<D, T>(V, lds_v0, 0, a.Nk, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  LdsOff<D, T> lo0(lane);
  // One key tile: prefetch tile t + 1 into (nk, nv), compute from (lk, lv), wait, barrier.
  auto tile = [&](int t, const T* lk, const T* lv, T* nk, T* nv) __attribute__((always_inline)) {
    LdsOff<D, T> lo = lo0;
    lo.opaque();
    if (t + 1 < T_) {
      load_tile<D, T>(K, nk, (t + 1) * kTile, a.Nk, wave, lane);
      load_tile<D, T>(V, nv, (t + 1) * kTile, a.Nk, wave, lane);
    }
    // S^T = K Q^T and dP^T = V dO^T: rows = the tile's 64 keys (two 32-blocks), columns = queries
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
    // The two waves of a SIMD come from different workgroups and drift in and out of step; the
    // raised priority lets a wave's S / dP burst issue ahead of the other wave's VALU work
    // (measured 1.5 % faster).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = Mma<T>::mma(row_frag_o<D, T>(lk, lo, kb, ks), qf[ks], s[kb]);
        dp[kb] = Mma<T>::mma(row_frag_o<D, T>(lv, lo, kb, ks), dof[ks], dp[kb]);
      }
    __builtin_amdgcn_s_setprio(0);
    // per 16-key step g: P^T = exp(S - L) (0 where masked), dS^T = P^T (dP^T - D), then
    // dQ^T += K^T dS^T. At d = 64 only a tile holding a key past the first row's last visible key
    // (the ragged end; the causal diagonal) takes the per-key mask (a wave-uniform test); at
    // d = 128 a second copy of the body does not fit in registers.
    auto grads = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kb = g >> 1;
        float ds[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * (g & 1) + i;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, -L2));
          if constexpr (decltype(masked)::value) {
            if (t * kTile + kb * 32 + acc_row(r, hf) > last_key) p = 0.f;
          }
          ds[i] = p * (dp[kb][r] - Dr);
        }
        const v8 dsf = pack8<T>(ds);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] = Mma<T>::mma(tr_frag_o<D, T>(lk, lo, g, db), dsf, acc[db]);
      }
    };
    if (D > 64 || (t + 1) * kTile - 1 > wave_last_key) grads(std::true_type());  // one body at d = 128
    else grads(std::false_type());
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int t = 0; t < T_; t += 2) {
    tile(t, lds_k0, lds_v0, lds_k1, lds_v1);
    if (t + 1 < T_) tile(t + 1, lds_k1, lds_v1, lds_k0, lds_v0);
  }

  if (row < a.Nq) {
    float* out = a.dq + (head * (size_t)a.Nq + row) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = db * 32 + 8 * g4 + 4 * hf;
        f32x4_t x = {a.scale * acc[db][4 * g4], a.scale * acc[db][4 * g4 + 1], a.scale * acc[db][4 * g4 + 2],
                     a.scale * acc[db][4 * g4 + 3]};
        *reinterpret_cast<f32x4_t*>(out + dd) = x;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV at d = 64, ping-pong: 8 waves in two groups (A = waves 0-3, B = 4-7; waves w and w + 4
// share a SIMD) in opposite phases, as in the forward kernel, so one wave of each SIMD keeps the
// matrix core busy while the other computes P and dS. A workgroup owns 256 keys of one
// (b, h_kv), 32 per wave, and streams the 64-row query tiles of every query head of the group.
//   MFMA phase of step t: dV^T += dO^T P and dK^T += Q^T dS of step t - 1, then S and dP - D of
//     step t.
//   VALU phase of step t: P and dS of step t, rounded as the next phase's B operands.
// Group B runs one phase behind group A. Group A loads the tiles of step t + 1 (Q, dO, L, D) at
// the top of its MFMA phase t and waits for them at the end of its VALU phase t; a tile is read
// in MFMA phases t (rows) and t + 1 (transposed), so three buffers rotate: the load into buffer
// (t + 1) % 3 starts after both groups' last reads of step t - 2, which ended at least one barrier
// earlier. The steady steps are unrolled by three so every buffer is a distinct object at each use.
// ---------------------------------------------------------------------------------------------
constexpr int kPpWaves = 8;
constexpr int kPpOwn = kPpWaves * 32;            // keys per workgroup

// Issue order of a full MFMA phase (16 dV / dK MFMAs fed by two transposing reads each, then the
// 8 reads of -D, then 16 S / dP MFMAs fed by one row read each): the reads of the MFMA PD
// positions ahead go before each MFMA, so LDS latency hides behind matrix-core work and only a
// few operands are in registers at once.
__host__ __device__ constexpr int pp_reads_needed(int i) { return i < 16 ? 2 * (i + 1) : 40 + (i - 15); }
template <int PD, int I>
__device__ __forceinline__ void dkdv_pp_order() {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NM = 32;
  constexpr int kMfma = 0x008, kDsRead = 0x100;  // sched_group_barrier instruction classes
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(kDsRead, pp_reads_needed(PD), 0);
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    constexpr int a = pp_reads_needed(I + PD < NM ? I + PD : NM - 1);
    constexpr int b = pp_reads_needed(I + 1 + PD < NM ? I + 1 + PD : NM - 1);
    if constexpr (b > a) __builtin_amdgcn_sched_group_barrier(kDsRead, b - a, 0);
    dkdv_pp_order<PD, I + 1>();
  }
#endif
}

template <typename T, bool CAUSAL>
__global__ __launch_bounds__(kPpWaves * 64, 1) void bwd_dkdv_pp_kernel(BwdArgs a, int n_ktiles) {
  constexpr int D = 64;
  typedef BCfg<D, T> C;
  typedef typename C::v8 v8;
  __shared__ __attribute__((aligned(16))) T lds_q0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_q1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_q2[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_do0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_do1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_do2[C::ELEMS];
  __shared__ __attribute__((aligned(16))) float lds_l0[kTile];
  __shared__ __attribute__((aligned(16))) float lds_l1[kTile];
  __shared__ __attribute__((aligned(16))) float lds_l2[kTile];
  __shared__ __attribute__((aligned(16))) float lds_d0[kTile];
  __shared__ __attribute__((aligned(16))) float lds_d1[kTile];
  __shared__ __attribute__((aligned(16))) float lds_d2[kTile];

  // work order: see the file header (dK, dV)
  int kt, rest;
  if constexpr (CAUSAL) {
    const int units = gridDim.x / n_ktiles;
    kt = (int)blockIdx.x / units;
    rest = (int)blockIdx.x % units;
  } else {
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    kt = wg % n_ktiles;
    rest = wg / n_ktiles;
  }
  const int hk = rest % a.H_kv;
  const int b = rest / a.H_kv;
  const int group = a.H / a.H_kv;
  const size_t kvh = (size_t)b * a.H_kv + hk;
  const T* __restrict__ K = static_cast<const T*>(a.k) + kvh * (size_t)a.Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + kvh * (size_t)a.Nk * D;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool group_a = wave < 4;
  const int gw = wave & 3;                         // wave index within its group (loads: group A)
  const int hf = lane >> 5;
  const int key = kt * kPpOwn + wave * 32 + (lane & 31);   // this lane's key (column of S)
  const int keyc = min(key, a.Nk - 1);

  v8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    kf[ks] = *reinterpret_cast<const v8*>(K + (size_t)keyc * D + ks * 16 + hf * 8);
    vf[ks] = *reinterpret_cast<const v8*>(V + (size_t)keyc * D + ks * 16 + hf * 8);
  }
  const float c2 = a.scale_log2e;

  f32x16_t dk[C::DB], dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.f;

  const int n_rtiles = (a.Nq + kTile - 1) / kTile;
  int r_begin = 0;
  if constexpr (CAUSAL) r_begin = max(0, kt * kPpOwn - a.causal_off) / kTile;
  const int per_head = n_rtiles - r_begin;
  const int n_steps = per_head * group;            // (query head, row tile) pairs, head-major
  auto row0 = [&](int st) { return (r_begin + st % per_head) * kTile; };

  // Group A: a quarter of each tile per wave (a whole tile: scalar base and per-lane 32-bit
  // offsets computed once, kept opaque; a tile past Nq: load_tile's clamped path); wave 0 the lse
  // rows, wave 1 the D rows.
  unsigned toff[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int ci = (gw * C::LPW + i) * 64 + lane;
    const int r = ci / C::CH, cpos = ci % C::CH;
    toff[i] = (unsigned)((r * D + ((cpos ^ swz_rt<D>(r)) << 3)) * sizeof(T));
  }
  auto tile_in = [&](const T* X, T* lx, int r0) __attribute__((always_inline)) {
    if (r0 + kTile <= a.Nq) {
      const char* g = reinterpret_cast<const char*>(X + (size_t)r0 * D);
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        unsigned o = toff[i];
        asm volatile("" : "+v"(o));
        global_to_lds16(g + o, &lx[(gw * C::LPW + i) * 64 * 8]);
      }
    } else {
      load_tile<D, T>(X, lx, r0, a.Nq, gw, lane);
    }
  };
  auto issue = [&](int st, T* lq, T* ldo, float* ll, float* ld) __attribute__((always_inline)) {
    const int h = hk * group + st / per_head;
    const int r0 = row0(st);
    const size_t head = (size_t)b * a.H + h;
    tile_in(static_cast<const T*>(a.q) + head * (size_t)a.Nq * D, lq, r0);
    tile_in(static_cast<const T*>(a.dout) + head * (size_t)a.Nq * D, ldo, r0);
    if (wave == 0) load_rowvec(a.lse + head * a.Nq, ll, r0, a.Nq, lane);
    if (wave == 1) load_rowvec(a.delta + head * a.Nq, ld, r0, a.Nq, lane);
  };
  // After the loads land (vmcnt(0) of the loading wave): lse * log2(e) (+inf past Nq), and -D.
  auto prep_rows = [&](float* ll, float* ld, int r0) __attribute__((always_inline)) {
    if (wave == 0) ll[lane] = r0 + lane < a.Nq ? ll[lane] * kLog2e : INFINITY;
    if (wave == 1) ld[lane] = -ld[lane];
  };

  const LdsOff<D, T> lo0(lane);
  f32x16_t s[2], dp[2];
  v8 pf[4], dsf[4];

  // do_dkdv / do_sdp are compile-time flags (std::true_type / std::false_type), so the issue
  // order sits in the same basic block as the reads and MFMAs it orders.
  auto phase_mfma = [&](int t, auto do_dkdv, auto do_sdp, const T* qp, const T* dop, const T* qc, const T* doc,
                        const float* dc, T* qn, T* don, float* ln, float* dn) __attribute__((always_inline)) {
    LdsOff<D, T> lo = lo0;
    lo.opaque();
    if (group_a && t + 1 < n_steps) issue(t + 1, qn, don, ln, dn);
    if constexpr (decltype(do_dkdv)::value) {
      // dV^T += dO^T P and dK^T += Q^T dS of step t - 1 (transposing reads of its tiles)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          dv[db] = Mma<T>::mma(tr_frag_o<D, T>(dop, lo, g, db), pf[g], dv[db]);
          dk[db] = Mma<T>::mma(tr_frag_o<D, T>(qp, lo, g, db), dsf[g], dk[db]);
        }
    }
    if constexpr (decltype(do_sdp)::value) {
      // S = Q K^T and dP - D = dO V^T - D of step t (the dP accumulator starts at -D)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4_t nD = *reinterpret_cast<const f32x4_t*>(&dc[qb * 32 + 8 * g4 + 4 * hf]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            s[qb][4 * g4 + u] = 0.f;
            dp[qb][4 * g4 + u] = nD[u];
          }
        }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb] = Mma<T>::mma(row_frag_o<D, T>(qc, lo, qb, ks), kf[ks], s[qb]);
          dp[qb] = Mma<T>::mma(row_frag_o<D, T>(doc, lo, qb, ks), vf[ks], dp[qb]);
        }
    }
    if constexpr (decltype(do_dkdv)::value && decltype(do_sdp)::value) dkdv_pp_order<6, 0>();
    __syncthreads();
  };

  auto phase_valu = [&](int t, const float* lc, float* ln, float* dn) __attribute__((always_inline)) {
    // P = exp(S - L) (0 past Nq through L = +inf; masked keys), dS = P (dP - D); register r of
    // lane half hf is row 32 qb + acc_row(r, hf)
    const int r0 = row0(t);
    int lim = 0;
    if constexpr (CAUSAL) lim = key - a.causal_off - r0 - 4 * hf;
    auto grads = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qb = g >> 1;
      float p[8], ds[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int g4 = 2 * (g & 1) + h2;
        const f32x4_t Lv = *reinterpret_cast<const f32x4_t*>(&lc[qb * 32 + 8 * g4 + 4 * hf]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * g4 + u;
          float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c2, -Lv[u]));
          if constexpr (decltype(masked)::value) {
            if (32 * qb + 8 * g4 + u < lim) x = 0.f;
          }
          p[4 * h2 + u] = x;
          ds[4 * h2 + u] = x * dp[qb][r];
        }
      }
      pf[g] = pack8<T>(p);
      dsf[g] = pack8<T>(ds);
    }
    };
    // the per-key mask only where the wave's last key lies past what the step's first row sees
    if (CAUSAL && kt * kPpOwn + wave * 32 + 31 > r0 + a.causal_off) grads(std::true_type());
    else grads(std::false_type());
    if (group_a) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (t + 1 < n_steps) prep_rows(ln, dn, row0(t + 1));
    }
    __syncthreads();
  };

  // prologue: step 0's tiles resident and prepared; group B then sits out one phase
  if (group_a && n_steps > 0) {
    issue(0, lds_q0, lds_do0, lds_l0, lds_d0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    prep_rows(lds_l0, lds_d0, row0(0));
  }
  __syncthreads();
  if (!group_a) __syncthreads();

  // Step t reads buffers t % 3 (its own tiles) and (t + 2) % 3 (step t - 1's, transposed) and
  // loads into (t + 1) % 3: step 0 (S / dP only), the steady steps unrolled by three, then the
  // last step's dV / dK. Every wave takes the same number of barriers.
  const std::true_type yes;
  const std::false_type no;
  if (n_steps > 0) {
    phase_mfma(0, no, yes, lds_q2, lds_do2, lds_q0, lds_do0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
    phase_valu(0, lds_l0, lds_l1, lds_d1);
  }
  for (int t = 1; t < n_steps; t += 3) {
    phase_mfma(t, yes, yes, lds_q0, lds_do0, lds_q1, lds_do1, lds_d1, lds_q2, lds_do2, lds_l2, lds_d2);
    phase_valu(t, lds_l1, lds_l2, lds_d2);
    if (t + 1 < n_steps) {
      phase_mfma(t + 1, yes, yes, lds_q1, lds_do1, lds_q2, lds_do2, lds_d2, lds_q0, lds_do0, lds_l0, lds_d0);
      phase_valu(t + 1, lds_l2, lds_l0, lds_d0);
    }
    if (t + 2 < n_steps) {
      phase_mfma(t + 2, yes, yes, lds_q2, lds_do2, lds_q0, lds_do0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
      phase_valu(t + 2, lds_l0, lds_l1, lds_d1);
    }
  }
  if (n_steps == 0) phase_mfma(0, no, no, lds_q0, lds_do0, lds_q0, lds_do0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
  else if ((n_steps - 1) % 3 == 0) phase_mfma(n_steps, yes, no, lds_q0, lds_do0, lds_q1, lds_do1, lds_d1, lds_q2, lds_do2, lds_l2, lds_d2);
  else if ((n_steps - 1) % 3 == 1) phase_mfma(n_steps, yes, no, lds_q1, lds_do1, lds_q2, lds_do2, lds_d2, lds_q0, lds_do0, lds_l0, lds_d0);
  else phase_mfma(n_steps, yes, no, lds_q2, lds_do2, lds_q0, lds_do0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
  if (group_a) __syncthreads();

  if (key < a.Nk) {
    float* outk = a.dk + (kvh * (size_t)a.Nk + key) * D;
    float* outv = a.dv + (kvh * (size_t)a.Nk + key) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = db * 32 + 8 * g4 + 4 * hf;
        f32x4_t xk = {a.scale * dk[db][4 * g4], a.scale * dk[db][4 * g4 + 1], a.scale * dk[db][4 * g4 + 2],
                      a.scale * dk[db][4 * g4 + 3]};
        f32x4_t xv = {dv[db][4 * g4], dv[db][4 * g4 + 1], dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]};
        *reinterpret_cast<f32x4_t*>(outk + dd) = xk;
        *reinterpret_cast<f32x4_t*>(outv + dd) = xv;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ at d = 64, ping-pong (the structure of bwd_dkdv_pp_kernel with the roles of queries and keys
// exchanged): a workgroup owns 256 query rows of one (b, h), 32 per wave, and streams the head's
// K and V in 64-key tiles.
//   MFMA phase of tile t: dQ^T += K^T dS^T of tile t - 1, then S^T = K Q^T and dP^T - D of tile t.
//   VALU phase of tile t: P^T and dS^T of tile t.
// K is read in MFMA phases t (rows) and t + 1 (transposed), so the tiles rotate through three
// buffers as in bwd_dkdv_pp_kernel.
// ---------------------------------------------------------------------------------------------
__host__ __device__ constexpr int dq_pp_reads_needed(int i) { return i < 8 ? 2 * (i + 1) : 16 + (i - 7); }
template <int PD, int I>
__device__ __forceinline__ void dq_pp_order() {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NM = 24;
  constexpr int kMfma = 0x008, kDsRead = 0x100;  // sched_group_barrier instruction classes
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(kDsRead, dq_pp_reads_needed(PD), 0);
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    constexpr int a = dq_pp_reads_needed(I + PD < NM ? I + PD : NM - 1);
    constexpr int b = dq_pp_reads_needed(I + 1 + PD < NM ? I + 1 + PD : NM - 1);
    if constexpr (b > a) __builtin_amdgcn_sched_group_barrier(kDsRead, b - a, 0);
    dq_pp_order<PD, I + 1>();
  }
#endif
}

template <typename T, bool CAUSAL>
__global__ __launch_bounds__(kPpWaves * 64, 1) void bwd_dq_pp_kernel(BwdArgs a, int n_qtiles) {
  constexpr int D = 64;
  typedef BCfg<D, T> C;
  typedef typename C::v8 v8;
  __shared__ __attribute__((aligned(16))) T lds_k0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_k1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_k2[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v2[C::ELEMS];

  // work order as in bwd_dq_kernel
  int qt, rest;
  if constexpr (CAUSAL) {
    const int units = gridDim.x / n_qtiles;
    qt = n_qtiles - 1 - (int)blockIdx.x / units;
    rest = (int)blockIdx.x % units;
  } else {
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    qt = wg % n_qtiles;
    rest = wg / n_qtiles;
  }
  const int h = rest % a.H;
  const int b = rest / a.H;
  const size_t head = (size_t)b * a.H + h;
  const size_t kvh = kv_head_index(b, h, a.H, a.H_kv);
  const T* __restrict__ Q = static_cast<const T*>(a.q) + head * (size_t)a.Nq * D;
  const T* __restrict__ dO = static_cast<const T*>(a.dout) + head * (size_t)a.Nq * D;
  const T* __restrict__ K = static_cast<const T*>(a.k) + kvh * (size_t)a.Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + kvh * (size_t)a.Nk * D;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool group_a = wave < 4;
  const int gw = wave & 3;
  const int hf = lane >> 5;
  const int row = qt * kPpOwn + wave * 32 + (lane & 31);   // this lane's query row (column of S^T)
  const int rowc = min(row, a.Nq - 1);

  int kend = a.Nk;
  if constexpr (CAUSAL) kend = min(kend, min(a.Nq, (qt + 1) * kPpOwn) + a.causal_off);
  const int T_ = (kend + kTile - 1) / kTile;

  v8 qf[C::KS], dof[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = *reinterpret_cast<const v8*>(Q + (size_t)rowc * D + ks * 16 + hf * 8);
    dof[ks] = *reinterpret_cast<const v8*>(dO + (size_t)rowc * D + ks * 16 + hf * 8);
  }
  const float L2 = a.lse[head * a.Nq + rowc] * kLog2e;
  // D_i = sum_c dO_ic O_ic of this lane's row, here rather than in a kernel of its own: the lane
  // holds dims 16 ks + 8 hf .. + 7 of dO, the lane 32 apart the other half. Stored for the dK dV
  // kernel, which runs after this one.
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const size_t e = (head * (size_t)a.Nq + rowc) * D + ks * 16 + hf * 8;
    if (a.o_dtype == kF32) {
      const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.o) + e);
      const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.o) + e + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) dsum = __builtin_fmaf((float)dof[ks][i], o0[i], dsum);
#pragma unroll
      for (int i = 0; i < 4; ++i) dsum = __builtin_fmaf((float)dof[ks][4 + i], o1[i], dsum);
    } else {
      const v8 o = *reinterpret_cast<const v8*>(static_cast<const T*>(a.o) + e);
#pragma unroll
      for (int i = 0; i < 8; ++i) dsum = __builtin_fmaf((float)dof[ks][i], (float)o[i], dsum);
    }
  }
  dsum += __shfl_xor(dsum, 32);
  if (hf == 0 && row < a.Nq) a.delta[head * a.Nq + row] = dsum;
  const float nDr = -dsum;
  const float c2 = a.scale_log2e;
  const int last_key = CAUSAL ? row + a.causal_off : a.Nk - 1;   // keys past it are masked
  const int wave_last_key = CAUSAL ? min(qt * kPpOwn + wave * 32 + a.causal_off, a.Nk - 1) : a.Nk - 1;

  f32x16_t acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  // Group A loads a quarter of each tile per wave (whole tiles: scalar base + opaque 32-bit
  // offsets; the ragged end: load_tile's clamped path).
  unsigned toff[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int ci = (gw * C::LPW + i) * 64 + lane;
    const int r = ci / C::CH, cpos = ci % C::CH;
    toff[i] = (unsigned)((r * D + ((cpos ^ swz_rt<D>(r)) << 3)) * sizeof(T));
  }
  auto tile_in = [&](const T* X, T* lx, int k0) __attribute__((always_inline)) {
    if (k0 + kTile <= a.Nk) {
      const char* g = reinterpret_cast<const char*>(X + (size_t)k0 * D);
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        unsigned o = toff[i];
        asm volatile("" : "+v"(o));
        global_to_lds16(g + o, &lx[(gw * C::LPW + i) * 64 * 8]);
      }
    } else {
      load_tile<D, T>(X, lx, k0, a.Nk, gw, lane);
    }
  };
  auto issue = [&](int t, T* lk, T* lv) __attribute__((always_inline)) {
    tile_in(K, lk, t * kTile);
    tile_in(V, lv, t * kTile);
  };

  const LdsOff<D, T> lo0(lane);
  f32x16_t s[2], dp[2];
  v8 dsf[4];

  auto phase_mfma = [&](int t, auto do_dq, auto do_sdp, const T* kp, const T* kc, const T* vc, T* kn, T* vn)
      __attribute__((always_inline)) {
    LdsOff<D, T> lo = lo0;
    lo.opaque();
    if (group_a && t + 1 < T_) issue(t + 1, kn, vn);
    if constexpr (decltype(do_dq)::value) {
      // dQ^T += K^T dS^T of tile t - 1 (transposing reads of its K tile)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] = Mma<T>::mma(tr_frag_o<D, T>(kp, lo, g, db), dsf[g], acc[db]);
    }
    if constexpr (decltype(do_sdp)::value) {
      // S^T = K Q^T and dP^T - D = V dO^T - D of tile t (the dP accumulator starts at -D)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = 0.f;
          dp[kb][r] = nDr;
        }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = Mma<T>::mma(row_frag_o<D, T>(kc, lo, kb, ks), qf[ks], s[kb]);
          dp[kb] = Mma<T>::mma(row_frag_o<D, T>(vc, lo, kb, ks), dof[ks], dp[kb]);
        }
    }
    if constexpr (decltype(do_dq)::value && decltype(do_sdp)::value) dq_pp_order<6, 0>();
    __syncthreads();
  };

  auto phase_valu = [&](int t) __attribute__((always_inline)) {
    // per 16-key step g: P^T = exp(S - L), dS^T = P^T (dP^T - D); only a tile holding a key past
    // the wave's first row's last visible key takes the per-key mask (a wave-uniform test)
    auto grads = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kb = g >> 1;
        float ds[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * (g & 1) + i;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, -L2));
          if constexpr (decltype(masked)::value) {
            if (t * kTile + kb * 32 + acc_row(r, hf) > last_key) p = 0.f;
          }
          ds[i] = p * dp[kb][r];
        }
        dsf[g] = pack8<T>(ds);
      }
    };
    if ((t + 1) * kTile - 1 > wave_last_key) grads(std::true_type());
    else grads(std::false_type());
    if (group_a) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // prologue: tile 0 resident; group B then sits out one phase
  if (group_a && T_ > 0) {
    issue(0, lds_k0, lds_v0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (!group_a) __syncthreads();

  // Tile t reads buffers t % 3 and (t + 2) % 3 (tile t - 1's K, transposed) and loads into
  // (t + 1) % 3: tile 0 (S / dP only), the steady tiles unrolled by three, then the last dQ.
  const std::true_type yes;
  const std::false_type no;
  if (T_ > 0) {
    phase_mfma(0, no, yes, lds_k2, lds_k0, lds_v0, lds_k1, lds_v1);
    phase_valu(0);
  }
  for (int t = 1; t < T_; t += 3) {
    phase_mfma(t, yes, yes, lds_k0, lds_k1, lds_v1, lds_k2, lds_v2);
    phase_valu(t);
    if (t + 1 < T_) {
      phase_mfma(t + 1, yes, yes, lds_k1, lds_k2, lds_v2, lds_k0, lds_v0);
      phase_valu(t + 1);
    }
    if (t + 2 < T_) {
      phase_mfma(t + 2, yes, yes, lds_k2, lds_k0, lds_v0, lds_k1, lds_v1);
      phase_valu(t + 2);
    }
  }
  if (T_ == 0) phase_mfma(0, no, no, lds_k0, lds_k0, lds_v0, lds_k1, lds_v1);
  else if ((T_ - 1) % 3 == 0) phase_mfma(T_, yes, no, lds_k0, lds_k1, lds_v1, lds_k2, lds_v2);
  else if ((T_ - 1) % 3 == 1) phase_mfma(T_, yes, no, lds_k1, lds_k2, lds_v2, lds_k0, lds_v0);
  else phase_mfma(T_, yes, no, lds_k2, lds_k0, lds_v0, lds_k1, lds_v1);
  if (group_a) __syncthreads();

  if (row < a.Nq) {
    float* out = a.dq + (head * (size_t)a.Nq + row) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = db * 32 + 8 * g4 + 4 * hf;
        f32x4_t x = {a.scale * acc[db][4 * g4], a.scale * acc[db][4 * g4 + 1], a.scale * acc[db][4 * g4 + 2],
                     a.scale * acc[db][4 * g4 + 3]};
        *reinterpret_cast<f32x4_t*>(out + dd) = x;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV at d = 128, ping-pong with 16 keys per wave. With 32 keys per wave the dK, dV
// accumulators and the K, V operands alone take 256 registers, so each SIMD runs one wave
// and its matrix core waits whenever that wave computes P and dS. Here a wave owns 16 keys on
// 16x16x32 MFMAs (about 200 registers), and the 8 waves of a workgroup (128 keys of one (b, h_kv))
// run in two groups in opposite matrix-core / VALU phases as in bwd_dkdv_pp_kernel:
//   MFMA phase of step t: dV^T += dO^T P and dK^T += Q^T dS of step t - 1, then S and dP - D of
//     step t (and this step's L into registers);
//   VALU phase of step t: P and dS of step t, rounded as the next phase's B operands; group A also
//     stages step t's dO^T / Q^T operands (below).
// Per 64-row query tile and wave (query rows m, the wave's keys n):
//   * S = Q K^T and dP - D = dO V^T - D: 4 blocks of 16 rows x 16 keys; A = Q (dO) rows read from
//     LDS (row 16 qb + lane % 16, dims 32 ks + 8 (lane / 16) + [0, 8)), B = K (V) in registers. A
//     lane holds rows 16 qb + 4 g + r (g = lane / 16, r < 4) of its key lane % 16.
//   * dV^T += dO^T P, dK^T += Q^T dS: M = 16 dims, N = the 16 keys, K = 32 rows per k-step kk, in
//     the k order that gives lane group g the rows 32 kk + 4 g + [0, 4) and 32 kk + 16 + 4 g +
//     [0, 4): exactly the P (dS) values the lane holds, so the B operand is its own registers.
//     Output block db holds dims 16 db + 4 g + r of key lane % 16.
//   * Those A operands (dO^T, Q^T in that row order) are the same for all 8 waves: group A builds
//     them once per tile in its VALU phase (two transposing LDS reads per fragment, wave gw the
//     dim blocks 2 gw, 2 gw + 1), and every wave reads each with one 16-byte read. Read per wave
//     with transposing reads, they were three quarters of the tile's LDS time.
// Buffers (two of each): group A loads step t + 1's tiles and row vectors at the top of its MFMA
// phase t, waits for them at the end of its VALU phase t; step t's tiles are read in the interval
// of A's MFMA phase t (rows, A) and the next (rows, B; staging, A), its fragments in MFMA phases
// t + 1 of both groups, and its L and -D rows in the MFMA phases t; each buffer is written only in
// an interval after the barrier that ends the last one reading it.
// ---------------------------------------------------------------------------------------------
constexpr int k16Waves = 8;
constexpr int k16Own = k16Waves * 16;            // keys per workgroup (= kOwn)

template <typename T> struct Mma16;
template <> struct Mma16<__bf16> {
  static __device__ __forceinline__ f32x4_t mma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma16<_Float16> {
  static __device__ __forceinline__ f32x4_t mma(f16x8_t a, f16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Issue order of a full MFMA phase of bwd_dkdv16_kernel (32 dV / dK MFMAs fed by one fragment read
// each, then the 8 reads of -D and L, then 32 S / dP MFMAs fed by one row read each): the reads of
// the MFMA PD positions ahead go before each MFMA. In the compiler's own order each MFMA waited
// for the read just before it, so LDS latency showed on almost every one.
__host__ __device__ constexpr int pp16_reads_needed(int i) { return i < 32 ? i + 1 : i + 9; }
template <int PD, int I>
__device__ __forceinline__ void dkdv16_order() {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NM = 64;
  constexpr int kMfma = 0x008, kDsRead = 0x100;  // sched_group_barrier instruction classes
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(kDsRead, pp16_reads_needed(PD), 0);
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    constexpr int a = pp16_reads_needed(I + PD < NM ? I + PD : NM - 1);
    constexpr int b = pp16_reads_needed(I + 1 + PD < NM ? I + 1 + PD : NM - 1);
    if constexpr (b > a) __builtin_amdgcn_sched_group_barrier(kDsRead, b - a, 0);
    dkdv16_order<PD, I + 1>();
  }
#endif
}

template <typename T, bool CAUSAL>
__global__ __launch_bounds__(k16Waves * 64, 1) void bwd_dkdv16_kernel(BwdArgs a, int n_ktiles) {
  constexpr int D = 128;
  typedef BCfg<D, T> C;
  typedef typename C::v8 v8;
  constexpr int TB = 16 * D * (int)sizeof(T);    // bytes of 16 tile rows
  __shared__ __attribute__((aligned(16))) T lds_q0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_q1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_do0[C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_do1[C::ELEMS];
  __shared__ __attribute__((aligned(16))) float lds_l0[kTile];
  __shared__ __attribute__((aligned(16))) float lds_l1[kTile];
  __shared__ __attribute__((aligned(16))) float lds_d0[kTile];
  __shared__ __attribute__((aligned(16))) float lds_d1[kTile];
  // staged A operands of a step: fragment (tensor, kk, db) = 64 lanes x 16 bytes at
  // ((tensor * 16 + kk * 8 + db) * 64 + lane) * 8, tensor 0 = dO^T, 1 = Q^T
  __shared__ __attribute__((aligned(16))) T lds_f0[32 * 64 * 8];
  __shared__ __attribute__((aligned(16))) T lds_f1[32 * 64 * 8];

  // work order: see the file header (dK, dV)
  int kt, rest;
  if constexpr (CAUSAL) {
    const int units = gridDim.x / n_ktiles;
    kt = (int)blockIdx.x / units;
    rest = (int)blockIdx.x % units;
  } else {
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    kt = wg % n_ktiles;
    rest = wg / n_ktiles;
  }
  const int hk = rest % a.H_kv;
  const int b = rest / a.H_kv;
  const int group = a.H / a.H_kv;
  const size_t kvh = (size_t)b * a.H_kv + hk;
  const T* __restrict__ K = static_cast<const T*>(a.k) + kvh * (size_t)a.Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + kvh * (size_t)a.Nk * D;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool group_a = wave < 4;
  const int gw = wave & 3;                       // wave index within its group (loads, staging: group A)
  const int n = lane & 15;
  const int g = lane >> 4;
  const int key = kt * k16Own + wave * 16 + n;   // this lane's key
  const int keyc = min(key, a.Nk - 1);

  // B operands of S and dP: K (V) row of this lane's key, dims 32 ks + 8 g + [0, 8)
  v8 kf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = *reinterpret_cast<const v8*>(K + (size_t)keyc * D + ks * 32 + g * 8);
    vf[ks] = *reinterpret_cast<const v8*>(V + (size_t)keyc * D + ks * 32 + g * 8);
  }
  const float c2 = a.scale_log2e;

  f32x4_t dk[8], dv[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) dk[db][r] = dv[db][r] = 0.f;

  const int n_rtiles = (a.Nq + kTile - 1) / kTile;
  int r_begin = 0;
  if constexpr (CAUSAL) r_begin = max(0, kt * k16Own - a.causal_off) / kTile;
  const int per_head = n_rtiles - r_begin;
  const int n_steps = per_head * group;          // (query head, row tile) pairs, head-major
  auto row0 = [&](int st) { return (r_begin + st % per_head) * kTile; };

  // Group A: a quarter of each tile per wave; wave 0 the lse rows, wave 1 the D rows.
  auto issue = [&](int st, T* lq, T* ldo, float* ll, float* ld) __attribute__((always_inline)) {
    const int h = hk * group + st / per_head;
    const int r0 = row0(st);
    const size_t head = (size_t)b * a.H + h;
    load_tile<D, T>(static_cast<const T*>(a.q) + head * (size_t)a.Nq * D, lq, r0, a.Nq, gw, lane);
    load_tile<D, T>(static_cast<const T*>(a.dout) + head * (size_t)a.Nq * D, ldo, r0, a.Nq, gw, lane);
    if (wave == 0) load_rowvec(a.lse + head * a.Nq, ll, r0, a.Nq, lane);
    if (wave == 1) load_rowvec(a.delta + head * a.Nq, ld, r0, a.Nq, lane);
  };
  // After the loads land (vmcnt(0) of the loading wave): lse * log2(e) (+inf past Nq), and -D.
  auto prep_rows = [&](float* ll, float* ld, int r0) __attribute__((always_inline)) {
    if (wave == 0) ll[lane] = r0 + lane < a.Nq ? ll[lane] * kLog2e : INFINITY;
    if (wave == 1) ld[lane] = -ld[lane];
  };

  // Byte offsets of this lane's LDS reads within a tile. Row read (S, dP): row n (+ 16 qb), chunk
  // 4 ks + g; the swizzle depends on row % 16 = n only. Transposing read for the staged fragment of
  // k-step kk, half h, block db (group A, db = 2 gw + j): source lane n gives rows 32 kk + 16 h +
  // 4 g + n / 4 (row % 16 = 4 g + n / 4), columns 16 db + 4 (n % 4) + [0, 4).
  unsigned roff[4], toff[2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    roff[ks] = (unsigned)((n * D + (((4 * ks + g) ^ swz128(n)) << 3)) * sizeof(T));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tr = 4 * g + (n >> 2);
    const int col = 16 * (2 * gw + j) + 4 * (n & 3);
    toff[j] = (unsigned)((tr * D + (((col >> 3) ^ swz128(tr)) << 3) + (col & 7)) * sizeof(T));
  }

  f32x4_t s[4], dp[4];
  f32x4_t Lr[4];                                 // this step's lse * log2(e) of the lane's rows
  v8 pf[2], dsf[2];

  // do_dkdv / do_sdp are compile-time flags (std::true_type / std::false_type)
  auto phase_mfma = [&](int t, auto do_dkdv, auto do_sdp, const T* fprev, const T* qc, const T* doc,
                        const float* lc, const float* dc, T* qn, T* don, float* ln, float* dn)
      __attribute__((always_inline)) {
    unsigned ro[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ro[i] = roff[i];
      asm volatile("" : "+v"(ro[i]));
    }
    if (group_a && t + 1 < n_steps) issue(t + 1, qn, don, ln, dn);
    if constexpr (decltype(do_dkdv)::value) {
      // dV^T += dO^T P and dK^T += Q^T dS of step t - 1 (its staged fragments)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const v8 dof = *reinterpret_cast<const v8*>(&fprev[((kk * 8 + db) * 64 + lane) * 8]);
          const v8 qf = *reinterpret_cast<const v8*>(&fprev[((16 + kk * 8 + db) * 64 + lane) * 8]);
          dv[db] = Mma16<T>::mma(dof, pf[kk], dv[db]);
          dk[db] = Mma16<T>::mma(qf, dsf[kk], dk[db]);
        }
    }
    if constexpr (decltype(do_sdp)::value) {
      // S and dP - D of step t (the dP accumulator starts at -D of rows 16 qb + 4 g + r)
      const char* bq = reinterpret_cast<const char*>(qc);
      const char* bdo = reinterpret_cast<const char*>(doc);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        s[qb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        dp[qb] = *reinterpret_cast<const f32x4_t*>(&dc[16 * qb + 4 * g]);
        Lr[qb] = *reinterpret_cast<const f32x4_t*>(&lc[16 * qb + 4 * g]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          const int o = ro[ks] + qb * TB;
          s[qb] = Mma16<T>::mma(*reinterpret_cast<const v8*>(bq + o), kf[ks], s[qb]);
          dp[qb] = Mma16<T>::mma(*reinterpret_cast<const v8*>(bdo + o), vf[ks], dp[qb]);
        }
    }
    // reads 16 MFMAs ahead (kernel time at the d = 128 backward workload: 1.24 ms at 6, 1.20 at 16)
    if constexpr (decltype(do_dkdv)::value && decltype(do_sdp)::value) dkdv16_order<16, 0>();
    __syncthreads();
  };

  auto phase_valu = [&](int t, const T* qc, const T* doc, T* fcur, float* ln, float* dn)
      __attribute__((always_inline)) {
    if (group_a) {
      // step t's dO^T / Q^T fragments of dim blocks 2 gw, 2 gw + 1
      unsigned to[2] = {toff[0], toff[1]};
      asm volatile("" : "+v"(to[0]), "+v"(to[1]));
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const char* bx = reinterpret_cast<const char*>(tq ? qc : doc);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int o1 = to[j] + 2 * kk * TB;
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(bx + o1));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(bx + o1 + TB));
            const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
            const u32x4_t x = {l2[0], l2[1], h2[0], h2[1]};
            *reinterpret_cast<u32x4_t*>(&fcur[((tq * 16 + kk * 8 + 2 * gw + j) * 64 + lane) * 8]) = x;
          }
      }
    }
    // P = 2^(s c - L log2 e) (0 past Nq through L = +inf), dS = P (dP - D). Under the causal mask
    // the row 16 qb + 4 g + r of the tile sees this lane's key when 16 qb + 4 g + r >= key -
    // causal_off - r0.
    int lim = 0;
    if constexpr (CAUSAL) lim = key - a.causal_off - row0(t) - 4 * g;
    float p[4][4], ds[4][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c2, -Lr[qb][r]));
        if constexpr (CAUSAL) {
          if (16 * qb + r < lim) x = 0.f;
        }
        p[qb][r] = x;
        ds[qb][r] = x * dp[qb][r];
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[kk][i] = (T)p[2 * kk][i];
        pf[kk][4 + i] = (T)p[2 * kk + 1][i];
        dsf[kk][i] = (T)ds[2 * kk][i];
        dsf[kk][4 + i] = (T)ds[2 * kk + 1][i];
      }
    if (group_a) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (t + 1 < n_steps) prep_rows(ln, dn, row0(t + 1));
    }
    __syncthreads();
  };

  // prologue: step 0's tiles resident and prepared; group B then sits out one phase
  if (group_a && n_steps > 0) {
    issue(0, lds_q0, lds_do0, lds_l0, lds_d0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    prep_rows(lds_l0, lds_d0, row0(0));
  }
  __syncthreads();
  if (!group_a) __syncthreads();

  // Step t reads tiles and rows t % 2 and fragments (t - 1) % 2, stages fragments t % 2 and loads
  // into (t + 1) % 2. Every wave takes the same number of barriers.
  const std::true_type yes;
  const std::false_type no;
  if (n_steps > 0) {
    phase_mfma(0, no, yes, lds_f1, lds_q0, lds_do0, lds_l0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
    phase_valu(0, lds_q0, lds_do0, lds_f0, lds_l1, lds_d1);
  }
  for (int t = 1; t < n_steps; t += 2) {
    phase_mfma(t, yes, yes, lds_f0, lds_q1, lds_do1, lds_l1, lds_d1, lds_q0, lds_do0, lds_l0, lds_d0);
    phase_valu(t, lds_q1, lds_do1, lds_f1, lds_l0, lds_d0);
    if (t + 1 < n_steps) {
      phase_mfma(t + 1, yes, yes, lds_f1, lds_q0, lds_do0, lds_l0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
      phase_valu(t + 1, lds_q0, lds_do0, lds_f0, lds_l1, lds_d1);
    }
  }
  if (n_steps == 0) phase_mfma(0, no, no, lds_f0, lds_q0, lds_do0, lds_l0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
  else if ((n_steps - 1) % 2 == 0) phase_mfma(n_steps, yes, no, lds_f0, lds_q1, lds_do1, lds_l1, lds_d1, lds_q0, lds_do0, lds_l0, lds_d0);
  else phase_mfma(n_steps, yes, no, lds_f1, lds_q0, lds_do0, lds_l0, lds_d0, lds_q1, lds_do1, lds_l1, lds_d1);
  if (group_a) __syncthreads();

  if (key < a.Nk) {
    float* outk = a.dk + (kvh * (size_t)a.Nk + key) * D;
    float* outv = a.dv + (kvh * (size_t)a.Nk + key) * D;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int dd = 16 * db + 4 * g;
      f32x4_t xk = {a.scale * dk[db][0], a.scale * dk[db][1], a.scale * dk[db][2], a.scale * dk[db][3]};
      *reinterpret_cast<f32x4_t*>(outk + dd) = xk;
      *reinterpret_cast<f32x4_t*>(outv + dd) = dv[db];
    }
  }
}

template <int D, typename T>
hipError_t launch_typed(const BwdArgs& a, hipStream_t s) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  const long long nd = (rows + (256 / (D / 8)) - 1) / (256 / (D / 8));
  const int n_qtiles = (a.Nq + kOwn - 1) / kOwn;
  const int n_ktiles = (a.Nk + kOwn - 1) / kOwn;
  const long long nq = (long long)n_qtiles * a.H * a.B;
  const long long nk = (long long)n_ktiles * a.H_kv * a.B;
  if (nd > 0x7fffffffLL || nq > 0x7fffffffLL || nk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  BwdArgs args = a;
  if (rows > 0) {  // D first (the other two kernels read it; at d = 64 the dQ kernel computes it), dQ, dK dV
    hipError_t e = hipSuccess;
    if constexpr (D != 64) {
      long long r = rows;
      void* kargs[] = {&args, &r};
      e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_delta_kernel<D, T>), dim3((unsigned)nd), dim3(256),
                          kargs, 0, s);
      if (e != hipSuccess) return e;
    }
    if constexpr (D == 64) {  // ping-pong kernel: 256 query rows per workgroup
      int n = (a.Nq + kPpOwn - 1) / kPpOwn;
      const long long nqp = (long long)n * a.H * a.B;
      void* kargs2[] = {&args, &n};
      const void* k = a.causal ? reinterpret_cast<const void*>(&bwd_dq_pp_kernel<T, true>)
                               : reinterpret_cast<const void*>(&bwd_dq_pp_kernel<T, false>);
      e = hipLaunchKernel(k, dim3((unsigned)nqp), dim3(kPpWaves * 64), kargs2, 0, s);
    } else {
      int n = n_qtiles;
      void* kargs2[] = {&args, &n};
      const void* k = a.causal ? reinterpret_cast<const void*>(&bwd_dq_kernel<D, T, true>)
                               : reinterpret_cast<const void*>(&bwd_dq_kernel<D, T, false>);
      e = hipLaunchKernel(k, dim3((unsigned)nq), dim3(kBwdThreads), kargs2, 0, s);
    }
    if (e != hipSuccess) return e;
  }
  if (nk == 0) return hipSuccess;
  if constexpr (D == 64) {  // ping-pong kernel: 256 keys per workgroup
    int n = (a.Nk + kPpOwn - 1) / kPpOwn;
    const long long nkp = (long long)n * a.H_kv * a.B;
    void* kargs[] = {&args, &n};
    const void* k = a.causal ? reinterpret_cast<const void*>(&bwd_dkdv_pp_kernel<T, true>)
                             : reinterpret_cast<const void*>(&bwd_dkdv_pp_kernel<T, false>);
    return hipLaunchKernel(k, dim3((unsigned)nkp), dim3(kPpWaves * 64), kargs, 0, s);
  } else {  // d = 128: 16 keys per wave, two waves per SIMD (128 keys per workgroup, as kOwn)
    static_assert(k16Own == kOwn, "the d = 128 dK dV grid uses n_ktiles of kOwn keys");
    int n = n_ktiles;
    void* kargs[] = {&args, &n};
    const void* k = a.causal ? reinterpret_cast<const void*>(&bwd_dkdv16_kernel<T, true>)
                             : reinterpret_cast<const void*>(&bwd_dkdv16_kernel<T, false>);
    return hipLaunchKernel(k, dim3((unsigned)nk), dim3(k16Waves * 64), kargs, 0, s);
  }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, int in_dtype, hipStream_t s) {
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
