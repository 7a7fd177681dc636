// Tiled FlashAttention forward for bf16 / fp16 inputs on the gfx950 matrix cores.
//
// What is computed ("FlashAttention 简化版：Tiling + Online Softmax", §2.3 and §3.1): one
// workgroup owns a tile of query rows of one (b, h) and streams that head's keys past it in
// tiles of 64 keys. Per query row it keeps a running maximum, the running sum l and the fp32
// output accumulator; each key tile computes the scores, adds exp(s - m) to l and exp(s - m) V
// to the accumulator, and when the maximum grows, first scales l and the accumulator by
// exp(m_old - m_new). The accumulator is divided by l once at the end.
//
// How it maps onto CDNA4:
//  * Two wave groups in opposite phases. A CDNA SIMD overlaps matrix-core and VALU work only
//    across different waves: one wave's MFMAs run while another wave issues VALU instructions
//    (a probe of one wave interleaving independent MFMA and VALU instructions showed no
//    overlap at all). A workgroup therefore has 8 waves, two per SIMD: group A (waves 0-3)
//    and group B (waves 4-7), each owning its own query rows. Every tile is two phases per
//    wave -- an MFMA phase (PV of the previous tile, then S of this tile) and a VALU phase
//    (the softmax update of this tile) -- and group B runs one phase behind group A, held there
//    by workgroup barriers (at d = 128 one after every phase; at d = 64 one per tile, A's after
//    its VALU phase and B's after its MFMA phase). So at any time one wave of each SIMD is on
//    the matrix core while the other is on the VALU.
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
//    no LDS write instructions), two buffers each, issued by group A. At d = 128 the loads of
//    K(t+1) and V(t) start in A's VALU phase of tile t (no LDS reads there, so no MFMA phase
//    stalls on them). At d = 64 they start in A's MFMA phase and A's VALU phase re-lays the raw
//    V tile in LDS as ready-made PV operand fragments, so the MFMA phase reads V^T with plain
//    16-byte reads instead of transposing ones. Both tiles are XOR-swizzled in 16-byte chunks
//    (K: chunk ^ (row / 2) % 8, V: chunk ^ 2 * (row % 4)) so the operand
//    reads spread over the LDS banks. The swizzle is applied on the global side: the lane that
//    fills LDS chunk (row, c) fetches global chunk (row, c ^ f(row)).
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
//    Calls that want no row statistics skip the running max altogether: the reference only
//    moves when a tile's row sum of 2^(raw*c - m_ref) leaves [0, 2^threshold] (the first
//    tile always does), which bounds every p the same way.
//  * P is rounded to the input type (round to nearest even) only as the PV operand; l sums
//    the fp32 values ("CS349E 第 11 讲 01_online_softmax.py", demo 4).
//  * Query rows per wave: 64 at d = 64 (two 32-column MFMA blocks share every K/V operand read
//    from LDS), 32 at d = 128 (the accumulator doubles); 512 or 256 rows per workgroup.

#include "fa_internal.h"
#include "mfma_common.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kWaves = 8;                    // two groups of four, one wave of each per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kBC = 64;                      // keys per tile

template <int D, typename T, int NB_ = (D <= 64) ? 2 : 1>
struct Cfg {
  typedef typename Mma<T>::v8 v8;
  static constexpr int NB = NB_;                   // 32-query MFMA column blocks per wave
  static constexpr int BR = kWaves * NB * 32;      // query rows per workgroup
  static constexpr int KS = D / 16;                // 16-wide k steps of S^T = K Q^T
  static constexpr int DB = D / 32;                // 32-row blocks of O^T
  static constexpr int CH = D / 8;                 // 16-byte chunks per K/V row
  static constexpr int ELEMS = kBC * D;            // elements per K (or V) tile
  static constexpr int CPW = ELEMS / 8 / 4;        // 16-byte chunks each group-A wave moves per tensor
  static constexpr int LPW = CPW / 64;             // direct-to-LDS loads per group-A wave per tensor
  static_assert(LPW >= 1 && LPW * 64 * 4 * 8 == ELEMS, "tile / wave mismatch");
};

// Online-softmax state of one wave's query rows (one value per lane each).
template <int NB>
struct RowState {
  float mraw[NB];   // true running max of the raw dot products (exact-max form only)
  float m2ref[NB];  // exponent reference, base-2 units
  float lsum[NB];   // sum of 2^(raw*c - m2ref)
};


// HBM -> LDS of one 64-row K or V tile, one quarter per group-A wave (gw = 0..3, wave-uniform).
// Load i of a wave moves LDS chunks gw * CPW + 64 i + lane, i.e. tile rows r = 16 gw + (64 / CH) i
// + lane / CH, chunk lane % CH, fetched from global chunk (lane % CH) ^ swz(r). `off` holds those
// per-lane byte offsets within the tile (computed once, see load_offsets), so a full tile costs one
// load per 1024 bytes with a scalar base; a tile that runs past `kend` (ragged end) repeats the
// last key of the range instead, and its scores are masked.
template <int D, typename T, bool KT>
__device__ __forceinline__ void load_tile2(const T* __restrict__ X, T* lx, int key0, int kend, int gw, int lane,
                                           const unsigned (&off)[Cfg<D, T>::LPW]) {
  typedef Cfg<D, T> C;
  if (key0 + kBC <= kend) {
    const char* g = reinterpret_cast<const char*>(X + (size_t)key0 * D);
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      // an opaque copy keeps the offset 32-bit: the compiler would otherwise hoist 64-bit
      // per-lane addresses out of the tile loop and spill them where registers are short
      unsigned o = off[i];
      asm volatile("" : "+v"(o));
      global_to_lds16(g + o, &lx[(gw * C::CPW + i * 64) * 8]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int base = gw * C::CPW + i * 64;  // first LDS chunk of this load (wave-uniform)
    const int ci = base + lane;
    const int r = ci / C::CH, cpos = ci % C::CH;
    const int key = min(key0 + r, kend - 1);
    const int gch = cpos ^ (KT ? swzk(r) : swzv(r));
    global_to_lds16(X + (size_t)key * D + (gch << 3), &lx[base * 8]);
  }
}

// Per-lane byte offsets of load_tile2's full-tile loads.
template <int D, typename T, bool KT>
__device__ __forceinline__ void load_offsets(int gw, int lane, unsigned (&off)[Cfg<D, T>::LPW]) {
  typedef Cfg<D, T> C;
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int ci = gw * C::CPW + i * 64 + lane;
    const int r = ci / C::CH, cpos = ci % C::CH;
    const int gch = cpos ^ (KT ? swzk(r) : swzv(r));
    off[i] = (unsigned)((r * D + (gch << 3)) * sizeof(T));
  }
}

// S^T = K Q^T for one tile: rows = 64 keys (two 32-blocks), columns = this wave's queries.
template <int D, typename T, int NB>
__device__ __forceinline__ void s_tile(const T* __restrict__ lk, const typename Cfg<D, T, NB>::v8 (&qf)[NB][Cfg<D, T, NB>::KS],
                                       f32x16_t (&s)[NB][2], int lane) {
  typedef Cfg<D, T, NB> C;
  typedef typename C::v8 v8;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
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
      const v8 kf = *reinterpret_cast<const v8*>(&lk[r * D + ((ch ^ swzk(r)) << 3)]);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) s[nb][kb] = Mma<T>::mma(kf, qf[nb][ks], s[nb][kb]);
    }
  }
}

// O^T += V^T P^T for one tile: 16 keys per MFMA step, V^T read transposed from row-major LDS.
template <int D, typename T, int NB>
__device__ __forceinline__ void pv_tile(const T* __restrict__ lv, const typename Cfg<D, T, NB>::v8 (&pf)[NB][4],
                                        f32x16_t (&acc)[NB][Cfg<D, T, NB>::DB], int lane) {
  typedef Cfg<D, T, NB> C;
  typedef typename C::v8 v8;
  const int hf = lane >> 5;
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
      const int off1 = row1 * D + (((col >> 3) ^ swzv(row1)) << 3) + (col & 7);
      const int off2 = (row1 + 8) * D + (((col >> 3) ^ swzv(row1 + 8)) << 3) + (col & 7);
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&lv[off1]);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&lv[off2]);
      const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
      const u32x4_t packed = {lo2[0], lo2[1], hi2[0], hi2[1]};
      const v8 vf = __builtin_bit_cast(v8, packed);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[nb][db] = Mma<T>::mma(vf, pf[nb][g], acc[nb][db]);
    }
  }
}

// Stage V(t) as ready-made MFMA A operands: fragment (g, db) of a tile is the 16 bytes every
// lane feeds the PV MFMA of 16-key step g and 32-dim block db -- V^T[dim][keys of step g] in the
// key order of the P operand -- stored lane after lane, so each wave later reads it with one
// conflict-free 16-byte read. The transposition itself (two ds_read_b64_tr_b16 per fragment)
// happens once per workgroup and tile instead of once per wave. Group-A wave gw stages
// fragments gw, gw + 4, ...
template <int D, typename T>
__device__ __forceinline__ void stage_v(const T* __restrict__ lv, T* vfrag, int gw, int lane) {
  constexpr int DB = D / 32;
  const int hf = lane >> 5;
  const int tj = lane & 15;
  const int ti = tj >> 2;
  const int tq = tj & 3;
  const int tgb = (lane >> 4) & 1;
#pragma unroll
  for (int f = gw; f < (kBC / 16) * DB; f += 4) {
    const int g = f / DB, db = f % DB;
    const int row1 = 16 * g + 4 * hf + ti;
    const int col = db * 32 + tgb * 16 + tq * 4;
    const int off1 = row1 * D + (((col >> 3) ^ swzv(row1)) << 3) + (col & 7);
    const int off2 = (row1 + 8) * D + (((col >> 3) ^ swzv(row1 + 8)) << 3) + (col & 7);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&lv[off1]);
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&lv[off2]);
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
    const u32x4_t packed = {lo2[0], lo2[1], hi2[0], hi2[1]};
    *reinterpret_cast<u32x4_t*>(&vfrag[(f * 64 + lane) * 8]) = packed;
  }
}

// O^T += V^T P^T for one tile from staged fragments: one 16-byte LDS read per MFMA A operand.
template <int D, typename T, int NB>
__device__ __forceinline__ void pv_staged(const T* __restrict__ vfrag, const typename Cfg<D, T, NB>::v8 (&pf)[NB][4],
                                          f32x16_t (&acc)[NB][Cfg<D, T, NB>::DB], int lane) {
  typedef Cfg<D, T, NB> C;
  typedef typename C::v8 v8;
#pragma unroll
  for (int g = 0; g < kBC / 16; ++g)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const v8 vf = *reinterpret_cast<const v8*>(&vfrag[((g * C::DB + db) * 64 + lane) * 8]);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[nb][db] = Mma<T>::mma(vf, pf[nb][g], acc[nb][db]);
    }
}

// Exponentials of one block's scores: p = 2^(s c2 - ref), and with TAIL 0 for the keys at or
// past the row's limit; returns the row sum. At d = 64 the P operands are also rounded here
// (measured 1.5 % faster there; at d = 128 rounding after the softmax update measured 2 % faster).
// Key index (within the tile, minus 4 hf) of value i = 16 kb + r of a 64-key block: key
// 32 kb + 8 (r / 4) + 4 hf + r % 4 is masked when tail_key(i) >= limh = lim - 4 hf.
__host__ __device__ constexpr int tail_key(int i) { return 32 * (i >> 4) + 8 * ((i & 15) >> 2) + (i & 3); }

template <int D, typename T, bool TAIL>
__device__ __forceinline__ float exps_block(const f32x16_t (&s)[2], float ref, float c2, float (&p)[32],
                                           typename Cfg<D, T>::v8 (&pf)[4], int limh) {
#pragma unroll
  for (int i = 0; i < 32; ++i) p[i] = __builtin_fmaf(s[i >> 4][i & 15], c2, -ref);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float x = __builtin_amdgcn_exp2f(p[i]);
    if constexpr (TAIL) {
      if (tail_key(i) >= limh) x = 0.f;
    }
    p[i] = x;
  }
  float r4[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
  for (int i = 4; i < 32; ++i) r4[i & 3] += p[i];
  if constexpr (D == 64) {
#pragma unroll
    for (int i = 0; i < 32; ++i) pf[i >> 3][i & 7] = (T)p[i];
  }
  return xhalf_sum((r4[0] + r4[1]) + (r4[2] + r4[3]));
}

// Maximum of one block's 32 scores (the masked ones as -inf): two chains of three-input maxima,
// 16 instructions (chains of fmaxf took 63: 31 maxima and 32 NaN-quieting copies).
template <bool TAIL>
__device__ __forceinline__ float max_block(const f32x16_t (&s)[2], int limh) {
  auto val = [&](int i) -> float {
    const float x = s[i >> 4][i & 15];
    return (TAIL && tail_key(i) >= limh) ? -INFINITY : x;
  };
  float m0 = max3f(val(0), val(1), val(2)), m1 = max3f(val(3), val(4), val(5));
#pragma unroll
  for (int i = 6; i < 30; i += 4) {
    m0 = max3f(m0, val(i), val(i + 1));
    m1 = max3f(m1, val(i + 2), val(i + 3));
  }
  return xhalf_max(max3f(m0, m1, max2f(val(30), val(31))));
}

// Move the exponent reference of the rows with `need` to `target`, scaling l and the block's
// accumulator by 2^(ref_old - ref_new). Wave-uniform branch: only some tiles move some rows.
template <int D>
__device__ __forceinline__ bool move_ref(bool need, float target, bool first, float& m2ref, float& lsum,
                                         f32x16_t (&acc)[D / 32]) {
  if (__ballot(need)) {
    asm volatile("" ::: "memory");
    const float ref = need ? target : m2ref;
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(m2ref - ref);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    m2ref = ref;
    return true;
  }
  return false;
}

// Softmax update of one tile for one 32-query block, given the tile scores s (raw dot
// products) of that block: moves the exponent reference when needed (scaling l and the block's
// accumulator), writes P as PV operands and adds its row sum to l.
//   FAST = false: exact running max, reference moves when the tile max exceeds it by > tau.
//   FAST = true:  no running max; reference moves when the tile's row sum leaves [0, 2^tau].
// TAIL: keys with tail_key >= limh (per lane) are masked (p = 0, and no part of the maximum).
template <int D, typename T, bool FAST, bool TAIL>
__device__ __forceinline__ void softmax_block(const f32x16_t (&s)[2], float& mraw, float& m2ref, float& lsum,
                                              typename Cfg<D, T>::v8 (&pf)[4], f32x16_t (&acc)[Cfg<D, T>::DB],
                                              bool first, float c2, float tau, float bound, int limh = 0) {
  float p[32];
  float rs;
  if constexpr (FAST) {
    rs = exps_block<D, T, TAIL>(s, m2ref, c2, p, pf, limh);
    const bool trig = first || !(rs <= bound);
    if (__ballot(trig)) {
      const float mx2 = max_block<TAIL>(s, limh) * c2;
      if (move_ref<D>(trig, first ? mx2 : fmaxf(m2ref, mx2), first, m2ref, lsum, acc))
        rs = exps_block<D, T, TAIL>(s, m2ref, c2, p, pf, limh);
    }
  } else {
    const float mx = max_block<TAIL>(s, limh);
    mraw = fmaxf(mraw, mx);
    const float mx2 = mx == -INFINITY ? -INFINITY : mx * c2;  // a wholly masked tile (scale may be 0)
    move_ref<D>(first || (mx2 > m2ref + tau), mx2, first, m2ref, lsum, acc);
    rs = exps_block<D, T, TAIL>(s, m2ref, c2, p, pf, limh);
  }
  lsum += rs;
  if constexpr (D != 64) {
#pragma unroll
    for (int i = 0; i < 32; ++i) pf[i >> 3][i & 7] = (T)p[i];
  }
}

// Issue order of the d = 128 MFMA phase (PV of the previous tile, then S): 32 MFMAs, the first
// 16 fed by two transposing V reads each, the last 16 by one K read each. The reads of the MFMA
// PD positions ahead are issued before each MFMA, so LDS latency hides behind matrix-core work
// (the compiler's own order fetches one MFMA group ahead; PD = 2 measured 6 % faster). At
// d = 64 the compiler's order measured as fast as any fixed one.
__host__ __device__ constexpr int pv_s_reads_before(int i) { return i < 16 ? 2 * i : 32 + (i - 16); }
template <int PD, int I>
__device__ __forceinline__ void mfma_phase_order_d128() {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NM = 32;
  constexpr int kMfma = 0x008, kDsRead = 0x100;  // sched_group_barrier instruction classes
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(kDsRead, pv_s_reads_before(PD), 0);
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    constexpr int a = pv_s_reads_before(I + PD < NM ? I + PD : NM);
    constexpr int b = pv_s_reads_before(I + 1 + PD < NM ? I + 1 + PD : NM);
    if constexpr (b > a) __builtin_amdgcn_sched_group_barrier(kDsRead, b - a, 0);
    mfma_phase_order_d128<PD, I + 1>();
  }
#endif
}

// The d = 64 MFMA phase (PV of the previous tile from staged V fragments, then S of this tile) as
// a fixed instruction sequence: 8 groups of 2 LDS reads + 4 MFMAs, the reads of each group issued
// between the MFMAs of the group before. A probe of one wave issuing 32x32x16 MFMAs with LDS
// operands measured 43.5 cycles per MFMA in the compiler's order (two reads, wait for both,
// four MFMAs: nothing in flight during the wait) and 35.6 in this one (32 is the matrix-core
// rate). Reads, waits and MFMAs are inline asm so that the order is kept. Each wait takes the
// registers it guards as in-out operands, so no MFMA that reads them can be placed before it.
// The compiler does not see the MFMA latency inside asm, so the sequence ends with the wait
// states a VALU read of an MFMA result needs, in an asm statement that takes every S and PV
// accumulator as an in-out operand: no instruction that reads or writes them can be placed
// between the last MFMA and the end of those wait states. (Written with compiler-visible
// MFMAs and LDS loads instead, the compiler must assume the loads may alias the direct-to-LDS
// tile loads in flight and waits for those before the first read: 2.4 % slower.)
#define FA_RD(dst, addr, off) asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(dst) : "v"(addr))
#define FA_WAIT0(x, y) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x), "+v"(y))
#define FA_MF_BF16(acc, a, b) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define FA_MF0_BF16(acc, a, b) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b))
#define FA_MF_F16(acc, a, b) asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define FA_MF0_F16(acc, a, b) asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b))

template <typename T>
__device__ __forceinline__ void mfma_acc(f32x16_t& acc, const typename Mma<T>::v8& a, const typename Mma<T>::v8& b) {
  if constexpr (std::is_same<T, __bf16>::value) FA_MF_BF16(acc, a, b); else FA_MF_F16(acc, a, b);
}
template <typename T>
__device__ __forceinline__ void mfma_zero(f32x16_t& acc, const typename Mma<T>::v8& a, const typename Mma<T>::v8& b) {
  if constexpr (std::is_same<T, __bf16>::value) FA_MF0_BF16(acc, a, b); else FA_MF0_F16(acc, a, b);
}

// vaddr: LDS byte address of this lane's first staged V fragment (buffer + lane * 16);
// kaddr[ks]: LDS byte address of this lane's K chunk of k-step ks in key block 0 (block 1 is +4096).
template <typename T>
__device__ __forceinline__ void mfma_phase_d64(unsigned vaddr, const unsigned (&kaddr)[4],
                                               const typename Mma<T>::v8 (&pf)[2][4], const typename Mma<T>::v8 (&qf)[2][4],
                                               f32x16_t (&acc)[2][2], f32x16_t (&s)[2][2]) {
  typedef typename Mma<T>::v8 v8;
  v8 r0a, r0b, r1a, r1b;
  // PV: group g = fragments (g, db 0) and (g, db 1) at (2g + db) * 1024
  FA_RD(r0a, vaddr, 0); FA_RD(r0b, vaddr, 1024);
  FA_WAIT0(r0a, r0b);
  mfma_acc<T>(acc[0][0], r0a, pf[0][0]); FA_RD(r1a, vaddr, 2048);
  mfma_acc<T>(acc[1][0], r0a, pf[1][0]); mfma_acc<T>(acc[0][1], r0b, pf[0][0]); FA_RD(r1b, vaddr, 3072);
  mfma_acc<T>(acc[1][1], r0b, pf[1][0]);
  FA_WAIT0(r1a, r1b);
  mfma_acc<T>(acc[0][0], r1a, pf[0][1]); FA_RD(r0a, vaddr, 4096);
  mfma_acc<T>(acc[1][0], r1a, pf[1][1]); mfma_acc<T>(acc[0][1], r1b, pf[0][1]); FA_RD(r0b, vaddr, 5120);
  mfma_acc<T>(acc[1][1], r1b, pf[1][1]);
  FA_WAIT0(r0a, r0b);
  mfma_acc<T>(acc[0][0], r0a, pf[0][2]); FA_RD(r1a, vaddr, 6144);
  mfma_acc<T>(acc[1][0], r0a, pf[1][2]); mfma_acc<T>(acc[0][1], r0b, pf[0][2]); FA_RD(r1b, vaddr, 7168);
  mfma_acc<T>(acc[1][1], r0b, pf[1][2]);
  FA_WAIT0(r1a, r1b);
  mfma_acc<T>(acc[0][0], r1a, pf[0][3]); FA_RD(r0a, kaddr[0], 0);
  mfma_acc<T>(acc[1][0], r1a, pf[1][3]); mfma_acc<T>(acc[0][1], r1b, pf[0][3]); FA_RD(r0b, kaddr[0], 4096);
  mfma_acc<T>(acc[1][1], r1b, pf[1][3]);
  // S: group ks = K chunks of key blocks 0 and 1
  FA_WAIT0(r0a, r0b);
  mfma_zero<T>(s[0][0], r0a, qf[0][0]); FA_RD(r1a, kaddr[1], 0);
  mfma_zero<T>(s[1][0], r0a, qf[1][0]); mfma_zero<T>(s[0][1], r0b, qf[0][0]); FA_RD(r1b, kaddr[1], 4096);
  mfma_zero<T>(s[1][1], r0b, qf[1][0]);
  FA_WAIT0(r1a, r1b);
  mfma_acc<T>(s[0][0], r1a, qf[0][1]); FA_RD(r0a, kaddr[2], 0);
  mfma_acc<T>(s[1][0], r1a, qf[1][1]); mfma_acc<T>(s[0][1], r1b, qf[0][1]); FA_RD(r0b, kaddr[2], 4096);
  mfma_acc<T>(s[1][1], r1b, qf[1][1]);
  FA_WAIT0(r0a, r0b);
  mfma_acc<T>(s[0][0], r0a, qf[0][2]); FA_RD(r1a, kaddr[3], 0);
  mfma_acc<T>(s[1][0], r0a, qf[1][2]); mfma_acc<T>(s[0][1], r0b, qf[0][2]); FA_RD(r1b, kaddr[3], 4096);
  mfma_acc<T>(s[1][1], r0b, qf[1][2]);
  FA_WAIT0(r1a, r1b);
  mfma_acc<T>(s[0][0], r1a, qf[0][3]);
  mfma_acc<T>(s[1][0], r1a, qf[1][3]); mfma_acc<T>(s[0][1], r1b, qf[0][3]);
  mfma_acc<T>(s[1][1], r1b, qf[1][3]);
  // On gfx950 a VALU or memory access of a 16-pass MFMA's result needs passes + 4 = 20 wait
  // states after the MFMA; these are 20 (s_nop N waits N + 1). The accumulators are operands, so
  // every access of them follows (tests/test_mfma_asm_hazards.py checks the built code).
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]), "+v"(acc[0][0]), "+v"(acc[0][1]),
                 "+v"(acc[1][0]), "+v"(acc[1][1])::"memory");
}

template <int D, typename T, bool FAST, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_mfma_kernel(FwdArgs a, int n_qtiles) {
  typedef Cfg<D, T> C;
  typedef typename C::v8 v8;
  constexpr int NB = C::NB;

  // At d = 64 group A also re-lays each V tile as ready-made PV operand fragments (see stage_v):
  // its VALU phase has room for it, and it takes the transposing reads off the MFMA phase. At
  // d = 128 the softmax phase is the shorter one and the plain transposing reads measured faster.
  constexpr bool STAGE = D == 64;
  // Barriers per tile. Two: one after each phase, for both groups. One (d = 64): group B's after
  // its MFMA phase, group A's after its VALU phase, so between two barriers A runs MFMA(t) then
  // VALU(t) and B runs VALU(t - 1) then MFMA(t), and neither waits for the other mid-tile. The
  // buffer rules below hold either way: a buffer is written only in a barrier interval in which no
  // wave reads it. At d = 64 one barrier measured 2 % faster; at d = 128 (loads issued in A's
  // VALU phase) 4 % slower.
  constexpr bool ONE_BAR = STAGE;
  __shared__ __attribute__((aligned(16))) T lds_k[2][C::ELEMS];
  __shared__ __attribute__((aligned(16))) T lds_v[2][C::ELEMS];                          // raw V tiles
  __shared__ __attribute__((aligned(16))) T lds_vf[STAGE ? 2 : 1][STAGE ? C::ELEMS : 8];  // staged fragments

  // ---- work item: (query tile, split, h, b) ----
  // Without the mask: the query tile varies fastest, and the XCD remap keeps a head's tiles on one
  // XCD (one L2). Under the causal mask later query tiles see more keys and are handed out first
  // (longest first: the hardware dispatches blocks in order as compute units free up); the query
  // tile varies slowest, and with a multiple of 8 (split, head) units a head's tiles all land on
  // the XCD that takes block index mod 8.
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
  const int split = rest % a.num_splits;
  rest /= a.num_splits;
  const int h = rest % a.H;
  const int b = rest / a.H;
  const size_t head = (size_t)b * a.H + h;
  const size_t kvh = kv_head_index(b, h, a.H, a.H_kv);
  const T* __restrict__ Q = static_cast<const T*>(a.q) + head * (size_t)a.Nq * D;
  const T* __restrict__ K = static_cast<const T*>(a.k) + kvh * (size_t)a.Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + kvh * (size_t)a.Nk * D;
  const int kbeg = split_begin(split, a.Nk, a.num_splits);
  int kend = split_begin(split + 1, a.Nk, a.num_splits);
  // Causal mask: row i sees keys <= i + causal_off. The workgroup's key range ends after the
  // last key its last row sees (key tiles wholly past it are skipped); in split mode the range
  // can be empty, and the rows then keep the empty state.
  if constexpr (CAUSAL) kend = min(kend, min(a.Nq, (qt + 1) * C::BR) + a.causal_off);
  const int nkeys = kend - kbeg;
  const int T_ = nkeys > 0 ? (nkeys + kBC - 1) / kBC : 0;  // key tiles
  // Tiles [0, n_plain) hold only keys every row of the wave sees: no masking there (under the
  // causal mask the bound is per wave, set below).
  int n_plain = (nkeys % kBC == 0) ? T_ : T_ - 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool group_a = wave < 4;
  const int gw = __builtin_amdgcn_readfirstlane(wave) & 3;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int qrow0 = qt * C::BR + wave * (NB * 32);

  // ---- Q^T fragments: B operand of S^T = K Q^T, lane = query column, 8 dims per lane ----
  v8 qf[NB][C::KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = qrow0 + nb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (row < a.Nq) raw = *reinterpret_cast<const u32x4_t*>(Q + (size_t)row * D + ks * 16 + hf * 8);
      qf[nb][ks] = __builtin_bit_cast(v8, raw);
    }
  }

  // d = 64: LDS byte addresses of this lane's MFMA-phase reads (per buffer)
  // (buffer 0; buffer 1 is ELEMS elements further)
  unsigned vaddr0 = 0u, kaddr0[4] = {0u, 0u, 0u, 0u};
  if constexpr (D == 64) {
    vaddr0 = (unsigned)(__UINTPTR_TYPE__)(lds_void_t*)&lds_vf[0][lane * 8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r = l32, ch = ks * 2 + hf;
      kaddr0[ks] = (unsigned)(__UINTPTR_TYPE__)(lds_void_t*)&lds_k[0][r * D + ((ch ^ swzk(r)) << 3)];
    }
  }
  unsigned koff[C::LPW], voff[C::LPW];
  load_offsets<D, T, true>(gw, lane, koff);
  load_offsets<D, T, false>(gw, lane, voff);
  const float c2 = a.scale_log2e;
  const float tau = a.rescale_threshold;
  const float bound = __builtin_amdgcn_exp2f(tau);
  RowState<NB> st;
  f32x16_t acc[NB][C::DB];
  f32x16_t s[NB][2];
  v8 pf[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    st.mraw[nb] = -INFINITY;
    st.m2ref[nb] = 0.f;
    st.lsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][db][r] = 0.f;
  }

  // Causal: no row of this wave sees a key of tile t (wave-uniform; once true, true for every
  // later tile).
  const int wave_row0 = __builtin_amdgcn_readfirstlane(qrow0);
  auto wave_masked = [&](int t) -> bool {
    if constexpr (CAUSAL) return wave_row0 + NB * 32 + a.causal_off <= kbeg + t * kBC;
    else return false;
  };
  // Causal: the tiles whose keys the wave's first row (and so every row of the wave) sees in
  // full. A wave further down the query tile sees more of the diagonal tiles in full than the
  // workgroup's first row does; it takes the unmasked softmax there. Every wave runs the same
  // barriers per tile on either path.
  if constexpr (CAUSAL) n_plain = min(n_plain, max(0, (wave_row0 + a.causal_off + 1 - kbeg) / kBC));

  // ---- the two phases of one tile ----
  // Loads (group A only; global -> LDS, asynchronous). Staged: K(t+1) and V(t+1) start at the top
  // of the MFMA phase of tile t. Otherwise K(t+1) and V(t) start at the top of the VALU phase of
  // tile t, which reads no LDS, so the MFMA phase never waits on an outstanding load. Either way
  // group A waits for them at the end of its VALU phase, and no wave reads a buffer before the
  // barrier that follows, nor while a load into it is in flight (every buffer's previous
  // contents were last read at least one barrier earlier).
  auto phase_mfma = [&](int t, bool do_pv, bool do_s) {
    if constexpr (STAGE) {
      if (group_a && t + 1 < T_) {
        load_tile2<D, T, true>(K, lds_k[(t + 1) & 1], kbeg + (t + 1) * kBC, kend, gw, lane, koff);
        load_tile2<D, T, false>(V, lds_v[(t + 1) & 1], kbeg + (t + 1) * kBC, kend, gw, lane, voff);
      }
      if constexpr (NB == 2) {
        if (do_pv && do_s) {
          const unsigned vo = ((t - 1) & 1) * (unsigned)(C::ELEMS * sizeof(T));
          const unsigned ko = (t & 1) * (unsigned)(C::ELEMS * sizeof(T));
          const unsigned kaddr[4] = {kaddr0[0] + ko, kaddr0[1] + ko, kaddr0[2] + ko, kaddr0[3] + ko};
          mfma_phase_d64<T>(vaddr0 + vo, kaddr, pf, qf, acc, s);
        } else if (do_pv) {
          pv_staged<D, T, NB>(lds_vf[(t - 1) & 1], pf, acc, lane);
        }
      } else if (do_pv) {
        pv_staged<D, T, NB>(lds_vf[(t - 1) & 1], pf, acc, lane);
      }
    } else {
      if (do_pv) pv_tile<D, T, NB>(lds_v[(t - 1) & 1], pf, acc, lane);
    }
    if (do_s && !(STAGE && NB == 2 && do_pv)) s_tile<D, T, NB>(lds_k[t & 1], qf, s, lane);
    if constexpr (D == 128) {
      if (do_pv && do_s) mfma_phase_order_d128<2, 0>();
    }
    // At d = 128 the phase's MFMAs stay before its barrier (the compiler would move the last ones
    // past it, into the other group's MFMA phase, where the softmax then waits for them): 0.8 %
    // on the long-sequence workload.
    if (!ONE_BAR || (!group_a && do_s)) {
      if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // VALU phase of tile t: (staged) group A re-lays V(t); the softmax update; group A waits for its
  // loads; barrier.
  auto valu_prologue = [&](int t) {
    if constexpr (STAGE) {
      if (group_a) stage_v<D, T>(lds_v[t & 1], lds_vf[t & 1], gw, lane);
    } else if (group_a) {
      if (t + 1 < T_) load_tile2<D, T, true>(K, lds_k[(t + 1) & 1], kbeg + (t + 1) * kBC, kend, gw, lane, koff);
      if (t < T_) load_tile2<D, T, false>(V, lds_v[t & 1], kbeg + t * kBC, kend, gw, lane, voff);
    }
  };
  auto phase_valu_full = [&](int t, bool first) {
    valu_prologue(t);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      softmax_block<D, T, FAST, false>(s[nb], st.mraw[nb], st.m2ref[nb], st.lsum[nb], pf[nb], acc[nb], first, c2, tau,
                                       bound);
    if (group_a) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!ONE_BAR || group_a) __syncthreads();
  };
  // Masked tiles: a row sees the tile's keys below lim (the range end: a ragged last tile; the
  // row's last visible key + 1: causal), and the keys at or past it are masked one by one. Under
  // the causal mask a tile of which no row of the wave sees any key (a wave-uniform test on the
  // wave's last row) takes a short path instead: P = 0 and the state is unchanged. The first tile
  // always takes the per-key path, which sets up the state.
  auto phase_valu_masked = [&](int t, bool first) {
    valu_prologue(t);
    const int k0 = kbeg + t * kBC;
    if (CAUSAL && !first && wave_masked(t)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 8; ++i) pf[nb][g][i] = (T)0.f;
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        int lim = kend - k0;
        if constexpr (CAUSAL) lim = min(lim, wave_row0 + nb * 32 + l32 + a.causal_off + 1 - k0);
        softmax_block<D, T, FAST, true>(s[nb], st.mraw[nb], st.m2ref[nb], st.lsum[nb], pf[nb], acc[nb], first, c2,
                                        tau, bound, lim - 4 * hf);
      }
    }
    if (group_a) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!ONE_BAR || group_a) __syncthreads();
  };

  if (T_ > 0) {
    // ---- prologue: K(0) (and, staged, V(0)) resident; with two barriers per tile group B then sits
    //      out one phase (with one, B runs its MFMA phase of tile 0 at once and waits at the barrier) ----
    if (group_a) {
      load_tile2<D, T, true>(K, lds_k[0], kbeg, kend, gw, lane, koff);
      if constexpr (STAGE) load_tile2<D, T, false>(V, lds_v[0], kbeg, kend, gw, lane, voff);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!ONE_BAR && !group_a) __syncthreads();

    // First tile, unmasked tiles, masked tiles, then the final PV; every tile is one MFMA
    // phase and one VALU phase. Only the first tile takes the first-tile logic, and the
    // steady-state loop carries the unmasked softmax body. Without the causal mask at most
    // the last tile is masked, and it is peeled out of the loop.
    phase_mfma(0, false, true);
    if (n_plain >= 1) phase_valu_full(0, true);
    else phase_valu_masked(0, true);
    for (int t = 1; t < n_plain; ++t) {
      phase_mfma(t, true, true);
      phase_valu_full(t, false);
    }
    if constexpr (CAUSAL) {
      // (d = 64, sum-checked) a wave whose rows saw no key of tile t - 1 sees none of the later
      // tiles either: it leaves the loop (its PV of a zero P and its unused S are skipped) and
      // only takes part in the loads, group A's V staging and the barriers, so the other wave of
      // its SIMD has the matrix core and the VALU to itself on the last diagonal tiles (causal
      // workload 148.6 -> 146.3 us). Its P is already 0, so the final PV adds nothing.
      int t = n_plain > 1 ? n_plain : 1;
      for (; t < T_ && !(STAGE && FAST && wave_masked(t - 1)); ++t) {
        phase_mfma(t, true, true);
        phase_valu_masked(t, false);
      }
      if constexpr (STAGE && FAST) {
        for (; t < T_; ++t) {
          if (group_a && t + 1 < T_) {
            load_tile2<D, T, true>(K, lds_k[(t + 1) & 1], kbeg + (t + 1) * kBC, kend, gw, lane, koff);
            load_tile2<D, T, false>(V, lds_v[(t + 1) & 1], kbeg + (t + 1) * kBC, kend, gw, lane, voff);
          }
          if (!group_a) __syncthreads();
          valu_prologue(t);
          if (group_a) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
          }
        }
      }
    } else if (n_plain < T_ && T_ > 1) {
      phase_mfma(T_ - 1, true, true);
      phase_valu_masked(T_ - 1, false);
    }
    phase_mfma(T_, true, false);
    if (!ONE_BAR && group_a) __syncthreads();
  }

  // ---- epilogue: re-express l (and o) relative to the true maximum; O = acc / l ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = qrow0 + nb * 32 + l32;
    if (row >= a.Nq) continue;
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
      if constexpr (!FAST) {
        if (hf == 0) {
          const float to_true = __builtin_amdgcn_exp2f(st.m2ref[nb] - st.mraw[nb] * c2);
          if (a.m_out) a.m_out[head * a.Nq + row] = a.scale * st.mraw[nb];
          if (a.l_out) a.l_out[head * a.Nq + row] = st.lsum[nb] * to_true;
          if (a.lse_out) a.lse_out[head * a.Nq + row] = a.scale * st.mraw[nb] + logf(st.lsum[nb] * to_true);
        }
      } else {
        // the log-sum-exp needs no maximum: sum_j e^(scale s_j) = 2^m2ref * lsum, whatever the
        // reference (every term of lsum is at most 2^tau, so it carries full fp32 precision)
        if (hf == 0 && a.lse_out)
          a.lse_out[head * a.Nq + row] = st.m2ref[nb] * 0.6931471805599453f + logf(st.lsum[nb]);
      }
    } else if constexpr (!FAST) {
      // A row that saw no key of this range (causal mask) keeps the empty state (-inf, 0, 0).
      // In the (lse, o / l) form the empty state is (-inf, 0).
      const bool empty = st.mraw[nb] == -INFINITY;
      const float to_true = empty ? 0.f : __builtin_amdgcn_exp2f(st.m2ref[nb] - st.mraw[nb] * c2);
      const bool lse_form = a.split_mode == 2;
      const float w = lse_form ? (empty ? 0.f : 1.f / st.lsum[nb]) : to_true;
      const size_t prow = ((size_t)split * a.B * a.H + head) * a.Nq + row;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dd = db * 32 + 8 * g4 + 4 * hf;
          store4(a.part_o, prow * D + dd, kF32, acc[nb][db][4 * g4] * w, acc[nb][db][4 * g4 + 1] * w,
                 acc[nb][db][4 * g4 + 2] * w, acc[nb][db][4 * g4 + 3] * w);
        }
      if (hf == 0) {
        if (lse_form) {
          a.part_m[prow] = empty ? -INFINITY : a.scale * st.mraw[nb] + logf(st.lsum[nb] * to_true);
        } else {
          a.part_m[prow] = empty ? -INFINITY : a.scale * st.mraw[nb];
          a.part_l[prow] = st.lsum[nb] * to_true;
        }
      }
    }
  }
}

template <int D, typename T>
hipError_t launch_typed(const FwdArgs& a, hipStream_t s) {
  const int n_qtiles = (a.Nq + Cfg<D, T>::BR - 1) / Cfg<D, T>::BR;
  const long long nwg = (long long)n_qtiles * a.num_splits * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  int nq = n_qtiles;
  void* kargs[] = {&args, &nq};
  // Full-output calls without m / l take the sum-checked softmax (also with the log-sum-exp, which
  // needs no maximum); m / l, split states and a zero threshold (the literal recurrence) take the
  // running-max form.
  const bool fast = a.split_mode == 0 && !a.m_out && !a.l_out && a.rescale_threshold >= 1.f;
  const void* k;
  if (a.causal) k = fast ? reinterpret_cast<const void*>(&fwd_mfma_kernel<D, T, true, true>)
                         : reinterpret_cast<const void*>(&fwd_mfma_kernel<D, T, false, true>);
  else k = fast ? reinterpret_cast<const void*>(&fwd_mfma_kernel<D, T, true, false>)
                : reinterpret_cast<const void*>(&fwd_mfma_kernel<D, T, false, false>);
  return hipLaunchKernel(k, dim3((unsigned)nwg), dim3(kThreads), kargs, 0, s);
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
