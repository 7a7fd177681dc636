// FlashAttention forward for fp32 inputs: three kernels.
//  * fwd_f32_kernel (this header): more than 16 query rows at d = 128, on the VALU.
//  * fwd_f32_mfma_kernel: more than 16 query rows at d = 64, the products on the fp32 matrix
//    cores (described above it).
//  * fwd_f32_rows_kernel: one workgroup per query row, keys spread over the lanes (described
//    above it): calls of up to 16 query rows, and small calls of more (up to 256 rows per launch
//    at d = 64, 1024 at d = 128), which it spreads over more compute units than the tiled
//    kernels would use.
//
// fwd_f32_kernel. Same recurrence as the matrix-core kernel ("FlashAttention 简化版：Tiling + Online Softmax",
// §2.3 and §3.1), written for accuracy: scores are s = scale * (q . k) in fp32, the running max
// is taken on s, and exp is the accurate expf, so the result tracks the float64 definition to a
// few fp32 ulps.
//
// Work decomposition. A workgroup owns 16 query rows of one (b, h) and 8 waves; each wave streams
// its own contiguous eighth of the key range and keeps its own online-softmax state for all 16
// rows, and the 8 states are merged at the end with the pairwise rule of "CS349E 第 11 讲
// 01_online_softmax.py" demo 2 (the key-split of flash-decoding, inside one workgroup). So a
// workload of few rows still spreads over many waves: 256 rows are 16 workgroups of 8 waves.
// Inside a wave 4 adjacent lanes share a query row, each owning D/4 of its columns of q and of
// the accumulator; a dot product is D/4 FMAs per lane plus two exchanges within the 4 lanes.
//
// K/V tiles go from HBM straight into a per-wave LDS region (direct-to-LDS loads, two buffers,
// the next tile in flight while the current one is used), so the key loop needs no workgroup
// barrier. Every lane of a wave reads the same key row at the same time (16 rows x 4 column
// slices), so the LDS reads are broadcasts.
//
// Accuracy of the sums. O's sum sum_j p_j v_j nearly cancels (|O| is small next to
// sum |p v| when many keys share the weight), so plain fp32 accumulation over thousands of keys
// would lose ~sqrt(Nk) ulps. Each tile's contribution (16 or 8 keys) is summed plainly and then
// added to the running l and accumulator with compensation (Kahan), and the merge of the 8 wave
// states is compensated too: the error grows with the tile length, not with Nk.

#include "fa_internal.h"
#include "mfma_common.h"

namespace fa {
namespace {

constexpr int kWavesF = 8;
constexpr int kThreadsF = kWavesF * 64;
constexpr int kLPR = 4;              // lanes per query row
constexpr int kRows = 64 / kLPR;     // query rows per workgroup (every wave holds all of them)

template <int D>
struct F32Cfg {
  static constexpr int DPL = D / kLPR;                  // columns per lane
  static constexpr int KT = D == 64 ? 16 : 8;           // keys per tile
  static constexpr int TILE = KT * D;                   // floats per K (or V) tile
  static constexpr int LOADS = TILE / 4 / 64;           // 16-byte direct-to-LDS loads per lane per tensor
  static_assert(LOADS * 4 * 64 == TILE, "tile / wave mismatch");
  static constexpr int WAVE_BUF = 2 * TILE;             // floats per wave and buffer: K then V
};

// sum += x with the rounding error carried in comp (Kahan): the compensated value is sum - comp.
__device__ __forceinline__ void kahan_add(float& sum, float& comp, float x) {
  const float y = x - comp;
  const float t = sum + y;
  comp = (t - sum) - y;
  sum = t;
}

// Sum of x over the 4 lanes of a query row (DPP quad permutes: swap neighbours, then pairs).
__device__ __forceinline__ float row_sum4(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  return x;
}

// HBM -> LDS of keys [key0, key0 + KT) of one tensor (rows past kend repeat row kend - 1; their
// scores are masked). Row-major [KT][D] in LDS.
template <int D>
__device__ __forceinline__ void load_tile_f32(const float* __restrict__ X, float* lx, int key0, int kend, int lane) {
  typedef F32Cfg<D> C;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int c = i * 64 + lane;            // 16-byte chunk of the tile
    const int r = c / (D / 4);
    const int key = min(key0 + r, kend - 1);
    global_to_lds16(X + (size_t)key * D + (c % (D / 4)) * 4, &lx[i * 256]);
  }
}

template <int D>
__global__ __launch_bounds__(kThreadsF) void fwd_f32_kernel(FwdArgs a, int n_qtiles) {
  typedef F32Cfg<D> C;
  constexpr int DPL = C::DPL, KT = C::KT;
  // The two tile buffers are separate objects, and the key loop steps two tiles at a time, so the
  // compiler sees that a step's reads do not alias the loads of the next tile in flight (it would
  // otherwise wait for those loads before the first read).
  __shared__ __attribute__((aligned(16))) float lds0[kWavesF * C::WAVE_BUF];
  __shared__ __attribute__((aligned(16))) float lds1[kWavesF * C::WAVE_BUF];

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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rloc = lane / kLPR;
  const int row = qt * kRows + rloc;
  const int col0 = (lane % kLPR) * DPL;
  const bool live = row < a.Nq;
  // Causal mask: this row sees keys < row_end; the workgroup's range ends after the last key its
  // last row sees (key tiles wholly past it are skipped).
  int row_end = kend;
  if (a.causal) {
    row_end = min(kend, row + a.causal_off + 1);
    kend = min(kend, min(a.Nq, (qt + 1) * kRows) + a.causal_off);
  }
  // This wave's share of the range: contiguous, in whole tiles.
  const int ntiles = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;
  const int t0 = (int)(((long long)wave * ntiles) / kWavesF);
  const int t1 = (int)(((long long)(wave + 1) * ntiles) / kWavesF);

  float q[DPL], acc[DPL], comp[DPL], tacc[DPL];
#pragma unroll
  for (int c = 0; c < DPL; c += 4) {
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    if (live) x = *reinterpret_cast<const f32x4_t*>(Q + (size_t)row * D + col0 + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[c + i] = x[i];
      acc[c + i] = comp[c + i] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f, lcomp = 0.f;

  float* w0 = lds0 + wave * C::WAVE_BUF;    // [K, V][TILE]
  float* w1 = lds1 + wave * C::WAVE_BUF;
  // One tile: wait for it, start the next one into the other buffer, then the online-softmax update.
  auto step = [&](int t, float* cur, float* nxt) {
    const int key0 = kbeg + t * KT;
    const float* lk = cur;
    const float* lv = cur + C::TILE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this tile has landed (this wave's own loads)
    if (t + 1 < t1) {
      load_tile_f32<D>(K, nxt, key0 + KT, kend, lane);
      load_tile_f32<D>(V, nxt + C::TILE, key0 + KT, kend, lane);
    }
    float s[KT];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < DPL; c += 4) {
        const f32x4_t kx = *reinterpret_cast<const f32x4_t*>(&lk[j * D + col0 + c]);
        dot = __builtin_fmaf(q[c], kx[0], dot);
        dot = __builtin_fmaf(q[c + 1], kx[1], dot);
        dot = __builtin_fmaf(q[c + 2], kx[2], dot);
        dot = __builtin_fmaf(q[c + 3], kx[3], dot);
      }
      dot = row_sum4(dot);
      s[j] = (key0 + j < row_end) ? a.scale * dot : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mnew = fmaxf(m, mt);
    if (mnew != -INFINITY) {               // a tile with no visible key for this row leaves its state alone
      if (mnew != m) {                     // the max grew: rescale l and the accumulator by exp(m_old - m_new)
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
        l *= alpha;
        lcomp *= alpha;
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          acc[c] *= alpha;
          comp[c] *= alpha;
        }
        m = mnew;
      }
      float tl = 0.f;
#pragma unroll
      for (int c = 0; c < DPL; ++c) tacc[c] = 0.f;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        const float p = (key0 + j < row_end) ? expf(s[j] - m) : 0.f;
        tl += p;
#pragma unroll
        for (int c = 0; c < DPL; c += 4) {
          const f32x4_t vx = *reinterpret_cast<const f32x4_t*>(&lv[j * D + col0 + c]);
          tacc[c] = __builtin_fmaf(p, vx[0], tacc[c]);
          tacc[c + 1] = __builtin_fmaf(p, vx[1], tacc[c + 1]);
          tacc[c + 2] = __builtin_fmaf(p, vx[2], tacc[c + 2]);
          tacc[c + 3] = __builtin_fmaf(p, vx[3], tacc[c + 3]);
        }
      }
      kahan_add(l, lcomp, tl);
#pragma unroll
      for (int c = 0; c < DPL; ++c) kahan_add(acc[c], comp[c], tacc[c]);
    }
  };
  if (t0 < t1) {
    load_tile_f32<D>(K, w0, kbeg + t0 * KT, kend, lane);
    load_tile_f32<D>(V, w0 + C::TILE, kbeg + t0 * KT, kend, lane);
  }
  int t = t0;
  for (; t + 1 < t1; t += 2) {
    step(t, w0, w1);
    step(t + 1, w1, w0);
  }
  if (t < t1) step(t, w0, w1);

  // ---- merge the 8 wave states of every row (compensated), then the epilogue ----
  __syncthreads();                         // every wave is done with its tiles: the LDS is reused
  // per wave: m[16], l[16], then the 16 x D compensated accumulator; waves 0-3 in lds0, 4-7 in lds1
  constexpr int WSTATE = 2 * kRows + kRows * D;
  static_assert(4 * WSTATE <= kWavesF * C::WAVE_BUF, "merge state does not fit");
  float* st = (wave < 4 ? lds0 : lds1) + (wave & 3) * WSTATE;
  if (lane % kLPR == 0) {
    st[rloc] = m;
    st[kRows + rloc] = l - lcomp;
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) st[2 * kRows + rloc * D + col0 + c] = acc[c] - comp[c];
  __syncthreads();

  // thread -> (row r, 16-column slice): D / 32 x ... columns per thread
  constexpr int CPT = D * kRows / kThreadsF;   // columns per thread (2 or 4)
  const int r = tid / (D / CPT);
  const int cc = (tid % (D / CPT)) * CPT;
  const int grow = qt * kRows + r;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWavesF; ++w) M = fmaxf(M, (w < 4 ? lds0 : lds1)[(w & 3) * WSTATE + r]);
  float L = 0.f, Lc = 0.f, o[CPT], oc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) o[i] = oc[i] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWavesF; ++w) {
      const float* ws = (w < 4 ? lds0 : lds1) + (w & 3) * WSTATE;
      const float mw = ws[r];
      if (mw == -INFINITY) continue;      // a wave that saw no key of this row weighs 0
      const float wgt = expf(mw - M);
      kahan_add(L, Lc, wgt * ws[kRows + r]);
#pragma unroll
      for (int i = 0; i < CPT; ++i) kahan_add(o[i], oc[i], wgt * ws[2 * kRows + r * D + cc + i]);
    }
  }
  L -= Lc;
#pragma unroll
  for (int i = 0; i < CPT; ++i) o[i] -= oc[i];
  if (grow >= a.Nq) return;

  if (a.split_mode == 0) {
    const float inv = 1.f / L;
    float* O = static_cast<float*>(a.o) + (head * (size_t)a.Nq + grow) * D + cc;
#pragma unroll
    for (int i = 0; i < CPT; ++i) O[i] = o[i] * inv;
    if (cc == 0) {
      if (a.m_out) a.m_out[head * a.Nq + grow] = M;
      if (a.l_out) a.l_out[head * a.Nq + grow] = L;
      if (a.lse_out) a.lse_out[head * a.Nq + grow] = M + logf(L);
    }
  } else {
    const size_t prow = ((size_t)split * a.B * a.H + head) * a.Nq + grow;
    float* P = a.part_o + prow * D + cc;
    // (lse, o / l) form: a row with no key in this range keeps (-inf, 0)
    const float w = (a.split_mode == 2) ? (L > 0.f ? 1.f / L : 0.f) : 1.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) P[i] = o[i] * w;
    if (cc == 0) {
      if (a.split_mode == 2) {
        a.part_m[prow] = (M == -INFINITY) ? -INFINITY : M + logf(L);
      } else {
        a.part_m[prow] = M;
        a.part_l[prow] = L;
      }
    }
  }
}

// ---- d = 64 on the fp32 matrix cores ----
// The same decomposition as fwd_f32_kernel (a workgroup owns 16 query rows of one head; each of
// its NW waves streams its own share of the key range and keeps its own online-softmax state; the
// NW states are merged with compensation at the end), with the two products on
// v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation, at twice the rate of plain fp32 FMAs
// on the VALU, which is left with the softmax.
//  * S^T = K Q^T per 16-key step: rows = keys, columns = the 16 queries. In the 16x16 result a
//    lane owns one query (lane % 16) and 4 consecutive keys (4 (lane / 16) + r), so the row max
//    and sum need two exchanges (lanes 16 and 32 apart). The 64 dimensions are taken in the order
//    that lets one 16-byte load feed four k-steps: k-step (G, i) gives group g = lane / 16 the
//    dimension 16 G + 4 g + i (Q^T, in registers, follows the same order).
//  * O^T += V^T P^T: the B operand of k-step kk is P at key 4 g + kk, the lane's own score
//    register kk, so P never leaves the lane. Row m of output block db is dimension 4 m + db, so
//    the A operands a lane feeds the 4 blocks at one key are 4 consecutive floats of one V row:
//    one 16-byte load per key.
//  * K and V go straight from memory into registers in exactly those operand layouts (a step is
//    8 16-byte buffer loads per lane, addressed by a scalar descriptor and immediates); no LDS
//    until the merge. The scores of step t + 1 are issued before the softmax of step t.
//  * Exponentials in base 2, as in the matrix-core kernel: with c = scale * log2(e), p =
//    2^(s c - m2) is one FMA and one v_exp_f32, against about 13 instructions for expf. VALU
//    instructions do not overlap the fp32 MFMAs of the same SIMD (a probe: 16 MFMAs take 512
//    cycles, and each VALU instruction beside them adds about 7), so the VALU count sets the
//    rate; the rounding of the argument s c - m2, which both forms share, dominates the error.
//    m_out is scale times the running max of the raw dot products, and m2 = that max times c.
//  * Accuracy as in fwd_f32_kernel otherwise: the PV products of 8 steps (128 keys) accumulate
//    plainly in the matrix core and are then added with compensation, as is l; the merge of the
//    wave states is compensated.
constexpr int kQM = 16;                     // query rows per workgroup
constexpr int kKM = 16;                     // keys per step
// Fourth word of a raw buffer descriptor (32-bit data format, no swizzle, no stride).
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Max / sum over the 4 lanes that hold one query (lanes 16 apart).
__device__ __forceinline__ float qrow_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_max(max2f(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float qrow_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void fwd_f32_mfma_kernel(FwdArgs a, int n_qtiles) {
  constexpr int D = 64;
  // merge state per wave: m2[16], l[16], mraw[16], then O[16][64] (compensated values)
  constexpr int WST = 3 * kQM + kQM * D;
  __shared__ float st_all[NW * WST];

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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;     // this lane's query (MFMA column) and the K row it supplies
  const int g = lane >> 4;     // its k-index group
  const int row = qt * kQM + n;
  const bool live = row < a.Nq;
  // Causal mask: this row sees keys < row_end; every row of the workgroup sees the keys below
  // all_end; the workgroup's range ends after the last key its last row sees.
  int row_end = kend, all_end = kend;
  if (a.causal) {
    row_end = min(kend, row + a.causal_off + 1);
    all_end = min(kend, qt * kQM + a.causal_off + 1);
    kend = min(kend, min(a.Nq, (qt + 1) * kQM) + a.causal_off);
  }
  const int nsteps = kend > kbeg ? (kend - kbeg + kKM - 1) / kKM : 0;
  const int t0 = (int)(((long long)wave * nsteps) / NW);
  const int t1 = (int)(((long long)(wave + 1) * nsteps) / NW);

  // Q^T operand: qv[4 G + i] = Q[row][16 G + 4 g + i]
  float qv[16];
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    if (live) x = *reinterpret_cast<const f32x4_t*>(Q + (size_t)row * D + 16 * G + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[4 * G + i] = x[i];
  }
  // Operands of one step, per lane: kx[4 G + i] = K[key0 + n][16 G + 4 g + i] (S^T A operands),
  // vx[4 kk + db] = V[key0 + 4 g + kk][4 n + db] (O^T A operands). Byte offsets from the step's
  // first key row: K n * 256 + g * 16 (+ 64 G), V 4 g * 256 + n * 16 (+ 256 kk).
  const unsigned koffb = (unsigned)(n * 256 + g * 16);
  const unsigned voffb = (unsigned)(g * 1024 + n * 16);
  // Buffer loads: the descriptor of a step starts at its first key row (a 64-bit address) and
  // holds that step's rows only, at most 16 (4 KB, so the 32-bit record count never overflows,
  // whatever Nk is), so the rows of a ragged last step that lie past kend read as 0 (the
  // hardware's range check; their scores are masked) and no load branches. Steps past the wave's
  // last one are clamped to it (those loads are not used).
  auto step_rsrc = [&](const float* X, int t) {
    const int key0 = kbeg + min(t, t1 - 1) * kKM;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(X + (size_t)key0 * D), 0,
                                             min(kend - key0, kKM) * D * (int)sizeof(float), kBufferWord3);
  };
  auto load_k = [&](int t, float (&kx)[16]) {
    const __amdgpu_buffer_rsrc_t r = step_rsrc(K, t);
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const f32x4_t x = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, koffb + 64 * G, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) kx[4 * G + i] = x[i];
    }
  };
  auto load_v = [&](int t, float (&vx)[16]) {
    const __amdgpu_buffer_rsrc_t r = step_rsrc(V, t);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f32x4_t x = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voffb + 256 * kk, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) vx[4 * kk + i] = x[i];
    }
  };

  // per lane: the query's running max of the raw dot products (shared by its 4 lanes) and its
  // base-2 exponent reference m2 = mraw * c, this lane's share of l = sum 2^(s c - m2), and
  // O^T[16 g + 4 r + db][query] in acc[db][r]; bl / bacc are the plain sums of the current 8 steps
  const float c = a.scale_log2e;
  float mraw = -INFINITY, m2 = -INFINITY, l = 0.f, lcomp = 0.f, bl = 0.f;
  float acc[4][4], comp[4][4];
  f32x4_t bacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[db][i] = comp[db][i] = bacc[db][i] = 0.f;
  auto flush = [&]() {
    kahan_add(l, lcomp, bl);
    bl = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kahan_add(acc[db][i], comp[db][i], (float)bacc[db][i]);
        bacc[db][i] = 0.f;
      }
  };

  auto scores = [&](const float (&kx)[16]) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) s = mfma_f32(kx[k], qv[k], s);
    return s;
  };
  // softmax update and O^T += V^T P^T of step t, given its raw scores
  auto update = [&](int t, const f32x4_t& s, const float (&vx)[16]) {
    const int key0 = kbeg + t * kKM;
    const bool full = key0 + kKM <= all_end;   // every key of the step is seen by every row
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = (full || key0 + 4 * g + r < row_end) ? s[r] : -INFINITY;
    float mt = qrow_max(max3f(sv[0], sv[1], max2f(sv[2], sv[3])));
    const bool grow = mt > mraw;             // false while the query has seen no key (both -inf)
    if (__ballot(grow)) {                    // rescale l and the accumulators by 2^(m2_old - m2_new)
      const float m2new = grow ? mt * c : m2;
      const float alpha = grow ? (mraw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - m2new)) : 1.f;
      l *= alpha;
      lcomp *= alpha;
      bl *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[db][i] *= alpha;
          comp[db][i] *= alpha;
          bacc[db][i] *= alpha;
        }
      if (grow) {
        mraw = mt;
        m2 = m2new;
      }
    }
    float p[4];
    if (full) {
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m2));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p[r] = (key0 + 4 * g + r < row_end) ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m2)) : 0.f;
    }
    bl += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int db = 0; db < 4; ++db) bacc[db] = mfma_f32(vx[4 * kk + db], p[kk], bacc[db]);
    if (((t - t0) & 7) == 7) flush();
  };

  // Software pipeline: iteration t issues the scores of step t + 1 (matrix cores) before the
  // softmax of step t (VALU), so a wave's own MFMAs run under its softmax. K is loaded two steps
  // ahead of its use (one step ahead of its scores), V one step ahead; the loop is unrolled by two
  // so the buffers are fixed registers: at the top of iteration t, K(t + 1) is in kb1, V(t) in vb0
  // and the scores of step t in s_cur.
  float kb0[16], vb0[16], kb1[16], vb1[16];
  if (t0 < t1) {
    load_k(t0, kb0);
    load_v(t0, vb0);
    load_k(t0 + 1, kb1);
    f32x4_t s_cur = scores(kb0);
    int t = t0;
    for (; t + 1 < t1; t += 2) {
      load_k(t + 2, kb0);
      load_v(t + 1, vb1);
      const f32x4_t s_nxt = scores(kb1);
      update(t, s_cur, vb0);
      load_k(t + 3, kb1);
      load_v(t + 2, vb0);
      s_cur = scores(kb0);
      update(t + 1, s_nxt, vb1);
    }
    if (t < t1) update(t, s_cur, vb0);
  }
  flush();

  // ---- merge the NW wave states of every row (compensated), then the epilogue ----
  {
    float* st = st_all + wave * WST;
    const float lq = qrow_sum(l - lcomp);
    if (g == 0) {
      st[n] = m2;
      st[kQM + n] = lq;
      st[2 * kQM + n] = mraw;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[3 * kQM + n * D + 16 * g + 4 * r + db] = acc[db][r] - comp[db][r];
  }
  __syncthreads();

  // thread -> (row r, 2 consecutive columns): 16 rows x 64 columns over the first 512 threads
  constexpr int CPT = 2;
  static_assert(NW * 64 >= kQM * D / CPT, "every output column needs a thread");
  if (tid >= kQM * D / CPT) return;
  const int r = tid / (D / CPT);
  const int cc = (tid % (D / CPT)) * CPT;
  const int grow_ = qt * kQM + r;
  float M2 = -INFINITY, MR = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    M2 = fmaxf(M2, st_all[w * WST + r]);
    MR = fmaxf(MR, st_all[w * WST + 2 * kQM + r]);
  }
  float L = 0.f, Lc = 0.f, o[CPT], oc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) o[i] = oc[i] = 0.f;
  if (M2 != -INFINITY) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* ws = st_all + w * WST;
      const float mw = ws[r];
      if (mw == -INFINITY) continue;      // a wave that saw no key of this row weighs 0
      const float wgt = __builtin_amdgcn_exp2f(mw - M2);
      kahan_add(L, Lc, wgt * ws[kQM + r]);
#pragma unroll
      for (int i = 0; i < CPT; ++i) kahan_add(o[i], oc[i], wgt * ws[3 * kQM + r * D + cc + i]);
    }
  }
  L -= Lc;
#pragma unroll
  for (int i = 0; i < CPT; ++i) o[i] -= oc[i];
  if (grow_ >= a.Nq) return;
  // m = scale * max of the raw dot products; L = sum 2^(s c - M2) with M2 = max * c (the same
  // rounded product every wave used), i.e. l relative to m; lse = M2 ln 2 + ln L
  const float M = a.scale * MR;
  const float lse = M2 * 0.6931471805599453f + logf(L);

  if (a.split_mode == 0) {
    const float inv = 1.f / L;
    float* O = static_cast<float*>(a.o) + (head * (size_t)a.Nq + grow_) * D + cc;
#pragma unroll
    for (int i = 0; i < CPT; ++i) O[i] = o[i] * inv;
    if (cc == 0) {
      if (a.m_out) a.m_out[head * a.Nq + grow_] = M;
      if (a.l_out) a.l_out[head * a.Nq + grow_] = L;
      if (a.lse_out) a.lse_out[head * a.Nq + grow_] = lse;
    }
  } else {
    const size_t prow = ((size_t)split * a.B * a.H + head) * a.Nq + grow_;
    float* P = a.part_o + prow * D + cc;
    // (lse, o / l) form: a row with no key in this range keeps (-inf, 0)
    const float w = (a.split_mode == 2) ? (L > 0.f ? 1.f / L : 0.f) : 1.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) P[i] = o[i] * w;
    if (cc == 0) {
      if (a.split_mode == 2) {
        a.part_m[prow] = (M2 == -INFINITY) ? -INFINITY : lse;
      } else {
        a.part_m[prow] = (M2 == -INFINITY) ? -INFINITY : M;
        a.part_l[prow] = L;
      }
    }
  }
}

// ---- few query rows (Nq <= 16): one workgroup per (key range, row, head), keys across lanes ----
// With one row per workgroup there is nothing to share through LDS, and the time goes to memory
// round trips, not arithmetic. So the roles of rows and keys swap inside a wave: the wave holds
// the one query row, and each group of LPK lanes (CPL columns each) takes a different key, so a
// key costs its group CPL FMAs, a short exchange and one expf. K and V go straight into registers,
// P steps ahead of their use, in 8 waves: about 128 KiB in flight per workgroup. Step i of wave
// w covers keys kbeg + (i * NW + w) * G + [0, G), so the waves walk the range together. Each group
// keeps its own (m, l, acc), summed plainly over 8 steps and then added with compensation; the
// groups of a wave are merged, then the waves (all compensated).
template <int D>
struct F32RowCfg {
  static constexpr int CPL = 8;           // columns per lane
  static constexpr int LPK = D / CPL;     // lanes per key: 8 (d = 64) or 16 (d = 128)
  static constexpr int G = 64 / LPK;      // keys per wave step
  static constexpr int NW = 8;            // waves per workgroup (16: single head 7.6 -> 6.5 us with 8)
  static constexpr int P = 4;             // steps in flight per wave
};
constexpr int kThreadsRows = F32RowCfg<64>::NW * 64;

// Sum over the LPK lanes of a key group (DPP: neighbours, pairs, then mirrored halves).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  if constexpr (LPK == 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
  return x;
}

// Lane j of a group owns columns r * 4 * LPK + 4 j + [0, 4) for r < CPL / 4, so one 16-byte load
// instruction of the wave covers whole contiguous row segments.
// NT: nontemporal loads (a stream only this workgroup reads).
template <int D, bool NT = false>
__device__ __forceinline__ void load_key_cols(const float* __restrict__ row, int j, float (&x)[F32RowCfg<D>::CPL]) {
  typedef F32RowCfg<D> C;
#pragma unroll
  for (int r = 0; r < C::CPL / 4; ++r) {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(row + r * 4 * C::LPK + 4 * j);
    const f32x4_t v = NT ? __builtin_nontemporal_load(p) : *p;
    x[4 * r] = v[0];
    x[4 * r + 1] = v[1];
    x[4 * r + 2] = v[2];
    x[4 * r + 3] = v[3];
  }
}

template <int D, bool NT>
__global__ __launch_bounds__(kThreadsRows) void fwd_f32_rows_kernel(FwdArgs a) {
  typedef F32RowCfg<D> C;
  constexpr int CPL = C::CPL, LPK = C::LPK, G = C::G, NW = C::NW, P = C::P;
  // merge state: per wave m[G], l[G], acc[G][D], then per wave (m, l, o[D])
  constexpr int WSTATE = 2 * G + G * D;
  __shared__ float st_all[NW * WSTATE];

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
  const float* __restrict__ K = static_cast<const float*>(a.k) + kvh * (size_t)a.Nk * D;
  const float* __restrict__ V = static_cast<const float*>(a.v) + kvh * (size_t)a.Nk * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane / LPK;
  const int j = lane % LPK;
  const int nsteps = kend > kbeg ? (kend - kbeg + NW * G - 1) / (NW * G) : 0;
  // key of this lane's group at step i
  auto key_at = [&](int i) { return kbeg + (i * NW + wave) * G + grp; };

  float q[CPL], acc[CPL], comp[CPL], tacc[CPL];
  load_key_cols<D>(static_cast<const float*>(a.q) + (head * a.Nq + row) * (size_t)D, j, q);
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = comp[c] = tacc[c] = 0.f;
  float m = -INFINITY, l = 0.f, lcomp = 0.f, tl = 0.f;
  auto flush = [&]() {
    kahan_add(l, lcomp, tl);
    tl = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      kahan_add(acc[c], comp[c], tacc[c]);
      tacc[c] = 0.f;
    }
  };

  float kb[P][CPL], vb[P][CPL];
  // rows past kend repeat row kend - 1 (their keys take no part)
  auto load_step = [&](int i, float (&kx)[CPL], float (&vx)[CPL]) {
    const size_t key = (size_t)min(key_at(i), kend - 1);
    load_key_cols<D, NT>(K + key * D, j, kx);
    load_key_cols<D, NT>(V + key * D, j, vx);
  };
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < nsteps) load_step(p, kb[p], vb[p]);
  for (int i0 = 0; i0 < nsteps; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int i = i0 + p;
      if (i >= nsteps) break;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) dot = __builtin_fmaf(q[c], kb[p][c], dot);
      dot = group_sum<LPK>(dot);
      if (key_at(i) < kend) {
        const float sc = a.scale * dot;
        if (sc > m) {                        // the max grew: rescale by exp(m_old - m_new)
          const float alpha = (m == -INFINITY) ? 0.f : expf(m - sc);
          l *= alpha;
          lcomp *= alpha;
          tl *= alpha;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            acc[c] *= alpha;
            comp[c] *= alpha;
            tacc[c] *= alpha;
          }
          m = sc;
        }
        const float pw = expf(sc - m);
        tl += pw;
#pragma unroll
        for (int c = 0; c < CPL; ++c) tacc[c] = __builtin_fmaf(pw, vb[p][c], tacc[c]);
      }
      if ((i & 7) == 7) flush();
      if (i + P < nsteps) load_step(i + P, kb[p], vb[p]);
    }
  }
  flush();

  // ---- merge: the G groups of each wave, then the NW waves (all compensated) ----
  float* st = st_all + wave * WSTATE;
  if (j == 0) {
    st[grp] = m;
    st[G + grp] = l - lcomp;
  }
#pragma unroll
  for (int r = 0; r < CPL / 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) st[2 * G + grp * D + r * 4 * LPK + 4 * j + c] = acc[4 * r + c] - comp[4 * r + c];
  __syncthreads();
  // each wave folds its own groups: lane -> D / 64 columns
  constexpr int CW = D / 64;
  float wm = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) wm = fmaxf(wm, st[g]);
  float wl = 0.f, wlc = 0.f, wo[CW], woc[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) wo[i] = woc[i] = 0.f;
  if (wm != -INFINITY) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mg = st[g];
      if (mg == -INFINITY) continue;         // a group that saw no key weighs 0
      const float w = expf(mg - wm);
      kahan_add(wl, wlc, w * st[G + g]);
#pragma unroll
      for (int i = 0; i < CW; ++i) kahan_add(wo[i], woc[i], w * st[2 * G + g * D + lane * CW + i]);
    }
  }
  __syncthreads();
  constexpr int WS2 = 2 + D;
  static_assert(NW * WS2 <= NW * WSTATE, "wave states do not fit");
  if (lane == 0) {
    st_all[wave * WS2] = wm;
    st_all[wave * WS2 + 1] = wl - wlc;
  }
#pragma unroll
  for (int i = 0; i < CW; ++i) st_all[wave * WS2 + 2 + lane * CW + i] = wo[i] - woc[i];
  __syncthreads();
  if (tid >= D) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, st_all[w * WS2]);
  float L = 0.f, Lc = 0.f, o = 0.f, oc = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = st_all[w * WS2];
      if (mw == -INFINITY) continue;
      const float wgt = expf(mw - M);
      kahan_add(L, Lc, wgt * st_all[w * WS2 + 1]);
      kahan_add(o, oc, wgt * st_all[w * WS2 + 2 + tid]);
    }
  }
  L -= Lc;
  o -= oc;
  const size_t qrow = head * a.Nq + row;
  if (a.split_mode == 0) {
    static_cast<float*>(a.o)[qrow * D + tid] = o / L;
    if (tid == 0) {
      if (a.m_out) a.m_out[qrow] = M;
      if (a.l_out) a.l_out[qrow] = L;
      if (a.lse_out) a.lse_out[qrow] = M + logf(L);
    }
  } else {
    const size_t prow = (size_t)split * a.B * a.H * a.Nq + qrow;
    // (lse, o / l) form: an empty range keeps (-inf, 0)
    a.part_o[prow * D + tid] = (a.split_mode == 2) ? (L > 0.f ? o / L : 0.f) : o;
    if (tid == 0) {
      if (a.split_mode == 2) {
        a.part_m[prow] = (M == -INFINITY) ? -INFINITY : M + logf(L);
      } else {
        a.part_m[prow] = M;
        a.part_l[prow] = L;
      }
    }
  }
}

template <int D>
hipError_t launch_typed(const FwdArgs& a, hipStream_t s) {
  const int n_qtiles = (a.Nq + kRows - 1) / kRows;
  const long long nwg = (long long)n_qtiles * a.num_splits * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  int nq = n_qtiles;
  void* kargs[] = {&args, &nq};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_f32_kernel<D>), dim3((unsigned)nwg), dim3(kThreadsF),
                         kargs, 0, s);
}

}  // namespace

hipError_t launch_fwd_f32_mfma(const FwdArgs& a, hipStream_t s) {
  // 8 waves (two per SIMD): 12 measured no faster, 16 slower (their registers spill)
  constexpr int NW = 8;
  const int n_qtiles = (a.Nq + kQM - 1) / kQM;
  const long long nwg = (long long)n_qtiles * a.num_splits * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  int nq = n_qtiles;
  void* kargs[] = {&args, &nq};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_f32_mfma_kernel<NW>), dim3((unsigned)nwg), dim3(NW * 64),
                         kargs, 0, s);
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_fwd_f32_mfma(a, s);
  if (d == 128) return launch_typed<128>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32_rows(const FwdArgs& a, int d, hipStream_t s) {
  const long long nwg = (long long)a.num_splits * a.Nq * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  void* kargs[] = {&args};
  // K and V stream nontemporally when each K/V head is read by one workgroup per key range (one
  // query row per K/V head: B=4, H=64, Nk=4096 one-query rows 96.7 -> 83.3 us at d = 64); with
  // several rows per K/V head the hint evicts lines the other rows' workgroups still read
  // (16 rows x 4 heads x 8192 keys: 49 -> 91 us), so those keep plain loads.
  const bool nt = a.Nq == 1 && a.H == a.H_kv;
  const void* k = d == 64 ? (nt ? reinterpret_cast<const void*>(&fwd_f32_rows_kernel<64, true>)
                                : reinterpret_cast<const void*>(&fwd_f32_rows_kernel<64, false>))
                : d == 128 ? (nt ? reinterpret_cast<const void*>(&fwd_f32_rows_kernel<128, true>)
                                 : reinterpret_cast<const void*>(&fwd_f32_rows_kernel<128, false>))
                           : nullptr;
  if (!k) return hipErrorInvalidValue;
  return hipLaunchKernel(k, dim3((unsigned)nwg), dim3(kThreadsRows), kargs, 0, s);
}

}  // namespace fa
