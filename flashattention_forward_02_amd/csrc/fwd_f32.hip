// Tiled FlashAttention forward for fp32 inputs (VALU, full fp32 arithmetic).
//
// Same recurrence as the matrix-core kernel ("FlashAttention 简化版：Tiling + Online Softmax",
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
//
// Up to 16 query rows go to fwd_f32_rows_kernel instead (one workgroup per key range, row and
// head, keys spread over the lanes; described above the kernel).

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

// ---- few query rows (Nq <= 16): one workgroup per (key range, row, head), keys across lanes ----
// With one row per workgroup there is nothing to share through LDS, and the time goes to memory
// round trips, not arithmetic. So the roles of rows and keys swap inside a wave: the wave holds
// the one query row, and each group of LPK lanes (CPL columns each) takes a different key, so a
// key costs its group CPL FMAs, a short exchange and one expf. K and V go straight into registers,
// P steps ahead of their use, in 16 waves: about 256 KiB in flight per workgroup. Step i of wave
// w covers keys kbeg + (i * NW + w) * G + [0, G), so the waves walk the range together. Each group
// keeps its own (m, l, acc), summed plainly over 8 steps and then added with compensation; the
// groups of a wave are merged, then the waves (all compensated).
template <int D>
struct F32RowCfg {
  static constexpr int CPL = 8;           // columns per lane
  static constexpr int LPK = D / CPL;     // lanes per key: 8 (d = 64) or 16 (d = 128)
  static constexpr int G = 64 / LPK;      // keys per wave step
  static constexpr int NW = 16;           // waves per workgroup
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
template <int D>
__device__ __forceinline__ void load_key_cols(const float* __restrict__ row, int j, float (&x)[F32RowCfg<D>::CPL]) {
  typedef F32RowCfg<D> C;
#pragma unroll
  for (int r = 0; r < C::CPL / 4; ++r) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + r * 4 * C::LPK + 4 * j);
    x[4 * r] = v[0];
    x[4 * r + 1] = v[1];
    x[4 * r + 2] = v[2];
    x[4 * r + 3] = v[3];
  }
}

template <int D>
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
    load_key_cols<D>(K + key * D, j, kx);
    load_key_cols<D>(V + key * D, j, vx);
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

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_typed<64>(a, s);
  if (d == 128) return launch_typed<128>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32_rows(const FwdArgs& a, int d, hipStream_t s) {
  const long long nwg = (long long)a.num_splits * a.Nq * a.H * a.B;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FwdArgs args = a;
  void* kargs[] = {&args};
  const void* k = d == 64 ? reinterpret_cast<const void*>(&fwd_f32_rows_kernel<64>)
                : d == 128 ? reinterpret_cast<const void*>(&fwd_f32_rows_kernel<128>) : nullptr;
  if (!k) return hipErrorInvalidValue;
  return hipLaunchKernel(k, dim3((unsigned)nwg), dim3(kThreadsRows), kargs, 0, s);
}

}  // namespace fa
