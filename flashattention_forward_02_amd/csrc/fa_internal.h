// Internal declarations shared by the host API (fa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum Dtype : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Arguments of one forward launch. In full mode (split_mode == 0) the kernels write the
// normalised O (out_dtype) and, when non-null, m_out / l_out. In split mode they write the
// unnormalised partial states part_m / part_l / part_o of each key range.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* m_out;
  float* l_out;
  float* lse_out;   // optional row log-sum-exp m + ln(l) (full mode)
  float* part_m;
  float* part_l;
  float* part_o;
  int B, H, Nq, Nk;
  int H_kv;         // K/V heads; query head h reads K/V head h / (H / H_kv)
  int causal;       // 1: query row i sees keys j <= i + causal_off only
  int causal_off;   // Nk - Nq
  int num_splits;   // 1 in full mode
  int split_mode;   // 0: final output, 1: partial states (m, l, o), 2: partial states (lse, o / l)
  int out_dtype;    // Dtype of o (full mode)
  float scale;      // softmax scale applied to q.k (natural-log units)
  float scale_log2e;  // scale * log2(e): scores in base-2 units for exp2
  float rescale_threshold;  // log2 units; see fwd_mfma.hip (0 = rescale whenever the max grows)
};

// Merge arguments. The merge order travels inside the kernel arguments.
constexpr int kMaxSplits = 256;
struct MergeArgs {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  void* o;
  float* m_out;
  float* l_out;
  int S, rows;      // rows = B * H * Nq
  int out_dtype;
  int lse_format;   // 1: parts are (lse, normalised o) in part_m / part_o; lse_out receives the total
  float* lse_out;
  unsigned short order[kMaxSplits];
};

// Key range [split_begin(c), split_begin(c + 1)) of part c of a split-KV partition.
__host__ __device__ inline int split_begin(int c, int Nk, int S) {
  return (int)(((long long)c * (long long)Nk) / (long long)S);
}

// Offset of K/V head (b, h / (H / H_kv)) in units of heads.
__host__ __device__ inline size_t kv_head_index(int b, int h, int H, int H_kv) {
  return (size_t)b * H_kv + h / (H / H_kv);
}

// Workgroup remap so that consecutive logical tiles run on one XCD. The dispatcher hands
// workgroup i of a 1-D grid to XCD i % 8; tiles of one head share K/V, and keeping them on
// one XCD keeps that K/V in one L2.
__device__ inline int xcd_remap(int wg, int nwg) {
  if ((nwg & 7) != 0) return wg;
  return (wg & 7) * (nwg >> 3) + (wg >> 3);
}

// Backward arguments (bf16 / fp16 inputs; gradients in fp32).
struct BwdArgs {
  const void* q;      // [B, H, Nq, d] in_dtype
  const void* k;      // [B, H_kv, Nk, d] in_dtype
  const void* v;      // [B, H_kv, Nk, d] in_dtype
  const void* o;      // [B, H, Nq, d] o_dtype (forward output)
  const void* dout;   // [B, H, Nq, d] in_dtype
  const float* lse;   // [B, H, Nq] row log-sum-exp of the scaled scores
  float* delta;       // [B, H, Nq] workspace: D_i = sum_c dO_ic O_ic
  float* dq;          // [B, H, Nq, d]
  float* dk;          // [B, H_kv, Nk, d]
  float* dv;          // [B, H_kv, Nk, d]
  int B, H, H_kv, Nq, Nk;
  int causal, causal_off;
  int o_dtype;
  float scale, scale_log2e;
};

hipError_t launch_fwd_mfma(const FwdArgs& a, int d, int in_dtype, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int d, int in_dtype, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_fwd_f32_rows(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_decode(const FwdArgs& a, int d, int in_dtype, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, int d, hipStream_t s);
hipError_t launch_probe_mfma(float* out, int nblocks, int iters, hipStream_t s);
hipError_t launch_probe_mfma_f32(float* out, int nblocks, int iters, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, unsigned* out, int nblocks, hipStream_t s);

// Query-row count up to which the split/decode kernel (one workgroup per query row and key
// range) is used instead of the tiled kernels.
constexpr int kDecodeMaxNq = 16;

}  // namespace fa
