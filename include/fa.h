/*
 * fa.h -- C ABI of libfa.so, a FlashAttention forward pass (and its gradients) for AMD MI355X
 * (gfx950).
 *
 * The operation (one attention head; every (b, h) pair is independent):
 *
 *     S = scale * Q K^T                        [Nq, Nk]
 *     P = softmax(S) along each row            [Nq, Nk]
 *     O = P V                                  [Nq, d]
 *
 * as defined by "FlashAttention 简化版：Tiling + Online Softmax" (forceinjection.github.io), §1.1,
 * and computed the way §2.3 and §3.1 of that page lay out: Q is cut into row tiles, K and V
 * stream past each Q tile in key tiles, and every query row keeps a running maximum m, a
 * running sum l of exp(s - m) and an accumulator; when a key tile raises m, l and the
 * accumulator are scaled by exp(m_old - m_new), and the accumulator is divided by l once,
 * after the last key tile. No [Nq, Nk] matrix is ever written to memory.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense and contiguous, row-major with d innermost: Q [B, H, Nq, d],
 *     K and V [B, H, Nk, d], O [B, H, Nq, d]. Element (b, h, i, c) sits at
 *     ((b*H + h)*N + i)*d + c. d (the head dimension) must be 64 or 128.
 *   - Every pointer is a device pointer (hipMalloc / torch memory) aligned to 16 bytes
 *     (m_out, l_out, part_m, part_l: 4 bytes). A pointer may be NULL only when its tensor
 *     holds no elements. The caller owns all memory. The library never allocates device memory.
 *   - Arithmetic: scores, the running maximum m, the running sum l and the output
 *     accumulator are fp32 for every input type. With bf16/fp16 inputs the two products
 *     QK^T and PV run on the matrix cores with fp32 accumulation; the probabilities P are
 *     rounded to the input type (round to nearest even) for PV only, while l sums the
 *     unrounded fp32 values -- the precision scheme of demo 4 of "CS349E 第 11 讲
 *     01_online_softmax.py".
 *   - m_out / l_out (optional, NULL to skip), shape [B, H, Nq] fp32: m is the row maximum of
 *     S and l = sum_j exp(S_ij - m), so softmax(S)_ij = exp(S_ij - m_i) / l_i (the statistics
 *     Exercise 5 of "Flash Attention 代码填空 (Level 2-3)" keeps for the backward pass).
 *   - All calls are asynchronous on `stream` (a hipStream_t; NULL means the null stream).
 *   - Errors: every call validates its arguments on the host before touching the device and
 *     returns a status; nothing aborts, throws or prints. FA_EINVAL: a bad pointer, size,
 *     dtype, scale or alignment. FA_EUNSUPPORTED: a valid request the library does not
 *     implement (e.g. d = 96). FA_EHIP: the HIP runtime reported an error when launching.
 *     fa_last_error() then returns a description (per thread, valid until the next call).
 *     B*H = 0 or Nq = 0 is a successful no-op. Nk must be >= 1 (softmax over no keys is
 *     undefined). Calls that overlap on one stream are ordered; calls on different streams
 *     that write the same buffers race.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 4
#define FA_MAX_SPLITS 256

typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_F16 = 2 } fa_dtype;

typedef enum { FA_OK = 0, FA_EINVAL = 1, FA_EUNSUPPORTED = 2, FA_EHIP = 3 } fa_status;

/*
 * fa_fwd -- O = softmax(scale * Q K^T) V for every (b, h).
 *
 * Defined by "FlashAttention 简化版：Tiling + Online Softmax" §1.1 (standard attention) and
 * computed as its §3.1 tiled loop with the online-softmax state of §2.3.
 *   q, k, v   [B,H,Nq,d], [B,H,Nk,d], [B,H,Nk,d] in `in_dtype` (FA_F32, FA_BF16, FA_F16).
 *   o         [B,H,Nq,d] in `out_dtype`, which is FA_F32 or equal to `in_dtype`.
 *   m_out, l_out  optional [B,H,Nq] fp32 row statistics (see above), or NULL.
 *   scale     finite and >= 0; usually 1/sqrt(d) (the pages' scale). 0 gives uniform weights.
 * No output (o, m_out, l_out) may overlap an input or another output (FA_EINVAL).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o,
                 float* m_out, float* l_out,
                 int B, int H, int Nq, int Nk, int d, float scale,
                 fa_dtype in_dtype, fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_split -- split-KV partial states (flash-decoding).
 *
 * The key range of every head is cut into `num_splits` contiguous parts; part c covers keys
 * [floor(c*Nk/num_splits), floor((c+1)*Nk/num_splits)) and is never empty. For each part the
 * call writes the partial state (m, l, o) of "CS349E 第 11 讲 01_online_softmax.py" demo 2:
 *   part_m [S,B,H,Nq] fp32   m = max over the part's keys of S_ij
 *   part_l [S,B,H,Nq] fp32   l = sum over the part's keys of exp(S_ij - m)
 *   part_o [S,B,H,Nq,d] fp32 o = sum over the part's keys of exp(S_ij - m) * V_j  (NOT divided by l)
 * with S = num_splits, 1 <= num_splits <= min(Nk, FA_MAX_SPLITS). fa_merge_states combines
 * them; the merged result equals fa_fwd's up to rounding. The caller owns the three buffers,
 * which must not overlap q, k, v or one another (FA_EINVAL).
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v,
                       float* part_m, float* part_l, float* part_o,
                       int num_splits, int B, int H, int Nq, int Nk, int d, float scale,
                       fa_dtype in_dtype, void* stream);

/*
 * fa_fwd_ext -- fa_fwd with grouped K/V heads and an optional causal mask.
 *
 * "FlashAttention 简化版：Tiling + Online Softmax" §7 names both as the next steps after the
 * plain forward pass (a causal mask folded into the tiling, for decoder models; multi-query /
 * grouped-query attention, to cut K/V memory) without fixing a convention; these are the ones
 * taken:
 *   H_kv      number of K/V heads: k, v are [B,H_kv,Nk,d]; H must be a multiple of H_kv.
 *             Query head h reads K/V head h / (H / H_kv) (consecutive query heads share one).
 *             H_kv = H is fa_fwd; H_kv = 1 is multi-query attention.
 *   causal    0: no mask. 1: query row i sees only keys j <= i + (Nk - Nq) -- the usual
 *             decoder mask when Nq = Nk; with Nq < Nk the queries are the last Nq positions of
 *             the key sequence (the last row sees every key). Requires Nq <= Nk, so every row
 *             keeps at least one key. Masked scores are -inf: they take part in neither m, l
 *             nor O.
 * Everything else (q, o, m_out, l_out, scale, dtypes, errors) is as in fa_fwd. Key tiles that
 * lie wholly past a query tile's last visible key are skipped, so a causal call does about
 * half the work of an unmasked one at Nq = Nk.
 */
fa_status fa_fwd_ext(const void* q, const void* k, const void* v, void* o,
                     float* m_out, float* l_out,
                     int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                     fa_dtype in_dtype, fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_lse -- fa_fwd_ext that also stores each row's log-sum-exp, the statistic the backward
 * pass needs.
 *
 * "Flash Attention 代码填空 (Level 2-3)" Exercise 5 keeps the row statistics m and l of the
 * forward pass so that the backward pass can recompute P without storing it; "CS349E 第 11 讲
 * 01_online_softmax.py" notes that FlashAttention-2 keeps a single number per row instead, the
 * log-sum-exp L = m + ln(l), from which P_ij = exp(S_ij - L_i).
 *   lse  [B,H,Nq] fp32, receives L_i = m_i + ln(l_i) of the scaled scores S (natural log).
 * Everything else as in fa_fwd_ext. lse must not overlap q, k, v or o.
 */
fa_status fa_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                     fa_dtype in_dtype, fa_dtype out_dtype, void* stream);

/*
 * fa_bwd -- gradients of O = softmax(scale * Q K^T) V with respect to Q, K and V.
 *
 * "Flash Attention 代码填空 (Level 2-3)" Exercise 5: the backward pass recomputes P from the
 * stored row statistics, P_ij = exp(S_ij - L_i), and accumulates dV_j = sum_i P_ij^T dO_i; the
 * other two gradients follow from the same definition by the chain rule
 * ("FlashAttention 简化版：Tiling + Online Softmax" §7 lists the backward pass, recomputation
 * plus blockwise gradients, as the first extension):
 *     dP = dO V^T,   dS_ij = P_ij (dP_ij - D_i),   D_i = sum_c dO_ic O_ic,
 *     dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
 *   q, k, v   the forward inputs (layouts and H_kv, causal as in fa_fwd_ext), FA_BF16 or FA_F16.
 *   o         [B,H,Nq,d] the forward output, in o_dtype (FA_F32 or in_dtype).
 *   dout      [B,H,Nq,d] dL/dO, in in_dtype.
 *   lse       [B,H,Nq] fp32 row log-sum-exp from fa_fwd_lse (same q, k, scale, causal).
 *   delta     [B,H,Nq] fp32 workspace owned by the caller; receives D_i.
 *   dq        [B,H,Nq,d] fp32; dk, dv [B,H_kv,Nk,d] fp32. With grouped heads dk and dv of a
 *             K/V head sum over the query heads that read it.
 * No [Nq, Nk] matrix is stored: P and dS are recomputed tile by tile, rounded to in_dtype only
 * as matrix-core operands, and accumulated in fp32. Every output element is written by exactly
 * one workgroup (no atomics), so results are bitwise reproducible. Outputs must not overlap any
 * input or each other. fp32 inputs return FA_EUNSUPPORTED. Nq = 0 gives dk = dv = 0.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, float* delta, float* dq, float* dk, float* dv,
                 int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                 fa_dtype in_dtype, fa_dtype o_dtype, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and results,
 * with no `delta` argument. D (one fp32 per query row) is kept in a buffer built into the library
 * -- a file-scope device array of FA_NOALLOC_MAX_ROWS floats (16 MiB) that every GPU the library
 * runs on holds until the process ends -- instead of a caller workspace. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine). Its first call on a device is its
 * set-up: it looks up that device's copy of the buffer, and the HIP runtime loads the buffer onto
 * the device at that point (about 18 MiB of device memory, once); later calls leave device memory
 * as it is. A caller that must not see even that can make one call outside the region it guards.
 *   B*H*Nq must be <= FA_NOALLOC_MAX_ROWS (FA_EINVAL otherwise; fa_bwd has no such limit).
 * All calls on one GPU share that GPU's buffer: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and give wrong gradients; calls ordered on
 * one stream do not. D is written before it is read within every call, so nothing left by an
 * earlier call is used. Everything else (arguments, layouts, errors) as in fa_bwd.
 */
#define FA_NOALLOC_MAX_ROWS 4194304
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, float* dq, float* dk, float* dv,
                         int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                         fa_dtype in_dtype, fa_dtype o_dtype, void* stream);

/*
 * fa_fwd_split_ext -- fa_fwd_split with grouped K/V heads and an optional causal mask.
 *
 * H_kv and causal as in fa_fwd_ext; the partition and the state layouts as in fa_fwd_split.
 * Under the mask a part that holds no key a row may see gives that row the empty state
 * m = -inf, l = 0, o = 0, which fa_merge_states weighs 0. (With Nq <= Nk part 0 always holds
 * key 0, which every row sees.)
 */
fa_status fa_fwd_split_ext(const void* q, const void* k, const void* v,
                           float* part_m, float* part_l, float* part_o,
                           int num_splits, int B, int H, int H_kv, int Nq, int Nk, int d, float scale,
                           int causal, fa_dtype in_dtype, void* stream);

/*
 * fa_merge_states -- fold partial states into the attention output.
 *
 * For every (b, h, i) the states of the `num_splits` parts are merged one after another in
 * the order given by `order` (a host array holding a permutation of 0..num_splits-1, read
 * during the call; NULL means 0, 1, ..., num_splits-1). One merge step is
 *   m = max(m_a, m_b); l = l_a e^(m_a - m) + l_b e^(m_b - m); o = o_a e^(m_a - m) + o_b e^(m_b - m),
 * the rule that makes the result independent of the order up to rounding ("CS349E 第 11 讲
 * 01_online_softmax.py" demo 2, derived from the recurrence of "从零手写 FlashAttention" §4).
 * A part with m = -inf (no keys) has weight 0. Finally O = o / l in `out_dtype` (FA_F32,
 * FA_BF16 or FA_F16), and, when not NULL, m_out / l_out receive the merged m and l. A row whose
 * parts are all empty (possible under the causal mask of fa_fwd_split_ext only for rows that see
 * no key at all) gets O = 0, m = -inf, l = 0.
 * Layouts as in fa_fwd_split; o is [B,H,Nq,d]. No output (o, m_out, l_out) may overlap a partial
 * state or another output (FA_EINVAL).
 */
fa_status fa_merge_states(const float* part_m, const float* part_l, const float* part_o,
                          const int* order, int num_splits, int B, int H, int Nq, int d,
                          void* o, fa_dtype out_dtype, float* m_out, float* l_out, void* stream);

/*
 * fa_fwd_split_lse -- split-KV partial states in the (lse, o) form.
 *
 * "CS349E 第 11 讲 01_online_softmax.py" (its note after demo 2): flash-decoding stores, per key
 * range s, the output already divided by that range's own l, o_s / l_s, and lse_s = m_s + ln(l_s)
 * -- one value fewer than (m, l, o) -- and combines the ranges with weights exp(lse_s - lse).
 *   part_lse [S,B,H,Nq] fp32   lse_s (-inf for a range holding no key the row may see)
 *   part_o   [S,B,H,Nq,d] fp32 o_s / l_s (0 for such a range)
 * Partition, H_kv, causal, dtypes and errors as in fa_fwd_split_ext.
 */
fa_status fa_fwd_split_lse(const void* q, const void* k, const void* v, float* part_lse, float* part_o,
                           int num_splits, int B, int H, int H_kv, int Nq, int Nk, int d, float scale,
                           int causal, fa_dtype in_dtype, void* stream);

/*
 * fa_merge_lse -- combine (lse, o) partial states into the attention output.
 *
 * lse = ln(sum_s exp(lse_s)) (computed as max_s lse_s + ln sum_s exp(lse_s - max)), then
 * O = sum_s exp(lse_s - lse) o_s, both sums taken in the order given by `order` (a host
 * permutation of 0..num_splits-1; NULL = ascending). Ranges with lse_s = -inf weigh 0; a row whose
 * ranges are all empty gets O = 0 and lse = -inf. o [B,H,Nq,d] in out_dtype; lse_out [B,H,Nq] fp32
 * (NULL to skip) receives lse, the row log-sum-exp of the whole key range.
 */
fa_status fa_merge_lse(const float* part_lse, const float* part_o, const int* order, int num_splits,
                       int B, int H, int Nq, int d, void* o, fa_dtype out_dtype, float* lse_out, void* stream);

/* Name of a status code ("FA_OK", ...); never NULL. */
const char* fa_status_string(int status);

/* Description of the last non-OK status returned on this thread ("" if none). */
const char* fa_last_error(void);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
