// Types and small device helpers shared by the matrix-core kernels (forward and backward).
#pragma once

#include "fa_internal.h"

namespace fa {

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

// Maxima of scores (finite, or -inf for masked ones). fmaxf would first quiet a possible
// signalling NaN in every operand the compiler cannot prove canonical (one extra v_max_f32 x, x
// per operand, and an MFMA result is such an operand), which doubles the cost of a row maximum.
// The NaN-propagating maximum needs no quieting and becomes v_maximum3_f32 on gfx950, two new
// values per instruction; for scores it is the same maximum.
__device__ __forceinline__ float max2f(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Max / sum of a value and its counterpart in the other half of the wave (lane l and l ^ 32).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2f(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// One 16-byte-per-lane global -> LDS copy: lane i's 16 bytes land at lds + 16 * i. (A plain
// function, not a template: the host compile pass rejects this target builtin inside templates.)
__device__ __forceinline__ void global_to_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

// XOR swizzles of the 16-byte chunks of LDS row r: chunk c of a K row is stored at c ^ swzk(r),
// of a V row at c ^ swzv(r). The K tile is read one row per lane, 16 bytes at a time. With 64
// four-byte banks (256 bytes per cycle, measured ~246 B/clk per CU), 16 lanes of a 16-byte read
// go in one cycle when they hit 16 different 16-byte bank groups; a 128-byte K row spans half of
// them, so rows r and r + 1 alternate halves and (r >> 1) & 7 spreads 16 consecutive rows over
// all 16 groups (r & 7 repeats after 8 rows: a two-way conflict). The V tile is read by
// transposing reads of 4 rows x 8 bytes per 16-lane group; its swizzle was picked by timing.
__device__ __forceinline__ int swzk(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swzv(int r) { return ((r & 3) << 1); }

// d = 128 (256-byte rows: every row spans all 64 banks): chunk c of row r at
// c ^ (4 (r % 4) + (r / 4) % 4). Sixteen consecutive rows get sixteen different chunks, so a
// 16-byte row read (16 lanes, 16 rows, one chunk column) meets no conflict; and the 32 lanes of
// an 8-byte transposing read cover rows 4 i + j (j = 0..3) by 4 column chunks (2 bits) times
// 2 halves of a chunk, and the swizzle moves row j's chunks by 4 j, into the two chunk bits the
// columns leave free, so those lanes also hit 32 different bank pairs. (The forward kernel keeps
// swzk / swzv at d = 128, which give both kinds of read two-way conflicts: there this swizzle
// took the conflicts to zero, counted with SQ_LDS_BANK_CONFLICT, but measured 2 % slower.)
__device__ __forceinline__ int swz128(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Tiles read both ways (rows and transposed; the backward kernels' Q, dO, K and V tiles). At
// d = 64 the bits of (r >> 1) % 8 in reverse order: still a different chunk for each row pair of
// 16 consecutive rows (row reads), and bit 1 of r, which tells the two row pairs of a
// transposing read's 4-row group apart, lands in chunk bit 2, which its column chunks leave free
// (swzk puts bit 3 there: a two-way conflict). At d = 128 swz128.
template <int D>
__device__ __forceinline__ int swz_rt(int r) {
  return D == 128 ? swz128(r) : ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1));
}

}  // namespace fa
