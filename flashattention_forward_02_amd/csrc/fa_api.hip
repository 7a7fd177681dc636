// C ABI of libfa.so: argument validation, kernel selection and error reporting.
// The contract of every entry point is documented in include/fa.h.

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "fa.h"
#include "fa_probe.h"
#include "fa_internal.h"

namespace {

thread_local char g_last_error[512];

fa_status fail(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bool valid_dtype(int dt) { return dt == FA_F32 || dt == FA_BF16 || dt == FA_F16; }
size_t dtype_size(int dt) { return dt == FA_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

// True when some output buffer overlaps an input buffer or another output (null or empty buffers
// overlap nothing).
bool outputs_overlap(const void* const* outs, const size_t* outsz, int nout, const void* const* ins,
                     const size_t* insz, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return true;
  }
  return false;
}

// Shape, dtype and scale checks shared by fa_fwd and fa_fwd_split.
fa_status check_common(const char* fn, const void* q, const void* k, const void* v, int B, int H, int Nq, int Nk,
                       int d, float scale, int in_dtype) {
  if (B < 0 || H < 0 || Nq < 0) return fail(FA_EINVAL, "%s: B=%d, H=%d, Nq=%d must be >= 0", fn, B, H, Nq);
  if (Nk < 1) return fail(FA_EINVAL, "%s: Nk=%d; softmax over an empty key set is undefined (Nk >= 1)", fn, Nk);
  // A pointer may be NULL only when its tensor holds no elements.
  const bool no_q = (size_t)B * H * Nq == 0, no_kv = (size_t)B * H == 0;
  if ((!q && !no_q) || ((!k || !v) && !no_kv))
    return fail(FA_EINVAL, "%s: q, k and v must be non-NULL device pointers", fn);
  if (!valid_dtype(in_dtype)) return fail(FA_EINVAL, "%s: in_dtype=%d is not FA_F32, FA_BF16 or FA_F16", fn, in_dtype);
  if (!(scale >= 0.f) || !isfinite(scale)) return fail(FA_EINVAL, "%s: scale=%g must be finite and >= 0", fn, (double)scale);
  if (d <= 0) return fail(FA_EINVAL, "%s: d=%d must be > 0", fn, d);
  if (d != 64 && d != 128) return fail(FA_EUNSUPPORTED, "%s: head dimension d=%d (supported: 64, 128)", fn, d);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(FA_EINVAL, "%s: q, k and v must be 16-byte aligned", fn);
  return FA_OK;
}

// Base-2 growth of the running max tolerated before the matrix-core kernel rescales its state
// (see fwd_mfma.hip). 8 keeps every p below 2^8; FA_RESCALE_THRESHOLD (read once, for tests)
// can set it, e.g. 0 to rescale whenever the max grows.
float rescale_threshold() {
  static const float tau = [] {
    const char* e = getenv("FA_RESCALE_THRESHOLD");
    if (!e || !*e) return 8.0f;
    const float v = strtof(e, nullptr);
    return (v >= 0.f && v <= 16.f) ? v : 8.0f;
  }();
  return tau;
}

fa::FwdArgs make_args(const void* q, const void* k, const void* v, int B, int H, int H_kv, int Nq, int Nk,
                      float scale, int causal) {
  fa::FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.causal = causal;
  a.causal_off = Nk - Nq;
  a.Nq = Nq;
  a.Nk = Nk;
  a.num_splits = 1;
  a.scale = scale;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.rescale_threshold = rescale_threshold();
  return a;
}

// fp32: the one-workgroup-per-row kernel takes every call with at most 16 query rows, and also
// small calls with more: it spreads the rows over the compute units, where a small launch of the
// tiled kernels leaves most of them idle. Measured faster up to 512 rows per launch at d = 64
// (B=H=1, N=256: 9.2 -> 6.4 us per call; B=1, H=2, N=256: 9.2 -> 8.1; 512 queries x 1024 keys:
// 17.4 -> 15.1) and up to 1024 at d = 128, where the tiled kernel is the VALU one (4 heads of
// 256 x 1024: 74 -> 42 us); slower beyond (1024 rows at d = 64: 9.3 -> 14.0 us).
bool f32_by_rows(const fa::FwdArgs& a, int d) {
  const long long rows = (long long)a.B * a.H * a.Nq * a.num_splits;
  return a.Nq <= fa::kDecodeMaxNq || rows <= (d == 64 ? 512 : 1024);
}

fa_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(FA_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return FA_OK;
}

// Checks of the grouped-head count and the mask flag (fa_fwd_ext, fa_fwd_split_ext).
fa_status check_ext(const char* fn, int H, int H_kv, int Nq, int Nk, int causal) {
  if (H_kv < 1 || (H > 0 && H % H_kv != 0))
    return fail(FA_EINVAL, "%s: H=%d must be a positive multiple of H_kv=%d", fn, H, H_kv);
  if (causal != 0 && causal != 1) return fail(FA_EINVAL, "%s: causal=%d must be 0 or 1", fn, causal);
  if (causal && Nq > Nk)
    return fail(FA_EINVAL, "%s: the causal mask needs Nq <= Nk (Nq=%d, Nk=%d): rows would see no key", fn, Nq, Nk);
  return FA_OK;
}

fa_status fwd_impl(const char* fn, const void* q, const void* k, const void* v, void* o, float* m_out, float* l_out,
                   float* lse_out, int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                   fa_dtype in_dtype, fa_dtype out_dtype, void* stream) {
  fa_status st = check_common(fn, q, k, v, B, H, Nq, Nk, d, scale, in_dtype);
  if (st != FA_OK) return st;
  if ((st = check_ext(fn, H, H_kv, Nq, Nk, causal)) != FA_OK) return st;
  if (!o && (size_t)B * H * Nq != 0) return fail(FA_EINVAL, "%s: o must be a non-NULL device pointer", fn);
  if (out_dtype != FA_F32 && out_dtype != in_dtype)
    return fail(FA_EINVAL, "%s: out_dtype=%d must be FA_F32 or equal to in_dtype=%d", fn, (int)out_dtype, (int)in_dtype);
  if (!aligned16(o)) return fail(FA_EINVAL, "%s: o must be 16-byte aligned", fn);
  if (!aligned4(m_out) || !aligned4(l_out) || !aligned4(lse_out))
    return fail(FA_EINVAL, "%s: m_out, l_out and lse must be 4-byte aligned", fn);
  if ((size_t)B * H == 0 || Nq == 0) return FA_OK;
  const size_t obytes = (size_t)B * H * Nq * d * dtype_size(out_dtype);
  const size_t qbytes = (size_t)B * H * Nq * d * dtype_size(in_dtype);
  const size_t kvbytes = (size_t)B * H_kv * Nk * d * dtype_size(in_dtype);
  const size_t rbytes = (size_t)B * H * Nq * sizeof(float);
  const void* ins[] = {q, k, v};
  const size_t insz[] = {qbytes, kvbytes, kvbytes};
  const void* outs[] = {o, m_out, l_out, lse_out};
  const size_t outsz[] = {obytes, m_out ? rbytes : 0, l_out ? rbytes : 0, lse_out ? rbytes : 0};
  if (outputs_overlap(outs, outsz, 4, ins, insz, 3))
    return fail(FA_EINVAL, "%s: an output (o, m_out, l_out, lse) overlaps q, k, v or another output", fn);

  fa::FwdArgs a = make_args(q, k, v, B, H, H_kv, Nq, Nk, scale, causal);
  a.o = o;
  a.m_out = m_out;
  a.l_out = l_out;
  a.lse_out = lse_out;
  a.out_dtype = out_dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (in_dtype == FA_F32) e = f32_by_rows(a, d) ? fa::launch_fwd_f32_rows(a, d, s) : fa::launch_fwd_f32(a, d, s);
  else if (Nq <= fa::kDecodeMaxNq) e = fa::launch_decode(a, d, in_dtype, s);
  else e = fa::launch_fwd_mfma(a, d, in_dtype, s);
  return launched(fn, e);
}

fa_status fwd_split_impl(const char* fn, const void* q, const void* k, const void* v, float* part_m, float* part_l,
                         float* part_o, int num_splits, int B, int H, int H_kv, int Nq, int Nk, int d, float scale,
                         int causal, fa_dtype in_dtype, void* stream, bool lse_form = false) {
  fa_status st = check_common(fn, q, k, v, B, H, Nq, Nk, d, scale, in_dtype);
  if (st != FA_OK) return st;
  if ((st = check_ext(fn, H, H_kv, Nq, Nk, causal)) != FA_OK) return st;
  if ((!part_m || (!part_l && !lse_form) || !part_o) && (size_t)B * H * Nq != 0)
    return fail(FA_EINVAL, lse_form ? "%s: part_lse and part_o must be non-NULL"
                                    : "%s: part_m, part_l and part_o must be non-NULL", fn);
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS || num_splits > Nk)
    return fail(FA_EINVAL, "%s: num_splits=%d must be in [1, min(Nk=%d, %d)]", fn, num_splits, Nk, FA_MAX_SPLITS);
  if (!aligned16(part_o) || !aligned4(part_m) || !aligned4(part_l))
    return fail(FA_EINVAL, "%s: part_o must be 16-byte and part_m, part_l 4-byte aligned", fn);
  if ((size_t)B * H == 0 || Nq == 0) return FA_OK;
  {
    const size_t es = dtype_size(in_dtype), rows = (size_t)num_splits * B * H * Nq;
    const size_t qbytes = (size_t)B * H * Nq * d * es, kvbytes = (size_t)B * H_kv * Nk * d * es;
    const void* ins[] = {q, k, v};
    const size_t insz[] = {qbytes, kvbytes, kvbytes};
    const void* outs[] = {part_m, lse_form ? nullptr : part_l, part_o};
    const size_t outsz[] = {rows * 4, lse_form ? 0 : rows * 4, rows * d * 4};
    if (outputs_overlap(outs, outsz, 3, ins, insz, 3))
      return fail(FA_EINVAL, "%s: a partial-state buffer overlaps q, k, v or another partial-state buffer", fn);
  }

  fa::FwdArgs a = make_args(q, k, v, B, H, H_kv, Nq, Nk, scale, causal);
  a.part_m = part_m;
  a.part_l = part_l;
  a.part_o = part_o;
  a.num_splits = num_splits;
  a.split_mode = lse_form ? 2 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (in_dtype == FA_F32) e = f32_by_rows(a, d) ? fa::launch_fwd_f32_rows(a, d, s) : fa::launch_fwd_f32(a, d, s);
  else if (Nq <= fa::kDecodeMaxNq) e = fa::launch_decode(a, d, in_dtype, s);
  else e = fa::launch_fwd_mfma(a, d, in_dtype, s);
  return launched(fn, e);
}

// Shared by fa_merge_states ((m, l, o) parts) and fa_merge_lse ((lse, o) parts: part_l unused).
fa_status merge_impl(const char* fn, bool lse_form, const float* part_m, const float* part_l, const float* part_o,
                     const int* order, int num_splits, int B, int H, int Nq, int d, void* o, fa_dtype out_dtype,
                     float* m_out, float* l_out, float* lse_out, void* stream) {
  if (B < 0 || H < 0 || Nq < 0) return fail(FA_EINVAL, "%s: B=%d, H=%d, Nq=%d must be >= 0", fn, B, H, Nq);
  if ((!part_m || (!part_l && !lse_form) || !part_o || !o) && (size_t)B * H * Nq != 0)
    return fail(FA_EINVAL, lse_form ? "%s: part_lse, part_o and o must be non-NULL"
                                    : "%s: part_m, part_l, part_o and o must be non-NULL", fn);
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS)
    return fail(FA_EINVAL, "%s: num_splits=%d must be in [1, %d]", fn, num_splits, FA_MAX_SPLITS);
  if (!valid_dtype(out_dtype)) return fail(FA_EINVAL, "%s: out_dtype=%d is not a fa_dtype", fn, (int)out_dtype);
  if (d <= 0) return fail(FA_EINVAL, "%s: d=%d must be > 0", fn, d);
  if (d != 64 && d != 128) return fail(FA_EUNSUPPORTED, "%s: head dimension d=%d (supported: 64, 128)", fn, d);
  if (!aligned16(part_o) || !aligned16(o) || !aligned4(part_m) || !aligned4(part_l) || !aligned4(m_out) ||
      !aligned4(l_out) || !aligned4(lse_out))
    return fail(FA_EINVAL, "%s: part_o and o must be 16-byte aligned, the rest 4-byte aligned", fn);

  fa::MergeArgs a;
  memset(&a, 0, sizeof(a));
  bool seen[FA_MAX_SPLITS] = {false};
  for (int i = 0; i < num_splits; ++i) {
    const int s = order ? order[i] : i;
    if (s < 0 || s >= num_splits || seen[s])
      return fail(FA_EINVAL, "%s: order is not a permutation of 0..%d (entry %d = %d)", fn, num_splits - 1, i, s);
    seen[s] = true;
    a.order[i] = (unsigned short)s;
  }
  const long long rows = (long long)B * H * Nq;
  if (rows == 0) return FA_OK;
  if (rows > 0x7fffffffLL) return fail(FA_EINVAL, "%s: B*H*Nq=%lld exceeds 2^31-1", fn, rows);
  {
    const size_t r = (size_t)rows, st = (size_t)num_splits * r;
    const void* ins[] = {part_m, lse_form ? nullptr : part_l, part_o};
    const size_t insz[] = {st * 4, lse_form ? 0 : st * 4, st * d * 4};
    const void* outs[] = {o, m_out, l_out, lse_out};
    const size_t outsz[] = {r * d * dtype_size(out_dtype), m_out ? r * 4 : 0, l_out ? r * 4 : 0,
                            lse_out ? r * 4 : 0};
    if (outputs_overlap(outs, outsz, 4, ins, insz, 3))
      return fail(FA_EINVAL, "%s: an output (o, m_out, l_out, lse) overlaps a partial state or another output", fn);
  }
  a.part_m = part_m;
  a.part_l = part_l;
  a.part_o = part_o;
  a.o = o;
  a.m_out = m_out;
  a.l_out = l_out;
  a.lse_out = lse_out;
  a.lse_format = lse_form ? 1 : 0;
  a.S = num_splits;
  a.rows = (int)rows;
  a.out_dtype = out_dtype;
  return launched(fn, fa::launch_merge(a, d, static_cast<hipStream_t>(stream)));
}

// ---- the built-in D buffer of fa_bwd_noalloc ----
// D (one fp32 per query row) lives in this file-scope device array instead of a caller workspace,
// for callers that cannot allocate device memory. Every GPU the library runs on holds its own copy
// until the process ends; its device address is looked up once per device (hipGetSymbolAddress
// with that device current) and the kernels receive that address. In host code the array's name is
// not a device address and is never passed to a kernel.
constexpr long long kScratchFloats = FA_NOALLOC_MAX_ROWS;   // 16 MiB of fp32
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device `stream` belongs to (the current device for the null
// stream), looked up on the first call for that device.
fa_status scratch_for_stream(const char* fn, void* stream, float** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_EHIP, "%s: cannot tell the stream's device: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_EUNSUPPORTED, "%s: device %d (at most %d devices)", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = (cur >= 0 && cur != dev) ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || !p)
      return fail(FA_EHIP, "%s: device address of the built-in D buffer on device %d: %s", fn, dev,
                  hipGetErrorString(e != hipSuccess ? e : hipErrorInvalidSymbol));
    if (e2 != hipSuccess) return fail(FA_EHIP, "%s: restoring device %d: %s", fn, cur, hipGetErrorString(e2));
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// fa_bwd and fa_bwd_noalloc. With use_scratch the D buffer is this device's copy of `scratch`
// (looked up after every argument check passed); otherwise it is the caller's `delta`.
fa_status bwd_impl(const char* fn, bool use_scratch, const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, float* delta, float* dq, float* dk, float* dv, int B, int H,
                   int H_kv, int Nq, int Nk, int d, float scale, int causal, fa_dtype in_dtype, fa_dtype o_dtype,
                   void* stream) {
  fa_status st = check_common(fn, q, k, v, B, H, Nq, Nk, d, scale, in_dtype);
  if (st != FA_OK) return st;
  if ((st = check_ext(fn, H, H_kv, Nq, Nk, causal)) != FA_OK) return st;
  if (in_dtype == FA_F32) return fail(FA_EUNSUPPORTED, "%s: fp32 inputs (supported: FA_BF16, FA_F16)", fn);
  if (o_dtype != FA_F32 && o_dtype != in_dtype)
    return fail(FA_EINVAL, "%s: o_dtype=%d must be FA_F32 or equal to in_dtype=%d", fn, (int)o_dtype, (int)in_dtype);
  const size_t nrows = (size_t)B * H * Nq;
  if ((!o || !dout || !lse || (!delta && !use_scratch) || !dq) && nrows != 0)
    return fail(FA_EINVAL, use_scratch ? "%s: o, dout, lse and dq must be non-NULL device pointers"
                                       : "%s: o, dout, lse, delta and dq must be non-NULL device pointers", fn);
  if (use_scratch && nrows > (size_t)kScratchFloats)
    return fail(FA_EINVAL, "%s: B*H*Nq=%zu exceeds the %lld rows of its built-in D buffer (use fa_bwd with a caller "
                "workspace)", fn, nrows, (long long)kScratchFloats);
  if ((!dk || !dv) && (size_t)B * H != 0) return fail(FA_EINVAL, "%s: dk and dv must be non-NULL device pointers", fn);
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse) ||
      !aligned4(delta))
    return fail(FA_EINVAL, "%s: o, dout, dq, dk, dv must be 16-byte and lse, delta 4-byte aligned", fn);
  if ((size_t)B * H == 0) return FA_OK;
  // Outputs must not overlap any input or each other (the built-in D buffer overlaps nothing).
  const size_t qb = nrows * d * 2, kvb = (size_t)B * H_kv * Nk * d * 2, ob = nrows * d * dtype_size(o_dtype);
  const size_t qf = nrows * d * 4, kvf = (size_t)B * H_kv * Nk * d * 4, rb = nrows * 4;
  const void* ins[] = {q, k, v, o, dout, lse};
  const size_t insz[] = {qb, kvb, kvb, ob, qb, rb};
  const void* outs[] = {delta, dq, dk, dv};
  const size_t outsz[] = {use_scratch ? 0 : rb, qf, kvf, kvf};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return fail(FA_EINVAL, "%s: an output overlaps an input", fn);
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return fail(FA_EINVAL, "%s: two outputs overlap", fn);
  }
  if (use_scratch) {   // every argument checked: now the device is touched
    fa_status st2 = scratch_for_stream(fn, stream, &delta);
    if (st2 != FA_OK) return st2;
  }
  fa::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.causal = causal;
  a.causal_off = Nk - Nq;
  a.o_dtype = o_dtype;
  a.scale = scale;
  a.scale_log2e = scale * 1.4426950408889634f;
  // (Nq = 0 launches only the dK / dV kernel, which then writes zeros.)
  return launched(fn, fa::launch_bwd(a, d, in_dtype, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* m_out, float* l_out, int B, int H,
                 int Nq, int Nk, int d, float scale, fa_dtype in_dtype, fa_dtype out_dtype, void* stream) {
  g_last_error[0] = 0;
  return fwd_impl("fa_fwd", q, k, v, o, m_out, l_out, nullptr, B, H, H > 0 ? H : 1, Nq, Nk, d, scale, 0, in_dtype,
                  out_dtype, stream);
}

fa_status fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* m_out, float* l_out, int B, int H,
                     int H_kv, int Nq, int Nk, int d, float scale, int causal, fa_dtype in_dtype, fa_dtype out_dtype,
                     void* stream) {
  g_last_error[0] = 0;
  return fwd_impl("fa_fwd_ext", q, k, v, o, m_out, l_out, nullptr, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype,
                  out_dtype, stream);
}

fa_status fa_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int Nq,
                     int Nk, int d, float scale, int causal, fa_dtype in_dtype, fa_dtype out_dtype, void* stream) {
  g_last_error[0] = 0;
  if (!lse && B > 0 && H > 0 && Nq > 0) return fail(FA_EINVAL, "fa_fwd_lse: lse must be a non-NULL device pointer");
  return fwd_impl("fa_fwd_lse", q, k, v, o, nullptr, nullptr, lse, B, H, H_kv, Nq, Nk, d, scale, causal, in_dtype,
                  out_dtype, stream);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 float* delta, float* dq, float* dk, float* dv, int B, int H, int H_kv, int Nq, int Nk, int d,
                 float scale, int causal, fa_dtype in_dtype, fa_dtype o_dtype, void* stream) {
  g_last_error[0] = 0;
  return bwd_impl("fa_bwd", false, q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, causal,
                  in_dtype, o_dtype, stream);
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, float* dq, float* dk, float* dv, int B, int H, int H_kv, int Nq, int Nk,
                         int d, float scale, int causal, fa_dtype in_dtype, fa_dtype o_dtype, void* stream) {
  g_last_error[0] = 0;
  return bwd_impl("fa_bwd_noalloc", true, q, k, v, o, dout, lse, nullptr, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale,
                  causal, in_dtype, o_dtype, stream);
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, float* part_m, float* part_l, float* part_o,
                       int num_splits, int B, int H, int Nq, int Nk, int d, float scale, fa_dtype in_dtype,
                       void* stream) {
  g_last_error[0] = 0;
  return fwd_split_impl("fa_fwd_split", q, k, v, part_m, part_l, part_o, num_splits, B, H, H > 0 ? H : 1, Nq, Nk, d,
                        scale, 0, in_dtype, stream);
}

fa_status fa_fwd_split_ext(const void* q, const void* k, const void* v, float* part_m, float* part_l, float* part_o,
                           int num_splits, int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                           fa_dtype in_dtype, void* stream) {
  g_last_error[0] = 0;
  return fwd_split_impl("fa_fwd_split_ext", q, k, v, part_m, part_l, part_o, num_splits, B, H, H_kv, Nq, Nk, d, scale,
                        causal, in_dtype, stream);
}

fa_status fa_merge_states(const float* part_m, const float* part_l, const float* part_o, const int* order,
                          int num_splits, int B, int H, int Nq, int d, void* o, fa_dtype out_dtype, float* m_out,
                          float* l_out, void* stream) {
  g_last_error[0] = 0;
  return merge_impl("fa_merge_states", false, part_m, part_l, part_o, order, num_splits, B, H, Nq, d, o, out_dtype,
                    m_out, l_out, nullptr, stream);
}

fa_status fa_fwd_split_lse(const void* q, const void* k, const void* v, float* part_lse, float* part_o,
                           int num_splits, int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                           fa_dtype in_dtype, void* stream) {
  g_last_error[0] = 0;
  return fwd_split_impl("fa_fwd_split_lse", q, k, v, part_lse, nullptr, part_o, num_splits, B, H, H_kv, Nq, Nk, d,
                        scale, causal, in_dtype, stream, true);
}

fa_status fa_merge_lse(const float* part_lse, const float* part_o, const int* order, int num_splits, int B, int H,
                       int Nq, int d, void* o, fa_dtype out_dtype, float* lse_out, void* stream) {
  g_last_error[0] = 0;
  return merge_impl("fa_merge_lse", true, part_lse, nullptr, part_o, order, num_splits, B, H, Nq, d, o, out_dtype,
                    nullptr, nullptr, lse_out, stream);
}

fa_status fa_probe_mfma_bf16(float* out, long long out_elems, int nblocks, int iters, void* stream) {
  g_last_error[0] = 0;
  const char* fn = "fa_probe_mfma_bf16";
  if (nblocks < 1 || nblocks > (1 << 20) || iters < 1 || iters > (1 << 20))
    return fail(FA_EINVAL, "%s: nblocks=%d and iters=%d must be in [1, 2^20]", fn, nblocks, iters);
  if (!out || !aligned4(out) || out_elems < (long long)nblocks * 256)
    return fail(FA_EINVAL, "%s: out must be a 4-byte aligned device buffer of >= nblocks * 256 = %lld floats", fn,
                (long long)nblocks * 256);
  return launched(fn, fa::launch_probe_mfma(out, nblocks, iters, static_cast<hipStream_t>(stream)));
}

fa_status fa_probe_mfma_f32(float* out, long long out_elems, int nblocks, int iters, void* stream) {
  g_last_error[0] = 0;
  const char* fn = "fa_probe_mfma_f32";
  if (nblocks < 1 || nblocks > (1 << 20) || iters < 1 || iters > (1 << 20))
    return fail(FA_EINVAL, "%s: nblocks=%d and iters=%d must be in [1, 2^20]", fn, nblocks, iters);
  if (!out || !aligned4(out) || out_elems < (long long)nblocks * 256)
    return fail(FA_EINVAL, "%s: out must be a 4-byte aligned device buffer of >= nblocks * 256 = %lld floats", fn,
                (long long)nblocks * 256);
  return launched(fn, fa::launch_probe_mfma_f32(out, nblocks, iters, static_cast<hipStream_t>(stream)));
}

fa_status fa_probe_hbm_read(const void* src, long long bytes, unsigned* out, long long out_elems, int nblocks,
                            void* stream) {
  g_last_error[0] = 0;
  const char* fn = "fa_probe_hbm_read";
  if (nblocks < 1 || nblocks > (1 << 20)) return fail(FA_EINVAL, "%s: nblocks=%d must be in [1, 2^20]", fn, nblocks);
  if (!src || !aligned16(src) || bytes <= 0 || bytes % 16 != 0)
    return fail(FA_EINVAL, "%s: src must be 16-byte aligned and bytes=%lld a positive multiple of 16", fn, bytes);
  if (!out || !aligned4(out) || out_elems < (long long)nblocks * 256)
    return fail(FA_EINVAL, "%s: out must be a 4-byte aligned device buffer of >= nblocks * 256 = %lld values", fn,
                (long long)nblocks * 256);
  if (overlaps(src, (size_t)bytes, out, (size_t)out_elems * 4)) return fail(FA_EINVAL, "%s: out overlaps src", fn);
  return launched(fn, fa::launch_probe_read(src, (size_t)bytes, out, nblocks, static_cast<hipStream_t>(stream)));
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_EINVAL: return "FA_EINVAL";
    case FA_EUNSUPPORTED: return "FA_EUNSUPPORTED";
    case FA_EHIP: return "FA_EHIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_last_error; }

int fa_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
