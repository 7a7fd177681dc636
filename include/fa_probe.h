/*
 * fa_probe.h -- measurement probes exported by libfa.so (not part of the attention path).
 *
 * The attention kernels are reported against two ceilings: the chip's published peaks and the
 * rates these probes sustain on the same GPU in the same process. Neither probe computes
 * anything of the attention method; they exist so that "% of measured" figures can be
 * reproduced from this library alone. Statuses and fa_last_error() as in fa.h.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_probe_mfma_bf16 -- a matrix-core throughput probe.
 *
 * Launches `nblocks` workgroups of 4 waves; every wave issues iters * 8 dense bf16 MFMAs of
 * shape 32x32x16 (32768 flops each) on register operands, with eight independent accumulators.
 * Total work: nblocks * 4 * iters * 8 * 32768 flops; the caller times the launch.
 *   out        device buffer of out_elems fp32 values; receives one checksum per thread, so it
 *              must hold nblocks * 256 values (FA_EINVAL otherwise).
 *   nblocks    1 .. 2^20;  iters  1 .. 2^20.
 */
fa_status fa_probe_mfma_bf16(float* out, long long out_elems, int nblocks, int iters, void* stream);

/*
 * fa_probe_mfma_f32 -- the same probe with fp32 MFMAs of shape 16x16x4 (2048 flops each): every
 * wave issues iters * 8 of them on register operands, eight independent accumulators. Total
 * work: nblocks * 4 * iters * 8 * 2048 flops. Arguments and errors as fa_probe_mfma_bf16.
 */
fa_status fa_probe_mfma_f32(float* out, long long out_elems, int nblocks, int iters, void* stream);

/*
 * fa_probe_hbm_read -- a streaming-read bandwidth probe.
 *
 * Reads every byte of `src` once with nontemporal 16-byte loads: workgroup b of `nblocks` (256
 * threads) reads the b-th of nblocks contiguous chunks, eight loads in flight per lane, and every
 * thread writes one XOR checksum.
 *   src        device buffer of `bytes` bytes, 16-byte aligned; bytes a positive multiple of 16.
 *   out        device buffer of out_elems uint32 values, at least nblocks * 256 (FA_EINVAL otherwise).
 *   nblocks    1 .. 2^20.
 * Use a buffer well above the 256 MB last-level cache so that the rate is HBM's.
 */
fa_status fa_probe_hbm_read(const void* src, long long bytes, unsigned* out, long long out_elems, int nblocks,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
