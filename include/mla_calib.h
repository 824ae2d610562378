/*
 * mla_calib.h -- calibration calls of libmla: the streaming HBM read rate, the
 * rate of the merges' several-reads-one-write pattern and the dense bf16 MFMA
 * rate that one gfx950 GPU actually delivers.
 *
 * They are measurement aids, not part of the attention path: the roofline
 * fractions of the decode and merge kernels are quoted against the vendor
 * peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s) and against what these
 * calls reach on the same GPU.  The caller times them (for example with HIP
 * events on hip_stream); the calls only enqueue one kernel each.
 *
 * Conventions as in mla.h: device pointers owned by the caller, work enqueued
 * on hip_stream (a hipStream_t, NULL = the null stream), status codes, no
 * host reads of device memory.
 */
#ifndef MLA_CALIB_H
#define MLA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* 32-bit words every sink must hold. */
#define MLA_CALIB_SINK_WORDS (1 << 20)
/* Launch shape of the MFMA loop: workgroups of MLA_CALIB_MFMA_THREADS threads
 * (two waves per SIMD on the 256-CU part). */
#define MLA_CALIB_MFMA_GROUPS 512
#define MLA_CALIB_MFMA_THREADS 256

/*
 * mla_calib_hbm_read -- read `bytes` bytes at `buf` once, 16 bytes per load,
 * with a grid of up to 4096 workgroups striding over the buffer (eight loads
 * in flight per thread).  nontemporal != 0 issues the loads with the
 * non-temporal hint (the hint the 16-head decode uses for cache rows).  Each
 * thread folds what it read with xor and writes one word to `sink` (uint32
 * [MLA_CALIB_SINK_WORDS]; the values are meaningless).  Use a buffer several
 * times the 256 MB last-level cache so that the rate is HBM's.
 * Returns MLA_OK (bytes == 0: nothing enqueued), MLA_ERR_NULL, MLA_ERR_SHAPE
 * (bytes or buf not a multiple of 16) or MLA_ERR_HIP.
 */
mla_status mla_calib_hbm_read(const void* buf, size_t bytes, int32_t nontemporal, uint32_t* sink,
                              void* hip_stream);

/*
 * mla_calib_hbm_gather -- the merges' access pattern: `inputs` (1, 2, 4 or 8)
 * buffers of bytes_per_input bytes, consecutive at `in`, each read once, and
 * one buffer of bytes_per_input bytes at `out` written once with their xor
 * (16-byte words, a grid of up to 1024 workgroups striding over them).  The
 * rate is (inputs + 1) * bytes_per_input over the call's time; use inputs
 * larger than the 256 MB last-level cache together.  Returns MLA_OK
 * (bytes_per_input == 0: nothing enqueued), MLA_ERR_NULL, MLA_ERR_SHAPE
 * (sizes or pointers not multiples of 16, inputs not 1, 2, 4 or 8) or
 * MLA_ERR_HIP.
 */
mla_status mla_calib_hbm_gather(const void* in, size_t bytes_per_input, int32_t inputs, void* out,
                                void* hip_stream);

/*
 * mla_calib_mfma_bf16 -- MLA_CALIB_MFMA_GROUPS workgroups, every wave running
 * `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16 accumulation
 * chains on operands held in registers; one float per thread goes to `sink`
 * (float [MLA_CALIB_SINK_WORDS]).  The flops it performs are
 * mla_calib_mfma_flops(iters).  Returns MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE
 * (iters < 0) or MLA_ERR_HIP.
 */
mla_status mla_calib_mfma_bf16(int32_t iters, float* sink, void* hip_stream);

/* Flops of one mla_calib_mfma_bf16 call with this iteration count (-1 for
 * iters < 0); pure host arithmetic. */
double mla_calib_mfma_flops(int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CALIB_H */
