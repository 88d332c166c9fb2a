/*
 * vsa_probe.h - measurement aids of the VSA library for one AMD Instinct
 * MI355X (gfx950). They are not steps of the operator: they measure
 * properties of the chip that bound its kernels, so that the bounds quoted
 * with those kernels can be reproduced (bench.py --mode probe).
 *
 * Conventions as in vsa.h: device pointers, 16-byte aligned; work is
 * enqueued on `stream` (a hipStream_t, NULL = the null stream) and is
 * asynchronous; the caller times it (HIP events) and owns every buffer;
 * host-checkable faults return a vsa_status before anything is enqueued,
 * launch failures VSA_ERR_HIP.
 */
#ifndef VSA_PROBE_H
#define VSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix cores against independent vector-ALU work (the softmax budget of the
 * fine attention kernels). Launches 256 * waves_per_simd workgroups of four
 * waves (one per SIMD of a CU; waves_per_simd 1 or 2 per SIMD, held by the
 * workgroups' LDS allocation). Each wave runs `iters` rounds of four
 * independent chains of 32x32x16 bf16 MFMAs (32768 FLOP each), every MFMA
 * followed by `valu` independent vector instructions of kind `op` (0: fp32
 * FMA, 1: exp2): 4 * iters * 32768 FLOP per wave, 1024 * waves_per_simd
 * waves.
 * valu: 0, 1, 2, 4, 8 or 16; out: 65536 * waves_per_simd floats, written
 * (their values only keep the work from being removed).
 * Errors: VSA_ERR_NULL (out), VSA_ERR_UNSUPPORTED (valu, op or
 * waves_per_simd out of range), VSA_ERR_SHAPE (iters < 1). */
int32_t vsa_probe_mfma_valu(int32_t valu, int32_t op, int32_t waves_per_simd, int32_t iters, float* out,
                            void* stream);

/* Streaming read of HBM (the ceiling of the kernels that read every input
 * element once: pool, combine backward). `blocks` workgroups of 256 threads
 * read all `bytes` of src in 16-byte loads, grid-stride, each thread keeping
 * `inflight` loads (1, 2, 4, 8 or 16) in flight, with the non-temporal hint
 * when `nontemporal` is 1 (0: plain loads), and write one float per thread to
 * out (blocks * 256 floats).
 * Errors: VSA_ERR_NULL, VSA_ERR_ALIGN (src or bytes not a multiple of 16),
 * VSA_ERR_SHAPE (bytes 0, blocks outside [1, 2^20]), VSA_ERR_UNSUPPORTED
 * (inflight, nontemporal). */
int32_t vsa_probe_stream_read(const void* src, size_t bytes, int32_t blocks, int32_t inflight, int32_t nontemporal,
                              float* out, void* stream);

/* L2-resident data into LDS (the chunk path of the fine kernels). `blocks`
 * workgroups of two waves, each with 40 KB of LDS (four per CU), run `iters`
 * iterations; iteration c moves the 16 KB chunk at byte offset
 * ((block * 7 + c) * 16384) mod src_bytes of src into one of two LDS stages,
 * by direct-to-LDS loads (mode 0) or by 16-byte loads into registers and LDS
 * writes (mode 1), with the next chunk's loads in flight and a barrier per
 * iteration: blocks * iters * 16384 bytes in all. src_bytes: a power of two
 * from 16384 to 2^30 (2 MB keeps the source in every XCD's L2); out:
 * blocks * 128 floats, written.
 * Errors: VSA_ERR_NULL, VSA_ERR_ALIGN (src), VSA_ERR_SHAPE (src_bytes, blocks
 * outside [1, 2^20], iters < 1), VSA_ERR_UNSUPPORTED (mode). */
int32_t vsa_probe_l2_to_lds(int32_t mode, const void* src, size_t src_bytes, int32_t blocks, int32_t iters,
                            float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_PROBE_H */
