/*
 * fa_probe.h -- C ABI of libfa_probe: two microbenchmarks that measure what
 * the MI355X (gfx950) in hand actually sustains, so that the attention
 * kernels' rates can be reported against a measured ceiling as well as the
 * published one.  The pages frame every kernel by a roofline of matrix rate
 * against memory bandwidth (Lensa ML explainer, Step 1, memory hierarchy and
 * arithmetic intensity); these calls measure the two roofs.
 *
 * Measurement support only: nothing in libfa calls these, and they compute
 * nothing the attention path needs.  Both calls only enqueue work on
 * `stream` (a hipStream_t, NULL = default stream) and return; the caller
 * times them (for example with HIP events on the same stream).
 * Return value: 0 on success, 1 NULL pointer, 2 bad size, 4 misaligned
 * pointer (nothing is enqueued on those), 7 the HIP runtime refused the
 * launch.  The caller owns every buffer.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroup size of both probes (four wave64 waves). */
#define FA_PROBE_THREADS 256
/* stream_read consumes the buffer in chunks of this many bytes
 * (FA_PROBE_THREADS lanes x 16 loads x 16 bytes). */
#define FA_PROBE_READ_CHUNK 65536

/*
 * Dense bf16 matrix-core rate.  `blocks` workgroups of four waves; every
 * wave runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
 * accumulate chains on register operands (no memory traffic inside the
 * loop), i.e. blocks * 4 * iters * 4 * 32768 FLOP in total.  The operands are
 * pseudo-random bf16 values in [-1, 1) with full mantissas: the clock the
 * matrix cores sustain depends on the data, and attention operands are of
 * this kind.
 *   out    : device float32 [blocks * FA_PROBE_THREADS], 4-byte aligned: one
 *            sum of each lane's accumulators (keeps the products live).
 *   stamps : device uint64 [4], 8-byte aligned: workgroup 0, wave 0 writes the
 *            shader-clock counter (s_memtime) and the constant-rate real-time
 *            counter (s_memrealtime) before and after its loop, as
 *            {memtime_start, realtime_start, memtime_end, realtime_end}; the
 *            ratio of the two differences gives the shader clock under this
 *            load.
 * blocks in [1, 2^20], iters in [1, 2^24].
 */
int fa_probe_mfma_bf16(float* out, unsigned long long* stamps, int blocks, int iters,
                       void* stream);

/*
 * Streaming HBM read rate.  `blocks` workgroups read every byte of buf once
 * with 16-byte non-temporal loads (sixteen in flight per lane) and XOR-reduce
 * them; each workgroup reads one contiguous run of chunks.
 *   buf   : device, 16-byte aligned, `bytes` bytes, bytes a non-zero multiple
 *           of FA_PROBE_READ_CHUNK.  Its contents do not matter.
 *   out   : device uint32 [blocks * FA_PROBE_THREADS], 4-byte aligned.
 * blocks in [1, 2^20].
 */
int fa_probe_stream_read(const void* buf, size_t bytes, unsigned* out, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
