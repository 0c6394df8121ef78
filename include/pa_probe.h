/*
 * pa_probe.h -- HBM read-bandwidth and matrix-core throughput probes for MI355X (libpa_probe.so).
 *
 * Measurement aids, not part of the paged-attention method: they give the achievable read
 * rates that the decode kernel's bandwidth is compared with (the 8 TB/s figure is the vendor's
 * peak; what a kernel can stream is lower).  Two access patterns:
 *   - a streaming read of one contiguous buffer;
 *   - a gather of 4 KiB chunks in a caller-given order: a shuffled order is the pattern of a
 *     decode over a pool whose blocks are scattered ([TT] "How the Architecture Works": logical
 *     blocks map to physical blocks anywhere in the pool; at B = 16, D = 128, bf16 a
 *     (block, kv-head) K or V tile is 4 KiB).
 * A third probe gives the matrix cores' sustained rate for the bf16 instruction shapes the
 * kernels use (the 2.5 PFLOP/s dense bf16 figure is the vendor's peak at the nominal clock).
 * Each probe only enqueues one kernel on `stream` (a hipStream_t, NULL = null stream); the caller
 * owns every buffer and times the launch.  Loads are 16-byte non-temporal loads; each thread folds
 * what it read into one word of `sink` so no load can be removed.  Return: 0, or -1 for an
 * argument outside what the kernels support, -7 for a launch error (as pa.h's codes).
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads the first floor(nbytes / (16 * workgroups * 256 * loads)) * (16 * workgroups * 256 *
 * loads) bytes of buf (device, 16-byte aligned) once; *read_bytes receives that count.
 * workgroups in [1, 65536] of 256 threads; loads in {1, 2, 4, 8}: 16-byte loads each lane keeps
 * in flight.  sink: device, workgroups * 256 uint32. */
int32_t pa_probe_read_stream(const void* buf, size_t nbytes, int32_t workgroups, int32_t loads,
                             uint32_t* sink, size_t* read_bytes, void* stream);

/* Reads chunks order[0..nchunks) of 4 KiB each from buf (device, nchunks * 4 KiB, 16-byte
 * aligned), every chunk once; order (device int32) holds chunk ids in [0, nchunks) (others are
 * clamped into range).  A wave reads `per_wave` chunks per iteration (in {1, 2, 4}), each as
 * four 1 KiB contiguous loads.  workgroups of 256 threads; sink as above. */
int32_t pa_probe_read_gather(const void* buf, const int32_t* order, int32_t nchunks,
                             int32_t per_wave, int32_t workgroups, uint32_t* sink, void* stream);

/* Back-to-back independent bf16 matrix-core instructions with register operands:
 * shape 16 = v_mfma_f32_16x16x32_bf16 (8 accumulators per wave), 32 = v_mfma_f32_32x32x16_bf16
 * (4 accumulators); each wave issues iters rounds.  operands 0: a fixed sparse pattern (few
 * bits switch between instructions); 1: random bf16 words of magnitude 0.5 .. 2 with random
 * signs, a different set per accumulator, so consecutive instructions see unrelated bits, as in
 * attention on real data (the chip's power draw, and so its clock, depends on this).
 * workgroups in [1, 65536] of waves_per_wg in {1, 2, 4, 8} waves; *flops receives the launch's
 * flop count (2 per multiply-add).  sink: device, workgroups * 64 * waves_per_wg floats.
 * clocks: NULL, or device, 2 * workgroups uint64: per workgroup, the shader-clock ticks
 * (s_memtime) and the 100 MHz reference ticks (s_memrealtime) its first wave spent in the
 * loop, so their ratio x 100 MHz is the clock it ran at.  Returns 0, -1 on a bad argument, -7 on
 * a launch error. */
int32_t pa_probe_mfma(int32_t shape, int32_t operands, int32_t workgroups, int32_t waves_per_wg,
                      int32_t iters, float* sink, uint64_t* clocks, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
