/*
 * b12x_probes.h - measurement probes of the benchmark harness (gfx950).
 */
#ifndef B12X_PROBES_H
#define B12X_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Measurement probes of the benchmark harness, in a library of their own
 * (libb12x_probes.so, not part of the MoE library).  They compute nothing of
 * the MoE: they measure what this device sustains, so that the MoE kernels'
 * rates can be read against achieved ceilings as well as datasheet peaks.
 *
 * b12x_probe_stream_read: `workgroups` workgroups of 256 threads each read a
 * contiguous share of floor(bytes / 16 / workgroups) 16-byte words at src
 * (four loads in flight per thread) and write to sink, per thread, the XOR
 * of every dword it read.  Thread t of a workgroup reads the words of its
 * share whose index is t mod 256, in whole chunks of 1024 words: the words
 * past the last whole chunk of a share are not read.
 *  src   device, 16-byte aligned, `bytes` a multiple of 16
 *  sink  u32 [workgroups * 256] device, overwritten with the digests
 * b12x_probe_mfma: `workgroups` workgroups of four waves; every wave runs
 * `iterations` rounds of 16 independent 16x16x32 MFMAs (f16 if f16 != 0,
 * else bf16) on register operands: 16384 * 16 * iterations flops per wave.
 *  sink  f32 [workgroups * 256] device, overwritten
 * Both enqueue one kernel on `stream` and return 0, 1 for NULL pointers or
 * counts below 1, 5 for a misaligned src or a size not a multiple of 16, or
 * 7 if the launch fails (the codes of b12x_status). */
int32_t b12x_probe_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int32_t workgroups,
                               void* stream);
int32_t b12x_probe_mfma(float* sink, int32_t workgroups, int32_t iterations, int32_t f16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* B12X_PROBES_H */
