/*
 * w4a16_probe.h -- measurement kernels of the W4A16 decode library
 * (libw4a16_probe.so, gfx950).  Not part of the product: the benchmark uses
 * them to measure what the hardware gives a plain streaming read, the
 * ceiling every weight-streaming kernel is judged against beside the 8 TB/s
 * HBM specification (tiny-llm W4 page, "Revisit the Decode Roofline": decode
 * time is the streamed bytes over the memory bandwidth); a test uses the
 * second to check a hardware conversion one product kernel relies on.
 */
#ifndef W4A16_PROBE_H
#define W4A16_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at `src` (device memory, 16-byte aligned, bytes a
 * multiple of 16) once with 16-byte loads: a grid-stride loop in which each
 * thread keeps two loads in flight and consecutive lanes read consecutive
 * 16-byte pieces; nontemporal != 0 marks the loads nontemporal (streamed data
 * that should not displace cached lines).  The loaded words are folded into
 * one value per thread, which is stored to sink[0] only if it equals a
 * constant no input of this benchmark produces (the store keeps the loads
 * alive and never happens in practice).
 * blocks: workgroups of 256 threads (0 = 3 per compute unit of device 0).
 * Returns 0, or a nonzero hipError_t value if the arguments are invalid
 * (NULL, misaligned, bytes not a multiple of 16) or the launch failed.
 */
int w4a16_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks, int nontemporal,
                            void *stream);

/*
 * Converts every one of the 2^32 fp32 bit patterns to bf16 twice, with the
 * hardware's packed conversion (v_cvt_pk_bf16_f32, which the LDS-tiled
 * prefill epilogue uses) and with the integer round-to-nearest-even rule
 * the other kernels use (NaNs quieted, sign and payload top bits kept), and
 * adds the number of patterns where the two differ to *mismatches (device
 * memory, 8-byte aligned; the caller sets it to 0) and lowers *first (device
 * memory, 4-byte aligned; the caller sets it to 0xFFFFFFFF) to the smallest
 * such pattern.  One launch of 2^18 workgroups on `stream`; the results are
 * there once the stream has run it.
 * Returns 0, or a nonzero hipError_t value if a pointer is NULL or
 * misaligned or the launch failed.
 */
int w4a16_probe_bf16_round_check(unsigned long long *mismatches, uint32_t *first, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_PROBE_H */
