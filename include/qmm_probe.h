/*
 * qmm_probe.h — measurement aids exported by the same library as qmm.h.
 *
 * Neither call computes any part of the product.  They measure what this chip
 * sustains for the two resources the product is bound by — streaming reads
 * from HBM (the decode GEMVs) and int8 MFMA issue (the prefill GEMMs) — so a
 * product rate can be reported against a measured ceiling as well as against
 * the vendor peak.  The page "llama.cpp and GGUF" ("CPU and Edge Inference:
 * When It Wins") sets a theoretical ceiling and a realistic figure side by
 * side in its worked table; these provide the realistic side on MI355X.
 *
 * Conventions are those of qmm.h: device pointers, caller-owned buffers, the
 * stream as void* (NULL = null stream), validation before anything is
 * enqueued, nothing allocated or synchronized, nothing thrown.
 */
#ifndef QMM_PROBE_H
#define QMM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the sink buffer both calls take (one per workgroup, at most). */
#define QMM_PROBE_SINK_WORDS 65536

/* Reads every byte of src once, with 16-byte loads that consecutive lanes
 * issue for consecutive 16-byte pieces.
 *   src        : device, `bytes` bytes, 16-byte aligned
 *   bytes      : > 0, a multiple of 16 (QMM_ERR_SHAPE otherwise)
 *   sink       : device, QMM_PROBE_SINK_WORDS uint32 (256 KiB); word g is
 *                set to the XOR of the 32-bit words that workgroup g read,
 *                so the XOR of all words written is the XOR of every 32-bit
 *                word of src; words past the last workgroup are not touched
 *   workgroups : workgroups of 256 threads, 1..QMM_PROBE_SINK_WORDS; 0 picks
 *                one workgroup per 4 KiB of src, at most 2048 (8 per
 *                compute unit)
 * Returns QMM_OK, QMM_ERR_NULL, QMM_ERR_ALIGN, QMM_ERR_SHAPE or QMM_ERR_HIP. */
int qmm_probe_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups, void* stream);

/* Runs back-to-back v_mfma_i32_32x32x32_i8 instructions on register operands:
 * `workgroups` workgroups of 4 waves, each wave 4 independent accumulator
 * chains of `iters` instructions.  Word g of sink (QMM_PROBE_SINK_WORDS
 * uint32) is set to a digest of workgroup g's accumulators, the same for
 * every call with the same arguments.  Integer operations performed:
 * qmm_probe_mfma_ops(workgroups, iters) = workgroups * 4 * 4 * iters * 65536.
 *   workgroups : 1..QMM_PROBE_SINK_WORDS;  iters : 1..2^30
 *   (QMM_ERR_SHAPE otherwise)
 * Returns QMM_OK, QMM_ERR_NULL, QMM_ERR_SHAPE or QMM_ERR_HIP. */
int qmm_probe_mfma(int workgroups, int64_t iters, uint32_t* sink, void* stream);

/* Integer operations (2 per multiply-add) of one qmm_probe_mfma call; 0 for
 * arguments it would reject. */
int64_t qmm_probe_mfma_ops(int workgroups, int64_t iters);

/* As qmm_probe_mfma, with v_mfma_i32_16x16x64_i8 (16x16 tiles, K = 64) and 8
 * independent accumulator chains per wave.  Integer operations performed:
 * qmm_probe_mfma16_ops(workgroups, iters) = workgroups * 4 * 8 * iters * 32768.
 *   workgroups : 1..QMM_PROBE_SINK_WORDS;  iters : 1..2^30
 *   (QMM_ERR_SHAPE otherwise)
 * Returns QMM_OK, QMM_ERR_NULL, QMM_ERR_SHAPE or QMM_ERR_HIP. */
int qmm_probe_mfma16(int workgroups, int64_t iters, uint32_t* sink, void* stream);

/* Integer operations of one qmm_probe_mfma16 call; 0 for arguments it would
 * reject. */
int64_t qmm_probe_mfma16_ops(int workgroups, int64_t iters);

#ifdef __cplusplus
}
#endif
#endif /* QMM_PROBE_H */
