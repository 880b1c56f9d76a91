/*
 * libvitattn_probe -- a measurement helper of the benchmark, not part of the
 * attention path: the bf16 MFMA throughput this GPU sustains on a kernel
 * that issues nothing but v_mfma_f32_32x32x16_bf16 (gfx950), so that the
 * attention kernel's rate can be read against a measured ceiling as well as
 * the vendor's dense bf16 peak.  Built as its own shared library.
 */
#ifndef VITATTN_PROBE_H
#define VITATTN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * vitattn_probe_mfma_loop -- enqueues `blocks` workgroups of 4 waves on
 * `stream` (a hipStream_t, NULL = null stream); every wave runs `iters`
 * iterations of 4 independent 32x32x16 bf16 MFMAs on register operands that
 * are all 1.0 (random = 0) or pseudo-random bf16 values (random != 0: random
 * sign and mantissa, exponent in [2^-7, 2^0]), then writes one float per lane to
 * out[block * 256 + lane_in_block], so `out` must hold blocks * 256 floats
 * (caller-owned device memory).  Returns 0, -1 (out is NULL), -2 (blocks or
 * iters < 1) or -8 (the launch failed).  Returns without waiting.
 */
int vitattn_probe_mfma_loop(float* out, int blocks, int iters, int random, void* stream);

/* Flops one vitattn_probe_mfma_loop launch performs (2 per multiply-add). */
double vitattn_probe_mfma_loop_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* VITATTN_PROBE_H */
