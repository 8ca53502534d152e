/*
 * lcsa_probe.h - measurement support in liblcsa.so. Not part of the attention method: a probe of the
 * bf16 matrix core's sustained throughput on the GPU it runs on, so that a benchmark can put the
 * attention kernel's rate beside what the MFMA unit delivers under the same clocks and power.
 */
#ifndef LCSA_PROBE_H_
#define LCSA_PROBE_H_

#include "lcsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Runs `workgroups` workgroups of 4 waves; each wave issues `iters` rounds of 8 dense
 * v_mfma_f32_32x32x16_bf16 (32x32x16 bf16 products with fp32 accumulation, operands held in registers,
 * four independent accumulators) and writes one float per lane to sink[workgroups * 256] (device,
 * caller-owned, 4-byte aligned; the values are meaningless). *flop (host, may be NULL) receives the
 * FLOP the launch executes: workgroups * 4 * iters * 8 * 2 * 32 * 32 * 16. Asynchronous on `stream`;
 * 1 <= workgroups <= 2^20 and 1 <= iters <= 2^24, else LCSA_ERR_INVALID before any launch. */
lcsa_status lcsa_mfma_probe(int32_t workgroups, int32_t iters, float* sink, double* flop, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LCSA_PROBE_H_ */
