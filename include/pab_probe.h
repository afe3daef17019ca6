/*
 * pab_probe.h - C ABI of libpab_probe: one 32x32x64 matrix product on the
 * gfx950 matrix cores, so that tests can document how the matrix
 * instructions accumulate E4M3 products.  It backs the kernel design choice
 * that the FP8 recipe's S = Q K^T is summed on the bf16 matrix instruction
 * from the exact values of the E4M3 codes: the recipe asks for the exact
 * products of the quantised values with fp32 accumulation
 * ["FP8量化与稀疏性协同加速视频扩散模型", §3.1 staged quantisation; §3.3 item 3,
 * FP8 tensor-core instructions].  Test infrastructure: the attention path does
 * not use this library.
 */
#ifndef PAB_PROBE_H
#define PAB_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pab_probe_mfma_e4m3 - D = C + A B^T for A, B of 32 rows x 64 E4M3 codes.
 *
 * a, b   device uint8 [32][64], row-major E4M3 (OCP "fn") codes.
 * c_d    device float32 [32][32], row-major: C on entry, D on return
 *        (D[i][j] = C[i][j] + sum_k decode(a[i][k]) decode(b[j][k])).
 * kind   0: one v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit
 *           (E8M0 127) scales;
 *        1: four v_mfma_f32_32x32x16_bf16 over k = 0..63 in steps of 16, on
 *           the exact bf16 values of the codes (each E4M3 value is exact in
 *           bf16), chained through the fp32 accumulator.
 * stream hipStream_t as void* (NULL = the null stream); asynchronous.
 * Returns 0, 1 for invalid arguments (null or misaligned pointers, unknown
 * kind), or 3 when the launch fails.  One wave of 64 work-items.
 */
int pab_probe_mfma_e4m3(const uint8_t* a, const uint8_t* b, float* c_d, int kind, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAB_PROBE_H */
