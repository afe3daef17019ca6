// libpab_probe: one 32x32x64 product of E4M3 codes on the gfx950 matrix cores
// (see include/pab_probe.h).  The operand layouts are those of the attention
// kernel: in a 32x32 result lane l holds column l % 32 and, in register j, row
// 8 (j / 4) + 4 (l / 32) + j % 4; for a K = 64 FP8 operand lane l holds row
// l % 32 and elements 32 (l / 32) .. + 31; for a K = 16 bf16 operand, row
// l % 32 and elements 8 (l / 32) .. + 7 of its step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pab_device.h"
#include "pab_probe.h"

namespace {

typedef short v8s __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void probe_mfma_kernel(const uint8_t* a, const uint8_t* b, float* cd,
                                                        int kind) {
  const int lane = threadIdx.x, lr = lane & 31, lg = lane >> 5;
  v16f acc;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = cd[(8 * (j / 4) + 4 * lg + j % 4) * 32 + lr];
  if (kind == 0) {
    const uint4* pa = reinterpret_cast<const uint4*>(a + lr * 64 + 32 * lg);
    const uint4* pb = reinterpret_cast<const uint4*>(b + lr * 64 + 32 * lg);
    const pab::v8i A = {(int)pa[0].x, (int)pa[0].y, (int)pa[0].z, (int)pa[0].w,
                        (int)pa[1].x, (int)pa[1].y, (int)pa[1].z, (int)pa[1].w};
    const pab::v8i B = {(int)pb[0].x, (int)pb[0].y, (int)pb[0].z, (int)pb[0].w,
                        (int)pb[1].x, (int)pb[1].y, (int)pb[1].z, (int)pb[1].w};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 0, 0, 0, 127, 0, 127);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint2 ca = *reinterpret_cast<const uint2*>(a + lr * 64 + 16 * s + 8 * lg);
      const uint2 cb = *reinterpret_cast<const uint2*>(b + lr * 64 + 16 * s + 8 * lg);
      const uint4 xa = make_uint4(pab::e4m3_bf16x2<false>(ca.x), pab::e4m3_bf16x2<true>(ca.x),
                                  pab::e4m3_bf16x2<false>(ca.y), pab::e4m3_bf16x2<true>(ca.y));
      const uint4 xb = make_uint4(pab::e4m3_bf16x2<false>(cb.x), pab::e4m3_bf16x2<true>(cb.x),
                                  pab::e4m3_bf16x2<false>(cb.y), pab::e4m3_bf16x2<true>(cb.y));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8s, xa), __builtin_bit_cast(v8s, xb),
                                                    acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) cd[(8 * (j / 4) + 4 * lg + j % 4) * 32 + lr] = acc[j];
}

}  // namespace

extern "C" int pab_probe_mfma_e4m3(const uint8_t* a, const uint8_t* b, float* c_d, int kind,
                                   void* stream) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (!a || !b || !c_d || !al(a) || !al(b) || !al(c_d) || (kind != 0 && kind != 1)) return 1;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), a, b,
                     c_d, kind);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
