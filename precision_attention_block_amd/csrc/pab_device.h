// Device-side helpers shared by the libpab kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace pab {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
// log2(448): P is produced directly in the 448-scaled domain, exp2(x + log2 448).
constexpr float kLog2_448 = 8.807354922057604f;
constexpr float kLog2e = 1.4426950408889634f;

// Stores four floats with the non-temporal hint (see store_o_rows).
__device__ inline void store4_stream(float* p, v4f v) {
  __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
}

// ---- input loads: 8 consecutive elements as fp32 -----------------------------
__device__ inline void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ inline void load8(const __hip_bfloat16* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

// Eight consecutive input elements kept in their storage type (bf16 holds 8
// values in 4 registers) and widened on use.
template <typename T> struct Raw8;
template <> struct Raw8<__hip_bfloat16> {
  uint4 v;
  __device__ void load(const __hip_bfloat16* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ void zero() { v = make_uint4(0u, 0u, 0u, 0u); }
  __device__ void get(float (&w)[8]) const {
    w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
    w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z); w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ void zero() { a = make_float4(0.f, 0.f, 0.f, 0.f); b = a; }
  __device__ void get(float (&w)[8]) const {
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
};

// ---- FP8 E4M3 (OCP) ----------------------------------------------------------
// The hardware conversion rounds to nearest-even and keeps subnormals, but
// returns the NaN code for magnitudes that round above 448; clamping first
// gives the saturating conversion of the recipe.
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> their exact values as two bf16
// (the hardware conversion to f32 is exact; an E4M3 value has at most 4
// significant bits, so its f32 bit pattern truncated to 16 bits is exact too).
template <bool HI>
__device__ inline uint32_t e4m3_bf16x2(uint32_t w) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
}

// s = fl32(448 / amax); 1 when amax is 0 or the quotient is not finite.
__device__ inline float fp8_scale(float amax) {
  const float s = __fdiv_rn(kE4M3Max, amax);
  return (amax == 0.0f || !isfinite(s)) ? 1.0f : s;
}

// ---- wave reductions -----------------------------------------------------------
__device__ inline float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ inline int wave_sum_i(int v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Combine across the four 16-lane rows of a wave: afterwards every lane holds
// the maximum (sum) of the four lanes with the same l % 16.
__device__ inline float max_rows(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ inline float sum_rows(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Work-item index for workgroup blockIdx.x such that consecutive work items
// land on the same XCD: the hardware deals workgroups round-robin over the 8
// XCDs, each with its own L2, so this keeps the query tiles of one head (which
// share K and V) on one L2.
__device__ inline int xcd_work_index(int bid, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int xcd = bid % 8, local = bid / 8;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + local;
}

}  // namespace pab
