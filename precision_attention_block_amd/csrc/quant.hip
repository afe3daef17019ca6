// Quantizer kernels of the staged precision recipe.
//
//  * Q/K per-block FP8 [FPS §2.1, §3.1]: one workgroup per (batch*head, block);
//    the block is read from HBM once and held in registers between the amax
//    reduction and the encode.
//  * V per-channel FP8 [FPS §3.1]: amax by atomics over token chunks, then an
//    encode pass that writes the codes transposed ([d][tokens]) in the operand
//    order of the attention kernel's P.V product, then a pass that turns the
//    amax into the scale.
//  * Q/K MXFP4 [FP4G §1]: one thread per 32-channel group.
//  * V MXFP4 along tokens (FP4 P.V, [FV §1] FP4 attention): a 64-token tile
//    of one head is transposed through LDS; one thread per (channel, group of
//    32 tokens) derives the E8M0 scale and writes the 32 codes in the operand
//    order of the attention kernel's FP4 P.V product.
// Optional token gather (perm) implements the block transpose of [FPS §3.3
// item 1]: kernel token p reads input token perm[p]; -1 yields a zero token.
//
//  [FPS]  "FP8量化与稀疏性协同加速视频扩散模型"
//  [FP4G] "Blackwell架构实战：如何用FP4量化让你的AI模型推理速度翻倍（附代码）"
#include "pab_device.h"
#include "pab_internal.h"

namespace pab {

template <typename T>
__device__ inline const T* token_ptr(const QuantArgs& a, int bh, int tok) {
  const int b = bh / a.H, h = bh % a.H;
  return reinterpret_cast<const T*>(a.x) + (int64_t)b * a.sb + (int64_t)h * a.sh +
         (int64_t)tok * a.sn;
}

// Source token of kernel token p, or -1 for a zero token.
__device__ inline int src_token(const QuantArgs& a, int p) {
  if (p >= a.n_out) return -1;
  return a.perm ? a.perm[p] : p;
}

// ------------------------------------------------------------ FP8 per block
// 256 threads; D/8 threads per token row, each thread owns 8 channels of one
// row per pass.  Up to CACHE passes are held in registers in the input type.
template <typename T, int D, int CACHE>
__global__ __launch_bounds__(256) void quant_fp8_block_kernel(QuantArgs a) {
  constexpr int TPR = D / 8;           // threads per row
  constexpr int RPP = 256 / TPR;       // rows per pass
  const int bh = blockIdx.y, blk_i = blockIdx.x;
  const int tid = threadIdx.x, col = (tid % TPR) * 8, r0 = tid / TPR;
  const int row_begin = blk_i * a.blk;
  const int row_end = min(row_begin + a.blk, (int)a.n_alloc);
  const int passes = (row_end - row_begin + RPP - 1) / RPP;
  __shared__ float red[4];

  Raw8<T> v[CACHE];
  float amax = 0.0f;
  if (passes <= CACHE) {
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
      const int row = row_begin + i * RPP + r0;
      const int src = (i < passes && row < row_end) ? src_token(a, row) : -1;
      if (src >= 0) v[i].load(token_ptr<T>(a, bh, src) + col);
      else v[i].zero();
    }
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
      float w[8];
      v[i].get(w);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(w[j]));
    }
  } else {
    for (int i = 0; i < passes; ++i) {
      const int row = row_begin + i * RPP + r0;
      const int src = row < row_end ? src_token(a, row) : -1;
      if (src >= 0) {
        float w[8];
        load8(token_ptr<T>(a, bh, src) + col, w);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(w[j]));
      }
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = fp8_scale(amax);
  if (tid == 0) a.scales_f32[(int64_t)bh * a.nblk + blk_i] = s;

  uint8_t* out = a.codes + (int64_t)bh * a.n_alloc * D;
  uint16_t* vals = a.values ? a.values + (int64_t)bh * a.n_alloc * D : nullptr;
  auto emit = [&](int row, const float (&w)[8]) {
    uint2 c;
    c.x = e4m3x4(__fmul_rn(w[0], s), __fmul_rn(w[1], s), __fmul_rn(w[2], s), __fmul_rn(w[3], s));
    c.y = e4m3x4(__fmul_rn(w[4], s), __fmul_rn(w[5], s), __fmul_rn(w[6], s), __fmul_rn(w[7], s));
    *reinterpret_cast<uint2*>(out + (int64_t)row * D + col) = c;
    if (vals) *reinterpret_cast<uint4*>(vals + (int64_t)row * D + col) = make_uint4(
        e4m3_bf16x2<false>(c.x), e4m3_bf16x2<true>(c.x), e4m3_bf16x2<false>(c.y), e4m3_bf16x2<true>(c.y));
  };
  if (passes <= CACHE) {
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
      const int row = row_begin + i * RPP + r0;
      if (i < passes && row < row_end) {
        float w[8];
        v[i].get(w);
        emit(row, w);
      }
    }
  } else {
    for (int i = 0; i < passes; ++i) {
      const int row = row_begin + i * RPP + r0;
      if (row >= row_end) continue;
      const int src = src_token(a, row);
      float w[8];
      if (src >= 0) {
        load8(token_ptr<T>(a, bh, src) + col, w);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = 0.0f;
      }
      emit(row, w);
    }
  }
}

// ------------------------------------------------------------ FP8 per channel
__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// amax over a chunk of 512 tokens per workgroup (one round of resident
// workgroups at 16K tokens x 40 heads); atomic max on the float bits
// (valid for non-negative floats) into the scale buffer, which holds amax
// until channel_finalize turns it into the scale.
template <typename T, int D>
__global__ __launch_bounds__(256) void channel_amax_kernel(QuantArgs a) {
  constexpr int TPR = D / 8, RPP = 256 / TPR, CHUNK = 512, ROUND = 256;
  const int bh = blockIdx.y, tid = threadIdx.x, col = (tid % TPR) * 8, r0 = tid / TPR;
  const int t0 = blockIdx.x * CHUNK;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // per round, all ROUND / RPP loads of a thread are issued before any is
  // consumed
  constexpr int NP = ROUND / RPP;
  for (int r = 0; r < CHUNK; r += ROUND) {
    Raw8<T> v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int src = src_token(a, t0 + r + r0 + i * RPP);
      if (src >= 0) v[i].load(token_ptr<T>(a, bh, src) + col);
      else v[i].zero();
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float w[8];
      v[i].get(w);
#pragma unroll
      for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(w[j]));
    }
  }
  __shared__ float red[RPP][D + 1];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[r0][col + j] = m[j];
  __syncthreads();
  if (tid < D) {
    float x = 0.0f;
    for (int r = 0; r < RPP; ++r) x = fmaxf(x, red[r][tid]);
    atomicMax(reinterpret_cast<unsigned int*>(a.scales_f32) + (int64_t)bh * D + tid,
              __float_as_uint(x));
  }
}

// Encode 128 tokens of all channels and write them transposed:
// codes[bh][c][n] with, inside each 64-token group, token t = 32a + 8b + 4g + c
// (a < 2, b < 4, g < 2, c < 4) stored at position 32g + 16a + 4b + c.
template <typename T, int D>
__global__ __launch_bounds__(256) void channel_encode_kernel(QuantArgs a) {
  constexpr int G = 128, ROW = G + 16;
  __shared__ float sc[D];
  __shared__ __align__(16) uint8_t tile[D * ROW];
  const int bh = blockIdx.y, g0 = blockIdx.x * G, tid = threadIdx.x;
  if (tid < D)
    sc[tid] = fp8_scale(__uint_as_float(
        reinterpret_cast<const uint32_t*>(a.scales_f32)[(int64_t)bh * D + tid]));
  __syncthreads();
  // unit = (token quad tq, channel octet co): 32 * D/8 units
  constexpr int UNITS = 32 * (D / 8);
  for (int u = tid; u < UNITS; u += 256) {
    const int tq = u % 32, co = u / 32;
    float w[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = src_token(a, g0 + 4 * tq + i);
      if (src >= 0) {
        load8(token_ptr<T>(a, bh, src) + co * 8, w[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[i][j] = 0.0f;
      }
    }
    const int lq = tq % 16;                    // quad inside its 64-token group
    const int pos = 64 * (tq / 16) + 32 * (lq % 2) + 16 * (lq / 8) + 4 * ((lq % 8) / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = co * 8 + j;
      const float s = sc[c];
      *reinterpret_cast<uint32_t*>(tile + c * ROW + pos) =
          e4m3x4(__fmul_rn(w[0][j], s), __fmul_rn(w[1][j], s), __fmul_rn(w[2][j], s),
                 __fmul_rn(w[3][j], s));
    }
  }
  __syncthreads();
  uint8_t* out = a.codes + (int64_t)bh * D * a.n_alloc + g0;
  for (int u = tid; u < D * 8; u += 256) {
    const int c = u / 8, ch = u % 8;
    *reinterpret_cast<uint4*>(out + (int64_t)c * a.n_alloc + 16 * ch) =
        *reinterpret_cast<const uint4*>(tile + c * ROW + 16 * ch);
  }
}

__global__ void channel_finalize_kernel(float* scales, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) scales[i] = fp8_scale(scales[i]);
}

// ------------------------------------------------------------ MXFP4
// A thread owns 8 consecutive channels (a quarter of a 32-channel group) of 4
// tokens: the lanes of a wave read 64 consecutive 16-byte chunks per load,
// the four lanes of a group combine their amax with two quad permutes (DPP),
// and every lane converts its 8 values with the hardware E2M1 conversion and
// writes its 4 bytes of packed codes.
__device__ inline float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

template <typename T>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(QuantArgs a) {
  constexpr int D = 128, NG = D / 32, CPT = D / 8;   // chunks of 8 channels per token
  constexpr int RPT = 4;                              // token rows per thread
  // grid: x covers the n_alloc tokens of one (b, h) in groups of 64 (n_alloc
  // is a multiple of 128, so every wave is whole and every lane reaches the
  // permutes below), y is b * H + h
  const int bh = blockIdx.y;
  const int chunk = threadIdx.x % CPT, g = chunk / 4, sub = chunk % 4;
  const int tok0 = blockIdx.x * 64 + threadIdx.x / CPT;
  Raw8<T> v[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int src = src_token(a, tok0 + 16 * i);
    if (src >= 0) v[i].load(token_ptr<T>(a, bh, src) + 8 * chunk);
    else v[i].zero();
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    float w[8];
    v[i].get(w);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(w[j]));
    amax = quad_max(amax);
    // floor(log2 amax) from the exponent field; a zero or subnormal amax has
    // floor(log2) <= -127, which the clamp maps to -127 either way.
    const int e32 = (int)(__float_as_uint(amax) >> 23);
    const int e = e32 == 0 ? -127 : max(e32 - 127 - 2, -127);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact
    // the hardware E2M1 conversion (round to nearest even on the code, which
    // is the tie rule of the recipe; |x / 2^e| < 8 saturates to 6); two
    // elements per byte, element 2k in the low nibble
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = __fmul_rn(w[j], inv);
    uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[2], y[3], 1.0f, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[4], y[5], 1.0f, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[6], y[7], 1.0f, 3);
    const int64_t rowid = (int64_t)bh * a.n_alloc + tok0 + 16 * i;
    *reinterpret_cast<uint32_t*>(a.codes + rowid * (D / 2) + 4 * chunk) = packed;
    if (sub == 0) a.scales_u8[rowid * NG + g] = (uint8_t)(e + 127);
  }
}

// ------------------------------------------------------------ MXFP4 V (tokens)
// Token slot j (0..31) of a 32-token group holds token pi(j): the K order of
// the FP4 P.V product, whose lanes hold keys 8b + r (first 16 slots) and
// 8b + 4 + r (last 16) of the group, b and r < 4.
__device__ constexpr int v4_token_of_slot(int j) { return 8 * ((j % 16) / 4) + 4 * (j / 16) + j % 4; }

template <typename T>
__global__ __launch_bounds__(256) void quant_mxfp4_v_kernel(QuantArgs a) {
  constexpr int D = 128, TT = 64, LD = TT + 1;   // LDS row: one channel, 64 tokens (+1 pad)
  __shared__ float tile[D * LD];
  const int bh = blockIdx.y, t0 = blockIdx.x * TT, tid = threadIdx.x;
  // load: unit = (token, 8-channel chunk), 64 x 16 units
  for (int u = tid; u < TT * (D / 8); u += 256) {
    const int t = u / (D / 8), ch = u % (D / 8);
    float w[8];
    const int src = src_token(a, t0 + t);
    if (src >= 0) {
      load8(token_ptr<T>(a, bh, src) + 8 * ch, w);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[(8 * ch + j) * LD + t] = w[j];
  }
  __syncthreads();
  const int c = tid % D, g = tid / D;            // channel, 32-token group of the tile
  const float* row = tile + c * LD + 32 * g;
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(row[j]));
  // the MX rule as for Q/K: e = floor(log2 amax) - 2 from the exponent field,
  // -127 for a zero or subnormal amax
  const int e32 = (int)(__float_as_uint(amax) >> 23);
  const int e = e32 == 0 ? -127 : max(e32 - 127 - 2, -127);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = __fmul_rn(row[v4_token_of_slot(8 * q + i)], inv);
    uint32_t p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, y[2], y[3], 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, y[4], y[5], 1.0f, 2);
    w[q] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, y[6], y[7], 1.0f, 3);
  }
  uint8_t* out = a.codes + ((int64_t)bh * D + c) * (a.n_alloc / 2) + (t0 + 32 * g) / 2;
  *reinterpret_cast<uint4*>(out) = make_uint4(w[0], w[1], w[2], w[3]);
  // scales [group][channel], channels interleaved: c at 4 (c % 32) + c / 32
  a.scales_u8[((int64_t)bh * (a.n_alloc / 32) + t0 / 32 + g) * D + 4 * (c % 32) + c / 32] =
      (uint8_t)(e + 127);
}

// ------------------------------------------------------------ non-finite count
__global__ void count_nonfinite_kernel(const float* x, int64_t n, int32_t* count) {
  int c = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    c += !isfinite(x[i]);
  c = wave_sum_i(c);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(count, c);
}

// ------------------------------------------------------------ launchers
template <typename T, int D>
static hipError_t launch_fp8_block(const QuantArgs& a, hipStream_t st) {
  dim3 grid(a.nblk, a.B * a.H);
  constexpr int CACHE = sizeof(T) == 2 ? 24 : 12;
  hipLaunchKernelGGL((quant_fp8_block_kernel<T, D, CACHE>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_channel(const QuantArgs& a, hipStream_t st) {
  const int64_t ns = (int64_t)a.B * a.H * D;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(a.scales_f32), ns, 0u);
  hipLaunchKernelGGL((channel_amax_kernel<T, D>), dim3((unsigned)((a.n_out + 511) / 512), a.B * a.H),
                     dim3(256), 0, st, a);
  hipLaunchKernelGGL((channel_encode_kernel<T, D>), dim3((unsigned)(a.n_alloc / 128), a.B * a.H),
                     dim3(256), 0, st, a);
  hipLaunchKernelGGL(channel_finalize_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st,
                     a.scales_f32, ns);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_mxfp4(const QuantArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_alloc / 64), (unsigned)(a.B * a.H));   // n_alloc % 128 == 0
  hipLaunchKernelGGL((quant_mxfp4_kernel<T>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_mxfp4_v(const QuantArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_alloc / 64), (unsigned)(a.B * a.H));   // n_alloc % 128 == 0
  hipLaunchKernelGGL((quant_mxfp4_v_kernel<T>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_quant(const QuantArgs& a, hipStream_t st) {
  switch (a.recipe) {
    case 0: return a.d == 128 ? launch_fp8_block<T, 128>(a, st) : launch_fp8_block<T, 64>(a, st);
    case 1: return a.d == 128 ? launch_channel<T, 128>(a, st) : launch_channel<T, 64>(a, st);
    case 3: return launch_mxfp4_v<T>(a, st);
    default: return launch_mxfp4<T>(a, st);
  }
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
  return a.in_bf16 ? dispatch_quant<__hip_bfloat16>(a, st) : dispatch_quant<float>(a, st);
}

hipError_t launch_count_nonfinite(const float* x, int64_t n, int32_t* count, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(count_nonfinite_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256),
                     0, st, x, n, count);
  return hipGetLastError();
}

}  // namespace pab
