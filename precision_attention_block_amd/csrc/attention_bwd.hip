// Attention backward pass for gfx950 (CDNA4).
//
// The FA4 page ("FA4极速LLM：10分钟搞定20倍内存直降！", co-design list: the
// backward pass and its intermediates S, P, dP, dS, dQ) and the FPSAttention
// page ("FP8量化与稀疏性协同加速视频扩散模型", introduction: training-aware FP8)
// fix what is computed up to the gradient of the quantisers, which passes
// straight through: with the dequantised operands Q^, K^, V^ of the forward
// pass, its output O and its row statistic LSE (log2 units),
//   P = 2^(S log2 e - LSE), S = Q^ K^T sm     dV^ = P^T dO
//   dP = dO V^^T    D_i = sum_c dO_ic O_ic    dS = P (dP - D)
//   dQ^ = sm dS K^  dK^ = sm dS^T Q^
// The products run on v_mfma_f32_32x32x16_bf16.  Q and K enter as the exact
// bf16 values of their codes (FP8) or as exactly dequantised values (MXFP4),
// with the FP8 block scales applied in fp32 to S and folded into dS; V enters
// as exact code values with its per-channel FP8 scale folded into dO.  P, dS
// and dO are rounded to bf16 for their products; every sum is fp32.
//
// Two kernels, FlashAttention-2 style, so no atomics and a deterministic sum
// order:
//  * dK/dV: a workgroup owns 128 keys (4 blocks of 32, each split over a
//    wave that keeps the K rows as B operands and forms P and dV, and a wave
//    that keeps the V rows and forms dP, dS and dK) and walks the queries in
//    steps of 32.
//  * dQ: a workgroup owns 128 queries; each wave keeps the Q and dO rows of
//    its queries in registers and walks the keys in steps of 32.
// In the 32x32 MFMA result layout a lane holds one column and 16 rows
// 8 i + 4 lg + r (i, r < 4, lg = lane / 32).  Registers 8h .. 8h+7 of a
// score tile are therefore exactly the B operand of the next product over
// the rows 16h .. 16h+15 when the other operand lists those rows with bits 2
// and 3 of the index swapped.  The prep kernels write Q^T, K^T and dO^T in
// that order ("block transpose" done ahead of the kernel, as the forward's V),
// so the scores never leave the registers.
// Tiles reach LDS by LDS-DMA into XOR-swizzled rows (conflict-free 16-byte
// operand reads), one step ahead of the step being computed.
#include <type_traits>

#include "pab_bwd.h"
#include "pab_device.h"
#include "pab_lds.h"

namespace pab {

typedef short v8s __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));

constexpr float kInf = __builtin_huge_valf();
constexpr int kD = 128;

int64_t bwd_workspace_layout(int64_t BH, int64_t n_alloc, int64_t d, int64_t off[13]) {
  const int64_t rows = BH * n_alloc * d * 2, toks = BH * n_alloc * 4;
  const int64_t sizes[12] = {rows, rows, rows, rows, rows, rows, rows, toks, toks, toks, toks,
                             n_alloc * 4};
  int64_t at = 0;
  for (int i = 0; i < 12; ++i) {
    off[i] = at;
    at += (sizes[i] + 255) / 256 * 256;
  }
  off[12] = at;
  return at;
}

// Token index with bits 2 and 3 swapped (an involution): the slot of token t
// in a transposed array, and the token of slot t.
__device__ constexpr int swap23(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

__device__ inline uint32_t bf16x2(float a, float b) {   // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{a, b}, b2v));
}
// two floats whose values are exact in bf16
__device__ inline uint32_t bf16x2_exact(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// E2M1 code (4 bits) -> its value: 0, 0.5, 1, 1.5, 2, 3, 4, 6 with sign bit 3
// ("Blackwell架构实战……", §1: E2M1).
__device__ inline float e2m1_value(uint32_t nib) {
  const uint32_t m = nib & 7;
  const uint32_t mag = m < 2 ? (m ? 0x3F000000u : 0u) : (((126u + (m >> 1)) << 23) | ((m & 1) << 22));
  return __uint_as_float(mag | ((nib & 8) << 28));
}

// Writes the transposed copy of a 64-token x 128-channel bf16 tile (row pitch
// TP elements) in the block-tiled layout [token block of 32][channel][32
// slots], slots in swap23 order: dst points at the tile's first block.  One
// 32-token step of a transposed operand is then 8 contiguous KB.
template <int TP>
__device__ inline void store_transposed(const uint16_t* tile, uint16_t* dst, int tid) {
  for (int u = tid; u < kD * 8; u += 256) {
    const int c = u / 8, ch = u % 8;   // channel, 8-slot chunk of the 64 tokens
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s0 = 8 * ch + 2 * j;
      w[j] = (uint32_t)tile[swap23(s0) * TP + c] | ((uint32_t)tile[swap23(s0 + 1) * TP + c] << 16);
    }
    *reinterpret_cast<uint4*>(dst + (ch / 4) * kD * 32 + c * 32 + 8 * (ch % 4)) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- prep: Q / K values, their transposed copies and per-token factors -----
// grid (n_alloc / 64, BH, 2): z = 0 Q, 1 K.
template <bool MX>
__global__ __launch_bounds__(256) void bwd_prep_qk_kernel(BwdArgs a) {
  constexpr int TP = kD + 8;
  __shared__ __align__(16) uint16_t tile[64 * TP];
  const int bh = blockIdx.y, t0 = blockIdx.x * 64, tid = threadIdx.x;
  const bool isk = blockIdx.z == 1;
  const int64_t tokb = (int64_t)bh * a.n_alloc + t0;
  for (int u = tid; u < 64 * 16; u += 256) {
    const int t = u / 16, c8 = u % 16;
    uint4 w;
    if (MX) {
      const uint32_t cw = *reinterpret_cast<const uint32_t*>((isk ? a.k_codes : a.q_codes) +
                                                             (tokb + t) * (kD / 2) + 4 * c8);
      const int e8 = (isk ? a.k_mx : a.q_mx)[(tokb + t) * (kD / 32) + c8 / 4];
      const float sc = __builtin_amdgcn_ldexpf(1.0f, e8 - 127);
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e2m1_value((cw >> (4 * j)) & 15) * sc;
      w = make_uint4(bf16x2_exact(v[0], v[1]), bf16x2_exact(v[2], v[3]), bf16x2_exact(v[4], v[5]),
                     bf16x2_exact(v[6], v[7]));
      *reinterpret_cast<uint4*>((isk ? a.k_rows : a.q_rows) + (tokb + t) * kD + 8 * c8) = w;
    } else {
      w = *reinterpret_cast<const uint4*>((isk ? a.k_val : a.q_val) + (tokb + t) * kD + 8 * c8);
    }
    *reinterpret_cast<uint4*>(&tile[t * TP + 8 * c8]) = w;
  }
  if (tid < 64) {
    float f = 1.0f;
    if (!MX) {
      const int t = t0 + tid;
      f = 1.0f / (isk ? a.k_scale[(int64_t)bh * a.nblk_k + t / a.blk_k]
                      : a.q_scale[(int64_t)bh * a.nblk_q + t / a.blk_q]);
    }
    (isk ? a.fk : a.fq)[tokb + tid] = f;
  }
  __syncthreads();
  store_transposed<TP>(tile, (isk ? a.kt : a.qt) + ((int64_t)bh * a.n_alloc + t0) * kD, tid);
}

// ---- prep: V values as bf16 rows ---------------------------------------------
// grid (n_alloc / 64, BH).  FP8: the exact values of the E4M3 codes (the
// channel scale is folded into dO); MXFP4: the exactly dequantised values.
template <bool MXV>
__global__ __launch_bounds__(256) void bwd_prep_v_kernel(BwdArgs a) {
  constexpr int RP = 80;   // LDS row pitch (bytes) of a channel
  __shared__ __align__(16) uint8_t tile[kD * RP];
  __shared__ uint8_t e8[2 * kD];
  const int bh = blockIdx.y, t0 = blockIdx.x * 64, tid = threadIdx.x;
  if (!MXV) {
    for (int u = tid; u < kD * 4; u += 256) {
      const int c = u / 4, ch = u % 4;
      *reinterpret_cast<uint4*>(tile + c * RP + 16 * ch) = *reinterpret_cast<const uint4*>(
          a.v_codes + ((int64_t)bh * kD + c) * a.n_alloc + t0 + 16 * ch);
    }
  } else {
    for (int u = tid; u < kD * 2; u += 256) {
      const int c = u / 2, ch = u % 2;
      *reinterpret_cast<uint4*>(tile + c * RP + 16 * ch) = *reinterpret_cast<const uint4*>(
          a.v_codes + ((int64_t)bh * kD + c) * (a.n_alloc / 2) + t0 / 2 + 16 * ch);
    }
    e8[tid] = a.v_e8[((int64_t)bh * (a.n_alloc / 32) + t0 / 32) * kD + tid];
  }
  __syncthreads();
  uint16_t* out = a.v_rows + ((int64_t)bh * a.n_alloc + t0) * kD;
  for (int u = tid; u < 64 * 16; u += 256) {
    const int t = u / 16, c8 = u % 16;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 8 * c8 + 2 * j;
      if (!MXV) {
        // the V quantizer's 64-token interleave: quad lq of the group sits at
        // 32 (lq % 2) + 16 (lq / 8) + 4 ((lq % 8) / 2)
        const int lq = t / 4;
        const int slot = 32 * (lq % 2) + 16 * (lq / 8) + 4 * ((lq % 8) / 2) + t % 4;
        w[j] = e4m3_bf16x2<false>((uint32_t)tile[c * RP + slot] | ((uint32_t)tile[(c + 1) * RP + slot] << 8));
      } else {
        // 32-token groups: token 8 a + 4 b + r sits at slot 16 b + 4 a + r,
        // two slots per byte, the even slot in the low nibble
        const int g = t / 32, tt = t % 32;
        const int slot = 16 * ((tt / 4) % 2) + 4 * (tt / 8) + tt % 4;
        float v2[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint32_t byte = tile[(c + x) * RP + 16 * g + slot / 2];
          const int e = e8[g * kD + 4 * ((c + x) % 32) + (c + x) / 32];
          v2[x] = e2m1_value((slot & 1) ? byte >> 4 : byte & 15) * __builtin_amdgcn_ldexpf(1.0f, e - 127);
        }
        w[j] = bf16x2_exact(v2[0], v2[1]);
      }
    }
    *reinterpret_cast<uint4*>(out + (int64_t)t * kD + 8 * c8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- prep: dO rows and dO^T, D = rowsum(dO * O), LSE and key validity -------
// grid (n_alloc / 64, BH).
template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_do_kernel(BwdArgs a) {
  constexpr int TP = kD + 8;
  __shared__ __align__(16) uint16_t tile[64 * TP];
  __shared__ float fv[kD];
  const int bh = blockIdx.y, t0 = blockIdx.x * 64, tid = threadIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  if (tid < kD) fv[tid] = a.v_mx ? 1.0f : 1.0f / a.v_scale[(int64_t)bh * kD + tid];
  __syncthreads();
  const int t = tid / 4, part = tid % 4, tok = t0 + t;
  const bool live = tok < a.N;
  const T* g = static_cast<const T*>(a.dout) + b * a.do_sb + h * a.do_sh + (int64_t)(live ? tok : 0) * a.do_sn;
  const float* o = a.o + b * a.o_sb + h * a.o_sh + (int64_t)(live ? tok : 0) * a.o_sn;
  uint16_t* drow = a.dos_rows + ((int64_t)bh * a.n_alloc + tok) * kD;
  float acc = 0.0f;
#pragma unroll
  for (int c8 = 0; c8 < 4; ++c8) {
    const int c0 = 8 * part + 32 * c8;   // the 4 threads of a token read 128 contiguous bytes
    float gv[8], ov[8];
    if (live) {
      load8(g + c0, gv);
      load8(o + c0, ov);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) gv[j] = ov[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(gv[j], ov[j], acc);
    uint32_t ws[4], wt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ws[j] = bf16x2(gv[2 * j] * fv[c0 + 2 * j], gv[2 * j + 1] * fv[c0 + 2 * j + 1]);
      wt[j] = bf16x2(gv[2 * j], gv[2 * j + 1]);
    }
    *reinterpret_cast<uint4*>(drow + c0) = make_uint4(ws[0], ws[1], ws[2], ws[3]);
    *reinterpret_cast<uint4*>(&tile[t * TP + c0]) = make_uint4(wt[0], wt[1], wt[2], wt[3]);
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  if (part == 0) {
    const int64_t at = (int64_t)bh * a.n_alloc + tok;
    a.dd[at] = live ? acc : 0.0f;
    const float l = live ? a.lse[(int64_t)bh * a.N + tok] : kInf;
    a.lse_e[at] = l == -kInf ? kInf : l;   // a row without a valid key: every P is 0
    if (bh == 0) a.kvf[tok] = (live && (!a.kv_valid || a.kv_valid[tok])) ? 1.0f : 0.0f;
  }
  __syncthreads();
  store_transposed<TP>(tile, a.dot + ((int64_t)bh * a.n_alloc + t0) * kD, tid);
}

#if defined(__HIP_DEVICE_COMPILE__)
// LDS stage of one 32-token step: two row tiles [32][256 B] (CPR 16), one or
// two transposed tiles [128][64 B] (CPR 4) and 256-byte copies of per-token
// floats (32 used).
struct Stage {
  static constexpr int R0 = 0, R1 = 8192, T0 = 16384, T1 = 24576, F0 = 32768, F1 = F0 + 256,
                       F2 = F1 + 256, BYTES = F2 + 256;
};
// LDS stage of the dQ kernel: K rows, V rows, K^T and two per-token floats.
struct DqStage {
  static constexpr int R0 = 0, R1 = 8192, T0 = 16384, F0 = 24576, F1 = F0 + 256, BYTES = F1 + 256;
};

__device__ inline v8s lds_row_operand(const uint8_t* base, int row, int chunk) {
  return *reinterpret_cast<const v8s*>(base + row * 256 + 16 * (chunk ^ swz<16>(row)));
}
__device__ inline v8s lds_t_operand(const uint8_t* base, int row, int chunk) {
  return *reinterpret_cast<const v8s*>(base + row * 64 + 16 * (chunk ^ swz<4>(row)));
}

// Copies of one step: 8 KB row tiles take 8 instructions of 1 KB (4 rows),
// 8 KB transposed tiles 8 instructions (16 rows of 64 bytes, contiguous in
// the block-tiled layout); each wave issues 2 of each tile's 8.  The
// per-token floats are one full-wave dword copy each, issued by every wave to
// the same place.
__device__ inline void issue_rows(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int t0, int wave,
                                  const DmaPlan<16>& pr) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int inst = 2 * wave + x;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + inst * 1024), 16, pr.off[inst % 4],
                                             (t0 + 4 * inst) * 2 * kD, 0, 0);
  }
}
__device__ inline void issue_trans(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int t0, int wave,
                                   const DmaPlan<4>& pt) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int inst = 2 * wave + x;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + inst * 1024), 16, pt.off[0],
                                             t0 * 2 * kD + inst * 1024, 0, 0);
  }
}
__device__ inline void issue_floats(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int t0, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 4, 4 * lane, t0 * 4, 0, 0);
}

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kRsrcWord3);
}

#endif  // __HIP_DEVICE_COMPILE__

// ---- dK, dV ---------------------------------------------------------------------
// A workgroup of 8 waves owns 128 keys and walks the queries in steps of 32.
// Each 32-key block is split over two waves, so that each holds one operand
// and one accumulator (about half the registers of one wave doing all four
// products) and two waves share every SIMD:
//  * P-wave (waves 0-3, key block w): K operand and the dV accumulator.  For
//    step t+1 it forms S = Q K^T, P = 2^(S c - LSE) (masked), stores P (fp32)
//    in an LDS exchange buffer and adds dV^T += dO^T P.
//  * dS-wave (waves 4-7, key block w - 4): V operand and the dK accumulator.
//    For step t it forms dP = (dO / s_V) V_codes^T, reads P of step t from the
//    exchange buffer, dS' = P (dP - D) sm / s_Q (zero wherever P was masked)
//    and adds dK^T += Q_vals^T dS'.
// Waves w and w + 4 run on the same SIMD.  Three LDS stages hold steps t,
// t+1 (read) and t+2 (being copied); the exchange buffer is double-buffered
// by step parity.  One barrier per step orders the copies, the exchange and
// the reuse of stages.
// UQ: the Q block scale is the same for all 32 queries of a step (MXFP4, or
// FP8 blocks of a multiple of 32 tokens), so one fma forms each exponent
// argument and dS takes one fma and one multiply.
#if defined(__HIP_DEVICE_COMPILE__)
struct PairLds {
  static constexpr int PX = 3 * Stage::BYTES;             // exchange buffers
  static constexpr int PX_BYTES = 4 * 64 * 16 * 4;        // 4 key blocks x 64 lanes x 16 floats
  static constexpr int BYTES = PX + 2 * PX_BYTES;
};

// One wave's share of a stage's copies with 8 waves: one instruction per tile;
// waves 0, 1 and 2 also copy the LSE, D and 1/s_Q floats of the step.
__device__ inline void issue_stage8(uint8_t* stg, int q0, int wave, int lane,
                                    __amdgpu_buffer_rsrc_t qr, __amdgpu_buffer_rsrc_t dr,
                                    __amdgpu_buffer_rsrc_t qtr, __amdgpu_buffer_rsrc_t dtr,
                                    __amdgpu_buffer_rsrc_t lsr, __amdgpu_buffer_rsrc_t ddr,
                                    __amdgpu_buffer_rsrc_t fqr, const DmaPlan<16>& pr,
                                    const DmaPlan<4>& pt) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void_t*)(stg + Stage::R0 + wave * 1024), 16,
                                           pr.off[wave % 4], (q0 + 4 * wave) * 2 * kD, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void_t*)(stg + Stage::R1 + wave * 1024), 16,
                                           pr.off[wave % 4], (q0 + 4 * wave) * 2 * kD, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(qtr, (lds_void_t*)(stg + Stage::T0 + wave * 1024), 16,
                                           pt.off[0], q0 * 2 * kD + wave * 1024, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(dtr, (lds_void_t*)(stg + Stage::T1 + wave * 1024), 16,
                                           pt.off[0], q0 * 2 * kD + wave * 1024, 0, 0);
  if (wave < 3)
    issue_floats(wave == 0 ? lsr : wave == 1 ? ddr : fqr, stg + Stage::F0 + 256 * wave, q0, lane);
}
#endif  // __HIP_DEVICE_COMPILE__

// STA: the queries are the tiles of the key tile's window list, each walked
// in 32-query steps (no causal mask).
template <bool CAUSAL, bool UQ, bool STA>
__global__ __launch_bounds__(512) void bwd_dkdv_pair_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __align__(16) uint8_t lds[PairLds::BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wave < 4;
  const int kblk = wave & 3;
  const int lr = lane & 31, lg = lane >> 5;
  const int n_kt = a.n_alloc / kBwdTile;
  const int work = xcd_work_index(blockIdx.x, gridDim.x);
  const int bh = work / n_kt, kt = work % n_kt;
  const int key0 = kt * kBwdTile + 32 * kblk;   // this wave's 32 keys
  const int j = key0 + lr;                      // this lane's key
  const int64_t tokb = (int64_t)bh * a.n_alloc;

  const auto qr = rsrc(a.q_rows + tokb * kD, (int64_t)a.n_alloc * kD * 2);
  const auto dr = rsrc(a.dos_rows + tokb * kD, (int64_t)a.n_alloc * kD * 2);
  const auto qtr = rsrc(a.qt + tokb * kD, (int64_t)a.n_alloc * kD * 2);
  const auto dtr = rsrc(a.dot + tokb * kD, (int64_t)a.n_alloc * kD * 2);
  const auto lsr = rsrc(a.lse_e + tokb, (int64_t)a.n_alloc * 4);
  const auto ddr = rsrc(a.dd + tokb, (int64_t)a.n_alloc * 4);
  const auto fqr = rsrc(a.fq + tokb, (int64_t)a.n_alloc * 4);
  DmaPlan<16> pr;
  pr.init(lane, 2 * kD);
  DmaPlan<4> pt;
  pt.init(lane, 64);
  auto stage = [&](int i) __attribute__((always_inline)) { return lds + (i % 3) * Stage::BYTES; };
  // exchange slot of (step parity, this key block); lane l's 16 floats sit at
  // 16-byte chunks k * 1024 + 16 l (k < 4), so every access is one
  // contiguous KB per instruction
  auto xch = [&](int t) __attribute__((always_inline)) {
    return lds + PairLds::PX + (t & 1) * PairLds::PX_BYTES + kblk * 4096 + 16 * lane;
  };
  const int q_begin = CAUSAL ? kt * kBwdTile : 0;   // earlier queries see none of these keys
  const int q_end = (a.N + 31) / 32 * 32;
  const int spt = STA ? a.tile_tokens / 32 : 1;     // steps per tile
  const int32_t* wl = nullptr;
  int n_steps = (q_end - q_begin) / 32;
  if (STA) {
    const int v = kt * kBwdTile / a.tile_tokens;
    wl = a.win_idx + a.win_off[v];
    n_steps = (a.win_off[v + 1] - a.win_off[v]) * spt;
    if (n_steps <= 0) {   // an empty window list: no query sees these keys
      if (j < a.N) {
        const int b = bh / a.H, h = bh % a.H;
        float* row = (pwave ? a.dv : a.dk) + b * a.g_sb + h * a.g_sh + (int64_t)j * a.g_sn;
        for (int c = 4 * lg; c < kD; c += 8)
          *reinterpret_cast<float4*>(row + c) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      return;
    }
  }
  // first query of step t; the copies issued past the last step repeat it
  auto qstart = [&](int t) __attribute__((always_inline)) -> int {
    if (!STA) return q_begin + 32 * t;
    const int tc = t < n_steps ? t : n_steps - 1;
    return a.tile_tokens * __builtin_amdgcn_readfirstlane(wl[tc / spt]) + 32 * (tc % spt);
  };
  auto issue = [&](int t) __attribute__((always_inline)) {
    issue_stage8(stage(t), qstart(t), wave, lane, qr, dr, qtr, dtr, lsr, ddr, fqr, pr, pt);
  };
  // step 0 has landed once at most one stage's copies of this wave (5 for
  // waves 0-2, 4 for the others) are outstanding
  auto wait_first = [&]() __attribute__((always_inline)) {
    if (wave < 3)
      wait_vm_le<5>();
    else
      wait_vm_le<4>();
  };

  // lane (key j, lg) of an accumulator holds channels 32 cb + 8 i + 4 lg + r
  auto store_rows = [&](float* base, const v16f (&acc)[4]) __attribute__((always_inline)) {
    if (j >= a.N) return;
    const int b = bh / a.H, h = bh % a.H;
    float* row = base + b * a.g_sb + h * a.g_sh + (int64_t)j * a.g_sn;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(row + 32 * cb + 8 * i + 4 * lg) =
            make_float4(acc[cb][4 * i], acc[cb][4 * i + 1], acc[cb][4 * i + 2], acc[cb][4 * i + 3]);
  };

  if (pwave) {
    v8s kb[8];
    {
      const uint4* kr = reinterpret_cast<const uint4*>(a.k_rows + (tokb + j) * kD);
#pragma unroll
      for (int s = 0; s < 8; ++s) kb[s] = __builtin_bit_cast(v8s, kr[2 * s + lg]);
    }
    const float ck = a.sm_log2 * a.fk[tokb + j];
    const bool kvalid = a.kvf[j] != 0.0f;
    const bool all_valid = __all(kvalid);
    v16f dvt[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) dvt[cb][e] = 0.0f;
    // S and P of step t (stage t % 3): P goes to exchange slot t & 1 and,
    // packed as bf16 B operands, to pb for dV.  `before` runs between the
    // score products and the vector work (the previous step's dV products,
    // which do not depend on these scores).
    auto pstep = [&](const int t, v8s (&pb)[2], auto&& before) __attribute__((always_inline)) {
      const uint8_t* cur = stage(t);
      const int q0 = qstart(t);
      v16f s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row_operand(cur + Stage::R0, lr, 2 * ks + lg), kb[ks],
                                                    s, 0, 0, 0);
      before();
      float cs = 0.0f;
      if (UQ) cs = ck * *reinterpret_cast<const float*>(cur + Stage::F2);
      const bool masked = !all_valid || (CAUSAL && q0 < key0 + 32);
      // register 4 i + r is query q0 + 8 i + 4 lg + r; masked steps keep it
      // only if 8 i + r >= thr (query >= key for causal masks; never for a
      // masked key)
      const int thr = !kvalid ? 64 : CAUSAL ? j - q0 - 4 * lg : -64;
      float p[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 l4 = *reinterpret_cast<const float4*>(cur + Stage::F0 + 4 * (8 * i + 4 * lg));
        float4 f4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!UQ) f4 = *reinterpret_cast<const float4*>(cur + Stage::F2 + 4 * (8 * i + 4 * lg));
        const float lse[4] = {l4.x, l4.y, l4.z, l4.w}, fq[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * i + r;
          p[e] = __builtin_amdgcn_exp2f(UQ ? fmaf(s[e], cs, -lse[r]) : fmaf(s[e] * ck, fq[r], -lse[r]));
        }
      }
      if (masked) {
#pragma unroll
        for (int e = 0; e < 16; ++e) p[e] = 8 * (e / 4) + e % 4 >= thr ? p[e] : 0.0f;
      }
      uint8_t* x = xch(t);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<float4*>(x + k * 1024) = make_float4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pb[h] = __builtin_bit_cast(v8s, make_uint4(bf16x2(p[8 * h], p[8 * h + 1]), bf16x2(p[8 * h + 2], p[8 * h + 3]),
                                                   bf16x2(p[8 * h + 4], p[8 * h + 5]),
                                                   bf16x2(p[8 * h + 6], p[8 * h + 7])));
    };
    // dV^T += dO^T P of step t (channels x keys, K = queries)
    auto dvstep = [&](const int t, const v8s (&pb)[2]) __attribute__((always_inline)) {
      const uint8_t* cur = stage(t);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          dvt[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_t_operand(cur + Stage::T1, 32 * cb + lr, 2 * h + lg), pb[h], dvt[cb], 0, 0, 0);
    };
    // dV runs one step behind: iteration t forms the scores of step t+1, adds
    // step t's dV products while they complete, then forms P of step t+1.
    // Stage t stays valid through iteration t (the copy of that iteration
    // goes to stage t+2).
    issue(0);
    issue(1);
    wait_first();
    barrier_lds();
    v8s pba[2], pbb[2];
    pstep(0, pba, [] {});
    auto body = [&](const int t, const v8s (&pb_cur)[2], v8s (&pb_nxt)[2]) __attribute__((always_inline)) {
      wait_vm_le<0>();
      barrier_lds();   // step t+1 has landed; stage (t+2) % 3 and slot (t+1) & 1 are free
      issue(t + 2);
      pstep(t + 1, pb_nxt, [&] { dvstep(t, pb_cur); });
    };
    int t = 0;
    for (; t + 3 <= n_steps; t += 2) {
      body(t, pba, pbb);
      body(t + 1, pbb, pba);
    }
    if (t + 2 <= n_steps) {   // one more step to form: P of step t+1 goes to pbb
      body(t, pba, pbb);
      ++t;
      wait_vm_le<0>();
      barrier_lds();   // the dS-waves' last step
      issue(n_steps + 1);
      dvstep(t, pbb);
    } else {
      wait_vm_le<0>();
      barrier_lds();   // the dS-waves' last step
      issue(n_steps + 1);
      dvstep(t, pba);
    }
    wait_vm_le<0>();   // no copy may still target this workgroup's LDS when it ends
    store_rows(a.dv, dvt);
  } else {
    v8s vb[8];
    {
      const uint4* vr = reinterpret_cast<const uint4*>(a.v_rows + (tokb + j) * kD);
#pragma unroll
      for (int s = 0; s < 8; ++s) vb[s] = __builtin_bit_cast(v8s, vr[2 * s + lg]);
    }
    v16f dkt[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) dkt[cb][e] = 0.0f;
    // dP, dS and dK of step t
    auto dstep = [&](const int t) __attribute__((always_inline)) {
      const uint8_t* cur = stage(t);
      v16f dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) dp[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row_operand(cur + Stage::R1, lr, 2 * ks + lg), vb[ks],
                                                     dp, 0, 0, 0);
      float sc = 0.0f;
      if (UQ) sc = a.sm * *reinterpret_cast<const float*>(cur + Stage::F2);
      const uint8_t* x = xch(t);
      float ds[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 p4 = *reinterpret_cast<const float4*>(x + i * 1024);
        const float4 d4 = *reinterpret_cast<const float4*>(cur + Stage::F1 + 4 * (8 * i + 4 * lg));
        float4 f4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!UQ) f4 = *reinterpret_cast<const float4*>(cur + Stage::F2 + 4 * (8 * i + 4 * lg));
        const float pv[4] = {p4.x, p4.y, p4.z, p4.w}, dd[4] = {d4.x, d4.y, d4.z, d4.w};
        const float fq[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * i + r;
          ds[e] = UQ ? pv[r] * fmaf(dp[e], sc, -dd[r] * sc) : pv[r] * (dp[e] - dd[r]) * (a.sm * fq[r]);
        }
      }
      v8s db[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        db[h] = __builtin_bit_cast(v8s, make_uint4(bf16x2(ds[8 * h], ds[8 * h + 1]), bf16x2(ds[8 * h + 2], ds[8 * h + 3]),
                                                   bf16x2(ds[8 * h + 4], ds[8 * h + 5]),
                                                   bf16x2(ds[8 * h + 6], ds[8 * h + 7])));
      // dK^T += Q_vals^T dS' (channels x keys, K = queries)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          dkt[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_t_operand(cur + Stage::T0, 32 * cb + lr, 2 * h + lg), db[h], dkt[cb], 0, 0, 0);
    };
    issue(0);
    issue(1);
    wait_first();
    barrier_lds();
    for (int t = 0; t < n_steps; ++t) {
      wait_vm_le<0>();
      barrier_lds();   // P of step t is in its slot; stage (t+2) % 3 is free
      issue(t + 2);
      dstep(t);
    }
    wait_vm_le<0>();
    store_rows(a.dk, dkt);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---- dQ -------------------------------------------------------------------------
// UK: the K block scale is the same for all 32 keys of a step (MXFP4, or FP8
// blocks of a multiple of 32 tokens).
// STA: the keys are the tiles of the query tile's window list.
template <bool CAUSAL, bool UK, bool STA>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __align__(16) uint8_t lds[3 * DqStage::BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int n_qt = a.n_alloc / kBwdTile;
  const int work = xcd_work_index(blockIdx.x, gridDim.x);
  const int bh = work / n_qt;
  int qt = work % n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;               // longest query tiles first
  const int qw0 = qt * kBwdTile + 32 * wave;     // this wave's 32 queries
  const int i = qw0 + lr;                        // this lane's query
  const int64_t tokb = (int64_t)bh * a.n_alloc;

  v8s qb[8], gb[8];
  {
    const uint4* qr = reinterpret_cast<const uint4*>(a.q_rows + (tokb + i) * kD);
    const uint4* gr = reinterpret_cast<const uint4*>(a.dos_rows + (tokb + i) * kD);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qb[s] = __builtin_bit_cast(v8s, qr[2 * s + lg]);
      gb[s] = __builtin_bit_cast(v8s, gr[2 * s + lg]);
    }
  }
  const float cq = a.sm_log2 * a.fq[tokb + i];
  const float lse = a.lse_e[tokb + i];
  const float ddi = a.dd[tokb + i];

  const auto kr = rsrc(a.k_rows + tokb * kD, (int64_t)a.n_alloc * kD * 2);
  const auto vr = rsrc(a.v_rows + tokb * kD, (int64_t)a.n_alloc * kD * 2);
  const auto ktr = rsrc(a.kt + tokb * kD, (int64_t)a.n_alloc * kD * 2);
  const auto fkr = rsrc(a.fk + tokb, (int64_t)a.n_alloc * 4);
  const auto kvr = rsrc(a.kvf, (int64_t)a.n_alloc * 4);
  DmaPlan<16> pr;
  pr.init(lane, 2 * kD);
  DmaPlan<4> pt;
  pt.init(lane, 64);   // transposed rows of one step are 64 bytes apart
  auto issue = [&](uint8_t* stg, int k0) __attribute__((always_inline)) {
    issue_rows(kr, stg + DqStage::R0, k0, wave, pr);
    issue_rows(vr, stg + DqStage::R1, k0, wave, pr);
    issue_trans(ktr, stg + DqStage::T0, k0, wave, pt);
    issue_floats(fkr, stg + DqStage::F0, k0, lane);
    issue_floats(kvr, stg + DqStage::F1, k0, lane);
  };

  v16f dqt[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqt[cb][e] = 0.0f;

  const int n_keys = (a.N + 31) / 32 * 32;
  const int k_end = CAUSAL ? min(qt * kBwdTile + kBwdTile, n_keys) : n_keys;
  const bool tail_mask = a.kv_valid != nullptr;

  // S^T (keys x queries) = K Q^T and dP^T = V_codes (dO / s_V)^T of the step
  // in stage `cur`; register 4 ii + r is key k0 + 8 ii + 4 lg + r
  auto products = [&](const uint8_t* cur, v16f& s, v16f& dp) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row_operand(cur + DqStage::R0, lr, 2 * ks + lg), qb[ks], s,
                                                  0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row_operand(cur + DqStage::R1, lr, 2 * ks + lg), gb[ks],
                                                   dp, 0, 0, 0);
    }
  };
  // dS'^T = P^T (dP^T - D) sm / s_K and dQ^T += K_vals^T dS'^T
  auto finish = [&](const int k0, const uint8_t* cur, const v16f& s, const v16f& dp)
      __attribute__((always_inline)) {
    float cs = 0.0f, sc = 0.0f;
    if (UK) {
      const float fk = *reinterpret_cast<const float*>(cur + DqStage::F0);
      cs = cq * fk;
      sc = a.sm * fk;
    }
    const bool masked = tail_mask || k0 + 32 > a.N || (CAUSAL && k0 + 31 > qw0);
    // masked steps keep register 4 ii + r only if the key is valid and (causal)
    // 8 ii + r <= thr, i.e. key <= query
    const int thr = CAUSAL ? i - k0 - 4 * lg : 64;
    v8s db[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float ds[8];
#pragma unroll
      for (int x2 = 0; x2 < 2; ++x2) {
        const int ii = 2 * h + x2;
        float4 f4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!UK) f4 = *reinterpret_cast<const float4*>(cur + DqStage::F0 + 4 * (8 * ii + 4 * lg));
        const float fk[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * ii + r;
          const float pe = __builtin_amdgcn_exp2f(UK ? fmaf(s[e], cs, -lse) : fmaf(s[e] * cq, fk[r], -lse));
          ds[4 * x2 + r] = UK ? pe * fmaf(dp[e], sc, -ddi * sc) : pe * (dp[e] - ddi) * (a.sm * fk[r]);
        }
      }
      if (masked) {
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
          const int ii = 2 * h + x2;
          const float4 kv4 = *reinterpret_cast<const float4*>(cur + DqStage::F1 + 4 * (8 * ii + 4 * lg));
          const float kv[4] = {kv4.x, kv4.y, kv4.z, kv4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool keep = kv[r] != 0.0f && 8 * ii + r <= thr;
            ds[4 * x2 + r] = keep ? ds[4 * x2 + r] : 0.0f;
          }
        }
      }
      db[h] = __builtin_bit_cast(v8s, make_uint4(bf16x2(ds[0], ds[1]), bf16x2(ds[2], ds[3]),
                                                 bf16x2(ds[4], ds[5]), bf16x2(ds[6], ds[7])));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        dqt[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_t_operand(cur + DqStage::T0, 32 * cb + lr, 2 * h + lg),
                                                          db[h], dqt[cb], 0, 0, 0);
  };

  // Software pipeline over 32-key steps t (three LDS stages): iteration t
  // copies step t+2, forms the scores of step t+1 while the vector unit works
  // on step t, then adds step t's products.  Steps past the diagonal (causal)
  // are computed and masked: a branch around the products makes the compiler
  // move the accumulators on every step.  Past the last step the copies (read
  // as padding or zeros, bounded by the buffer descriptors) and the score
  // products are never used.
  auto stage = [&](int t) __attribute__((always_inline)) { return lds + (t % 3) * DqStage::BYTES; };
  constexpr int kIssues = 8;   // copy instructions per wave per stage
  const int spt = STA ? a.tile_tokens / 32 : 1;     // steps per tile
  const int32_t* wl = nullptr;
  int n_steps = k_end / 32;
  if (STA) {
    const int u = qt * kBwdTile / a.tile_tokens;
    wl = a.win_idx + a.win_off[u];
    n_steps = (a.win_off[u + 1] - a.win_off[u]) * spt;
    if (n_steps <= 0) {   // an empty window list: this query sees no key
      if (i < a.N) {
        const int b = bh / a.H, h = bh % a.H;
        float* row = a.dq + b * a.g_sb + h * a.g_sh + (int64_t)i * a.g_sn;
        for (int c = 4 * lg; c < kD; c += 8)
          *reinterpret_cast<float4*>(row + c) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      return;
    }
  }
  // first key of step t; the copies issued past the last step repeat it
  auto kstart = [&](int t) __attribute__((always_inline)) -> int {
    if (!STA) return 32 * t;
    const int tc = t < n_steps ? t : n_steps - 1;
    return a.tile_tokens * __builtin_amdgcn_readfirstlane(wl[tc / spt]) + 32 * (tc % spt);
  };
  issue(stage(0), kstart(0));
  issue(stage(1), kstart(1));
  wait_vm_le<kIssues>();
  barrier_lds();
  v16f sa, dpa, sb, dpb;
  products(stage(0), sa, dpa);
  auto body = [&](const int t, v16f& s_cur, v16f& dp_cur, v16f& s_nxt, v16f& dp_nxt)
      __attribute__((always_inline)) {
    wait_vm_le<0>();
    barrier_lds();   // step t+1 has landed everywhere; stage (t+2) % 3 is free
    issue(stage(t + 2), kstart(t + 2));
    products(stage(t + 1), s_nxt, dp_nxt);
    finish(kstart(t), stage(t), s_cur, dp_cur);
  };
  int t = 0;
  for (; t + 2 <= n_steps; t += 2) {
    body(t, sa, dpa, sb, dpb);
    body(t + 1, sb, dpb, sa, dpa);
  }
  if (t < n_steps) finish(kstart(t), stage(t), sa, dpa);   // odd count: the last step
  wait_vm_le<0>();
  if (i < a.N) {
    const int b = bh / a.H, h = bh % a.H;
    float* row = a.dq + b * a.g_sb + h * a.g_sh + (int64_t)i * a.g_sn;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        *reinterpret_cast<float4*>(row + 32 * cb + 8 * ii + 4 * lg) =
            make_float4(dqt[cb][4 * ii], dqt[cb][4 * ii + 1], dqt[cb][4 * ii + 2], dqt[cb][4 * ii + 3]);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

hipError_t launch_attention_backward(const BwdArgs& a, hipStream_t st) {
  const unsigned BH = (unsigned)(a.B * a.H);
  const dim3 g64((unsigned)(a.n_alloc / 64), BH);
  if (a.qk_mx)
    hipLaunchKernelGGL(bwd_prep_qk_kernel<true>, dim3(g64.x, g64.y, 2), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_prep_qk_kernel<false>, dim3(g64.x, g64.y, 2), dim3(256), 0, st, a);
  if (a.v_mx)
    hipLaunchKernelGGL(bwd_prep_v_kernel<true>, g64, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_prep_v_kernel<false>, g64, dim3(256), 0, st, a);
  if (a.dout_bf16)
    hipLaunchKernelGGL(bwd_prep_do_kernel<__hip_bfloat16>, g64, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_prep_do_kernel<float>, g64, dim3(256), 0, st, a);
  const dim3 gt(BH * (unsigned)(a.n_alloc / kBwdTile));
  // the Q scale is uniform over 32-query steps for MXFP4 (1) and for FP8 blocks of 32k tokens
  const bool uq = a.qk_mx || a.blk_q % 32 == 0;
  const bool uk = a.qk_mx || a.blk_k % 32 == 0;
  if (a.win_idx) {
    if (uq)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<false, true, true>), gt, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<false, false, true>), gt, dim3(512), 0, st, a);
    if (uk)
      hipLaunchKernelGGL((bwd_dq_kernel<false, true, true>), gt, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<false, false, true>), gt, dim3(256), 0, st, a);
  } else if (a.causal) {
    if (uq)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<true, true, false>), gt, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<true, false, false>), gt, dim3(512), 0, st, a);
    if (uk)
      hipLaunchKernelGGL((bwd_dq_kernel<true, true, false>), gt, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<true, false, false>), gt, dim3(256), 0, st, a);
  } else {
    if (uq)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<false, true, false>), gt, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<false, false, false>), gt, dim3(512), 0, st, a);
    if (uk)
      hipLaunchKernelGGL((bwd_dq_kernel<false, true, false>), gt, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<false, false, false>), gt, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace pab
