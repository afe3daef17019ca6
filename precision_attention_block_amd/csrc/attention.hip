// Fused block-scaled attention forward for gfx950 (CDNA4).
//
// O = softmax(Q K^T * sm_scale) V computed FlashAttention-style: tiles of
// BN = 64 keys are visited in ascending order with an online softmax, so no
// N x N matrix leaves the chip ["FA4极速LLM：10分钟搞定20倍内存直降！",
// FlashAttention section: tiling, online softmax, fusion].
// Precision recipe ["FP8量化与稀疏性协同加速视频扩散模型", §3.1 staged
// quantisation]: Q/K FP8 per block (or MXFP4 per 32 channels, "Blackwell架构实战：
// 如何用FP4量化让你的AI模型推理速度翻倍（附代码）", §1), V FP8 per channel,
// P requantised to FP8 with the fixed tensor scale 1/448.
// Sparse schedule [FPSAttention page, §2.2]: a query tile visits only the key
// tiles in its window list.
//
// Mapping onto CDNA4.  A workgroup of 4 waves owns BM = 128 queries of one
// head; each wave owns 32 queries (one 32-wide MFMA column block).
//  * S^T = K Q^T with 32x32 MFMAs.  In the 32x32 result layout lane l holds
//    query l % 32 and 16 keys of each 32-key block, so the row max / row sum
//    are in-lane reductions plus one lane swap (l <-> l ^ 32).
//    - FP8 recipe: the E4M3 values are fed to v_mfma_f32_32x32x16_bf16 as
//      exact bf16 copies written by the quantizer.  The f8f6f4 MFMAs sum FP8
//      products with only ~12 bits below the largest product (measured:
//      errors up to 4e-4 of sum |q_k k_k| on quantised N(0,1) data with
//      outlier channels), which after exponentiation breaks the 1e-2 output
//      agreement; the bf16 MFMA sums the same exact products to fp32
//      accuracy.
//    - MXFP4 recipe: v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and
//      the E8M0 group scale of each lane's 32 channels fed to the MFMA.
//  * P = exp2(S c - m + log2 448) is formed directly in the 448-scaled domain
//    and converted to E4M3 in registers; the lane then holds one query and 32
//    keys, which is exactly the B operand of O^T += V^T P~^T
//    (v_mfma_scale_f32_32x32x64_f8f6f4, FP8 x FP8): no data movement.  The V
//    quantizer stores V^T in the matching key order.
//  * the running output is rescaled only when some row maximum of the wave
//    moved (conditional rescaling, FA4 co-design list; threshold 0, so the
//    result equals an unconditional rescale).
//  * K and V^T tiles are double-buffered in LDS and copied by LDS-DMA
//    (buffer_load ... lds: no registers involved) into XOR-swizzled layouts
//    with conflict-free 16-byte operand reads; the copy of the next tile is in
//    flight while the current one is computed.
//  * workgroups are dealt to XCDs so that all query tiles of a head share an
//    L2; causal query tiles are issued longest-first (LPT).
#include "pab_device.h"
#include "pab_internal.h"

namespace pab {

constexpr float kNegInf = -__builtin_huge_valf();
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v8s __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Slot of 16-byte chunk c of row r in a swizzled LDS tile with CPR chunks per
// row is c ^ swz(r).  Every operand read below has the 16 lanes of one LDS
// phase read the same chunk index of 16 consecutive rows; the swizzle sends
// them to 16 disjoint 4-bank groups.
template <int CPR>
__device__ constexpr int swz(int row) {
  return CPR == 16 ? (row & 15) : CPR == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

template <int D, bool MX>
struct Tile {
  // K ring stage: FP8 recipe: K as bf16 (exact E4M3 values); MXFP4: packed
  // E2M1 plus the E8M0 group scales.
  static constexpr int KROW = MX ? D / 2 : 2 * D;   // bytes of one key row
  static constexpr int K_CPR = KROW / 16;
  static constexpr int K_BYTES = kBN * KROW;
  static constexpr int S_BYTES = MX ? kBN * (D / 32) : 0;
  static constexpr int KBUF = K_BYTES + S_BYTES;
  // V ring stage: V^T codes, the key padding mask and (FP8) the K block scales
  static constexpr int V_BYTES = D * kBN;           // D rows of kBN E4M3 codes
  static constexpr int M_BYTES = kBN;
  static constexpr int C_BYTES = MX ? 0 : 16;       // K block scales of the tile (<= 4)
  static constexpr int VBUF = V_BYTES + M_BYTES + C_BYTES;
  static constexpr int KI = K_BYTES / 1024 / 4;     // LDS-DMA instructions per wave
  static constexpr int VI = V_BYTES / 1024 / 4;
  static_assert(KBUF % 16 == 0 && VBUF % 16 == 0, "LDS stages must stay 16-byte aligned");
  static_assert(K_BYTES % 4096 == 0 && V_BYTES % 4096 == 0, "copy must split over 4 waves");
};

// Lane offsets of the LDS-DMA copy of a region of rows (16 CPR bytes each,
// gstride bytes apart in HBM).  Instruction `inst` fills region bytes
// [1024 inst, 1024 inst + 1024), lane i writing 16 bytes at 1024 inst + 16 i
// and fetching the global chunk that belongs in that slot.  The swizzle of
// row inst * RPI + lane / CPR depends on inst only through inst % PER.
template <int CPR>
struct DmaPlan {
  static constexpr int RPI = 64 / CPR;                            // rows per instruction
  static constexpr int PER = CPR == 16 ? 4 : CPR == 8 ? 2 : 1;    // swizzle period
  uint32_t off[PER];
  __device__ void init(int lane, int64_t gstride) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int row = p * RPI + lane / CPR;
      off[p] = (uint32_t)((lane / CPR) * gstride + 16 * ((lane % CPR) ^ swz<CPR>(row)));
    }
  }
};

#if defined(__HIP_DEVICE_COMPILE__)
// (buffer descriptors and everything that uses them exist in the device pass only)
struct HeadBuffers {
  __amdgpu_buffer_rsrc_t k, v, s, m, c;
  bool has_mask;
  int blk_k;
};
constexpr int kRsrcWord3 = 0x00020000;   // raw byte buffer

// Every wave issues the same number of LDS-DMA instructions per stage (K for
// a K stage, V for a V stage), and every pipeline iteration copies one K and
// one V stage, so one outstanding-copy count serves every wave and iteration.
template <int D, bool MX>
struct Issues {
  static constexpr int K = Tile<D, MX>::KI + (MX ? 1 : 0);
  static constexpr int V = Tile<D, MX>::VI + 1 + (MX ? 0 : 1);
};

// Copies the K (and MXFP4 group scales) of the key tile at `ks` into a K stage.
template <int D, bool MX, typename KPlan>
__device__ inline void issue_k(uint8_t* kbuf, const HeadBuffers& hb, int ks, int wave, int lane,
                               const KPlan& kp) {
  using TL = Tile<D, MX>;
  constexpr int KRPI = DmaPlan<TL::K_CPR>::RPI, KPER = DmaPlan<TL::K_CPR>::PER;
#pragma unroll
  for (int j = 0; j < TL::KI; ++j) {
    const int inst = wave * TL::KI + j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.k, (lds_void_t*)(kbuf + inst * 1024), 16,
                                             kp.off[inst % KPER], (ks + inst * KRPI) * TL::KROW, 0, 0);
  }
  if (MX && lane < 4)   // 256 bytes of E8M0 scales: 4 lanes x 16 bytes per wave
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.s, (lds_void_t*)(kbuf + TL::K_BYTES + 64 * wave), 16,
                                             16 * (lane & 3), ks * (D / 32) + 64 * wave, 0, 0);
}

// Copies V^T, the padding mask and (FP8) the K block scales of the key tile at
// `ks` into a V stage.  Each LDS-DMA instruction writes 16 bytes per active
// lane, so the small copies run on lane 0 only (every wave copies the same K
// scales to the same place, which is harmless).
template <int D, bool MX, typename VPlan>
__device__ inline void issue_v(uint8_t* vbuf, const HeadBuffers& hb, int n_alloc, int ks, int wave,
                               int lane, const VPlan& vp) {
  using TL = Tile<D, MX>;
#pragma unroll
  for (int j = 0; j < TL::VI; ++j) {
    const int inst = wave * TL::VI + j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.v, (lds_void_t*)(vbuf + inst * 1024), 16, vp.off[0],
                                             ks + inst * 16 * n_alloc, 0, 0);
  }
  if (lane == 0)   // 64 mask bytes, 16 per wave (zeros when there is no mask: ignored then)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.m, (lds_void_t*)(vbuf + TL::V_BYTES + 16 * wave), 16,
                                             0, ks + 16 * wave, 0, 0);
  if (!MX && lane == 0)   // the K block scales covering keys ks .. ks + BN - 1 (block size >= 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.c, (lds_void_t*)(vbuf + TL::V_BYTES + TL::M_BYTES),
                                             16, 0, (ks / hb.blk_k) * 4, 0, 0);
}

// Workgroup barrier that does not wait for outstanding LDS-DMA copies (a
// plain __syncthreads() fences every memory operation, including the copies
// that are meant to stay in flight); this wave's LDS reads are complete first.
// The waits use the s_waitcnt builtin (simm16: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8) rather than inline asm so that the compiler's own
// wait-count tracking sees them and adds no conservative waits of its own.
__device__ inline void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Waits until at most N of this wave's LDS-DMA copies are outstanding.
template <int N>
__device__ inline void wait_vm_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ inline v8i make_v8(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// True if some byte of w is zero.
__device__ inline bool has_zero_byte(uint32_t w) {
  return ((w - 0x01010101u) & ~w & 0x80808080u) != 0u;
}
#endif  // __HIP_DEVICE_COMPILE__

__device__ inline float swap_max(float v) {
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ inline float swap_sum(float v) {
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// MODE: 0 dense, 1 causal (top-left aligned), 2 sliding-tile.
// UK: the K scale is constant over each key tile (FP8 blocks a multiple of BN).
//
// Software pipeline over key tiles t = 0, 1, ...: iteration t issues the
// copies of K(t+3) and V(t+2), the QK^T MFMAs of tile t+1, the softmax of
// tile t (interleaved with those MFMAs) and the P.V MFMAs of tile t.  K and
// V each have a 3-stage LDS ring, so every copy has two iterations to land.
template <int D, bool MX, int MODE, bool UK>
__global__ __launch_bounds__(256, (MX && MODE != 2) ? 3 : 2) void attn_fwd_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using TL = Tile<D, MX>;
  constexpr int DB = D / 32;            // 32-channel blocks of O^T
  constexpr int QI = D / 16;            // bf16 32x32x16 MFMAs over d (FP8 recipe)
  constexpr int NK = Issues<D, MX>::K, NV = Issues<D, MX>::V;
  constexpr int QK_MFMA = MX ? 4 : 2 * QI;          // QK^T MFMAs per key tile
  constexpr int VALU_PER_MFMA = MX ? 30 : 8;
  constexpr int PRE_DS = 8;                          // LDS reads issued ahead
  constexpr int DS_PER_MFMA = MX ? 2 : 1;
  constexpr bool INTERLEAVE = true;
  // Distinct LDS objects per stage: the compiler can then see that a copy
  // into one stage does not alias reads of another and does not wait for it.
  __shared__ __align__(16) uint8_t k0[TL::KBUF], k1[TL::KBUF], k2[TL::KBUF];
  __shared__ __align__(16) uint8_t v0[TL::VBUF], v1[TL::VBUF], v2[TL::VBUF];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform; saying so keeps LDS-DMA addresses (M0) scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;     // MFMA column (query) and k-group
  const int work = xcd_work_index(blockIdx.x, gridDim.x);

  int bh, q0, n_steps, u = 0;
  const int spt = MODE == 2 ? a.tile_tokens / kBN : 1;
  if (MODE == 2) {
    const int sub = a.tile_tokens / kBM;               // query tiles per window tile
    const int per_bh = a.n_tiles * sub;
    bh = work / per_bh;
    const int r = work % per_bh;
    u = a.tile_order[r / sub];
    q0 = u * a.tile_tokens + (r % sub) * kBM;
    n_steps = (a.win_off[u + 1] - a.win_off[u]) * spt;
  } else {
    bh = work / a.n_qtiles;
    int qt = work % a.n_qtiles;
    if (MODE == 1) qt = a.n_qtiles - 1 - qt;   // longest query tiles first
    q0 = qt * kBM;
    const int all = (a.N + kBN - 1) / kBN;
    n_steps = MODE == 1 ? min((q0 + kBM) / kBN, all) : all;
  }
  const int wq0 = q0 + wave * 32;             // first query of this wave
  const int myq = wq0 + lr;                   // this lane's query
  const int32_t* wlist = MODE == 2 ? a.win_idx + a.win_off[u] : nullptr;
  auto step_start = [&](int t) -> int {
    if (MODE == 2) return wlist[t / spt] * a.tile_tokens + (t % spt) * kBN;
    return t * kBN;
  };

  const int64_t tok0 = (int64_t)bh * a.n_alloc;
  const uint8_t* kbh = (MX ? a.k : a.k16) + tok0 * TL::KROW;
  const uint8_t* vbh = a.vt + (int64_t)bh * D * a.n_alloc;

  // ---- Q operand (B of S^T = K Q^T), kept in registers for the whole pass.
  // FP8: at MFMA step i lane (query lr, group lg) holds the 8 channels of
  // chunk QI * lg + i; K is read with the same chunk order, so every channel
  // pairs exactly once.  MXFP4: at step i the 32 channels of group 2 i + lg.
  v8s qop16[QI];
  v8i qop8[2];
  int qsc[2] = {127, 127};
  float cq;
  {
    const int64_t qrow = tok0 + myq;
    if (MX) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
        const uint4 x = *reinterpret_cast<const uint4*>(a.q + qrow * (D / 2) + 16 * (2 * i + lg));
        r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
        qop8[i] = r;
        qsc[i] = a.q_mx[qrow * (D / 32) + 2 * i + lg];
      }
      cq = a.sm_log2;
    } else {
      const uint8_t* qp = a.q16 + qrow * (2 * D) + 16 * QI * lg;
#pragma unroll
      for (int i = 0; i < QI; ++i)
        qop16[i] = __builtin_bit_cast(v8s, *reinterpret_cast<const uint4*>(qp + 16 * i));
      cq = a.sm_log2 / a.q_scale[(int64_t)bh * a.nblk_q + myq / a.blk_q];
    }
  }

  float m_run = kNegInf, l_run = 0.0f;
  v16f o[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[cb][j] = 0.0f;

  DmaPlan<TL::K_CPR> kp;
  DmaPlan<4> vp;
  kp.init(lane, TL::KROW);
  vp.init(lane, a.n_alloc);
  HeadBuffers hb;
  hb.k = __builtin_amdgcn_make_buffer_rsrc((void*)kbh, 0, a.n_alloc * TL::KROW, kRsrcWord3);
  hb.v = __builtin_amdgcn_make_buffer_rsrc((void*)vbh, 0, a.n_alloc * D, kRsrcWord3);
  hb.s = __builtin_amdgcn_make_buffer_rsrc((void*)(MX ? a.k_mx + tok0 * (D / 32) : kbh), 0,
                                           MX ? a.n_alloc * (D / 32) : 0, kRsrcWord3);
  hb.has_mask = a.kv_valid != nullptr;
  hb.m = __builtin_amdgcn_make_buffer_rsrc((void*)(hb.has_mask ? a.kv_valid : kbh), 0,
                                           hb.has_mask ? a.N : 0, kRsrcWord3);
  hb.blk_k = MX ? 1 : a.blk_k;
  hb.c = __builtin_amdgcn_make_buffer_rsrc((void*)(MX ? kbh : (const void*)(a.k_scale + (int64_t)bh * a.nblk_k)),
                                           0, MX ? 0 : a.nblk_k * 4, kRsrcWord3);

  // Per-lane byte offsets of this lane's operand chunks inside a stage; the
  // rows are 32 kb + lr, so the swizzle depends on lr only (32, the rows per
  // block, is a multiple of every swizzle period).
  int k_off[MX ? 2 : QI];
  if (MX) {
#pragma unroll
    for (int i = 0; i < 2; ++i) k_off[i] = lr * TL::KROW + 16 * ((2 * i + lg) ^ swz<4>(lr));
  } else {
#pragma unroll
    for (int i = 0; i < QI; ++i) k_off[i] = lr * TL::KROW + 16 * ((QI * lg + i) ^ swz<TL::K_CPR>(lr));
  }
  const int v_off0 = lr * kBN + 16 * ((2 * lg) ^ swz<4>(lr));
  const int v_off1 = lr * kBN + 16 * ((2 * lg + 1) ^ swz<4>(lr));

  // S^T (keys x queries) of the key tile in K stage `Ks`, fp32 accumulate:
  // s[kb][j] is key 32 kb + 8 (j / 4) + 4 lg + j % 4 of the tile, query myq.
  auto qk = [&](const uint8_t* Ks, v16f (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      v16f acc;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
      if (MX) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          v8i kr = {0, 0, 0, 0, 0, 0, 0, 0};
          const uint4 x = *reinterpret_cast<const uint4*>(Ks + kb * 32 * TL::KROW + k_off[i]);
          kr[0] = x.x; kr[1] = x.y; kr[2] = x.z; kr[3] = x.w;
          const int ksc = Ks[TL::K_BYTES + (32 * kb + lr) * (D / 32) + 2 * i + lg];
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr, qop8[i], acc, 4, 4, 0, ksc, 0,
                                                                qsc[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < QI; ++i) {
          const v8s kr = __builtin_bit_cast(
              v8s, *reinterpret_cast<const uint4*>(Ks + kb * 32 * TL::KROW + k_off[i]));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr, qop16[i], acc, 0, 0, 0);
        }
      }
      s[kb] = acc;
    }
  };

  // Online softmax of the tile at key `ks` (scores s, V stage Vs) and
  // O^T += V^T P~^T.  `overlap` runs just before the exponentials, in the same
  // straight-line block, so that independent MFMAs can be interleaved with the
  // softmax arithmetic.
  auto softmax_pv = [&](const int ks, v16f (&s)[2], const uint8_t* Vs, auto overlap)
      __attribute__((always_inline)) {
    const uint8_t* Ms = Vs + TL::V_BYTES;
    const float* Cs = reinterpret_cast<const float*>(Ms + TL::M_BYTES);
    // dequantisation factor c (log2 domain): c = sm_scale log2(e) / (s_Q s_K),
    // per group of 4 keys (kb, j / 4); constant over the tile when UK.
    float c[8];
    if (MX) {
#pragma unroll
      for (int g = 0; g < 8; ++g) c[g] = cq;
    } else if (UK) {
      const float ck = cq * __builtin_amdgcn_rcpf(Cs[0]);
#pragma unroll
      for (int g = 0; g < 8; ++g) c[g] = ck;
    } else {
#pragma unroll
      for (int g = 0; g < 8; ++g) {   // Cs[i] is the scale of block ks / blk + i
        const int key = ks + 32 * (g / 4) + 8 * (g % 4);
        c[g] = cq * __builtin_amdgcn_rcpf(Cs[key / a.blk_k - ks / a.blk_k]);
      }
    }
    // masks: padding keys (staged in LDS with the tile), keys past N, the
    // causal diagonal; the test is wave-uniform, the masking branch-free
    uint32_t kvw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    bool partial = false;
    if (hb.has_mask) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        kvw[g] = *reinterpret_cast<const uint32_t*>(Ms + 32 * (g / 4) + 8 * (g % 4) + 4 * lg);
        partial |= has_zero_byte(kvw[g]);
      }
    }
    const bool need_mask = (ks + kBN > a.N) || (MODE == 1 && ks + kBN - 1 > wq0) ||
                           (__builtin_amdgcn_ballot_w64(partial) != 0);
    if (need_mask) {
      const int lim = MODE == 1 ? min(a.N - 1, myq) : a.N - 1;   // last admissible key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = ks + 32 * kb + 8 * (j / 4) + 4 * lg + (j % 4);
          const uint32_t byte = (kvw[4 * kb + j / 4] >> (8 * (j % 4))) & 0xFFu;
          const bool ok = (key <= lim) & (!hb.has_mask | (byte != 0u));
          s[kb][j] = ok ? s[kb][j] : kNegInf;
        }
    }
    // running max; with one factor c for the whole tile (c > 0) the max of
    // c s is c times the max of s
    float mx;
    if (MX || UK) {
      float m = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; j += 2) m = fmaxf(m, fmaxf(s[kb][j], s[kb][j + 1]));
      mx = c[0] * m;
    } else {
      mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float m4 = fmaxf(fmaxf(s[kb][4 * g4], s[kb][4 * g4 + 1]),
                                 fmaxf(s[kb][4 * g4 + 2], s[kb][4 * g4 + 3]));
          mx = fmaxf(mx, c[4 * kb + g4] * m4);
        }
    }
    mx = swap_max(mx);
    const float mnew = fmaxf(m_run, mx);
    const float alpha = mnew == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mnew);
    const float msh = mnew == kNegInf ? 0.0f : mnew - kLog2_448;
    m_run = mnew;
    // conditional rescale of the running output
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int cb = 0; cb < DB; ++cb) o[cb] *= alpha;
    }
    overlap();
    // P in the 448-scaled domain, E4M3 in registers
    float sum = 0.0f;
    v8i pk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float cc = c[4 * kb + g4];
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * g4 + 0], cc, -msh));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * g4 + 1], cc, -msh));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * g4 + 2], cc, -msh));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * g4 + 3], cc, -msh));
        sum += (p0 + p1) + (p2 + p3);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
        pk[4 * kb + g4] = w;
      }
    // interleave: the next tile's QK^T MFMAs (and their LDS operand reads)
    // spread over the softmax arithmetic above
    // (LDS reads run PRE_DS ahead of the MFMAs that consume them; the V
    // operand reads of the P.V product join the same stream)
    if (INTERLEAVE) {
      __builtin_amdgcn_sched_group_barrier(0x100, PRE_DS, 0);    // LDS reads in flight
#pragma unroll
      for (int i = 0; i < QK_MFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, DS_PER_MFMA, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);
      }
    }
    l_run = l_run * alpha + sum;
    // O^T += V^T P~^T (FP8 x FP8)
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {
      const v8i vr = make_v8(*reinterpret_cast<const uint4*>(Vs + cb * 32 * kBN + v_off0),
                             *reinterpret_cast<const uint4*>(Vs + cb * 32 * kBN + v_off1));
      o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vr, pk, o[cb], 0, 0, 0, 127, 0, 127);
    }
  };

  // ---- prologue: K(0), V(0), K(1), V(1), K(2) in flight; wait for the first three.
  // Past the last tile the copies repeat the last tile into stages nobody
  // reads, which keeps the number of outstanding copies fixed.
  auto tile_at = [&](int t) { return step_start(min(t, n_steps - 1)); };
  issue_k<D, MX>(k0, hb, tile_at(0), wave, lane, kp);
  issue_v<D, MX>(v0, hb, a.n_alloc, tile_at(0), wave, lane, vp);
  issue_k<D, MX>(k1, hb, tile_at(1), wave, lane, kp);
  issue_v<D, MX>(v1, hb, a.n_alloc, tile_at(1), wave, lane, vp);
  issue_k<D, MX>(k2, hb, tile_at(2), wave, lane, kp);
  wait_vm_le<NV + NK>();          // V(1) and K(2) may still be in flight
  barrier_lds();

  v16f s_cur[2], s_nxt[2];
  qk(k0, s_cur);

  // Iteration t with K stages (Kn1 = t+1, Kn3 = t+3) and V stages (Vc = t, Vn2 = t+2).
  auto iter = [&](const int t, const uint8_t* Kn1, uint8_t* Kn3, const uint8_t* Vc, uint8_t* Vn2)
      __attribute__((always_inline)) {
    const int ks = step_start(t);
    issue_k<D, MX>(Kn3, hb, tile_at(t + 3), wave, lane, kp);
    issue_v<D, MX>(Vn2, hb, a.n_alloc, tile_at(t + 2), wave, lane, vp);
    // (on the last iteration Kn1 holds a repeat of the last tile; the scores
    // computed from it are not used - computing them keeps this code one
    // straight-line block with the exponentials)
    softmax_pv(ks, s_cur, Vc, [&]() __attribute__((always_inline)) { qk(Kn1, s_nxt); });
    // K(t+2) and V(t+1) must have landed; this iteration's copies may not have
    wait_vm_le<NK + NV>();
    barrier_lds();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_nxt[kb];
  };
  for (int t = 0; t < n_steps; t += 3) {
    iter(t, k1, k0, v0, v2);
    if (t + 1 < n_steps) iter(t + 1, k2, k1, v1, v0);
    if (t + 2 < n_steps) iter(t + 2, k0, k2, v2, v1);
  }

  // ---- epilogue: O = acc / (448 l) / s_V, stored through the output permutation
  const float lt = swap_sum(l_run);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (myq < a.N) {
    const int tok = a.out_perm ? a.out_perm[myq] : myq;
    if (tok >= 0) {
      const int b = bh / a.H, h = bh % a.H;
      float* orow = a.out + b * a.osb + h * a.osh + (int64_t)tok * a.osn;
      const float* vs = a.v_scale + (int64_t)bh * D;
#pragma unroll
      for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c0 = 32 * cb + 8 * g4 + 4 * lg;
          float4 r;
          r.x = o[cb][4 * g4 + 0] * inv / vs[c0 + 0];
          r.y = o[cb][4 * g4 + 1] * inv / vs[c0 + 1];
          r.z = o[cb][4 * g4 + 2] * inv / vs[c0 + 2];
          r.w = o[cb][4 * g4 + 3] * inv / vs[c0 + 3];
          *reinterpret_cast<float4*>(orow + c0) = r;
        }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool MX, int MODE>
static hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const bool uk = MX || a.blk_k % kBN == 0;
  const int64_t blocks = MODE == 2 ? (int64_t)a.B * a.H * a.n_tiles * (a.tile_tokens / kBM)
                                   : (int64_t)a.B * a.H * a.n_qtiles;
  if (uk)
    hipLaunchKernelGGL((attn_fwd_kernel<D, MX, MODE, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, MX, MODE, false>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, bool MX>
static hipError_t launch_mode(const AttnArgs& a, int mode, hipStream_t st) {
  if (mode == 1) return launch_t<D, MX, 1>(a, st);
  if (mode == 2) return launch_t<D, MX, 2>(a, st);
  return launch_t<D, MX, 0>(a, st);
}

hipError_t launch_attention(const AttnArgs& a, int d, bool mx, int mode, hipStream_t st) {
  if (mx) return launch_mode<128, true>(a, mode, st);
  if (d == 64) return launch_mode<64, false>(a, mode, st);
  return launch_mode<128, false>(a, mode, st);
}

}  // namespace pab
