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
//  * K and V^T tiles live in 3-stage LDS rings filled by LDS-DMA
//    (buffer_load ... lds: no registers involved) in XOR-swizzled layouts
//    with conflict-free 16-byte operand reads; copies run two to three tiles
//    ahead of the tile being computed.
//  * one wave keeps both units busy: the softmax of tile t is interleaved
//    with the P.V MFMAs of tile t-1 and the QK^T MFMAs of tile t+1.
//  * workgroups are dealt to XCDs so that all query tiles of a head share an
//    L2; a causal workgroup computes a long and a short query tile of its
//    head in turn (tiles n - 1 - p and p), so all causal workgroups carry the
//    same work and the launch has no tail of short tiles (FP8 and FP4 P.V;
//    see the pairing note in the kernel).
//  * a workgroup whose queries are all padding ends at once; the output is
//    staged through LDS and written with streaming stores of whole 128-byte
//    row segments (store_o_rows).
// Dense FP8 attention with d = 128 over all key tiles runs on the ping-pong
// kernel further below instead.
#include "pab_device.h"
#include "pab_internal.h"
#include "pab_lds.h"

namespace pab {

constexpr float kNegInf = -__builtin_huge_valf();
typedef short v8s __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int D, bool MX, bool V4 = false>
struct Tile {
  // K ring stage: FP8 recipe: K as bf16 (exact E4M3 values); MXFP4: packed
  // E2M1 plus the E8M0 group scales.
  static constexpr int KROW = MX ? D / 2 : 2 * D;   // bytes of one key row
  static constexpr int K_CPR = KROW / 16;
  static constexpr int K_BYTES = kBN * KROW;
  static constexpr int S_BYTES = MX ? kBN * (D / 32) : 0;   // 256: one full-wave dword copy
  static constexpr int KBUF = K_BYTES + S_BYTES;
  // V ring stage: D rows of kBN E4M3 codes of V^T; FP4 P.V (V4): D rows of
  // kBN E2M1 codes (32 bytes) followed by the 256 E8M0 scale bytes of the tile
  static constexpr int VROW = V4 ? kBN / 2 : kBN;
  static constexpr int V_CPR = VROW / 16;
  static constexpr int VCODES = D * VROW;
  static constexpr int VSB = V4 ? 2 * D : 0;
  static constexpr int VBUF = VCODES + VSB;
  // side ring stage: the key padding mask bytes and (FP8) the K block scales,
  // each copied as one full-wave 256-byte LDS-DMA (only the first kBN mask
  // bytes and the first few scales are used)
  static constexpr int M_BYTES = 256;
  static constexpr int ABUF = M_BYTES + (MX ? 0 : 256);
  static constexpr int KI = K_BYTES / 1024 / 4;     // LDS-DMA instructions per wave
  static constexpr int VI = VCODES / 1024 / 4;
  static_assert(KBUF % 16 == 0 && VBUF % 16 == 0 && ABUF % 16 == 0,
                "LDS stages must stay 16-byte aligned");
  static_assert(K_BYTES % 4096 == 0 && VCODES % 4096 == 0, "copy must split over 4 waves");
  static_assert(!V4 || (MX && D == 128), "FP4 P.V runs with MXFP4 Q/K and d = 128");
};

#if defined(__HIP_DEVICE_COMPILE__)
// (buffer descriptors and everything that uses them exist in the device pass only)
struct HeadBuffers {
  __amdgpu_buffer_rsrc_t k, v, s, m, c, vs;   // vs: E8M0 V scales (FP4 P.V)
  bool has_mask;
  int blk_k;
};

// Every wave issues the same number of LDS-DMA instructions per copy (K for
// a K stage, V for a V stage plus a side stage), and every pipeline iteration
// issues one of each, so one outstanding-copy count serves every wave and
// iteration.
template <int D, bool MX, bool V4 = false>
struct Issues {
  static constexpr int K = Tile<D, MX, V4>::KI + (MX ? 1 : 0);
  static constexpr int V = Tile<D, MX, V4>::VI + (V4 ? 1 : 0);   // V4: plus the V scales
  static constexpr int A = MX ? 1 : 2;
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
  // the 256 bytes of E8M0 scales: one dword per lane; every wave copies the
  // same bytes to the same place, which keeps the copy a full-wave one
  if (MX)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.s, (lds_void_t*)(kbuf + TL::K_BYTES), 4, 4 * lane,
                                             ks * (D / 32), 0, 0);
}

// V^T copy instruction `inst` of the key tile at `ks` into a V stage (rows of
// VROW bytes, 1024 / VROW rows per instruction, n_alloc * VROW / kBN bytes
// apart in HBM).
template <int D, bool MX, bool V4, typename VPlan>
__device__ inline void issue_v_inst(uint8_t* vbuf, const HeadBuffers& hb, int n_alloc, int ks,
                                    int inst, const VPlan& vp) {
  using TL = Tile<D, MX, V4>;
  constexpr int RPI = 1024 / TL::VROW;
  const int gstride = V4 ? n_alloc / 2 : n_alloc;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.v, (lds_void_t*)(vbuf + inst * 1024), 16, vp.off[0],
                                           (V4 ? ks / 2 : ks) + inst * RPI * gstride, 0, 0);
}

// FP4 P.V: the 256 E8M0 V scale bytes of the key tile at `ks` (two 32-token
// groups x 128 channels), one dword per lane; every wave copies the same
// bytes to the same place.
template <int D, bool MX, bool V4>
__device__ inline void issue_vscale(uint8_t* vbuf, const HeadBuffers& hb, int ks, int lane) {
  using TL = Tile<D, MX, V4>;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.vs, (lds_void_t*)(vbuf + TL::VCODES), 4, 4 * lane,
                                           (ks / 32) * D, 0, 0);
}

// Copies V^T (and, FP4 P.V, its scales) of the key tile at `ks` into a V stage.
template <int D, bool MX, bool V4, typename VPlan>
__device__ inline void issue_v(uint8_t* vbuf, const HeadBuffers& hb, int n_alloc, int ks, int wave,
                               int lane, const VPlan& vp) {
  using TL = Tile<D, MX, V4>;
#pragma unroll
  for (int j = 0; j < TL::VI; ++j) issue_v_inst<D, MX, V4>(vbuf, hb, n_alloc, ks, wave * TL::VI + j, vp);
  if (V4) issue_vscale<D, MX, V4>(vbuf, hb, ks, lane);
}

// Copies the padding mask and (FP8) the K block scales of the key tile at `ks`
// into a side stage: full-wave dword copies of 256 bytes each (past the end of
// either buffer the copy reads zeros); every wave copies the same bytes to the
// same place.
template <int D, bool MX>
__device__ inline void issue_aux(uint8_t* abuf, const HeadBuffers& hb, int ks, int lane) {
  using TL = Tile<D, MX>;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.m, (lds_void_t*)abuf, 4, 4 * lane, ks, 0, 0);
  if (!MX)   // scales of the blocks from ks / blk on (a tile spans at most 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.c, (lds_void_t*)(abuf + TL::M_BYTES), 4, 4 * lane,
                                             (ks / hb.blk_k) * 4, 0, 0);
}

// The bf16 operand of S = K Q^T for one lane of the FP8 recipe, converted in
// registers from the lane's QI chunks of 8 consecutive E4M3 codes (channels
// 8 (QI lg + i) .. + 7 at step i): every E4M3 value is exact in bf16, so this
// equals the decoded value of each code.
template <int QI>
__device__ inline void load_q_codes(const uint8_t* p, v8s (&qop)[QI]) {
#pragma unroll
  for (int i = 0; i < QI; i += 2) {
    const uint4 c = *reinterpret_cast<const uint4*>(p + 8 * i);   // chunks i and i + 1
    const uint4 lo = make_uint4(e4m3_bf16x2<false>(c.x), e4m3_bf16x2<true>(c.x),
                                e4m3_bf16x2<false>(c.y), e4m3_bf16x2<true>(c.y));
    const uint4 hi = make_uint4(e4m3_bf16x2<false>(c.z), e4m3_bf16x2<true>(c.z),
                                e4m3_bf16x2<false>(c.w), e4m3_bf16x2<true>(c.w));
    qop[i] = __builtin_bit_cast(v8s, lo);
    qop[i + 1] = __builtin_bit_cast(v8s, hi);
  }
}

// Writes one wave's 32 output rows (lane (lr, lg) holds row lr, channels
// 32 cb + 8 g4 + 4 lg + j as o[cb][4 g4 + j], already normalised) through the
// wave's 4 KB LDS region `stage`, one 32-channel block at a time, so that
// every store instruction writes whole 128-byte row segments (8 lanes of 16
// bytes per row).  The stores carry the non-temporal hint: O is written once
// and not read back, and kept in the L2 it would push out the K and V tiles
// that the head's other workgroups still read; whole segments keep the hint
// from splitting the rows into partial writes.  Measured on dense MXFP4 16K
// (fetched + written per launch): plain stores of 16-byte pieces 0.53 + 0.35
// GB, the hint on those pieces 0.26 + 0.72 GB, staged whole segments with the
// hint 0.28 + 0.36 GB.
// dst[i]: the output row of row 8 i + lane / 8, or nullptr to skip it.  The
// caller has made every wave of the workgroup done with `stage`.
template <int DB>
__device__ inline void store_o_rows(uint8_t* stage, const v16f (&o)[DB], int lane,
                                    float* const (&dst)[4]) {
  const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) {
    // row r, 16-byte chunk k at r * 128 + 16 (k ^ (r & 7)): the XOR keeps the
    // 32 rows written at once on distinct banks
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const v4f v = {o[cb][4 * g4], o[cb][4 * g4 + 1], o[cb][4 * g4 + 2], o[cb][4 * g4 + 3]};
      *reinterpret_cast<v4f*>(stage + lr * 128 + 16 * ((2 * g4 + lg) ^ (lr & 7))) = v;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the writes have landed
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + lane / 8, k = lane % 8;
      const v4f v = *reinterpret_cast<const v4f*>(stage + r * 128 + 16 * (k ^ (r & 7)));
      if (dst[i]) store4_stream(dst[i] + 32 * cb + 4 * k, v);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the reads are done before the next block
    __builtin_amdgcn_wave_barrier();
  }
}

__device__ inline v8i make_v8(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
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
__device__ inline float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// MODE: 0 dense, 1 causal (top-left aligned), 2 sliding-tile, 3 dense over
// listed key tiles.
// UK: the K scale is constant over each key tile (FP8 blocks a multiple of BN).
//
// Software pipeline over key tiles t = 0, 1, ...: iteration t
//   - copies K(t+3) into a K stage, V(t+1) into a V stage and the mask/scales
//     of tile t+2 into a side stage (3-stage rings; every copy has at least
//     two iterations to land);
//   - computes the online softmax of tile t from S(t), interleaved with the
//     MFMAs of O^T += V(t-1)^T P~(t-1)^T and of S(t+1) = K(t+1) Q^T, so the
//     matrix cores run while the vector ALUs exponentiate;
//   - rescales O by alpha(t-1) first (the product of tile t-2 has landed).
// Iteration t first rescales O by alpha(t-1) and then adds P~(t-1) V(t-1), so
// after it O equals the eager accumulator after tile t-1
// (acc(t-1) = alpha(t-1) acc(t-2) + P~(t-1) V(t-1)); the last tile's rescale
// and product follow the loop.
// V4: FP4 P.V - V in MXFP4 along tokens and P requantised to MXFP4 per 32
// keys (MXFP4 Q/K only).
template <int D, bool MX, int MODE, bool UK, bool V4>
__global__ __launch_bounds__(256, MX ? 3 : 2) void attn_fwd_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using TL = Tile<D, MX, V4>;
  constexpr int DB = D / 32;            // 32-channel blocks of O^T
  constexpr int QI = D / 16;            // bf16 32x32x16 MFMAs over d (FP8 recipe)
  constexpr int NK = Issues<D, MX, V4>::K, NV = Issues<D, MX, V4>::V, NA = Issues<D, MX, V4>::A;
  // Distinct LDS objects per stage: the compiler can then see that a copy
  // into one stage does not alias reads of another and does not wait for it.
  __shared__ __align__(16) uint8_t k0[TL::KBUF], k1[TL::KBUF], k2[TL::KBUF];
  __shared__ __align__(16) uint8_t v0[TL::VBUF], v1[TL::VBUF], v2[TL::VBUF];
  __shared__ __align__(16) uint8_t x0[TL::ABUF], x1[TL::ABUF], x2[TL::ABUF];
  static_assert(TL::KBUF >= 4096 && TL::VBUF >= 4096, "each wave stages its output rows in 4 KB");

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform; saying so keeps LDS-DMA addresses (M0) scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;     // MFMA column (query) and k-group
  const int work = xcd_work_index(blockIdx.x, gridDim.x);

  int bh, q0 = 0, n_steps = 0, u = 0;
  // causal: workgroup p of a head computes query tile n - 1 - p and then query
  // tile p, so that every workgroup visits the same number of key tiles (n + 1
  // steps of pairs of tiles) and the launch has no short tail.  The MXFP4
  // kernel with FP8 V runs at 3 waves per SIMD with no registers to spare for
  // the second pass (its Q operands would be reloaded from scratch inside the
  // key loop, 12% slower on causal 8K): there each workgroup computes one
  // query tile, longest first.  With FP4 P.V the pairs are 6% faster.
  constexpr bool PAIR = MODE == 1 && (!MX || V4);
  int pair = 0, n_pass = 1, qt1 = 0;
  // steps per window-list entry: an entry is a whole key tile (key_unit =
  // tile_tokens) or one BN-key step (key_unit = BN)
  const int spt = MODE == 2 ? a.key_unit / kBN : 1;
  if (PAIR) {
    const int n_pairs = (a.n_qtiles + 1) / 2;
    bh = work / n_pairs;
    pair = work % n_pairs;
    n_pass = pair < a.n_qtiles - 1 - pair ? 2 : 1;
  } else if (MODE == 1) {
    bh = work / a.n_qtiles;
    qt1 = a.n_qtiles - 1 - work % a.n_qtiles;
  } else if (MODE == 2) {
    const int sub = a.tile_tokens / kBM;               // query tiles per window tile
    const int per_bh = a.n_tiles * sub;
    bh = work / per_bh;
    const int r = work % per_bh;
    u = a.tile_order[r / sub];
    q0 = u * a.tile_tokens + (r % sub) * kBM;
    n_steps = (a.win_off[u + 1] - a.win_off[u]) * spt;
  } else {
    bh = work / a.n_qtiles;
    q0 = (work % a.n_qtiles) * kBM;
    n_steps = MODE == 3 ? a.n_key_tiles : (a.N + kBN - 1) / kBN;
  }
  // Padding queries are stored nowhere: a workgroup made only of them (and
  // asked for no row statistic) has nothing to do.  Every wave checks all
  // 128 queries, so the whole workgroup leaves together, before any copy.
  if ((MODE == 2 || MODE == 3) && a.out_perm && !a.lse) {
    const bool mine = (q0 + lane < a.N && a.out_perm[q0 + lane] >= 0) ||
                      (q0 + 64 + lane < a.N && a.out_perm[q0 + 64 + lane] >= 0);
    if (!__any(mine)) return;
  }
  for (int pass = 0; pass < n_pass; ++pass) {
    if (MODE == 1) {
      q0 = (PAIR ? (pass == 0 ? a.n_qtiles - 1 - pair : pair) : qt1) * kBM;
      n_steps = min((q0 + kBM) / kBN, (a.N + kBN - 1) / kBN);
    }
    const int wq0 = q0 + wave * 32;             // first query of this wave
    const int myq = wq0 + lr;                   // this lane's query
    // The window list does not change during the launch: read through the
    // constant address space its entries become scalar loads, whose completion
    // counter is not the one the tile copies count on (a vector load would make
    // every step wait for the copies issued before it).
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const_i32* wlist = MODE == 2 ? (const_i32*)(a.win_idx + a.win_off[u])
                       : MODE == 3 ? (const_i32*)a.key_tiles : nullptr;
    auto step_start = [&](int t) -> int {
      if (MODE == 2) return wlist[t / spt] * a.key_unit + (t % spt) * kBN;
      if (MODE == 3) return wlist[t] * kBN;
      return t * kBN;
    };

    const int64_t tok0 = (int64_t)bh * a.n_alloc;
    const uint8_t* kbh = (MX ? a.k : a.k16) + tok0 * TL::KROW;
    const uint8_t* vbh = a.vt + (int64_t)bh * D * (V4 ? a.n_alloc / 2 : a.n_alloc);

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
          // E2M1 operands occupy the lower four registers; the upper four are
          // never read and stay unset
          v8i r;
          const uint4 x = *reinterpret_cast<const uint4*>(a.q + qrow * (D / 2) + 16 * (2 * i + lg));
          r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
          qop8[i] = r;
          qsc[i] = a.q_mx[qrow * (D / 32) + 2 * i + lg];
        }
        cq = a.sm_log2;
      } else {
        load_q_codes<QI>(a.q + qrow * D + 8 * QI * lg, qop16);
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
    DmaPlan<TL::V_CPR> vp;
    kp.init(lane, TL::KROW);
    vp.init(lane, V4 ? a.n_alloc / 2 : a.n_alloc);
    HeadBuffers hb;
    hb.k = __builtin_amdgcn_make_buffer_rsrc((void*)kbh, 0, a.n_alloc * TL::KROW, kRsrcWord3);
    hb.v = __builtin_amdgcn_make_buffer_rsrc((void*)vbh, 0, (V4 ? a.n_alloc / 2 : a.n_alloc) * D,
                                             kRsrcWord3);
    hb.vs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(V4 ? a.v_mx + (int64_t)bh * (a.n_alloc / 32) * D : kbh), 0,
        V4 ? (a.n_alloc / 32) * D : 0, kRsrcWord3);
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
    // FP4 P.V: the lane's 16-byte chunk (32 keys of group lg) of V^T row lr of
    // a 32-channel block, and its dword of four E8M0 V scales (byte cb is the
    // scale of channel 32 cb + lr and key group lg)
    const int v_off4 = lr * TL::VROW + 16 * (lg ^ swz<2>(lr));
    const int vsc_off = TL::VCODES + 128 * lg + 4 * lr;

    // V^T operand of channel block cb from a V stage (FP4: only the lower four
    // registers are set; the product below reads no more)
    auto v_operand = [&](const uint8_t* Vs, const int cb) __attribute__((always_inline)) {
      if (V4) {
        const uint4 x = *reinterpret_cast<const uint4*>(Vs + cb * 32 * TL::VROW + v_off4);
        v8i r;
        r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
        return r;
      }
      return make_v8(*reinterpret_cast<const uint4*>(Vs + cb * 32 * kBN + v_off0),
                     *reinterpret_cast<const uint4*>(Vs + cb * 32 * kBN + v_off1));
    };
    // O^T[cb] += V^T P~^T: FP8 x FP8 with unit scales, or (FP4 P.V) E2M1 x E2M1
    // with the V scale byte cb of vsc and the P scale ps of the lane's key group
    auto pv_mfma = [&](const int cb, const v8i& vr, const v8i& pk, const uint32_t vsc, const int ps)
        __attribute__((always_inline)) {
      if (!V4) {
        o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vr, pk, o[cb], 0, 0, 0, 127, 0, 127);
        return;
      }
      // E2M1 operands occupy four registers; the zero upper halves are never read
      v8i a4 = {0, 0, 0, 0, 0, 0, 0, 0}, b4 = {0, 0, 0, 0, 0, 0, 0, 0};
      a4[0] = vr[0]; a4[1] = vr[1]; a4[2] = vr[2]; a4[3] = vr[3];
      b4[0] = pk[0]; b4[1] = pk[1]; b4[2] = pk[2]; b4[3] = pk[3];
      if (cb == 0)
        o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, b4, o[cb], 4, 4, 0, vsc, 0, ps);
      else if (cb == 1)
        o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, b4, o[cb], 4, 4, 1, vsc, 0, ps);
      else if (cb == 2)
        o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, b4, o[cb], 4, 4, 2, vsc, 0, ps);
      else
        o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, b4, o[cb], 4, 4, 3, vsc, 0, ps);
    };

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
            v8i kr;   // E2M1: only the lower four registers are read
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

    // O^T += V^T P~^T for the tile in V stage `Vs`
    auto pv = [&](const uint8_t* Vs, const v8i& pk, const int ps) __attribute__((always_inline)) {
      const uint32_t vsc = V4 ? *reinterpret_cast<const uint32_t*>(Vs + vsc_off) : 0u;
#pragma unroll
      for (int cb = 0; cb < DB; ++cb) pv_mfma(cb, v_operand(Vs, cb), pk, vsc, ps);
    };

    // The MFMAs of one pipeline iteration, in issue order: m < DB is the P.V
    // product of channel block m; m >= DB is step m - DB of S = K Q^T (key
    // block kb = (m - DB) / QPB, step i = (m - DB) % QPB).
    constexpr int QPB = MX ? 2 : QI;
    constexpr int NM = DB + 2 * QPB;
    constexpr int LA = MX ? 2 : 1;        // operand read lookahead, in slots
    struct Op { v8i a; int sc; };
    auto slot_lo = [](int g) constexpr { return g >= 8 ? NM : NM * g / 8; };
    auto read_op = [&](const int m, const uint8_t* Vs, const uint8_t* Ks, Op& op)
        __attribute__((always_inline)) {
      if (m < DB) {
        op.a = v_operand(Vs, m);
      } else {
        const int kb = (m - DB) / QPB, i = (m - DB) % QPB;
        const uint4 x = *reinterpret_cast<const uint4*>(Ks + kb * 32 * TL::KROW + k_off[i]);
        op.a[0] = x.x; op.a[1] = x.y; op.a[2] = x.z; op.a[3] = x.w;
        if (MX) op.sc = Ks[TL::K_BYTES + (32 * kb + lr) * (D / 32) + 2 * i + lg];
      }
    };
    auto issue_op = [&](const int m, const Op& op, v16f& acc0, v16f& acc1, const v8i& pk_in,
                        const uint32_t vsc, const int ps_in) __attribute__((always_inline)) {
      if (m < DB) {
        pv_mfma(m, op.a, pk_in, vsc, ps_in);
      } else {
        const int kb = (m - DB) / QPB, i = (m - DB) % QPB;
        v16f c0;
#pragma unroll
        for (int j = 0; j < 16; ++j) c0[j] = 0.0f;
        if (MX) {
          v8i kr;   // E2M1: only the lower four registers are read
          kr[0] = op.a[0]; kr[1] = op.a[1]; kr[2] = op.a[2]; kr[3] = op.a[3];
          v16f& acc = kb == 0 ? acc0 : acc1;
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr, qop8[i], i == 0 ? c0 : acc,
                                                                    4, 4, 0, op.sc, 0, qsc[i]);
        } else {
          v8s kr;
          const v4i x = {op.a[0], op.a[1], op.a[2], op.a[3]};
          kr = __builtin_bit_cast(v8s, x);
          v16f& acc = kb == 0 ? acc0 : acc1;
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr, qop16[i], i == 0 ? c0 : acc, 0, 0, 0);
        }
      }
    };

    // ---- prologue.  V stage v2 stands for tile -1: zero codes, so the first
    // iteration's product with the zero P adds nothing.
    // Copies run up to three tiles past the last one.  Dense and causal tiles
    // past the end read zeros or in-bounds bytes of the same head (buffer
    // loads check their range) into stages that are never read; list-driven
    // steps (sliding-tile windows, listed key tiles) repeat the last listed
    // tile, since the list ends there.
    auto tile_at = [&](int t) { return MODE >= 2 ? step_start(min(t, n_steps - 1)) : t * kBN; };
    issue_k<D, MX>(k0, hb, tile_at(0), wave, lane, kp);
    issue_aux<D, MX>(x0, hb, tile_at(0), lane);
    issue_k<D, MX>(k1, hb, tile_at(1), wave, lane, kp);
    issue_aux<D, MX>(x1, hb, tile_at(1), lane);
    issue_v<D, MX, V4>(v0, hb, a.n_alloc, tile_at(0), wave, lane, vp);
    issue_k<D, MX>(k2, hb, tile_at(2), wave, lane, kp);
#pragma unroll
    for (int i = tid * 16; i < TL::VBUF; i += 256 * 16)
      *reinterpret_cast<uint4*>(v2 + i) = make_uint4(0u, 0u, 0u, 0u);
    wait_vm_le<NV + NK>();          // V(0) and K(2) may still be in flight
    barrier_lds();

    // Score tiles: S(t) = (c0, c1) and S(t+1) = (n0, n1).  MXFP4 forms the
    // next tile's key block 0 in slots 4-5, after this tile's block 0 has been
    // read (slots 0-3), so the two share registers (ga): three tiles rotate
    // instead of four, which saves 16 registers.  FP8 starts block 0 in slot 1.
    v16f ga[2], gb[2], gc;
    qk(k0, ga);
    // P~ of the previous tile (read by the P.V MFMAs) and of the current one
    // alternate between pa and pb like the score buffers
    v8i pa = {0, 0, 0, 0, 0, 0, 0, 0}, pb = {0, 0, 0, 0, 0, 0, 0, 0};
    int psa = 127, psb = 127;       // FP4 P.V: E8M0 scale of pa / pb for this lane's key group
    barrier_lds();                  // every wave is done with k0 before K(3) is copied there
    float alpha_prev = 1.0f;

    // Iteration t: K stages Kr (t+1, read) and Kw (t+3, written); V stages Vr
    // (t-1, read) and Vw (t+1, written); side stages Ar (t, read), Aw (t+2, written).
    auto iter = [&](const int t, const uint8_t* Kr, uint8_t* Kw, const uint8_t* Vr, uint8_t* Vw,
                    const uint8_t* Ar, uint8_t* Aw, v16f& c0s, v16f& c1s, v16f& n0s, v16f& n1s,
                    const v8i& pk_in, v8i& pk, const int ps_in, int& ps_out)
        __attribute__((always_inline)) {
      auto s_cur = [&](int kb) __attribute__((always_inline)) -> v16f& { return kb == 0 ? c0s : c1s; };
      const int ks = step_start(t);
      // this iteration's copies (K(t+3), V(t+1), side data of t+2) are issued
      // one instruction per slot below: issued back to back by every wave they
      // would queue up at the texture unit and stall the issuing waves
      const int ks_k = tile_at(t + 3), ks_v = tile_at(t + 1), ks_a = tile_at(t + 2);
      auto copy_item = [&](const int j) __attribute__((always_inline)) {
        constexpr int KRPI = DmaPlan<TL::K_CPR>::RPI, KPER = DmaPlan<TL::K_CPR>::PER;
        if (j < TL::KI) {
          const int inst = wave * TL::KI + j;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.k, (lds_void_t*)(Kw + inst * 1024), 16,
                                                   kp.off[inst % KPER], (ks_k + inst * KRPI) * TL::KROW, 0, 0);
        } else if (MX && j == TL::KI) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.s, (lds_void_t*)(Kw + TL::K_BYTES), 4, 4 * lane,
                                                   ks_k * (D / 32), 0, 0);
        } else if (j < NK + TL::VI) {
          issue_v_inst<D, MX, V4>(Vw, hb, a.n_alloc, ks_v, wave * TL::VI + (j - NK), vp);
        } else if (V4 && j == NK + TL::VI) {
          issue_vscale<D, MX, V4>(Vw, hb, ks_v, lane);
        } else if (j == NK + NV) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.m, (lds_void_t*)Aw, 4, 4 * lane, ks_a, 0, 0);
        } else if (!MX && j == NK + NV + 1) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.c, (lds_void_t*)(Aw + TL::M_BYTES), 4, 4 * lane,
                                                   (ks_a / hb.blk_k) * 4, 0, 0);
        }
      };
      static_assert(NK + NV + NA <= 8, "one copy instruction per slot");

      // dequantisation factor c (log2 domain): c = sm_scale log2(e) / (s_Q s_K),
      // per group of 4 keys (kb, j / 4); constant over the tile when UK.
      const float* Cs = reinterpret_cast<const float*>(Ar + TL::M_BYTES);
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
      // O = alpha(t-1) O: the product of tile t-2 (issued one iteration ago)
      // has landed, that of tile t-1 is issued below; only when some row max
      // moved
      if (__builtin_amdgcn_ballot_w64(alpha_prev != 1.0f) != 0) {
#pragma unroll
        for (int cb = 0; cb < DB; ++cb) o[cb] *= alpha_prev;
      }
      // masks: padding keys (staged with the tile), keys past N, the causal
      // diagonal; the tests are wave-uniform, the masking branch-free
      const bool edge = (ks + kBN > a.N) || (MODE == 1 && ks + kBN - 1 > wq0);
      if (edge || hb.has_mask) {
        const bool partial = hb.has_mask && Ar[lane] == 0;
        if (edge || __builtin_amdgcn_ballot_w64(partial) != 0) {
          const int lim = MODE == 1 ? min(a.N - 1, myq) : a.N - 1;   // last admissible key
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const uint32_t w = hb.has_mask
                  ? *reinterpret_cast<const uint32_t*>(Ar + 32 * kb + 8 * g4 + 4 * lg) : 0x01010101u;
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const int key = ks + 32 * kb + 8 * g4 + 4 * lg + jj;
                const bool ok = (key <= lim) & (((w >> (8 * jj)) & 0xFFu) != 0u);
                s_cur(kb)[4 * g4 + jj] = ok ? s_cur(kb)[4 * g4 + jj] : kNegInf;
              }
            }
        }
      }

      // operands of the first LA slots (and the FP4 V scales of the tile)
      Op ops[NM];
#pragma unroll
      for (int m = 0; m < slot_lo(LA); ++m) read_op(m, Vr, Kr, ops[m]);
      const uint32_t vsc = V4 ? *reinterpret_cast<const uint32_t*>(Vr + vsc_off) : 0u;

      // running max; with one factor c for the whole tile (c > 0) the max of
      // c s is c times the max of s
      float mx;
      float gmax[2];   // FP4 P.V: maximum score of each 32-key group of the row
      if (V4) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const v16f& x = s_cur(kb);
          const float t0 = max3f(x[0], x[1], x[2]), t1 = max3f(x[3], x[4], x[5]);
          const float t2 = max3f(x[6], x[7], x[8]), t3 = max3f(x[9], x[10], x[11]);
          const float t4 = max3f(x[12], x[13], x[14]);
          gmax[kb] = swap_max(max3f(max3f(t0, t1, t2), t3, fmaxf(t4, x[15])));
        }
        mx = c[0] * fmaxf(gmax[0], gmax[1]);
      } else if (MX || UK) {
        // max3 tree over the lane's 32 scores
        float m11[11];
#pragma unroll
        for (int i = 0; i < 10; ++i) {
          const int e = 3 * i;
          m11[i] = max3f(s_cur(e / 16)[e % 16], s_cur((e + 1) / 16)[(e + 1) % 16],
                         s_cur((e + 2) / 16)[(e + 2) % 16]);
        }
        m11[10] = fmaxf(s_cur(1)[14], s_cur(1)[15]);
        const float m = max3f(max3f(m11[0], m11[1], m11[2]), max3f(m11[3], m11[4], m11[5]),
                              max3f(max3f(m11[6], m11[7], m11[8]), m11[9], m11[10]));
        mx = c[0] * m;
      } else {
        mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float m4 = fmaxf(fmaxf(s_cur(kb)[4 * g4], s_cur(kb)[4 * g4 + 1]),
                                   fmaxf(s_cur(kb)[4 * g4 + 2], s_cur(kb)[4 * g4 + 3]));
            mx = fmaxf(mx, c[4 * kb + g4] * m4);
          }
      }
      if (!V4) mx = swap_max(mx);
      // the reference maximum moves only when the row maximum exceeds it by
      // more than tau (tau = 0: on every rise); P = 2^(S c - m) <= 2^tau is
      // quantised with the scale 448 / 2^tau
      const float cand = fmaxf(m_run, mx);
      const float mnew = cand > m_run + a.tau ? cand : m_run;
      const float alpha = mnew == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mnew);
      const float msh = mnew == kNegInf ? 0.0f : mnew - kLog2_448 + a.tau;
      m_run = mnew;
      // FP4 P.V: the MX rule per key group, e = floor(log2 max P) - 2 read from
      // the exponent of 2^(c gmax - m) (-127 for an empty or subnormal group);
      // the exponentials below then give P / 2^e in [0, 8).  c gmax is rounded
      // as a product of its own, exactly as the row maximum above, so that the
      // group holding the maximum gets 2^0 = 1 (a fused multiply-add would
      // leave the product's rounding error, and 2^-tiny sets e one too low);
      // the empty asm keeps the compiler from fusing the two.
      int eg[2] = {0, 0};
      float mshg[2] = {msh, msh};
      if (V4) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float cg = c[0] * gmax[kb];
          asm volatile("" : "+v"(cg));
          const float pmax = gmax[kb] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(cg - mnew);
          const int eb = (int)(__float_as_uint(pmax) >> 23);   // 0 for 0 and subnormals
          eg[kb] = max(eb - 129, -127);
          mshg[kb] = mnew == kNegInf ? 0.0f : mnew + (float)eg[kb];
        }
      }

      // The previous tile's P.V and the next tile's S are independent MFMAs;
      // they are dealt over 8 slots, one per group of 4 exponentials, and each
      // slot's operands are read from LDS LA slots ahead (a slot is shorter
      // than an LDS read's latency).  The order is pinned
      // with empty volatile asm statements (kept in program order): a slot's
      // MFMAs take their operands from one, and its exponentials end in one.
      float gs[8];
      float pq[4];   // exponentials of the previous group, packed one slot later
      uint32_t pk4[4];   // FP4 P.V: E2M1 codes, 8 per dword, dwords 0-1 key group 0
      // packs group g's four P values (E4M3, or E2M1 for FP4 P.V) and sums them;
      // runs one slot after their exponentials so that the exp latency is hidden
      // by other work
      auto finish = [&](const int g) __attribute__((always_inline)) {
        gs[g] = (pq[0] + pq[1]) + (pq[2] + pq[3]);
        if (V4) {
          uint32_t w;
          if ((g & 1) == 0) {
            asm volatile("" : "=v"(w));   // bytes 0-1 written here, 2-3 by group g + 1
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pq[0], pq[1], 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pq[2], pq[3], 1.0f, 1);
          } else {
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk4[g / 2], pq[0], pq[1], 1.0f, 2);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pq[2], pq[3], 1.0f, 3);
          }
          asm volatile("" : "+v"(w), "+v"(gs[g]));
          pk4[g / 2] = w;
          return;
        }
        int w;
        asm volatile("" : "=v"(w));   // the two conversions below write all four bytes
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pq[0], pq[1], w, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pq[2], pq[3], w, true);
        asm volatile("" : "+v"(w), "+v"(gs[g]));
        pk[g] = w;
      };
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        copy_item(g);
#pragma unroll
        for (int m = slot_lo(g); m < slot_lo(g + 1); ++m) {
          if (MX && !V4 && m >= DB) {
            // an E2M1 K operand lives in its lower four registers
            v4i lo = {ops[m].a[0], ops[m].a[1], ops[m].a[2], ops[m].a[3]};
            asm volatile("" : "+v"(lo));
            ops[m].a[0] = lo[0]; ops[m].a[1] = lo[1]; ops[m].a[2] = lo[2]; ops[m].a[3] = lo[3];
          } else {
            asm volatile("" : "+v"(ops[m].a));
          }
          issue_op(m, ops[m], n0s, n1s, pk_in, vsc, ps_in);
        }
#pragma unroll
        for (int m = slot_lo(g + LA); m < slot_lo(g + LA + 1); ++m) read_op(m, Vr, Kr, ops[m]);
        const int kb = g / 4, g4 = g % 4;
        const float cc = c[g];
        const float sh = V4 ? mshg[kb] : msh;
        float pn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pn[j] = __builtin_amdgcn_exp2f(fmaf(s_cur(kb)[4 * g4 + j], cc, -sh));
        if (g > 0) finish(g - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) pq[j] = pn[j];
      }
      finish(7);
      float sum;
      if (V4) {
        // B operand of the FP4 P.V product: lane half lg takes key group lg, its
        // own 16 codes of that group and the other half's 16 (K slot order
        // 8 b + r, then 8 b + 4 + r of the group, b, r < 4)
        const auto t0 = __builtin_amdgcn_permlane32_swap(pk4[0], pk4[2], false, false);
        const auto t1 = __builtin_amdgcn_permlane32_swap(pk4[1], pk4[3], false, false);
        pk[0] = (int)t0[0]; pk[1] = (int)t1[0]; pk[2] = (int)t0[1]; pk[3] = (int)t1[1];
        ps_out = 127 + (lg == 0 ? eg[0] : eg[1]);
        sum = ldexpf((gs[0] + gs[1]) + (gs[2] + gs[3]), eg[0]) +
              ldexpf((gs[4] + gs[5]) + (gs[6] + gs[7]), eg[1]);
      } else {
        sum = ((gs[0] + gs[1]) + (gs[2] + gs[3])) + ((gs[4] + gs[5]) + (gs[6] + gs[7]));
      }
      l_run = l_run * alpha + sum;
      alpha_prev = alpha;
      // K(t+2), V(t) and the side stage of t+1 must have landed; this
      // iteration's copies may not have
      wait_vm_le<NK + NV + NA>();
      barrier_lds();
    };
    // unrolled by 6: the stage rings have period 3 and the two score buffers
    // alternate, so no buffer is ever copied
    for (int t = 0; t < n_steps; t += 6) {
      // even t: S(t) in (ga0, ga1) -> S(t+1) in (MX ? ga0 : gb0, MX ? gc : gb1);
      // odd t: S(t) in (MX ? ga0 : gb0, MX ? gc : gb1) -> S(t+1) in (ga0, ga1)
      v16f& e0 = ga[0];
      v16f& e1 = ga[1];
      v16f& o0 = MX ? ga[0] : gb[0];
      v16f& o1 = MX ? gc : gb[1];
      iter(t, k1, k0, v2, v1, x0, x2, e0, e1, o0, o1, pa, pb, psa, psb);
      if (t + 1 < n_steps) iter(t + 1, k2, k1, v0, v2, x1, x0, o0, o1, e0, e1, pb, pa, psb, psa);
      if (t + 2 < n_steps) iter(t + 2, k0, k2, v1, v0, x2, x1, e0, e1, o0, o1, pa, pb, psa, psb);
      if (t + 3 < n_steps) iter(t + 3, k1, k0, v2, v1, x0, x2, o0, o1, e0, e1, pb, pa, psb, psa);
      if (t + 4 < n_steps) iter(t + 4, k2, k1, v0, v2, x1, x0, e0, e1, o0, o1, pa, pb, psa, psb);
      if (t + 5 < n_steps) iter(t + 5, k0, k2, v1, v0, x2, x1, o0, o1, e0, e1, pb, pa, psb, psa);
    }
    // the last tile's product: V(n_steps - 1) sits in stage (n_steps - 1) % 3
    {
#pragma unroll
      for (int cb = 0; cb < DB; ++cb) o[cb] *= alpha_prev;
      const int r = (n_steps - 1) % 3;
      pv(r == 0 ? v0 : r == 1 ? v1 : v2, (n_steps & 1) ? pb : pa, (n_steps & 1) ? psb : psa);
      // keep these MFMAs here, with every lane active: sunk into the store
      // branch below they would run on a partial EXEC mask, which drops the
      // operand rows of the inactive lanes
#pragma unroll
      for (int cb = 0; cb < DB; ++cb) asm volatile("" : "+v"(o[cb]));
    }
    wait_vm_le<0>();   // no copy may still target this workgroup's LDS when it ends

    // ---- epilogue: O = acc / (448 l) / s_V (FP4 P.V: acc / l), stored through
    // the output permutation
    const float lt = swap_sum(l_run);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    // row statistic for the backward pass: LSE = m + log2(sum_j 2^(S_j - m));
    // l carries the factor 448 / 2^tau of the FP8 P (FP4 P.V: none)
    if (myq < a.N && a.lse && lg == 0)
      a.lse[(int64_t)bh * a.N + myq] =
          lt > 0.0f ? m_run + __log2f(lt) - (V4 ? 0.0f : kLog2_448 - a.tau) : kNegInf;
    {
      const float* vs = V4 ? nullptr : a.v_scale + (int64_t)bh * D;
#pragma unroll
      for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = 32 * cb + 8 * g4 + 4 * lg + j;
            o[cb][4 * g4 + j] = V4 ? o[cb][4 * g4 + j] * inv : o[cb][4 * g4 + j] * inv / vs[c];
          }
    }
    float* dst[4];
    {
      const int b = bh / a.H, h = bh % a.H;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = wq0 + 8 * i + lane / 8;
        const int tok = q < a.N ? (a.out_perm ? a.out_perm[q] : q) : -1;
        dst[i] = tok >= 0 ? a.out + b * a.osb + h * a.osh + (int64_t)tok * a.osn : nullptr;
      }
    }
    // every wave is done with the stages (its last operand reads) before
    // they hold output rows: wave w stages through a 4 KB piece of one of them
    barrier_lds();
    store_o_rows<DB>(wave == 0 ? v0 : wave == 1 ? v1 : wave == 2 ? v2 : k0, o, lane, dst);
    // every wave is done with the stages before the next pass copies into them
    if (pass + 1 < n_pass) barrier_lds();
  }  // pass
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// Ping-pong variant for dense attention with d = 128 over all key tiles
// (optionally with a key padding mask).  Causal attention and the listed key
// tiles of padded grids go to the 4-wave kernel, which measures faster there
// (it pairs causal tiles and skips query tiles that hold only padding).
//
// A workgroup of 8 waves owns 256 queries of one head (32 per wave).  Waves w
// and w + 4 share a SIMD; they form two groups that alternate between a
// vector phase (the online softmax of tile t: masks, max, exponentials, P~
// packing, row sums, rescale of O) and a matrix phase (O^T += V(t)^T P~(t)^T
// and S(t+1) = K(t+1) Q^T), switching at every workgroup barrier, so that one
// wave's MFMAs run while the other wave's exponentials use the vector ALU.
// Per tile t the order of operations of each wave is the eager one:
// softmax(t) rescales O by alpha(t), then P~(t) V(t) is added.
//
//   step 2t    group 0: vector phase t       group 1: matrix phase t-1
//   step 2t+1  group 0: matrix phase t       group 1: vector phase t
//
// Tiles live in 4-stage LDS rings (K, V^T, side data).  At the start of its
// matrix phase t each wave copies its share of K(t+3), V(t+2) and the side
// data of t+2 (group 1 one step after group 0), and at the end of it waits
// for its copies of the previous iteration.  Every wave issues the same
// number of LDS-DMA instructions per iteration.
template <bool MX>
struct PP {
  static constexpr int D = 128;
  using TL = Tile<D, MX>;
  static constexpr int NST = 4;                         // ring stages
  static constexpr int BMW = 256;                       // queries per workgroup
  // K copy: FP8 16 x 1 KB instructions (2 per wave); MXFP4 4 x 1 KB (waves
  // 0-3) plus the 256 E8M0 scale bytes (waves 4-7)
  static constexpr int KI8 = MX ? 1 : TL::K_BYTES / 1024 / 8;
  static constexpr int VI8 = TL::VBUF / 1024 / 8;        // 1
  static constexpr int NA = MX ? 1 : 2;
  static constexpr int ISSUES = KI8 + VI8 + NA;
  static_assert(VI8 == 1 && (MX || KI8 == 2), "copy split assumes d = 128");
};

#if defined(__HIP_DEVICE_COMPILE__)
// koff: the lane offset of this wave's K copy instructions (wave + 8 j has
// the swizzle phase of the wave for every j).
template <bool MX>
__device__ inline void pp_issue_k(uint8_t* kbuf, const HeadBuffers& hb, int ks, int wave, int lane,
                                  uint32_t koff) {
  using TL = typename PP<MX>::TL;
  constexpr int KRPI = DmaPlan<TL::K_CPR>::RPI;
  if (MX) {
    if (wave < 4) {
      const int inst = wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.k, (lds_void_t*)(kbuf + inst * 1024), 16, koff,
                                               (ks + inst * KRPI) * TL::KROW, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.s, (lds_void_t*)(kbuf + TL::K_BYTES), 4, 4 * lane,
                                               ks * (PP<MX>::D / 32), 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < PP<MX>::KI8; ++j) {
      const int inst = wave + 8 * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.k, (lds_void_t*)(kbuf + inst * 1024), 16, koff,
                                               (ks + inst * KRPI) * TL::KROW, 0, 0);
    }
  }
}

template <bool MX, typename VPlan>
__device__ inline void pp_issue_v(uint8_t* vbuf, const HeadBuffers& hb, int n_alloc, int ks, int wave,
                                  const VPlan& vp) {
  const int inst = wave;   // 8 x 1 KB: 16 channel rows of kBN codes each
  __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.v, (lds_void_t*)(vbuf + inst * 1024), 16, vp.off[0],
                                           ks + inst * 16 * n_alloc, 0, 0);
}
#endif  // __HIP_DEVICE_COMPILE__

template <bool MX, bool UK>
__global__ __launch_bounds__(512, 1) void attn_pp_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = PP<MX>;
  using TL = typename P::TL;
  constexpr int D = P::D;
  constexpr int DB = D / 32;
  constexpr int QI = D / 16;
  __shared__ __align__(16) uint8_t k0[TL::KBUF], k1[TL::KBUF], k2[TL::KBUF], k3[TL::KBUF];
  __shared__ __align__(16) uint8_t v0[TL::VBUF], v1[TL::VBUF], v2[TL::VBUF], v3[TL::VBUF];
  __shared__ __align__(16) uint8_t x0[TL::ABUF], x1[TL::ABUF], x2[TL::ABUF], x3[TL::ABUF];
  uint8_t* const KS[4] = {k0, k1, k2, k3};
  uint8_t* const VS[4] = {v0, v1, v2, v3};
  uint8_t* const XS[4] = {x0, x1, x2, x3};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int lr = lane & 31, lg = lane >> 5;
  const int work = xcd_work_index(blockIdx.x, gridDim.x);
  const int n_qt = (a.n_alloc + P::BMW - 1) / P::BMW;
  const int bh = work / n_qt;
  const int q0 = (work % n_qt) * P::BMW;
  const int n_steps = (a.N + kBN - 1) / kBN;
  // first key of step t (past the last step: copies of keys past N, which
  // read zeros into stages that are never read)
  auto key_at = [&](int t) __attribute__((always_inline)) -> int { return t * kBN; };
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + lr;
  const bool q_live = wq0 < a.n_alloc;      // the wave's 32 queries have token slots

  const int64_t tok0 = (int64_t)bh * a.n_alloc;
  const uint8_t* kbh = (MX ? a.k : a.k16) + tok0 * TL::KROW;
  const uint8_t* vbh = a.vt + (int64_t)bh * D * a.n_alloc;

  v8s qop16[QI];
  v8i qop8[2];
  int qsc[2] = {127, 127};
  float cq = a.sm_log2;
  {
    const int64_t qrow = tok0 + (q_live ? myq : 0);
    if (MX) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
        if (q_live) {
          const uint4 x = *reinterpret_cast<const uint4*>(a.q + qrow * (D / 2) + 16 * (2 * i + lg));
          r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
          qsc[i] = a.q_mx[qrow * (D / 32) + 2 * i + lg];
        }
        qop8[i] = r;
      }
    } else {
      if (q_live) {
        load_q_codes<QI>(a.q + qrow * D + 8 * QI * lg, qop16);
        cq = a.sm_log2 / a.q_scale[(int64_t)bh * a.nblk_q + myq / a.blk_q];
      } else {
#pragma unroll
        for (int i = 0; i < QI; ++i) qop16[i] = __builtin_bit_cast(v8s, make_uint4(0u, 0u, 0u, 0u));
      }
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
  // every K copy instruction of this wave (wave + 8 j) has the swizzle phase
  // wave % PER: its lane offset is chosen once, with uniform selects (an
  // index into kp.off would be a dynamic one, and the array would be placed in
  // LDS and read back on every copy)
  constexpr int KPER = DmaPlan<TL::K_CPR>::PER;
  uint32_t koff = kp.off[0];
#pragma unroll
  for (int p = 1; p < KPER; ++p) koff = wave % KPER == p ? kp.off[p] : koff;
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

  // Copy item j of iteration t (r = t % 4): this wave's shares of K(t+3) and
  // V(t+2) and the side data of tile t+2, into the stages of tiles t+3 and t+2.
  // Tiles past the end read zeros or in-bounds bytes of the same head into
  // stages that are never read.  The items are spread over the matrix phase:
  // issued back to back by every wave they would queue up at the texture
  // unit and stall the issuing waves.
  auto copy_item = [&](const int j, const int t, const int r) __attribute__((always_inline)) {
    constexpr int KRPI = DmaPlan<TL::K_CPR>::RPI;
    uint8_t* kbuf = KS[(r + 3) & 3];
    const int ks_k = key_at(t + 3), ks_a = key_at(t + 2);
    if (j < P::KI8) {
      if (MX) {
        if (wave < 4)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.k, (lds_void_t*)(kbuf + wave * 1024), 16, koff,
                                                   (ks_k + wave * KRPI) * TL::KROW, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.s, (lds_void_t*)(kbuf + TL::K_BYTES), 4, 4 * lane,
                                                   ks_k * (D / 32), 0, 0);
      } else {
        const int inst = wave + 8 * j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.k, (lds_void_t*)(kbuf + inst * 1024), 16, koff,
                                                 (ks_k + inst * KRPI) * TL::KROW, 0, 0);
      }
    } else if (j == P::KI8) {
      pp_issue_v<MX>(VS[(r + 2) & 3], hb, a.n_alloc, key_at(t + 2), wave, vp);
    } else if (j == P::KI8 + 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.m, (lds_void_t*)XS[(r + 2) & 3], 4, 4 * lane, ks_a, 0, 0);
    } else if (!MX && j == P::KI8 + 2) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(hb.c, (lds_void_t*)(XS[(r + 2) & 3] + TL::M_BYTES), 4,
                                               4 * lane, (ks_a / hb.blk_k) * 4, 0, 0);
    }
  };

  // S^T (keys x queries) of the tile in K stage Ks
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
  auto pv = [&](const uint8_t* Vs, const v8i& pk) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {
      const v8i vr = make_v8(*reinterpret_cast<const uint4*>(Vs + cb * 32 * kBN + v_off0),
                             *reinterpret_cast<const uint4*>(Vs + cb * 32 * kBN + v_off1));
      o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vr, pk, o[cb], 0, 0, 0, 127, 0, 127);
    }
  };
  // matrix phase t: O^T += V(t)^T P~(t)^T (V stage Vs), then S(t+1) (K stage Kn).
  // The MFMAs are issued in order with their LDS operands read MLA MFMAs
  // ahead (pinned with empty volatile asm), which bounds the registers held
  // by operands in flight.  After the last tile S(t+1) is computed from a
  // stage holding a copy past the end and never used, which keeps the phase
  // free of branches.
  constexpr int QPB = MX ? 2 : QI;
  constexpr int NMM = DB + 2 * QPB;
  constexpr int MLA = 4;
  struct MOp { v8i a; int sc; };
  auto mphase = [&](const int t, const int r, const uint8_t* Vs, const uint8_t* Kn, const v8i& pk,
                    v16f (&s_out)[2]) __attribute__((always_inline)) {
    auto read = [&](const int m, MOp& op) __attribute__((always_inline)) {
      if (m < DB) {
        op.a = make_v8(*reinterpret_cast<const uint4*>(Vs + m * 32 * kBN + v_off0),
                       *reinterpret_cast<const uint4*>(Vs + m * 32 * kBN + v_off1));
      } else {
        const int kb = (m - DB) / QPB, i = (m - DB) % QPB;
        const uint4 x = *reinterpret_cast<const uint4*>(Kn + kb * 32 * TL::KROW + k_off[i]);
        op.a[0] = x.x; op.a[1] = x.y; op.a[2] = x.z; op.a[3] = x.w;
        if (MX) op.sc = Kn[TL::K_BYTES + (32 * kb + lr) * (D / 32) + 2 * i + lg];
      }
    };
    MOp ops[NMM];
    v16f acc[2];
#pragma unroll
    for (int m = 0; m < MLA; ++m) read(m, ops[m]);
    constexpr int CSTEP = NMM / P::ISSUES;   // MFMAs between two copy items
#pragma unroll
    for (int m = 0; m < NMM; ++m) {
      if (m % CSTEP == 0 && m / CSTEP < P::ISSUES) copy_item(m / CSTEP, t, r);
      asm volatile("" : "+v"(ops[m].a));
      if (m < DB) {
        o[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ops[m].a, pk, o[m], 0, 0, 0, 127, 0, 127);
      } else {
        const int kb = (m - DB) / QPB, i = (m - DB) % QPB;
        v16f c0;
#pragma unroll
        for (int j = 0; j < 16; ++j) c0[j] = 0.0f;
        if (MX) {
          v8i kr = {0, 0, 0, 0, 0, 0, 0, 0};
          kr[0] = ops[m].a[0]; kr[1] = ops[m].a[1]; kr[2] = ops[m].a[2]; kr[3] = ops[m].a[3];
          acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr, qop8[i], i == 0 ? c0 : acc[kb],
                                                                    4, 4, 0, ops[m].sc, 0, qsc[i]);
        } else {
          const v4i x = {ops[m].a[0], ops[m].a[1], ops[m].a[2], ops[m].a[3]};
          acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8s, x), qop16[i],
                                                            i == 0 ? c0 : acc[kb], 0, 0, 0);
        }
      }
      if (m + MLA < NMM) read(m + MLA, ops[m + MLA]);
    }
    s_out[0] = acc[0];
    s_out[1] = acc[1];
    // the phase ends here: its MFMAs may not drift past the barrier into the
    // vector phase (they would then compete with the other wave's MFMAs)
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) asm volatile("" : "+v"(o[cb]));
    asm volatile("" : "+v"(s_out[0]), "+v"(s_out[1]));
  };
  // vector phase t: masks, running max, P~(t), row sums, rescale of O
  auto vphase = [&](const int t, const uint8_t* Ar, v16f (&s)[2], v8i& pk) __attribute__((always_inline)) {
    const int ks = key_at(t);
    const float* Cs = reinterpret_cast<const float*>(Ar + TL::M_BYTES);
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
      for (int g = 0; g < 8; ++g) {
        const int key = ks + 32 * (g / 4) + 8 * (g % 4);
        c[g] = cq * __builtin_amdgcn_rcpf(Cs[key / a.blk_k - ks / a.blk_k]);
      }
    }
    const bool edge = ks + kBN > a.N;
    if (edge || hb.has_mask) {
      const bool partial = hb.has_mask && Ar[lane] == 0;
      if (edge || __builtin_amdgcn_ballot_w64(partial) != 0) {
        const int lim = a.N - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const uint32_t w = hb.has_mask
                ? *reinterpret_cast<const uint32_t*>(Ar + 32 * kb + 8 * g4 + 4 * lg) : 0x01010101u;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int key = ks + 32 * kb + 8 * g4 + 4 * lg + jj;
              const bool ok = (key <= lim) & (((w >> (8 * jj)) & 0xFFu) != 0u);
              s[kb][4 * g4 + jj] = ok ? s[kb][4 * g4 + jj] : kNegInf;
            }
          }
      }
    }
    float mx;
    if (MX || UK) {
      float m11[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int e = 3 * i;
        m11[i] = max3f(s[e / 16][e % 16], s[(e + 1) / 16][(e + 1) % 16], s[(e + 2) / 16][(e + 2) % 16]);
      }
      m11[10] = fmaxf(s[1][14], s[1][15]);
      const float m = max3f(max3f(m11[0], m11[1], m11[2]), max3f(m11[3], m11[4], m11[5]),
                            max3f(max3f(m11[6], m11[7], m11[8]), m11[9], m11[10]));
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
    // the reference maximum moves only when the row maximum exceeds it by
    // more than tau (tau = 0: on every rise); P = 2^(S c - m) <= 2^tau is
    // quantised with the scale 448 / 2^tau
    const float cand = fmaxf(m_run, mx);
    const float mnew = cand > m_run + a.tau ? cand : m_run;
    const float alpha = mnew == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mnew);
    const float msh = mnew == kNegInf ? 0.0f : mnew - kLog2_448 + a.tau;
    m_run = mnew;
    float gs[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int kb = g / 4, g4 = g % 4;
      const float cc = c[g];
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * g4 + j], cc, -msh));
      gs[g] = (p[0] + p[1]) + (p[2] + p[3]);
      int w;
      asm volatile("" : "=v"(w));   // the two conversions below write all four bytes
      w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], w, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
      pk[g] = w;
    }
    const float sum = ((gs[0] + gs[1]) + (gs[2] + gs[3])) + ((gs[4] + gs[5]) + (gs[6] + gs[7]));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int cb = 0; cb < DB; ++cb) o[cb] *= alpha;
    }
    l_run = l_run * alpha + sum;
    // likewise the vector work stays in its phase
    asm volatile("" : "+v"(pk), "+v"(l_run));
  };

  // ---- prologue: K(0..2), V(0..1), side data of tiles 0 and 1; S(0)
#pragma unroll
  for (int t = 0; t < 3; ++t) pp_issue_k<MX>(KS[t], hb, key_at(t), wave, lane, koff);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    pp_issue_v<MX>(VS[t], hb, a.n_alloc, key_at(t), wave, vp);
    issue_aux<D, MX>(XS[t], hb, key_at(t), lane);
  }
  wait_vm_le<0>();
  barrier_lds();
  v16f sa[2], sb[2];
  v8i pa, pb;
  qk(KS[0], sa);

  // iteration t (r = t % 4, a constant in every unrolled copy); S(t) and
  // P~(t) live in the buffers of parity t.  Both groups run the same
  // sequence; group 1 starts one barrier late, which makes its vector phases
  // coincide with group 0's matrix phases.  Copies issued in one iteration
  // have landed for every wave by the end of the next one (each wave waits
  // for its own, then the barrier), which is before their first use.
  auto iteration = [&](const int t, const int r, v16f (&s_t)[2], v16f (&s_t1)[2], v8i& p_t)
      __attribute__((always_inline)) {
    vphase(t, XS[r], s_t, p_t);
    barrier_lds();
    mphase(t, r, VS[r], KS[(r + 1) & 3], p_t, s_t1);
    wait_vm_le<P::ISSUES>();
    barrier_lds();
  };
  if (grp == 1) barrier_lds();
  for (int t = 0; t < n_steps; t += 4) {
    iteration(t, 0, sa, sb, pa);
    if (t + 1 < n_steps) iteration(t + 1, 1, sb, sa, pb);
    if (t + 2 < n_steps) iteration(t + 2, 2, sa, sb, pa);
    if (t + 3 < n_steps) iteration(t + 3, 3, sb, sa, pb);
  }
  // keep the last P.V MFMAs here, with every lane active (see the store below)
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) asm volatile("" : "+v"(o[cb]));
  wait_vm_le<0>();

  const float lt = swap_sum(l_run);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (myq < a.N && a.lse && lg == 0)   // as in the 4-wave kernel
    a.lse[(int64_t)bh * a.N + myq] = lt > 0.0f ? m_run + __log2f(lt) - (kLog2_448 - a.tau) : kNegInf;
  {
    const float* vs = a.v_scale + (int64_t)bh * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[cb][4 * g4 + j] = o[cb][4 * g4 + j] * inv / vs[32 * cb + 8 * g4 + 4 * lg + j];
  }
  float* dst[4];
  {
    const int b = bh / a.H, h = bh % a.H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wq0 + 8 * i + lane / 8;
      const int tok = q < a.N ? (a.out_perm ? a.out_perm[q] : q) : -1;
      dst[i] = tok >= 0 ? a.out + b * a.osb + h * a.osh + (int64_t)tok * a.osn : nullptr;
    }
  }
  // group 0 meets group 1's last barrier: after it no wave reads a stage
  // (group 1's last matrix phase is behind it), and wave w stages its output
  // rows through a 4 KB piece of one of them
  if (grp == 0) barrier_lds();
  uint8_t* const stage = wave == 0 ? v0 : wave == 1 ? v1 : wave == 2 ? v2 : wave == 3 ? v3
                        : wave == 4 ? k0 : wave == 5 ? k1 : wave == 6 ? k2 : k3;
  store_o_rows<DB>(stage, o, lane, dst);
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool MX, int MODE, bool V4>
static hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const bool uk = MX || a.blk_k % kBN == 0;
  const int64_t blocks = MODE == 2   ? (int64_t)a.B * a.H * a.n_tiles * (a.tile_tokens / kBM)
                         : MODE == 1 ? (int64_t)a.B * a.H * (MX && !V4 ? a.n_qtiles : (a.n_qtiles + 1) / 2)
                                     : (int64_t)a.B * a.H * a.n_qtiles;
  if (uk)
    hipLaunchKernelGGL((attn_fwd_kernel<D, MX, MODE, true, V4>), dim3((unsigned)blocks), dim3(256), 0, st,
                       a);
  else if constexpr (!MX)
    hipLaunchKernelGGL((attn_fwd_kernel<D, MX, MODE, false, false>), dim3((unsigned)blocks), dim3(256), 0,
                       st, a);
  return hipGetLastError();
}

template <int D, bool MX, bool V4 = false>
static hipError_t launch_mode(const AttnArgs& a, int mode, hipStream_t st) {
  if (mode == 1) return launch_t<D, MX, 1, V4>(a, st);
  if (mode == 2) return launch_t<D, MX, 2, V4>(a, st);
  if (mode == 3) return launch_t<D, MX, 3, V4>(a, st);
  return launch_t<D, MX, 0, V4>(a, st);
}

template <bool MX>
static hipError_t launch_pp(const AttnArgs& a, hipStream_t st) {
  const bool uk = MX || a.blk_k % kBN == 0;
  const int64_t blocks = (int64_t)a.B * a.H * ((a.n_alloc + PP<MX>::BMW - 1) / PP<MX>::BMW);
  if (uk)
    hipLaunchKernelGGL((attn_pp_kernel<MX, true>), dim3((unsigned)blocks), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((attn_pp_kernel<MX, false>), dim3((unsigned)blocks), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int d, bool mx, bool v4, int mode, hipStream_t st) {
  // dense FP8 with d = 128: the ping-pong kernel (its matrix phase, with QK^T
  // on the bf16 MFMA, is long enough to balance the vector phase; for MXFP4,
  // causal masks and listed key tiles the 4-wave kernel measures faster)
  if (v4) return mx && d == 128 ? launch_mode<128, true, true>(a, mode, st) : hipErrorInvalidValue;
  if (!mx && d == 128 && mode == 0) return launch_pp<false>(a, st);
  if (mx) return launch_mode<128, true>(a, mode, st);
  if (d == 64) return launch_mode<64, false>(a, mode, st);
  return launch_mode<128, false>(a, mode, st);
}

}  // namespace pab
