// Internal argument blocks and launchers of libpab (host and device).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace pab {

// Arguments of the quantizer kernels (validated by the C ABI layer).
struct QuantArgs {
  const void* x;          // input base pointer
  int64_t sb, sh, sn;     // element strides of batch, head, token (channel stride 1)
  int B, H, N_in, d;
  int recipe;             // 0 FP8 per block, 1 FP8 per channel, 2 MXFP4, 3 MXFP4 V (tokens)
  bool in_bf16;
  int blk, nblk;          // FP8 per block: tokens per block, blocks per (b, h)
  const int32_t* perm;    // nullable token gather
  int n_out, n_alloc;     // kernel tokens, allocated token slots
  uint8_t* codes;
  uint16_t* values;       // FP8 per block: bf16 copy of each code's exact value (nullable)
  float* scales_f32;      // FP8 recipes
  uint8_t* scales_u8;     // MXFP4 recipes
};

// Arguments of the attention kernel.
struct AttnArgs {
  const uint8_t* q;       // MXFP4 codes [BH][n_alloc][d/2]; FP8 E4M3 codes [BH][n_alloc][d]
  const uint8_t* k;
  const uint8_t* k16;     // FP8 recipe: bf16 values of K's E4M3 codes [BH][n_alloc][d]
  const uint8_t* vt;      // FP8 V^T [BH][d][n_alloc], operand-ordered per 64 tokens;
                          // FP4 P.V: MXFP4 V^T [BH][d][n_alloc/2]
  const uint8_t* v_mx;    // FP4 P.V: E8M0 V scales [BH][n_alloc/32][d] (channels interleaved)
  const float* q_scale;   // FP8: [BH][nblk_q]
  const float* k_scale;   // FP8: [BH][nblk_k]
  const uint8_t* q_mx;    // MXFP4: [BH][n_alloc][d/32]
  const uint8_t* k_mx;
  const float* v_scale;   // [BH][d]
  const uint8_t* kv_valid;    // nullable, [N]
  const int32_t* out_perm;    // nullable, [N]
  float* out;
  int64_t osb, osh, osn;      // output element strides (channel stride 1)
  float* lse;                 // nullable, [BH][N]: log2-sum-exp row statistic (kernel order)
  int B, H, N, n_alloc;
  int blk_q, blk_k, nblk_q, nblk_k;
  float sm_log2;          // sm_scale * log2(e)
  float tau;              // softmax rescale threshold (log2 units, an integer)
  int n_qtiles;           // query tiles of kBM per (b, h) (dense / causal)
  // sliding-tile schedule
  const int32_t* win_off;
  const int32_t* win_idx;
  const int32_t* tile_order;
  int n_tiles, tile_tokens;
  int key_unit;               // keys per window-list entry: tile_tokens, or BN (step lists)
  // dense over listed key tiles (mode 3): ascending BN-key tile indices
  const int32_t* key_tiles;
  int n_key_tiles;
};

constexpr int kBM = 128;      // queries per workgroup (4 waves x 32)
constexpr int kBN = 64;       // keys per online-softmax step

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);
hipError_t launch_count_nonfinite(const float* x, int64_t n, int32_t* count, hipStream_t st);
// mode: 0 dense, 1 causal, 2 sliding-tile, 3 dense over listed key tiles
// v4: V in MXFP4 along tokens (FP4 P.V; MXFP4 Q/K, d = 128)
hipError_t launch_attention(const AttnArgs& a, int d, bool mx, bool v4, int mode, hipStream_t st);

}  // namespace pab
