// Internal arguments and launchers of the attention backward pass (host and
// device).  The C ABI layer validates everything before filling these.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pab {

// Device arrays of the backward pass.  Token arrays have n_alloc slots per
// (batch, head); "rows" are [BH][n_alloc][d] bf16, "transposed" arrays are
// block-tiled [BH][n_alloc/32][d][32] bf16 with, inside every 16-token group,
// token t at slot t with bits 2 and 3 swapped (the K order in which a 32x32
// MFMA result lane holds its 16 values, see attention_bwd.hip).
struct BwdArgs {
  int B, H, N, n_alloc, d;
  float sm;                    // sm_scale
  float sm_log2;               // sm_scale * log2(e)
  bool causal;
  // forward inputs (quantised operands)
  bool qk_mx;                  // Q/K MXFP4 (else FP8 per block)
  const uint8_t* q_codes;      // MXFP4: [BH][n_alloc][d/2]
  const uint8_t* k_codes;
  const uint8_t* q_mx;         // MXFP4: E8M0 [BH][n_alloc][d/32]
  const uint8_t* k_mx;
  const uint16_t* q_val;       // FP8: bf16 values of the E4M3 codes [BH][n_alloc][d]
  const uint16_t* k_val;
  const float* q_scale;        // FP8: [BH][nblk_q]
  const float* k_scale;
  int blk_q, blk_k, nblk_q, nblk_k;
  bool v_mx;                   // V in MXFP4 along tokens (else FP8 per channel)
  const uint8_t* v_codes;      // FP8: V^T [BH][d][n_alloc] (64-token interleave);
                               // MXFP4: [BH][d][n_alloc/2] (32-token slot order)
  const float* v_scale;        // FP8: [BH][d]
  const uint8_t* v_e8;         // MXFP4: [BH][n_alloc/32][d] (channels interleaved)
  const uint8_t* kv_valid;     // nullable [N]
  // sliding-tile attention (nullable): CSR window lists of the tiles of
  // tile_tokens tokens (kernel token order).  The window relation is
  // symmetric, so W(v) lists both the key tiles of query tile v and the
  // query tiles that see key tile v.
  const int32_t* win_off;
  const int32_t* win_idx;
  int tile_tokens;
  // forward outputs and the upstream gradient
  const float* o;              // [B,H,N,d], strides o_s*
  int64_t o_sb, o_sh, o_sn;
  const void* dout;            // [B,H,N,d] float32 or bf16, strides do_s*
  bool dout_bf16;
  int64_t do_sb, do_sh, do_sn;
  const float* lse;            // [BH][N], log2 units
  // gradients (float32 [B,H,N,d], strides g_s*)
  float* dq;
  float* dk;
  float* dv;
  int64_t g_sb, g_sh, g_sn;
  // workspace arrays
  uint16_t* q_rows;            // MXFP4 Q/K: dequantised rows (FP8 uses q_val / k_val)
  uint16_t* k_rows;
  uint16_t* v_rows;            // V values: FP8 code values (scale folded into dos), MXFP4 dequantised
  uint16_t* dos_rows;          // bf16(dO / s_V) (FP8 V), bf16(dO) (MXFP4 V)
  uint16_t* qt;                // transposed Q values
  uint16_t* kt;                // transposed K values
  uint16_t* dot;               // transposed bf16(dO)
  float* lse_e;                // [BH][n_alloc]: LSE, +inf where the row has no valid key or is padding
  float* dd;                   // [BH][n_alloc]: D_i = sum_c dO_ic O_ic (0 for padding)
  float* fq;                   // [BH][n_alloc]: 1 / s_Q of the token's block (MXFP4: 1)
  float* fk;                   // [BH][n_alloc]: 1 / s_K (MXFP4: 1)
  float* kvf;                  // [n_alloc]: 1 for a valid key, 0 for masked keys and padding
};

constexpr int kBwdTile = 128;   // keys (dK/dV kernel) or queries (dQ kernel) per workgroup

// Byte offsets of the workspace arrays (256-byte aligned); returns the total.
int64_t bwd_workspace_layout(int64_t BH, int64_t n_alloc, int64_t d, int64_t off[13]);

hipError_t launch_attention_backward(const BwdArgs& a, hipStream_t st);

}  // namespace pab
