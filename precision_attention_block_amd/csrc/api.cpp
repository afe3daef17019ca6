// libpab C ABI: argument validation, launch configuration and the host-side
// sliding-tile planner.  Every check runs before the first HIP call, so a call
// rejected here has touched neither the device nor the stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>
#include <algorithm>
#include <mutex>
#include <numeric>

#include "../../include/pab.h"
#include "pab_bwd.h"
#include "pab_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

pab_status hip_status(hipError_t e, hipStream_t st) {
  if (e == hipSuccess) {
    const char* dbg = std::getenv("PAB_SYNC_DEBUG");
    if (dbg && dbg[0] == '1') {
      e = hipStreamSynchronize(st);
      if (e == hipSuccess) e = hipGetLastError();
    }
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return PAB_HIP_ERROR;
  }
  return PAB_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t round_up(int64_t n, int64_t a) { return (n + a - 1) / a * a; }

// Size limits.  They keep every launch inside the device's grid limits (fewer
// than 2^32 work-items along a grid dimension, at most 65536 workgroups along
// y) and every per-head buffer descriptor of the attention kernels below 2^31
// bytes (the descriptors take 32-bit byte counts and offsets).
constexpr int64_t kMaxAttnTokens = (int64_t)1 << 22;   // N per head: bf16 K operand, n_alloc * 256 B
constexpr int64_t kMaxAttnRows = (int64_t)1 << 31;     // B*H*n_alloc (exclusive): 2 work-items per token slot
constexpr int64_t kMaxGridY = 65536;                   // B*H of the quantiser and backward grids (y)
constexpr int64_t kMaxQuantTokens = (int64_t)1 << 27;  // n_out: up to 16 work-items per token slot
constexpr int64_t kMaxBwdTokens = (int64_t)1 << 20;    // N of the backward

// Validates a quantised operand view; `role` 0 = Q/K, 1 = V.  An FP8 Q/K
// view must carry its bf16 operand copy when `need_operand` is set (the
// forward reads K's copy and converts Q's codes itself; the backward reads
// both copies).
pab_status check_view(const pab_qview* v, int role, bool need_operand = true) {
  if (!v || !v->codes || !v->scales) return PAB_INVALID_ARG;
  if (v->B < 1 || v->H < 1 || v->N < 1 || v->d < 1) return PAB_INVALID_ARG;
  if (v->B > (int64_t)1 << 24 || v->H > (int64_t)1 << 24 || v->B * v->H > (int64_t)1 << 24 ||
      v->N > kMaxAttnTokens)
    return PAB_UNSUPPORTED;
  if (v->B * v->H * round_up(v->N, PAB_TOKEN_ALIGN) >= kMaxAttnRows) return PAB_UNSUPPORTED;
  if (!aligned(v->codes, 16)) return PAB_INVALID_ARG;
  if (role == 1) {
    if (v->recipe == PAB_MXFP4_V) return v->d == 128 ? PAB_OK : PAB_UNSUPPORTED;
    if (v->recipe != PAB_FP8_CHANNEL) return PAB_INVALID_ARG;
    if (v->d != 64 && v->d != 128) return PAB_UNSUPPORTED;
    return PAB_OK;
  }
  if (v->recipe == PAB_FP8_TOKEN_BLOCK) {
    if (v->d != 64 && v->d != 128) return PAB_UNSUPPORTED;
    if (v->block_tokens < 16 || v->block_tokens > 16384 || v->block_tokens % 16) return PAB_INVALID_ARG;
    if (need_operand && !v->operand) return PAB_INVALID_ARG;
    if (v->operand && !aligned(v->operand, 16)) return PAB_INVALID_ARG;
    return PAB_OK;
  }
  if (v->recipe == PAB_MXFP4_D32) return v->d == 128 ? PAB_OK : PAB_UNSUPPORTED;
  return PAB_INVALID_ARG;
}

// True for a call with nothing to compute: the three views agree on
// (B, H, N, d), no size is negative and B, H or N is 0.  Such a call reads and
// writes nothing, so its pointers are not examined.
bool empty_views(const pab_qview* q, const pab_qview* k, const pab_qview* v) {
  if (!q || !k || !v) return false;
  for (const pab_qview* x : {q, k, v})
    if (x->B < 0 || x->H < 0 || x->N < 0 || x->d < 1) return false;
  if (q->B != k->B || q->B != v->B || q->H != k->H || q->H != v->H || q->N != k->N ||
      q->N != v->N || q->d != k->d || q->d != v->d)
    return false;
  return q->B == 0 || q->H == 0 || q->N == 0;
}

pab_status fill_attn_args(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                          float sm_scale, int tau, const uint8_t* kv_valid, const int32_t* out_perm,
                          int64_t n_out_tokens, float* out, const int64_t out_strides[4],
                          pab::AttnArgs& a) {
  pab_status s;
  if ((s = check_view(q, 0, false)) != PAB_OK) return s;
  if ((s = check_view(k, 0)) != PAB_OK) return s;
  if ((s = check_view(v, 1)) != PAB_OK) return s;
  if (q->recipe != k->recipe) return PAB_INVALID_ARG;
  if (v->recipe == PAB_MXFP4_V && q->recipe != PAB_MXFP4_D32) return PAB_UNSUPPORTED;
  if (q->B != k->B || q->B != v->B || q->H != k->H || q->H != v->H || q->N != k->N ||
      q->N != v->N || q->d != k->d || q->d != v->d)
    return PAB_INVALID_ARG;
  if (!out || !out_strides) return PAB_INVALID_ARG;
  if (out_strides[3] != 1 || out_strides[0] < 0 || out_strides[1] < 0 || out_strides[2] < 0)
    return PAB_INVALID_ARG;
  if (out_strides[0] % 4 || out_strides[1] % 4 || out_strides[2] % 4 || !aligned(out, 16))
    return PAB_INVALID_ARG;
  if (n_out_tokens < 1) return PAB_INVALID_ARG;
  if (!out_perm && n_out_tokens < q->N) return PAB_INVALID_ARG;
  if (kv_valid && !aligned(kv_valid, 4)) return PAB_INVALID_ARG;
  if (tau < 0 || tau > PAB_MAX_TAU) return PAB_INVALID_ARG;
  if (!(std::isfinite(sm_scale))) return PAB_INVALID_ARG;
  const bool mx = q->recipe == PAB_MXFP4_D32;
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt((float)q->d);
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint8_t*>(q->codes);
  a.k = static_cast<const uint8_t*>(k->codes);
  a.k16 = static_cast<const uint8_t*>(k->operand);
  a.vt = static_cast<const uint8_t*>(v->codes);
  if (mx) {
    a.q_mx = static_cast<const uint8_t*>(q->scales);
    a.k_mx = static_cast<const uint8_t*>(k->scales);
  } else {
    a.q_scale = static_cast<const float*>(q->scales);
    a.k_scale = static_cast<const float*>(k->scales);
    a.blk_q = q->block_tokens;
    a.blk_k = k->block_tokens;
  }
  if (v->recipe == PAB_MXFP4_V)
    a.v_mx = static_cast<const uint8_t*>(v->scales);
  else
    a.v_scale = static_cast<const float*>(v->scales);
  a.kv_valid = kv_valid;
  a.out_perm = out_perm;
  a.out = out;
  a.osb = out_strides[0];
  a.osh = out_strides[1];
  a.osn = out_strides[2];
  a.B = (int)q->B;
  a.H = (int)q->H;
  a.N = (int)q->N;
  a.n_alloc = (int)round_up(q->N, PAB_TOKEN_ALIGN);
  if (!mx) {
    a.nblk_q = (int)((a.n_alloc + a.blk_q - 1) / a.blk_q);
    a.nblk_k = (int)((a.n_alloc + a.blk_k - 1) / a.blk_k);
  }
  a.sm_log2 = scale * 1.4426950408889634f;
  a.tau = (float)tau;
  a.n_qtiles = a.n_alloc / pab::kBM;
  return PAB_OK;
}

}  // namespace

extern "C" {

int pab_abi_version(void) { return PAB_ABI_VERSION; }

const char* pab_status_str(pab_status s) {
  switch (s) {
    case PAB_OK: return "ok";
    case PAB_INVALID_ARG: return "invalid argument";
    case PAB_UNSUPPORTED: return "unsupported configuration";
    case PAB_HIP_ERROR: return "HIP runtime error";
  }
  return "unknown status";
}

int pab_last_hip_error(void) { return g_last_hip_error; }

int64_t pab_token_alloc(int64_t n) {
  if (n <= 0) return 0;
  if (n > INT64_MAX - (PAB_TOKEN_ALIGN - 1)) return -1;   // not representable
  return round_up(n, PAB_TOKEN_ALIGN);
}

pab_status pab_attention_info(pab_recipe qk_recipe, int d, int mode, int* BM, int* BN) {
  if (!BM || !BN) return PAB_INVALID_ARG;
  if (mode < 0 || mode > 3) return PAB_INVALID_ARG;
  if (qk_recipe == PAB_FP8_TOKEN_BLOCK) {
    if (d != 64 && d != 128) return PAB_UNSUPPORTED;
  } else if (qk_recipe == PAB_MXFP4_D32) {
    if (d != 128) return PAB_UNSUPPORTED;
  } else {
    return PAB_INVALID_ARG;
  }
  // dense FP8 attention with d = 128 over all key tiles runs the 8-wave
  // kernel (256 queries)
  *BM = (qk_recipe == PAB_FP8_TOKEN_BLOCK && d == 128 && mode == 0) ? 2 * pab::kBM : pab::kBM;
  *BN = pab::kBN;
  return PAB_OK;
}

pab_status pab_quantize(const void* x, pab_dtype in_dt, const int64_t shape[4],
                        const int64_t strides[4], pab_recipe recipe, int block_tokens,
                        const int32_t* perm, int64_t n_out, void* codes, void* scales,
                        void* operand, void* stream) {
  if (!shape || !strides) return PAB_INVALID_ARG;
  {
    const int64_t B = shape[0], H = shape[1], N = shape[2], d = shape[3];
    if (B < 0 || H < 0 || N < 0 || d < 1 || n_out < 0) return PAB_INVALID_ARG;
    if (!perm && n_out != N) return PAB_INVALID_ARG;
    if (B == 0 || H == 0 || n_out == 0) return PAB_OK;   // empty output: nothing to do
  }
  if (!x || !codes || !scales) return PAB_INVALID_ARG;
  if (operand && (recipe != PAB_FP8_TOKEN_BLOCK || !aligned(operand, 16))) return PAB_INVALID_ARG;
  if (in_dt != PAB_F32 && in_dt != PAB_BF16) return PAB_INVALID_ARG;
  const int64_t B = shape[0], H = shape[1], N = shape[2], d = shape[3];
  if (B < 1 || H < 1 || N < 1 || d < 1) return PAB_INVALID_ARG;
  if (strides[3] != 1) return PAB_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (strides[i] < 0 || strides[i] % 8) return PAB_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return PAB_INVALID_ARG;
  if (n_out < 1) return PAB_INVALID_ARG;
  if (!perm && n_out != N) return PAB_INVALID_ARG;
  if (B * H > kMaxGridY || n_out > kMaxQuantTokens || N > INT32_MAX) return PAB_UNSUPPORTED;
  if (recipe == PAB_FP8_TOKEN_BLOCK) {
    if (d != 64 && d != 128) return PAB_UNSUPPORTED;
    if (block_tokens < 16 || block_tokens > 16384 || block_tokens % 16) return PAB_INVALID_ARG;
  } else if (recipe == PAB_FP8_CHANNEL) {
    if (d != 64 && d != 128) return PAB_UNSUPPORTED;
  } else if (recipe == PAB_MXFP4_D32 || recipe == PAB_MXFP4_V) {
    if (d != 128) return PAB_UNSUPPORTED;
  } else {
    return PAB_INVALID_ARG;
  }
  pab::QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x = x;
  a.sb = strides[0];
  a.sh = strides[1];
  a.sn = strides[2];
  a.B = (int)B;
  a.H = (int)H;
  a.N_in = (int)N;
  a.d = (int)d;
  a.recipe = (int)recipe;
  a.in_bf16 = in_dt == PAB_BF16;
  a.perm = perm;
  a.n_out = (int)n_out;
  a.n_alloc = (int)round_up(n_out, PAB_TOKEN_ALIGN);
  a.codes = static_cast<uint8_t*>(codes);
  a.values = static_cast<uint16_t*>(operand);
  if (recipe == PAB_MXFP4_D32 || recipe == PAB_MXFP4_V) {
    a.scales_u8 = static_cast<uint8_t*>(scales);
  } else {
    a.scales_f32 = static_cast<float*>(scales);
  }
  if (recipe == PAB_FP8_TOKEN_BLOCK) {
    a.blk = block_tokens;
    a.nblk = (int)((a.n_alloc + block_tokens - 1) / block_tokens);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(pab::launch_quantize(a, st), st);
}

pab_status pab_attention_dense(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                               int causal, float sm_scale, int tau, const uint8_t* kv_valid,
                               const int32_t* out_perm, int64_t n_out_tokens, float* out,
                               const int64_t out_strides[4], float* lse, void* stream) {
  if (empty_views(q, k, v) && n_out_tokens >= 0) return PAB_OK;
  pab::AttnArgs a;
  pab_status s = fill_attn_args(q, k, v, sm_scale, tau, kv_valid, out_perm, n_out_tokens, out,
                                out_strides, a);
  if (s != PAB_OK) return s;
  if (lse && !aligned(lse, 4)) return PAB_INVALID_ARG;
  a.lse = lse;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(pab::launch_attention(a, (int)q->d, q->recipe == PAB_MXFP4_D32,
                                          v->recipe == PAB_MXFP4_V, causal ? 1 : 0, st),
                    st);
}

pab_status pab_attention_dense_tiles(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                     float sm_scale, int tau, const int32_t* key_tiles,
                                     int n_key_tiles, const uint8_t* kv_valid,
                                     const int32_t* out_perm, int64_t n_out_tokens, float* out,
                                     const int64_t out_strides[4], float* lse, void* stream) {
  if (!key_tiles || !kv_valid || !aligned(key_tiles, 4)) return PAB_INVALID_ARG;
  pab::AttnArgs a;
  pab_status s = fill_attn_args(q, k, v, sm_scale, tau, kv_valid, out_perm, n_out_tokens, out,
                                out_strides, a);
  if (s != PAB_OK) return s;
  if (n_key_tiles < 1 || (int64_t)n_key_tiles * pab::kBN > round_up(q->N, pab::kBN))
    return PAB_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return PAB_INVALID_ARG;
  a.lse = lse;
  a.key_tiles = key_tiles;
  a.n_key_tiles = n_key_tiles;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(pab::launch_attention(a, (int)q->d, q->recipe == PAB_MXFP4_D32,
                                          v->recipe == PAB_MXFP4_V, 3, st),
                    st);
}

pab_status pab_key_tiles(const uint8_t* kv_valid, int64_t n, int bn, int32_t* tiles,
                         int64_t* count) {
  if (!kv_valid || !count || n < 1 || bn != pab::kBN || n > ((int64_t)1 << 28))
    return PAB_INVALID_ARG;
  int64_t c = 0;
  for (int64_t t = 0; t * bn < n; ++t) {
    const int64_t e = std::min<int64_t>(n, (t + 1) * bn);
    bool any = false;
    for (int64_t j = t * bn; j < e && !any; ++j) any = kv_valid[j] != 0;
    if (any) {
      if (tiles) tiles[c] = (int32_t)t;
      ++c;
    }
  }
  *count = c;
  return PAB_OK;
}

namespace {

// Sliding-tile attention with window-list entries of key_unit keys (a whole
// key tile, or one BN-key step).
pab_status run_sta(const pab_qview* q, const pab_qview* k, const pab_qview* v, float sm_scale, int tau,
                   const int32_t* win_off, const int32_t* win_idx, const int32_t* tile_order,
                   int n_tiles, int tile_tokens, int key_unit, const uint8_t* kv_valid,
                   const int32_t* out_perm, int64_t n_out_tokens, float* out,
                   const int64_t out_strides[4], float* lse, void* stream) {
  if (!win_off || !win_idx || !tile_order) return PAB_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return PAB_INVALID_ARG;
  if (n_tiles < 1 || tile_tokens < PAB_TOKEN_ALIGN || tile_tokens % PAB_TOKEN_ALIGN)
    return PAB_INVALID_ARG;
  pab::AttnArgs a;
  pab_status s = fill_attn_args(q, k, v, sm_scale, tau, kv_valid, out_perm, n_out_tokens, out,
                                out_strides, a);
  if (s != PAB_OK) return s;
  if ((int64_t)n_tiles * tile_tokens != q->N) return PAB_INVALID_ARG;
  a.lse = lse;
  a.win_off = win_off;
  a.win_idx = win_idx;
  a.tile_order = tile_order;
  a.n_tiles = n_tiles;
  a.tile_tokens = tile_tokens;
  a.key_unit = key_unit;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(pab::launch_attention(a, (int)q->d, q->recipe == PAB_MXFP4_D32,
                                          v->recipe == PAB_MXFP4_V, 2, st),
                    st);
}

}  // namespace

pab_status pab_attention_sta(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                             float sm_scale, int tau, const int32_t* win_off, const int32_t* win_idx,
                             const int32_t* tile_order, int n_tiles, int tile_tokens,
                             const uint8_t* kv_valid, const int32_t* out_perm,
                             int64_t n_out_tokens, float* out, const int64_t out_strides[4],
                             float* lse, void* stream) {
  return run_sta(q, k, v, sm_scale, tau, win_off, win_idx, tile_order, n_tiles, tile_tokens,
                 tile_tokens, kv_valid, out_perm, n_out_tokens, out, out_strides, lse, stream);
}

pab_status pab_attention_sta_steps(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                   float sm_scale, int tau, const int32_t* step_off,
                                   const int32_t* step_idx, const int32_t* tile_order, int n_tiles,
                                   int tile_tokens, const uint8_t* kv_valid,
                                   const int32_t* out_perm, int64_t n_out_tokens, float* out,
                                   const int64_t out_strides[4], float* lse, void* stream) {
  return run_sta(q, k, v, sm_scale, tau, step_off, step_idx, tile_order, n_tiles, tile_tokens,
                 pab::kBN, kv_valid, out_perm, n_out_tokens, out, out_strides, lse, stream);
}

pab_status pab_sta_steps(const int32_t* win_off, const int32_t* win_idx, int n_tiles,
                         int tile_tokens, const uint8_t* kv_valid, int64_t n, int bn,
                         int32_t* step_off, int32_t* step_idx, int64_t* n_steps) {
  if (!win_off || !win_idx || !n_steps || n_tiles < 1 || bn != pab::kBN || tile_tokens < bn ||
      tile_tokens % bn || (int64_t)n_tiles * tile_tokens != n)
    return PAB_INVALID_ARG;
  const int spt = tile_tokens / bn;
  auto valid = [&](int64_t kt) {
    if (!kv_valid) return true;
    for (int64_t j = kt * bn; j < (kt + 1) * bn; ++j)
      if (kv_valid[j]) return true;
    return false;
  };
  int64_t c = 0;
  for (int u = 0; u < n_tiles; ++u) {
    if (step_off) step_off[u] = (int32_t)c;
    if (win_off[u] > win_off[u + 1]) return PAB_INVALID_ARG;
    for (int32_t e = win_off[u]; e < win_off[u + 1]; ++e) {
      const int32_t w = win_idx[e];
      if (w < 0 || w >= n_tiles) return PAB_INVALID_ARG;
      for (int s = 0; s < spt; ++s) {
        const int64_t kt = (int64_t)w * spt + s;
        if (!valid(kt)) continue;
        if (step_idx) step_idx[c] = (int32_t)kt;
        ++c;
      }
    }
  }
  if (step_off) step_off[n_tiles] = (int32_t)c;
  *n_steps = c;
  return PAB_OK;
}

int64_t pab_attention_backward_workspace(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  if (B == 0 || H == 0 || N == 0) return 0;
  if (B > kMaxGridY || H > kMaxGridY || B * H > kMaxGridY || N > kMaxBwdTokens || d > 128)
    return -1;
  int64_t off[13];
  return pab::bwd_workspace_layout(B * H, round_up(N, PAB_TOKEN_ALIGN), d, off);
}

// The backward of dense / causal attention (win_idx NULL) or of sliding-tile
// attention over the CSR window lists (validated by the caller).
static pab_status backward_impl(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                int causal, float sm_scale, const uint8_t* kv_valid,
                                const int32_t* win_off, const int32_t* win_idx, int tile_tokens,
                                const float* out, const int64_t out_strides[4],
                                const void* dout, pab_dtype dout_dtype,
                                const int64_t dout_strides[4], const float* lse, float* dq,
                                float* dk, float* dv, const int64_t grad_strides[4],
                                void* workspace, int64_t workspace_bytes, void* stream,
                                bool launch = true) {
  if (empty_views(q, k, v)) return PAB_OK;
  pab_status s;
  if ((s = check_view(q, 0)) != PAB_OK) return s;
  if ((s = check_view(k, 0)) != PAB_OK) return s;
  if ((s = check_view(v, 1)) != PAB_OK) return s;
  if (q->recipe != k->recipe) return PAB_INVALID_ARG;
  if (q->B != k->B || q->B != v->B || q->H != k->H || q->H != v->H || q->N != k->N ||
      q->N != v->N || q->d != k->d || q->d != v->d)
    return PAB_INVALID_ARG;
  if (q->d != 128 || q->N > kMaxBwdTokens || q->B * q->H > kMaxGridY) return PAB_UNSUPPORTED;
  if (dout_dtype != PAB_F32 && dout_dtype != PAB_BF16) return PAB_INVALID_ARG;
  if (!out || !out_strides || !dout || !dout_strides || !lse || !dq || !dk || !dv ||
      !grad_strides || !workspace)
    return PAB_INVALID_ARG;
  const int64_t dq_align = dout_dtype == PAB_BF16 ? 8 : 4;
  for (int i = 0; i < 3; ++i) {
    if (out_strides[i] < 0 || out_strides[i] % 4 || grad_strides[i] < 0 || grad_strides[i] % 4 ||
        dout_strides[i] < 0 || dout_strides[i] % dq_align)
      return PAB_INVALID_ARG;
  }
  if (out_strides[3] != 1 || dout_strides[3] != 1 || grad_strides[3] != 1) return PAB_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(lse, 4) || !aligned(workspace, 256))
    return PAB_INVALID_ARG;
  if (kv_valid && !aligned(kv_valid, 4)) return PAB_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return PAB_INVALID_ARG;
  const int64_t BH = q->B * q->H, n_alloc = round_up(q->N, PAB_TOKEN_ALIGN);
  int64_t off[13];
  if (workspace_bytes < pab::bwd_workspace_layout(BH, n_alloc, q->d, off)) return PAB_INVALID_ARG;
  if (!launch) return PAB_OK;   // validation only

  pab::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = (int)q->B;
  a.H = (int)q->H;
  a.N = (int)q->N;
  a.n_alloc = (int)n_alloc;
  a.d = (int)q->d;
  a.sm = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt((float)q->d);
  a.sm_log2 = a.sm * 1.4426950408889634f;
  a.causal = causal != 0;
  a.qk_mx = q->recipe == PAB_MXFP4_D32;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto ws16 = [&](int i) { return reinterpret_cast<uint16_t*>(ws + off[i]); };
  auto ws32 = [&](int i) { return reinterpret_cast<float*>(ws + off[i]); };
  if (a.qk_mx) {
    a.q_codes = static_cast<const uint8_t*>(q->codes);
    a.k_codes = static_cast<const uint8_t*>(k->codes);
    a.q_mx = static_cast<const uint8_t*>(q->scales);
    a.k_mx = static_cast<const uint8_t*>(k->scales);
    a.q_rows = ws16(0);
    a.k_rows = ws16(1);
  } else {
    a.q_val = static_cast<const uint16_t*>(q->operand);
    a.k_val = static_cast<const uint16_t*>(k->operand);
    a.q_scale = static_cast<const float*>(q->scales);
    a.k_scale = static_cast<const float*>(k->scales);
    a.blk_q = q->block_tokens;
    a.blk_k = k->block_tokens;
    a.nblk_q = (int)((n_alloc + a.blk_q - 1) / a.blk_q);
    a.nblk_k = (int)((n_alloc + a.blk_k - 1) / a.blk_k);
    a.q_rows = const_cast<uint16_t*>(a.q_val);   // read only
    a.k_rows = const_cast<uint16_t*>(a.k_val);
  }
  a.v_mx = v->recipe == PAB_MXFP4_V;
  a.v_codes = static_cast<const uint8_t*>(v->codes);
  if (a.v_mx)
    a.v_e8 = static_cast<const uint8_t*>(v->scales);
  else
    a.v_scale = static_cast<const float*>(v->scales);
  a.kv_valid = kv_valid;
  a.win_off = win_off;
  a.win_idx = win_idx;
  a.tile_tokens = tile_tokens;
  a.o = out;
  a.o_sb = out_strides[0];
  a.o_sh = out_strides[1];
  a.o_sn = out_strides[2];
  a.dout = dout;
  a.dout_bf16 = dout_dtype == PAB_BF16;
  a.do_sb = dout_strides[0];
  a.do_sh = dout_strides[1];
  a.do_sn = dout_strides[2];
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.g_sb = grad_strides[0];
  a.g_sh = grad_strides[1];
  a.g_sn = grad_strides[2];
  a.v_rows = ws16(2);
  a.dos_rows = ws16(3);
  a.qt = ws16(4);
  a.kt = ws16(5);
  a.dot = ws16(6);
  a.lse_e = ws32(7);
  a.dd = ws32(8);
  a.fq = ws32(9);
  a.fk = ws32(10);
  a.kvf = ws32(11);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(pab::launch_attention_backward(a, st), st);
}

pab_status pab_attention_backward(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                  int causal, float sm_scale, const uint8_t* kv_valid,
                                  const float* out, const int64_t out_strides[4],
                                  const void* dout, pab_dtype dout_dtype,
                                  const int64_t dout_strides[4], const float* lse, float* dq,
                                  float* dk, float* dv, const int64_t grad_strides[4],
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, causal, sm_scale, kv_valid, nullptr, nullptr, 0, out, out_strides,
                       dout, dout_dtype, dout_strides, lse, dq, dk, dv, grad_strides, workspace,
                       workspace_bytes, stream);
}

namespace {

// Workspace of pab_attention_backward_noalloc.  In host code the array's name
// stands for a host-side shadow, not a device address: the device address of
// each device's copy comes from hipGetSymbolAddress and is the only form that
// reaches a kernel.
static __device__ __align__(256) uint8_t scratch[PAB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the device of `st`, looked up once per device
// with that device current.
pab_status scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, st);
  if (dev < 0 || dev >= kMaxScratchDevices) return PAB_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e, st);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, st);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, st);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PAB_OK;
}

}  // namespace

pab_status pab_attention_backward_noalloc(const pab_qview* q, const pab_qview* k,
                                          const pab_qview* v, int causal, float sm_scale,
                                          const uint8_t* kv_valid, const float* out,
                                          const int64_t out_strides[4], const void* dout,
                                          pab_dtype dout_dtype, const int64_t dout_strides[4],
                                          const float* lse, float* dq, float* dk, float* dv,
                                          const int64_t grad_strides[4], void* stream) {
  if (empty_views(q, k, v)) return PAB_OK;
  if (!q) return PAB_INVALID_ARG;
  const int64_t need = pab_attention_backward_workspace(q->B, q->H, q->N, q->d);
  if (need < 0) return PAB_INVALID_ARG;
  if (need > PAB_NOALLOC_SCRATCH_BYTES) return PAB_UNSUPPORTED;
  // every argument is checked (with a stand-in workspace address) before the
  // device is touched
  pab_status s = backward_impl(q, k, v, causal, sm_scale, kv_valid, nullptr, nullptr, 0, out,
                               out_strides, dout, dout_dtype, dout_strides, lse, dq, dk, dv,
                               grad_strides, reinterpret_cast<void*>(256), PAB_NOALLOC_SCRATCH_BYTES,
                               stream, false);
  if (s != PAB_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((s = scratch_address(st, &ws)) != PAB_OK) return s;
  return backward_impl(q, k, v, causal, sm_scale, kv_valid, nullptr, nullptr, 0, out, out_strides,
                       dout, dout_dtype, dout_strides, lse, dq, dk, dv, grad_strides, ws,
                       PAB_NOALLOC_SCRATCH_BYTES, stream);
}

pab_status pab_attention_sta_backward(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                      float sm_scale, const int32_t* win_off,
                                      const int32_t* win_idx, int n_tiles, int tile_tokens,
                                      const uint8_t* kv_valid, const float* out,
                                      const int64_t out_strides[4], const void* dout,
                                      pab_dtype dout_dtype, const int64_t dout_strides[4],
                                      const float* lse, float* dq, float* dk, float* dv,
                                      const int64_t grad_strides[4], void* workspace,
                                      int64_t workspace_bytes, void* stream) {
  if (empty_views(q, k, v)) return PAB_OK;
  if (!q || !win_off || !win_idx || !aligned(win_off, 4) || !aligned(win_idx, 4))
    return PAB_INVALID_ARG;
  if (n_tiles < 1 || tile_tokens < PAB_TOKEN_ALIGN || tile_tokens % PAB_TOKEN_ALIGN)
    return PAB_INVALID_ARG;
  if ((int64_t)n_tiles * tile_tokens != q->N) return PAB_INVALID_ARG;
  return backward_impl(q, k, v, 0, sm_scale, kv_valid, win_off, win_idx, tile_tokens, out,
                       out_strides, dout, dout_dtype, dout_strides, lse, dq, dk, dv, grad_strides,
                       workspace, workspace_bytes, stream);
}

pab_status pab_sta_plan(const int grid[3], const int real_grid[3], const int tile[3],
                        const int window[3], int32_t* perm, int32_t* inv_perm,
                        uint8_t* kv_valid, int32_t* win_off, int32_t* win_idx,
                        int32_t* lpt_order, int64_t* n_tokens, int64_t* n_tiles,
                        int64_t* n_pairs) {
  if (!grid || !real_grid || !tile || !window) return PAB_INVALID_ARG;
  int nt[3], rad[3];
  int64_t tokens = 1, tiles = 1, real = 1;
  for (int i = 0; i < 3; ++i) {
    if (grid[i] < 1 || tile[i] < 1 || real_grid[i] < 1 || window[i] < 1) return PAB_INVALID_ARG;
    if (grid[i] % tile[i] || real_grid[i] > grid[i]) return PAB_INVALID_ARG;
    nt[i] = grid[i] / tile[i];
    rad[i] = window[i] / 2;
    tokens *= grid[i];
    tiles *= nt[i];
    real *= real_grid[i];
    if (tokens > (int64_t)1 << 30) return PAB_UNSUPPORTED;   // checked per axis: no overflow
  }
  // window size per tile: product over axes of the clipped interval length
  auto axis_count = [&](int a, int c) {
    return std::min(c + rad[a], nt[a] - 1) - std::max(c - rad[a], 0) + 1;
  };
  int64_t pairs = 0;
  for (int ut = 0; ut < nt[0]; ++ut)
    for (int uh = 0; uh < nt[1]; ++uh)
      for (int uw = 0; uw < nt[2]; ++uw)
        pairs += (int64_t)axis_count(0, ut) * axis_count(1, uh) * axis_count(2, uw);
  if (n_tokens) *n_tokens = tokens;
  if (n_tiles) *n_tiles = tiles;
  if (n_pairs) *n_pairs = pairs;

  if (perm || inv_perm || kv_valid) {
    // inside a tile its real tokens come first, in raster order, and its
    // padding slots last, so that padding fills whole key steps and query
    // tiles wherever it can
    const int64_t tile_tokens = (int64_t)tile[0] * tile[1] * tile[2];
    int64_t base = 0;
    for (int ut = 0; ut < nt[0]; ++ut)
      for (int uh = 0; uh < nt[1]; ++uh)
        for (int uw = 0; uw < nt[2]; ++uw, base += tile_tokens) {
          int64_t p = base;
          for (int dt = 0; dt < tile[0]; ++dt)
            for (int dh = 0; dh < tile[1]; ++dh)
              for (int dw = 0; dw < tile[2]; ++dw) {
                const int t = ut * tile[0] + dt, h = uh * tile[1] + dh, w = uw * tile[2] + dw;
                if (t >= real_grid[0] || h >= real_grid[1] || w >= real_grid[2]) continue;
                const int64_t r = ((int64_t)t * real_grid[1] + h) * real_grid[2] + w;
                if (perm) perm[p] = (int32_t)r;
                if (kv_valid) kv_valid[p] = 1;
                if (inv_perm) inv_perm[r] = (int32_t)p;
                ++p;
              }
          for (; p < base + tile_tokens; ++p) {
            if (perm) perm[p] = -1;
            if (kv_valid) kv_valid[p] = 0;
          }
        }
  }
  if (win_off || win_idx || lpt_order) {
    std::vector<int32_t> sizes(tiles);
    int64_t pos = 0, u = 0;
    if (win_off) win_off[0] = 0;
    for (int ut = 0; ut < nt[0]; ++ut)
      for (int uh = 0; uh < nt[1]; ++uh)
        for (int uw = 0; uw < nt[2]; ++uw, ++u) {
          const int t0 = std::max(ut - rad[0], 0), t1 = std::min(ut + rad[0], nt[0] - 1);
          const int h0 = std::max(uh - rad[1], 0), h1 = std::min(uh + rad[1], nt[1] - 1);
          const int w0 = std::max(uw - rad[2], 0), w1 = std::min(uw + rad[2], nt[2] - 1);
          for (int vt = t0; vt <= t1; ++vt)
            for (int vh = h0; vh <= h1; ++vh)
              for (int vw = w0; vw <= w1; ++vw) {
                if (win_idx) win_idx[pos] = (int32_t)(((int64_t)vt * nt[1] + vh) * nt[2] + vw);
                ++pos;
              }
          sizes[u] = (t1 - t0 + 1) * (h1 - h0 + 1) * (w1 - w0 + 1);
          if (win_off) win_off[u + 1] = (int32_t)pos;
        }
    if (lpt_order) {
      // longest window lists first; among equal sizes, tiles with the same
      // window list next to each other (ordered by the list, then by index),
      // so that their workgroups run together and read the same key tiles
      // in the same order, sharing the L2
      std::vector<std::vector<int32_t>> lists(tiles);
      int64_t v = 0;
      for (int ut = 0; ut < nt[0]; ++ut)
        for (int uh = 0; uh < nt[1]; ++uh)
          for (int uw = 0; uw < nt[2]; ++uw, ++v) {
            const int t0 = std::max(ut - rad[0], 0), t1 = std::min(ut + rad[0], nt[0] - 1);
            const int h0 = std::max(uh - rad[1], 0), h1 = std::min(uh + rad[1], nt[1] - 1);
            const int w0 = std::max(uw - rad[2], 0), w1 = std::min(uw + rad[2], nt[2] - 1);
            for (int vt = t0; vt <= t1; ++vt)
              for (int vh = h0; vh <= h1; ++vh)
                for (int vw = w0; vw <= w1; ++vw)
                  lists[v].push_back((int32_t)(((int64_t)vt * nt[1] + vh) * nt[2] + vw));
          }
      std::vector<int32_t> order(tiles);
      std::iota(order.begin(), order.end(), 0);
      std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
        if (sizes[x] != sizes[y]) return sizes[x] > sizes[y];
        return std::lexicographical_compare(lists[x].begin(), lists[x].end(), lists[y].begin(),
                                            lists[y].end());
      });
      std::copy(order.begin(), order.end(), lpt_order);
    }
  }
  return PAB_OK;
}

pab_status pab_count_nonfinite(const float* x, int64_t n, int32_t* dev_count, void* stream) {
  if (!x || !dev_count || n < 0) return PAB_INVALID_ARG;
  if (n == 0) return PAB_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(pab::launch_count_nonfinite(x, n, dev_count, st), st);
}

}  // extern "C"
