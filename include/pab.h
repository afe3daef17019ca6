/*
 * pab.h - C ABI of libpab: block-scaled FP8 / MXFP4 FlashAttention forward
 * with optional 3D sliding-tile sparsity, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *  [FPS]  "FP8量化与稀疏性协同加速视频扩散模型" (FPSAttention): §2.1 block FP8
 *         quantisation, §2.2 sliding-tile attention, §3.1 staged quantisation
 *         strategy, §3.3 kernel design (block transpose, fusion).
 *  [FP4G] "Blackwell架构实战：如何用FP4量化让你的AI模型推理速度翻倍（附代码）",
 *         §1: E2M1 and micro-scaled (MX) 4-bit quantisation.
 *  [FA4]  "FA4极速LLM：10分钟搞定20倍内存直降！": tiling, online softmax,
 *         conditional rescaling, LPT scheduling for causal masks.
 *  [FV]   FastVideo FP4 attention kernel article (wmrh.cn): §2.1 attention
 *         definition, §5.2 the fp4_attention(qkv, mask, head_dim,
 *         scaling_factor) call, §8.2 fall back when the output is not finite.
 *
 * Conventions for every call
 *  - Tensors are in device memory the caller allocated; the library never
 *    allocates device memory and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every device call is asynchronous on that stream and does not
 *    synchronise, except when the environment variable PAB_SYNC_DEBUG=1 is
 *    set (then each call synchronises the stream and reports kernel errors).
 *  - All arguments are validated before any launch; a call that returns an
 *    error other than PAB_HIP_ERROR has written nothing.
 *  - Element counts and strides are in elements, not bytes.
 *  - Empty inputs: pab_quantize with B, H or n_out equal to 0, and
 *    pab_attention_dense / pab_attention_backward with B, H or N equal to 0
 *    (the three views agreeing on their sizes), return PAB_OK, launch
 *    nothing and do not examine their pointers, which may be NULL.
 *    Negative sizes are PAB_INVALID_ARG.  The sliding-tile calls need a
 *    plan, which always holds tokens.
 *  - Size limits (PAB_UNSUPPORTED beyond them), from the device's grid limits
 *    and the kernels' 32-bit buffer offsets: pab_quantize B*H <= 65536,
 *    n_out <= 2^27 and N_in < 2^31; the attention calls N <= 2^22,
 *    B*H <= 2^24 and B*H*pab_token_alloc(N) < 2^31; the backward N <= 2^20
 *    and B*H <= 65536.  Larger batches are split by the caller.
 *  - Quantised token buffers are padded: a tensor with n tokens is stored with
 *    n_alloc = pab_token_alloc(n) token slots (a multiple of PAB_TOKEN_ALIGN);
 *    the quantizers write zero codes into slots n..n_alloc-1.
 *  - No C++ exception crosses this interface.  Thread-safe (no globals other
 *    than the thread-local last HIP error).
 */
#ifndef PAB_H
#define PAB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAB_ABI_VERSION 9
#define PAB_TOKEN_ALIGN 128  /* query tile of the attention kernel */
#define PAB_MAX_TAU 8        /* largest softmax rescale threshold (log2 units) */

typedef enum {
  PAB_OK = 0,
  PAB_INVALID_ARG = 1,   /* null pointer, bad shape, stride or size */
  PAB_UNSUPPORTED = 2,   /* valid but not implemented (e.g. d not in {64,128}) */
  PAB_HIP_ERROR = 3      /* a HIP runtime call failed; see pab_last_hip_error */
} pab_status;

typedef enum { PAB_F32 = 0, PAB_BF16 = 1 } pab_dtype;

/* Quantisation recipes of the staged precision strategy [FPS §3.1] and the
 * MX variant [FP4G §1]. */
typedef enum {
  /* Q/K: FP8 E4M3 (OCP "fn", largest 448), one fp32 scale per block of
   * `block_tokens` consecutive tokens x all d channels of one (batch, head):
   * s = fl32(448 / amax) (s = 1 if amax is 0 or the quotient is not finite),
   * code = E4M3(fl32(x * s)), round-to-nearest-even, saturating at +-448;
   * dequantised x ~= decode(code) / s  [FPS §2.1]. */
  PAB_FP8_TOKEN_BLOCK = 0,
  /* V: FP8 E4M3 with one fp32 scale per (batch, head, channel) over all tokens,
   * same scale rule [FPS §3.1]. */
  PAB_FP8_CHANNEL = 1,
  /* Q/K MXFP4: E2M1 codes with one E8M0 scale per 32 consecutive channels:
   * e = clamp(floor(log2 amax) - 2, -127, 127) (-127 for an all-zero group),
   * scale byte e + 127, code = E2M1(x * 2^-e), round-to-nearest-even on the
   * code, saturating at +-6; dequantised x = decode(code) * 2^e [FP4G §1]. */
  PAB_MXFP4_D32 = 2,
  /* V for FP4 P.V [FV §1, FP4 attention]: MXFP4 along the token axis, one
   * E8M0 scale per (batch, head, channel, 32 consecutive kernel tokens), same
   * MX rule; zero padding slots count as tokens of their group. */
  PAB_MXFP4_V = 3
} pab_recipe;

/* ABI version (PAB_ABI_VERSION of the built library). */
int pab_abi_version(void);
/* Static description of a status code. */
const char* pab_status_str(pab_status s);
/* hipError_t of the last failing HIP call on this thread (0 if none). */
int pab_last_hip_error(void);
/* Token slots a quantised buffer for n tokens must hold (n rounded up to
 * PAB_TOKEN_ALIGN; 0 for n <= 0, -1 when the rounded count is not
 * representable). */
int64_t pab_token_alloc(int64_t n);

/* Tile sizes of the attention kernel for a recipe / head dim: BM queries per
 * workgroup (256 for dense FP8 attention with d = 128 over all key tiles,
 * mode 0; else 128), BN keys per online-softmax step (64).  The online
 * softmax visits key tiles of BN keys in ascending order and requantises P
 * against the running maximum including the current tile, so BN is part of
 * the result's definition (the reference oracle takes it as a parameter).
 * mode: 0 dense, 1 causal, 2 sliding-tile, 3 dense over listed key tiles. */
pab_status pab_attention_info(pab_recipe qk_recipe, int d, int mode, int* BM, int* BN);

/*
 * pab_quantize - quantise one tensor with one recipe [FPS §2.1, §3.1; FP4G §1].
 *
 * x        device, logical [B, H, N_in, d] of in_dt with element strides
 *          `strides` (any non-negative strides; the innermost must be 1).
 * perm     device int32 [n_out] or NULL.  If given, kernel token p takes input
 *          token perm[p] (a value of -1 gives a zero token: padding).  This is
 *          the block transpose of [FPS §3.3 item 1] that makes each 3D tile
 *          contiguous.  If NULL, n_out must equal N_in and token p is input
 *          token p.
 * block_tokens  tokens per scale block for PAB_FP8_TOKEN_BLOCK (a multiple of
 *          16, at most 16384); ignored otherwise.
 * Outputs (n_alloc = pab_token_alloc(n_out)):
 *  PAB_FP8_TOKEN_BLOCK: codes uint8 [B, H, n_alloc, d];
 *                       scales float32 [B, H, ceil(n_alloc / block_tokens)]
 *                       (blocks holding no token below n_out get scale 1);
 *                       operand (if not NULL) bfloat16 [B, H, n_alloc, d]: the
 *                       exact value decode(code) of every code (not divided by
 *                       the scale) - the attention kernel reads K in this
 *                       form, see pab_attention_dense; Q needs it only for
 *                       the backward calls.
 *  PAB_FP8_CHANNEL:     codes uint8 [B, H, d, n_alloc] - transposed, and inside
 *                       every 64-token group the token t = 32a + 8b + 4g + c
 *                       (a < 2, b < 4, g < 2, c < 4) is stored at position
 *                       32g + 16a + 4b + c (the operand order of the kernel's
 *                       P.V product); scales float32 [B, H, d].
 *  PAB_MXFP4_D32:       codes uint8 [B, H, n_alloc, d/2], two E2M1 codes per
 *                       byte, channel 2k in the low nibble;
 *                       scales uint8 (E8M0) [B, H, n_alloc, d/32].
 *  PAB_MXFP4_V:         codes uint8 [B, H, d, n_alloc/2] - transposed, two
 *                       E2M1 codes per byte, slot 2k in the low nibble; slot
 *                       j of every 32-token group holds token
 *                       8 ((j mod 16) / 4) + 4 (j / 16) + j mod 4 of the group
 *                       (the operand order of the FP4 P.V product);
 *                       scales uint8 (E8M0) [B, H, n_alloc/32, d] with channel
 *                       c of a group at position 4 (c mod 32) + c / 32.
 *                       d must be 128.
 * `operand` must be NULL for the other recipes.  x must be 16-byte aligned
 * and the batch/head/token strides multiples of 8.
 * d must be 64 or 128 (128 for MXFP4).  Inputs are assumed finite.
 */
pab_status pab_quantize(const void* x, pab_dtype in_dt, const int64_t shape[4],
                        const int64_t strides[4], pab_recipe recipe, int block_tokens,
                        const int32_t* perm, int64_t n_out, void* codes, void* scales,
                        void* operand, void* stream);

/* A quantised operand as pab_quantize wrote it (all device pointers). */
typedef struct {
  const void* codes;
  const void* scales;
  const void* operand;   /* PAB_FP8_TOKEN_BLOCK: the bf16 operand copy; required for K,
                            and for Q and K in the backward calls; the forward calls
                            do not read Q's (NULL allowed) */
  pab_recipe recipe;
  int block_tokens;      /* PAB_FP8_TOKEN_BLOCK only */
  int64_t B, H, N, d;    /* N = tokens (n_out of pab_quantize) */
} pab_qview;

/*
 * pab_attention_dense - O = softmax(Q K^T * sm_scale) V, FlashAttention-style
 * [FV §2.1; FA4 FlashAttention section], on quantised operands:
 *  Q, K: PAB_FP8_TOKEN_BLOCK or PAB_MXFP4_D32 (both the same recipe);
 *  V:    PAB_FP8_CHANNEL, or PAB_MXFP4_V with MXFP4 Q/K (FP4 P.V, below);
 *  P:    requantised to FP8 E4M3 with the fixed per-tensor scale 1/448
 *        [FPS §3.1]: P~ = E4M3(448 P) against the running row maximum.
 * For each query row the kernel visits key tiles of BN keys in ascending
 * order (causal: keys j <= i, top-left aligned) and keeps the running max m,
 * the sum l of the unquantised P and the accumulator of P~ V in fp32.
 * Q K^T of the FP8 recipe is summed from the exact products of the decoded
 * E4M3 values (K's bf16 operand copy; Q's codes are decoded in registers) with
 * fp32 accumulation; P~ V uses the FP8 matrix instructions.
 * O[i,c] = acc[i,c] / (448 l_i) / s_V[c]; a row with no valid key gives 0.
 * FP4 P.V (V in PAB_MXFP4_V) [FV §1, FP4 attention]: P is requantised to
 * MXFP4 instead, per query row and per 32 consecutive keys of the tile, by the
 * MX rule of PAB_MXFP4_D32 applied to P (e = floor(log2 max P) - 2); both
 * products run on the FP4 matrix instructions, and O = acc / l (the scales
 * sit inside the products).  tau applies as below; there is no 448 factor.
 * sm_scale <= 0 means 1/sqrt(d)  [FV §5.2 scaling_factor].
 * tau       softmax rescale threshold, an integer in log2 units, 0 ..
 *           PAB_MAX_TAU [FA4 co-design list: conditional rescaling]: the
 *           reference maximum m of a row moves only when the row maximum
 *           exceeds m + tau (a float32 comparison); until then P = 2^(S - m)
 *           may reach 2^tau, and P~ = E4M3(448 / 2^tau * P), l and acc are
 *           kept against the stale m (O divides by 448 / 2^tau instead of
 *           448).  tau = 0 is the recipe above; a larger tau skips most
 *           rescales of the accumulator at the cost of tau bits of P~ range
 *           at the small end.  Out of range: PAB_INVALID_ARG.
 * kv_valid  device uint8 [N] or NULL: keys with 0 are masked (padding).
 * out_perm  device int32 [N] or NULL: query p is stored at output token
 *           out_perm[p] (skipped if -1); NULL stores query p at token p.
 * out       device float32 [B, H, n_out_tokens, d] with element strides
 *           out_strides (innermost 1); rows that no query maps to are not
 *           written.
 * lse       device float32 [B, H, N] or NULL: the row statistic
 *           LSE_i = m_i + log2(sum_j 2^(S_ij - m_i)) in the log2 units of S
 *           (S = Q K^T * sm_scale * log2(e)), stored per query in the kernel's
 *           token order whatever out_perm is; -inf for a row without a valid
 *           key.  The backward pass recovers P from it.
 */
pab_status pab_attention_dense(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                               int causal, float sm_scale, int tau, const uint8_t* kv_valid,
                               const int32_t* out_perm, int64_t n_out_tokens, float* out,
                               const int64_t out_strides[4], float* lse, void* stream);

/*
 * pab_attention_dense_tiles - pab_attention_dense without a causal mask that
 * visits only the BN-key tiles listed in key_tiles (tile t = keys t*BN ..
 * t*BN+BN-1; BN from pab_attention_info): a padded sequence skips the tiles
 * that hold no valid key.  key_tiles is a device int32 array of n_key_tiles
 * ascending tile indices.  Every key outside the listed tiles must be masked
 * by kv_valid (required here); the result then equals pab_attention_dense
 * with the same kv_valid bit for bit, since a tile without a valid key leaves
 * the online softmax unchanged.  pab_key_tiles builds the list.  Query tiles
 * whose queries out_perm maps nowhere are skipped when lse is NULL.
 */
pab_status pab_attention_dense_tiles(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                     float sm_scale, int tau, const int32_t* key_tiles,
                                     int n_key_tiles, const uint8_t* kv_valid,
                                     const int32_t* out_perm, int64_t n_out_tokens, float* out,
                                     const int64_t out_strides[4], float* lse, void* stream);

/*
 * pab_key_tiles - host helper: the indices of the BN-key tiles of kv_valid
 * (host uint8 [n]) that hold at least one nonzero entry, ascending, into
 * tiles (host int32, may be NULL to count only); *count receives their
 * number.  bn must be the kernel's BN (pab_attention_info).
 */
pab_status pab_key_tiles(const uint8_t* kv_valid, int64_t n, int bn, int32_t* tiles,
                         int64_t* count);

/*
 * pab_attention_sta - sliding-tile sparse attention [FPS §2.2]: the N tokens
 * (kernel order, see pab_sta_plan) form n_tiles tiles of tile_tokens tokens;
 * query tile u attends only to the key tiles win_idx[win_off[u] ..
 * win_off[u+1]-1] (ascending), each visited as tile_tokens/BN key tiles in
 * ascending order.  Everything else is as in pab_attention_dense (no causal
 * mask).  A window list holding every tile gives the dense result bit for bit.
 * win_off int32 [n_tiles+1], win_idx int32 [win_off[n_tiles]], tile_order
 * int32 [n_tiles] (a permutation of the tiles: the order work is issued, e.g.
 * longest window first [FA4, LPT scheduling]) - device pointers.
 * tile_tokens must be a multiple of PAB_TOKEN_ALIGN and N == n_tiles *
 * tile_tokens.  lse as in pab_attention_dense.
 */
pab_status pab_attention_sta(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                             float sm_scale, int tau, const int32_t* win_off, const int32_t* win_idx,
                             const int32_t* tile_order, int n_tiles, int tile_tokens,
                             const uint8_t* kv_valid, const int32_t* out_perm,
                             int64_t n_out_tokens, float* out, const int64_t out_strides[4],
                             float* lse, void* stream);

/*
 * pab_attention_sta_steps - pab_attention_sta with window lists in BN-key
 * steps instead of whole key tiles: query tile u visits the BN-key tiles
 * step_idx[step_off[u] .. step_off[u+1]-1] (ascending; tile t = keys t*BN ..
 * t*BN+BN-1).  pab_sta_steps expands tile window lists into these and drops
 * the steps without a valid key, which leaves the result unchanged (bit for
 * bit): a padded grid then skips its padding keys.
 */
pab_status pab_attention_sta_steps(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                   float sm_scale, int tau, const int32_t* step_off,
                                   const int32_t* step_idx, const int32_t* tile_order, int n_tiles,
                                   int tile_tokens, const uint8_t* kv_valid,
                                   const int32_t* out_perm, int64_t n_out_tokens, float* out,
                                   const int64_t out_strides[4], float* lse, void* stream);

/*
 * pab_sta_steps - host helper: expands the window lists of pab_sta_plan
 * (win_off [n_tiles+1], win_idx) into BN-key step lists, keeping the steps
 * that hold a valid key of kv_valid (host uint8 [n], NULL = all valid), in
 * ascending order.  n = n_tiles * tile_tokens.  Two-call pattern: with
 * step_off / step_idx NULL only *n_steps is returned.
 */
pab_status pab_sta_steps(const int32_t* win_off, const int32_t* win_idx, int n_tiles,
                         int tile_tokens, const uint8_t* kv_valid, int64_t n, int bn,
                         int32_t* step_off, int32_t* step_idx, int64_t* n_steps);

/*
 * pab_attention_backward - gradients of the attention of pab_attention_dense
 * [FA4 co-design list: the backward pass, intermediates S, P, dP, dS, dQ],
 * for training-aware quantisation [FPS introduction].  The quantisers pass
 * gradients straight through: the results are the gradients with respect to
 * the dequantised operands Q^, K^, V^ of
 *     O = softmax(Q^ K^T * sm_scale) V^,
 * evaluated with the forward's row statistic and output:
 *     P = 2^(S - LSE) with S = Q^ K^T * sm_scale * log2(e)
 *     dV = P^T dO,  dP = dO V^^T,  D_i = sum_c dO_ic O_ic,
 *     dS = P (dP - D),  dQ = sm_scale dS K^,  dK = sm_scale dS^T Q^.
 * q, k, v   the views the forward pass used: Q/K PAB_FP8_TOKEN_BLOCK (with its
 *           operand copy) or PAB_MXFP4_D32; V PAB_FP8_CHANNEL or PAB_MXFP4_V;
 *           d = 128.
 * causal, sm_scale, kv_valid   as passed to the forward (sm_scale <= 0 means
 *           1/sqrt(d)).
 * out       the forward output O, float32 [B, H, N, d] in the kernel's token
 *           order (the forward called without out_perm), strides out_strides.
 * dout      dO, float32 or bf16 (dout_dtype) [B, H, N, d], strides
 *           dout_strides (innermost 1).
 * lse       the forward's lse, float32 [B, H, N].
 * dq, dk, dv  float32 [B, H, N, d] with strides grad_strides (innermost 1);
 *           every element of rows 0..N-1 is written.
 * workspace device memory of at least
 *           pab_attention_backward_workspace(B, H, N, d) bytes, 256-byte
 *           aligned, owned by the caller; contents on entry do not matter.
 * P, dS and dO enter their matrix products rounded to bf16; sums are fp32.
 * Strides must be multiples of 4 (float32) or 8 (bf16) elements and the
 * pointers 16-byte aligned.  PAB_UNSUPPORTED for d != 128, N > 2^20 or
 * B*H > 65536.
 * The workspace size is 0 for an empty input and -1 for a negative size or
 * one beyond the backward's limits (B*H > 65536, N > 2^20, d > 128).
 */
int64_t pab_attention_backward_workspace(int64_t B, int64_t H, int64_t N, int64_t d);
pab_status pab_attention_backward(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                  int causal, float sm_scale, const uint8_t* kv_valid,
                                  const float* out, const int64_t out_strides[4],
                                  const void* dout, pab_dtype dout_dtype,
                                  const int64_t dout_strides[4], const float* lse, float* dq,
                                  float* dk, float* dv, const int64_t grad_strides[4],
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* Largest workspace (bytes) of pab_attention_backward_noalloc: the size of
 * the library's own device array. */
#define PAB_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)

/*
 * pab_attention_backward_noalloc - pab_attention_backward for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same gradients from the same
 * kernels, with the workspace taken from a file-scope device array of
 * PAB_NOALLOC_SCRATCH_BYTES inside the library instead of a caller buffer.
 * Every argument but the workspace is as for pab_attention_backward.
 * The array's address on a device is looked up once, at the first call on
 * that device (the stream's device); the call itself allocates nothing.
 * Each device holds one array for the life of the process, shared by every
 * call on that device: calls that overlap in time on one device (on
 * different streams, or from different threads) race on it and must be
 * serialised by the caller.  The kernels write every workspace byte they
 * read, so no state carries over between calls.
 * PAB_UNSUPPORTED when the problem needs more than PAB_NOALLOC_SCRATCH_BYTES
 * of workspace (pab_attention_backward_workspace gives the need), before any
 * launch; PAB_HIP_ERROR if the address lookup fails.
 */
pab_status pab_attention_backward_noalloc(const pab_qview* q, const pab_qview* k,
                                          const pab_qview* v, int causal, float sm_scale,
                                          const uint8_t* kv_valid, const float* out,
                                          const int64_t out_strides[4], const void* dout,
                                          pab_dtype dout_dtype, const int64_t dout_strides[4],
                                          const float* lse, float* dq, float* dk, float* dv,
                                          const int64_t grad_strides[4], void* stream);

/* Backward of sliding-tile attention (pab_attention_sta): the gradients of
 * pab_attention_backward, with key j visible to query i when the tile of j is
 * in the window list of the tile of i and kv_valid[j] is nonzero [FPS] §2.2.
 * The tokens are in the kernel's tile-major order (the forward called without
 * out_perm, which gives out and lse in that order).  The window relation must
 * be symmetric (v in W(u) exactly when u in W(v)), as the windows of
 * pab_sta_plan are: the key tiles of query tile u are read from W(u) and the
 * query tiles that see key tile v from W(v); a tile with an empty list gets
 * zero gradients.  win_off int32 [n_tiles + 1],
 * win_idx int32 [win_off[n_tiles]] on the device; n_tiles * tile_tokens = N,
 * tile_tokens a multiple of PAB_TOKEN_ALIGN.  Every other argument, the
 * workspace and the errors are as for pab_attention_backward. */
pab_status pab_attention_sta_backward(const pab_qview* q, const pab_qview* k, const pab_qview* v,
                                      float sm_scale, const int32_t* win_off,
                                      const int32_t* win_idx, int n_tiles, int tile_tokens,
                                      const uint8_t* kv_valid, const float* out,
                                      const int64_t out_strides[4], const void* dout,
                                      pab_dtype dout_dtype, const int64_t dout_strides[4],
                                      const float* lse, float* dq, float* dk, float* dv,
                                      const int64_t grad_strides[4], void* workspace,
                                      int64_t workspace_bytes, void* stream);

/*
 * pab_sta_plan - host-side planner for sliding-tile attention [FPS §2.2,
 * §3.3 item 1].  grid = (T, H, W) of the padded latent grid (each a multiple
 * of tile), real_grid <= grid the unpadded grid whose tokens the caller holds
 * in raster order, tile = (t, h, w) tokens per tile, window = (w_t, w_h, w_w)
 * in tiles: key tile v is in the window of query tile u iff
 * |u_a - v_a| <= floor(w_a / 2) on every axis, clipped at the grid border.
 * Kernel token order: tiles in raster order over the tile grid; inside a
 * tile its real tokens in raster order, then its padding slots (so padding
 * fills whole key steps and query tiles where it can, which the step lists
 * and the query-tile skip then leave out).
 * Outputs (host memory; pass NULL to skip an array; call once with all NULL
 * to get the sizes):
 *   perm       int32 [n_tokens]: raster index in real_grid of kernel token p,
 *              -1 for padding;
 *   inv_perm   int32 [T_r*H_r*W_r]: kernel position of each real token;
 *   kv_valid   uint8 [n_tokens]: 1 where perm >= 0;
 *   win_off    int32 [n_tiles+1], win_idx int32 [n_pairs]: window lists,
 *              ascending within each tile;
 *   lpt_order  int32 [n_tiles]: an issue order (results do not depend on
 *              it): tiles by decreasing window size [FA4, LPT scheduling],
 *              tiles with the same window list next to each other (ordered
 *              by the list, then by index) so that their workgroups run
 *              together and share the key tiles they read.
 * Pure host code, deterministic.
 */
pab_status pab_sta_plan(const int grid[3], const int real_grid[3], const int tile[3],
                        const int window[3], int32_t* perm, int32_t* inv_perm,
                        uint8_t* kv_valid, int32_t* win_off, int32_t* win_idx,
                        int32_t* lpt_order, int64_t* n_tokens, int64_t* n_tiles,
                        int64_t* n_pairs);

/*
 * pab_count_nonfinite - adds the number of NaN/Inf values among x[0..n) to
 * *dev_count (device int32; the caller zeroes it).  Lets a caller fall back
 * to another attention path when an output is not finite [FV §8.2].
 */
pab_status pab_count_nonfinite(const float* x, int64_t n, int32_t* dev_count, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PAB_H */
