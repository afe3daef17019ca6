// Host-side driver for a sanitizer build of libpab's C ABI (address and
// undefined-behaviour sanitizers on the host code of api.cpp).  It needs no
// GPU: it runs the pure host entry points (the sliding-tile planner, the
// step and key-tile lists, the size helpers) on valid and hostile sizes with
// output arrays of exactly the size the count-only call reported, so a write
// past the end is caught, and drives every validation path of the device
// entry points with arguments that must be rejected before the first HIP call.
// Prints "checks passed: N" and exits 0, or names the failed check and exits 1.
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "pab.h"

static int g_checks = 0;
static int g_failed = 0;

#define EXPECT(cond)                                                         \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_failed;                                                            \
    }                                                                        \
  } while (0)

// Rejected by validation, before any HIP call (a HIP error would mean a call
// got through to the device).
static bool rejected(pab_status s) { return s == PAB_INVALID_ARG || s == PAB_UNSUPPORTED; }

static const int64_t kBig = std::numeric_limits<int64_t>::max();

// One planner run with exact-size outputs; checks the invariants the device
// entry points rely on (a permutation, ascending in-range window lists).
static void plan_case(const int grid[3], const int real[3], const int tile[3], const int win[3],
                      pab_status expect) {
  int64_t nt = -1, nti = -1, npr = -1;
  pab_status s = pab_sta_plan(grid, real, tile, win, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, &nt, &nti, &npr);
  EXPECT(s == expect);
  if (s != PAB_OK) return;
  const int64_t n_real = (int64_t)real[0] * real[1] * real[2];
  const int tile_tokens = tile[0] * tile[1] * tile[2];
  std::vector<int32_t> perm(nt), inv(n_real), off(nti + 1), idx(npr), lpt(nti);
  std::vector<uint8_t> kv(nt);
  s = pab_sta_plan(grid, real, tile, win, perm.data(), inv.data(), kv.data(), off.data(),
                   idx.data(), lpt.data(), &nt, &nti, &npr);
  EXPECT(s == PAB_OK);
  EXPECT(nt == nti * tile_tokens);
  std::vector<int> seen(n_real, 0);
  for (int64_t t = 0; t < nt; ++t) {
    EXPECT(perm[t] >= -1 && perm[t] < n_real);
    EXPECT((perm[t] >= 0) == (kv[t] != 0));
    if (perm[t] >= 0) {
      ++seen[perm[t]];
      EXPECT(inv[perm[t]] == t);
    }
  }
  for (int64_t i = 0; i < n_real; ++i) EXPECT(seen[i] == 1);
  EXPECT(off[0] == 0 && off[nti] == npr);
  std::vector<int> used(nti, 0);
  for (int64_t u = 0; u < nti; ++u) {
    EXPECT(off[u] < off[u + 1]);
    for (int32_t j = off[u]; j < off[u + 1]; ++j) {
      EXPECT(idx[j] >= 0 && idx[j] < nti);
      if (j > off[u]) EXPECT(idx[j] > idx[j - 1]);
    }
    EXPECT(lpt[u] >= 0 && lpt[u] < nti);
    if (lpt[u] >= 0 && lpt[u] < nti) ++used[lpt[u]];
  }
  for (int64_t u = 0; u < nti; ++u) EXPECT(used[u] == 1);

  // step lists (BN = 64) and key tiles over the plan's valid-key mask
  int bm = 0, bn = 0;
  EXPECT(pab_attention_info(PAB_FP8_TOKEN_BLOCK, 128, 2, &bm, &bn) == PAB_OK);
  int64_t n_steps = -1;
  EXPECT(pab_sta_steps(off.data(), idx.data(), (int)nti, tile_tokens, kv.data(), nt, bn, nullptr,
                       nullptr, &n_steps) == PAB_OK);
  std::vector<int32_t> soff(nti + 1), sidx(n_steps);
  EXPECT(pab_sta_steps(off.data(), idx.data(), (int)nti, tile_tokens, kv.data(), nt, bn,
                       soff.data(), sidx.data(), &n_steps) == PAB_OK);
  EXPECT(soff[nti] == n_steps);
  for (int64_t j = 0; j < n_steps; ++j) EXPECT(sidx[j] >= 0 && (int64_t)sidx[j] * bn < nt);
  int64_t n_tiles = -1;
  EXPECT(pab_key_tiles(kv.data(), nt, bn, nullptr, &n_tiles) == PAB_OK);
  std::vector<int32_t> tiles(n_tiles);
  EXPECT(pab_key_tiles(kv.data(), nt, bn, tiles.data(), &n_tiles) == PAB_OK);
  for (int64_t j = 1; j < n_tiles; ++j) EXPECT(tiles[j] > tiles[j - 1]);
}

static pab_qview view(pab_recipe r, int64_t B, int64_t H, int64_t N, int64_t d, void* codes,
                      void* scales, void* operand, int block) {
  pab_qview v;
  v.codes = codes;
  v.scales = scales;
  v.operand = operand;
  v.recipe = r;
  v.block_tokens = block;
  v.B = B;
  v.H = H;
  v.N = N;
  v.d = d;
  return v;
}

int main() {
  // size helpers on hostile sizes
  EXPECT(pab_token_alloc(0) == 0 && pab_token_alloc(-5) == 0);
  EXPECT(pab_token_alloc(1) == PAB_TOKEN_ALIGN && pab_token_alloc(129) == 2 * PAB_TOKEN_ALIGN);
  EXPECT(pab_token_alloc(kBig) < 0);
  EXPECT(pab_attention_backward_workspace(-1, 1, 1, 128) < 0);
  EXPECT(pab_attention_backward_workspace(1, 1, 1, 0) < 0);
  EXPECT(pab_attention_backward_workspace(0, 4, 100, 128) == 0);
  EXPECT(pab_attention_backward_workspace(2, 3, 700, 128) > 0);
  EXPECT(pab_attention_backward_workspace(kBig, kBig, kBig, 128) < 0);
  EXPECT(pab_attention_backward_workspace(1, 1, kBig, kBig) < 0);
  // enum arguments take their declared values only (in C++ no other value of
  // these enums can be formed without undefined behaviour)
  for (int s = 0; s <= 3; ++s) EXPECT(pab_status_str((pab_status)s) != nullptr);
  EXPECT(pab_abi_version() == PAB_ABI_VERSION);
  int bm = 0, bn = 0;
  for (int r = 0; r <= 3; ++r)
    for (int d : {0, 32, 64, 128, 256})
      for (int mode = -1; mode <= 4; ++mode) {
        pab_status s = pab_attention_info((pab_recipe)r, d, mode, &bm, &bn);
        EXPECT(s == PAB_OK || s == PAB_INVALID_ARG || s == PAB_UNSUPPORTED);
      }
  EXPECT(pab_attention_info(PAB_MXFP4_D32, 128, 0, nullptr, &bn) == PAB_INVALID_ARG);

  // the planner: padded and exact grids, windows as wide as the grid,
  // single-tile axes, and rejected shapes
  {
    const int g1[3] = {4, 16, 24}, r1[3] = {3, 15, 22}, t1[3] = {2, 8, 8}, w1[3] = {1, 3, 3};
    plan_case(g1, r1, t1, w1, PAB_OK);
    const int g2[3] = {8, 16, 16}, t2[3] = {4, 8, 8}, w2[3] = {2, 2, 2};
    plan_case(g2, g2, t2, w2, PAB_OK);
    const int w3[3] = {1, 1, 1};
    plan_case(g2, g2, t2, w3, PAB_OK);
    const int g4[3] = {2, 8, 8};
    plan_case(g4, g4, g4, w3, PAB_OK);
    const int bad_tile[3] = {3, 8, 8};
    plan_case(g2, g2, bad_tile, w3, PAB_INVALID_ARG);
    const int bad_real[3] = {9, 16, 16};
    plan_case(g2, bad_real, t2, w3, PAB_INVALID_ARG);
    const int zero_real[3] = {0, 16, 16};
    pab_status s = pab_sta_plan(g2, zero_real, t2, w3, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr);
    EXPECT(s != PAB_OK);
    const int even_win[3] = {2, 4, 3};   // radius floor(w / 2) per axis
    plan_case(g1, r1, t1, even_win, PAB_OK);
    const int neg[3] = {-4, 16, 16};
    plan_case(neg, neg, t2, w3, PAB_INVALID_ARG);
    const int huge[3] = {1 << 30, 1 << 30, 1 << 30};
    plan_case(huge, huge, t2, w3, PAB_UNSUPPORTED);
  }
  // step and key-tile lists: hostile sizes are rejected, not walked
  {
    const int32_t off[2] = {0, 1}, idx[1] = {0};
    int64_t cnt = -1;
    EXPECT(pab_sta_steps(off, idx, 1, 128, nullptr, 128, 64, nullptr, nullptr, &cnt) == PAB_OK &&
           cnt == 2);
    EXPECT(pab_sta_steps(off, idx, 1, 128, nullptr, 256, 64, nullptr, nullptr, &cnt) ==
           PAB_INVALID_ARG);
    EXPECT(pab_sta_steps(off, idx, 1, 100, nullptr, 100, 64, nullptr, nullptr, &cnt) !=
           PAB_OK);
    EXPECT(pab_sta_steps(nullptr, idx, 1, 128, nullptr, 128, 64, nullptr, nullptr, &cnt) ==
           PAB_INVALID_ARG);
    const int32_t bad_idx[1] = {3};
    EXPECT(pab_sta_steps(off, bad_idx, 1, 128, nullptr, 128, 64, nullptr, nullptr, &cnt) ==
           PAB_INVALID_ARG);
    const int32_t bad_off[2] = {0, -1};
    EXPECT(pab_sta_steps(bad_off, idx, 1, 128, nullptr, 128, 64, nullptr, nullptr, &cnt) ==
           PAB_INVALID_ARG);
    const uint8_t kv[3] = {0, 1, 0};
    EXPECT(pab_key_tiles(kv, 3, 64, nullptr, &cnt) == PAB_OK && cnt == 1);
    EXPECT(pab_key_tiles(kv, 3, 0, nullptr, &cnt) == PAB_INVALID_ARG);
    EXPECT(pab_key_tiles(kv, -3, 64, nullptr, &cnt) == PAB_INVALID_ARG);
    EXPECT(pab_key_tiles(kv, 3, 64, nullptr, nullptr) == PAB_INVALID_ARG);
  }

  // device entry points: every call below must be rejected by validation
  // (the pointers are stand-ins that are never dereferenced)
  alignas(256) static uint8_t fake[4096];
  void* p = fake;
  const int64_t shape[4] = {1, 2, 300, 128}, strides[4] = {76800, 38400, 128, 1};
  const int64_t huge_shape[4] = {kBig, kBig, kBig, 128};
  EXPECT(pab_quantize(nullptr, PAB_BF16, shape, strides, PAB_FP8_TOKEN_BLOCK, 64, nullptr, 300,
                      p, p, p, nullptr) == PAB_INVALID_ARG);
  EXPECT(pab_quantize(p, PAB_BF16, shape, strides, PAB_FP8_CHANNEL, 64, nullptr, 299, p, p,
                      nullptr, nullptr) == PAB_INVALID_ARG);
  EXPECT(rejected(pab_quantize(p, PAB_BF16, huge_shape, strides, PAB_FP8_TOKEN_BLOCK, 64,
                               nullptr, 300, p, p, p, nullptr)));
  EXPECT(rejected(pab_quantize(p, PAB_BF16, shape, strides, PAB_FP8_TOKEN_BLOCK, 64, nullptr,
                               kBig, p, p, p, nullptr)));
  EXPECT(pab_quantize(p, PAB_BF16, shape, strides, PAB_FP8_TOKEN_BLOCK, 0, nullptr, 300, p, p, p,
                      nullptr) == PAB_INVALID_ARG);
  const int64_t neg_strides[4] = {76800, 38400, -128, 1};
  EXPECT(pab_quantize(p, PAB_BF16, shape, neg_strides, PAB_FP8_TOKEN_BLOCK, 64, nullptr, 300, p,
                      p, p, nullptr) == PAB_INVALID_ARG);

  pab_qview q = view(PAB_FP8_TOKEN_BLOCK, 1, 2, 300, 128, p, p, p, 64);
  pab_qview k = q;
  pab_qview v = view(PAB_FP8_CHANNEL, 1, 2, 300, 128, p, p, nullptr, 0);
  const int64_t ostr[4] = {76800, 38400, 128, 1};
  pab_qview hq = q;
  hq.B = kBig;
  hq.H = kBig;
  pab_qview hk = hq, hv = v;
  hv.B = kBig;
  hv.H = kBig;
  EXPECT(rejected(pab_attention_dense(&hq, &hk, &hv, 0, 0.f, 0, nullptr, nullptr, 300,
                                      (float*)p, ostr, nullptr, nullptr)));
  pab_qview nq = q;
  nq.N = kBig;
  pab_qview nk = nq, nv = v;
  nv.N = kBig;
  EXPECT(rejected(pab_attention_dense(&nq, &nk, &nv, 0, 0.f, 0, nullptr, nullptr, kBig,
                                      (float*)p, ostr, nullptr, nullptr)));
  pab_qview mism = k;
  mism.N = 299;
  EXPECT(pab_attention_dense(&q, &mism, &v, 0, 0.f, 0, nullptr, nullptr, 300, (float*)p, ostr,
                             nullptr, nullptr) == PAB_INVALID_ARG);
  EXPECT(pab_attention_dense(&q, &k, &v, 0, 0.f, 0, nullptr, nullptr, 300, nullptr, ostr, nullptr,
                             nullptr) == PAB_INVALID_ARG);
  const int64_t bad_ostr[4] = {76800, 38400, 128, 2};
  EXPECT(pab_attention_dense(&q, &k, &v, 0, 0.f, 0, nullptr, nullptr, 300, (float*)p, bad_ostr,
                             nullptr, nullptr) == PAB_INVALID_ARG);
  EXPECT(pab_attention_dense(&q, &k, &v, 0, std::numeric_limits<float>::quiet_NaN(), 0, nullptr,
                             nullptr, 300, (float*)p, ostr, nullptr, nullptr) == PAB_INVALID_ARG);
  const int32_t woff[2] = {0, 1}, widx[1] = {0}, order[1] = {0};
  EXPECT(rejected(pab_attention_sta(&q, &k, &v, 0.f, 0, woff, widx, order, 1, 100, nullptr,
                                    nullptr, 300, (float*)p, ostr, nullptr, nullptr)));
  EXPECT(rejected(pab_attention_sta(&q, &k, &v, 0.f, 0, woff, widx, order, -1, 128, nullptr,
                                    nullptr, 300, (float*)p, ostr, nullptr, nullptr)));
  EXPECT(rejected(pab_attention_dense_tiles(&q, &k, &v, 0.f, 0, widx, -1, (const uint8_t*)p,
                                            nullptr, 300, (float*)p, ostr, nullptr, nullptr)));
  // backward: d = 64, a workspace that is too small, and sizes beyond the
  // allocation-free entry point's scratch array
  pab_qview q64 = view(PAB_FP8_TOKEN_BLOCK, 1, 2, 300, 64, p, p, p, 64);
  pab_qview v64 = view(PAB_FP8_CHANNEL, 1, 2, 300, 64, p, p, nullptr, 0);
  EXPECT(pab_attention_backward(&q64, &q64, &v64, 0, 0.f, nullptr, (float*)p, ostr, p, PAB_F32,
                                ostr, (float*)p, (float*)p, (float*)p, (float*)p, ostr, p, 4096,
                                nullptr) == PAB_UNSUPPORTED);
  EXPECT(pab_attention_backward(&q, &k, &v, 0, 0.f, nullptr, (float*)p, ostr, p, PAB_F32, ostr,
                                (float*)p, (float*)p, (float*)p, (float*)p, ostr, p, 16,
                                nullptr) == PAB_INVALID_ARG);
  pab_qview bq = view(PAB_FP8_TOKEN_BLOCK, 64, 64, 1 << 16, 128, p, p, p, 64);
  pab_qview bv = view(PAB_FP8_CHANNEL, 64, 64, 1 << 16, 128, p, p, nullptr, 0);
  EXPECT(rejected(pab_attention_backward_noalloc(&bq, &bq, &bv, 0, 0.f, nullptr, (float*)p, ostr,
                                                 p, PAB_F32, ostr, (float*)p, (float*)p, (float*)p,
                                                 (float*)p, ostr, nullptr)));
  EXPECT(rejected(pab_attention_sta_backward(&q, &k, &v, 0.f, woff, widx, 1, 100, nullptr,
                                             (float*)p, ostr, p, PAB_F32, ostr, (float*)p,
                                             (float*)p, (float*)p, (float*)p, ostr, p, 4096,
                                             nullptr)));
  EXPECT(pab_count_nonfinite(nullptr, 10, (int32_t*)p, nullptr) == PAB_INVALID_ARG);
  EXPECT(pab_count_nonfinite((const float*)p, -1, (int32_t*)p, nullptr) == PAB_INVALID_ARG);

  std::printf("checks passed: %d of %d\n", g_checks - g_failed, g_checks);
  return g_failed == 0 ? 0 : 1;
}
