"""Pins for the oracle's attention recipe: the online-softmax core against a
float64 brute force with the natural exponential, special cases where P's
quantisation is exact, masks, and sliding-tile windows against a token-level
mask built from 3D coordinates."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import quant as Q
from oracle import sta as S


def _ops(q, k, v, blk=64, recipe="fp8"):
    if recipe == "fp8":
        qc, qs = Q.fp8_block_quantize(q, blk)
        kc, ks = Q.fp8_block_quantize(k, blk)
        qo, ko = A.Operand("fp8_block", qc, qs, blk), A.Operand("fp8_block", kc, ks, blk)
        qh, kh = Q.fp8_block_dequantize(qc, qs, blk), Q.fp8_block_dequantize(kc, ks, blk)
    else:
        qc, qe = Q.mxfp4_quantize(q)
        kc, ke = Q.mxfp4_quantize(k)
        qo, ko = A.Operand("mxfp4", qc, qe), A.Operand("mxfp4", kc, ke)
        qh, kh = Q.mxfp4_dequantize(qc, qe), Q.mxfp4_dequantize(kc, ke)
    vc, vs = Q.fp8_channel_quantize(v)
    vo = A.Operand("fp8_channel", vc, vs)
    vh = Q.fp8_channel_dequantize(vc, vs)
    return qo, ko, vo, qh, kh, vh


def _rand(n, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal((n, d)) * scale).astype(np.float32) for _ in range(3)]


@pytest.mark.parametrize("recipe", ["fp8", "mxfp4"])
@pytest.mark.parametrize("bn", [32, 64, 128])
def test_core_equals_brute_force_on_dequantised_inputs(recipe, bn):
    q, k, v = _rand(200, 64, 10, 2.0)
    qo, ko, vo, qh, kh, vh = _ops(q, k, v, recipe=recipe)
    rows = np.arange(200)
    sm = 1 / np.sqrt(64)
    o = A.recipe_attention(qo, ko, vo, rows, sm_scale=sm, bn=bn, quantize_p=False, fp64_core=True)
    ref = A.brute_force(qh, kh, vh, sm)
    # the recipe's output is rounded to float32 at the end
    assert np.allclose(o, ref, rtol=2e-7, atol=1e-7)
    # with float32 scores and P the difference stays at float32 rounding level
    o32 = A.recipe_attention(qo, ko, vo, rows, sm_scale=sm, bn=bn, quantize_p=False)
    assert np.abs(o32 - ref).max() < 1e-5


def test_rows_sum_to_one():
    q, k, _ = _rand(130, 64, 11, 3.0)
    v = np.ones((130, 64), np.float32)
    qo, ko, vo, *_ = _ops(q, k, v)
    assert np.all(vo.scales == 448) and np.all(vo.codes == 0x7E)
    rows = np.arange(130)
    o = A.recipe_attention(qo, ko, vo, rows, sm_scale=0.125, bn=64, quantize_p=False, fp64_core=True)
    assert np.abs(o - 1).max() < 1e-6
    # with P requantised to E4M3 the weights are off by at most 2^-4 relative
    oq = A.recipe_attention(qo, ko, vo, rows, sm_scale=0.125, bn=64)
    assert np.abs(oq - 1).max() <= 2.0 ** -4


def test_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((64, 64)).astype(np.float32)
    k = np.repeat(rng.standard_normal((1, 64)).astype(np.float32), 256, axis=0)
    v = rng.standard_normal((256, 64)).astype(np.float32)
    qo, ko, vo, qh, kh, vh = _ops(q, k, v)
    o = A.recipe_attention(qo, ko, vo, np.arange(64), sm_scale=0.125, bn=64)
    assert np.allclose(o, vh.mean(axis=0)[None, :], rtol=1e-6, atol=1e-7)


def test_dominant_logit_selects_one_value_row():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((256, 64)).astype(np.float32) * 0.01
    k[77] = 8.0
    q = np.full((4, 64), 8.0, np.float32)
    v = rng.standard_normal((256, 64)).astype(np.float32)
    qo, ko, vo, qh, kh, vh = _ops(q, k, v)
    o = A.recipe_attention(qo, ko, vo, np.arange(4), sm_scale=1.0, bn=64)
    assert np.allclose(o, vh[77][None, :], rtol=1e-6, atol=0)


def test_causal_first_row_and_single_token():
    q, k, v = _rand(96, 64, 14)
    qo, ko, vo, qh, kh, vh = _ops(q, k, v, blk=32)
    o = A.recipe_attention(qo, ko, vo, np.arange(96), sm_scale=0.125, bn=32, causal=True)
    assert np.allclose(o[0], vh[0], rtol=1e-6, atol=0)
    # causal = brute force with a lower-triangular mask when P is not quantised
    o2 = A.recipe_attention(qo, ko, vo, np.arange(96), sm_scale=0.125, bn=32, causal=True,
                            quantize_p=False, fp64_core=True)
    ref = A.brute_force(qh, kh, vh, 0.125, mask=np.tril(np.ones((96, 96), bool)))
    assert np.allclose(o2, ref, rtol=2e-7, atol=1e-7)
    q1, k1, v1 = _rand(1, 64, 15)
    qo, ko, vo, qh, kh, vh = _ops(q1, k1, v1)
    o = A.recipe_attention(qo, ko, vo, np.arange(1), sm_scale=0.125, bn=64)
    assert np.allclose(o, vh, rtol=1e-6, atol=0)


def test_key_padding_mask_and_fully_masked_rows():
    q, k, v = _rand(160, 64, 16)
    qo, ko, vo, qh, kh, vh = _ops(q, k, v, blk=32)
    valid = np.ones(160, np.uint8)
    valid[[3, 50, 51, 52, 159]] = 0
    valid[64:96] = 0                    # a whole BN=32 tile masked
    o = A.recipe_attention(qo, ko, vo, np.arange(160), sm_scale=0.1, bn=32, kv_valid=valid,
                           quantize_p=False, fp64_core=True)
    ref = A.brute_force(qh, kh, vh, 0.1, mask=np.broadcast_to(valid.astype(bool), (160, 160)))
    assert np.allclose(o, ref, rtol=2e-7, atol=1e-7)
    none = np.zeros(160, np.uint8)
    o = A.recipe_attention(qo, ko, vo, np.arange(10), sm_scale=0.1, bn=32, kv_valid=none)
    assert np.all(o == 0)


def test_quantised_recipe_close_to_unquantised_attention():
    # reported, not a parity gate: the pages give no number for this error
    q, k, v = _rand(256, 64, 17)
    qo, ko, vo, *_ = _ops(q, k, v)
    o = A.recipe_attention(qo, ko, vo, np.arange(256), sm_scale=0.125, bn=64)
    ref = A.brute_force(q, k, v, 0.125)
    err = np.abs(o - ref)
    assert err.max() < 0.1 and err.mean() < 0.02


def _token_tile_coords(p, real_grid, tile, grid):
    """Tile coordinates of each kernel position, from the raster index for real
    tokens; padding tokens take the coordinates implied by their position."""
    Tr, Hr, Wr = real_grid
    coords = []
    nt, nh, nw = (g // t for g, t in zip(grid, tile))
    for pos in range(p.n_tokens):
        r = p.perm[pos]
        if r >= 0:
            t, rem = divmod(int(r), Hr * Wr)
            h, w = divmod(rem, Wr)
            coords.append((t // tile[0], h // tile[1], w // tile[2]))
        else:
            u = pos // p.tile_tokens
            coords.append((u // (nh * nw), (u // nw) % nh, u % nw))
    return np.array(coords)


@pytest.mark.parametrize("window", [(1, 1, 1), (3, 3, 3), (3, 5, 5), (9, 9, 9)])
def test_sta_equals_token_level_mask(window):
    grid, real, tile = (4, 8, 8), (3, 7, 8), (2, 4, 4)
    p = S.plan(grid, real, tile, window)
    n = p.n_tokens
    rng = np.random.default_rng(18)
    q, k, v = (rng.standard_normal((n, 32)).astype(np.float32) for _ in range(3))
    q[p.perm < 0] = 0
    k[p.perm < 0] = 0
    v[p.perm < 0] = 0
    qo, ko, vo, qh, kh, vh = _ops(q, k, v, blk=p.tile_tokens)
    tc = _token_tile_coords(p, real, tile, grid)
    rad = np.array(window) // 2
    mask = np.all(np.abs(tc[:, None, :] - tc[None, :, :]) <= rad, axis=-1)
    mask &= p.kv_valid.astype(bool)[None, :]
    ref = A.brute_force(qh, kh, vh, 0.2, mask=mask)
    out = np.zeros((n, 32), np.float32)
    for u in range(p.n_tiles):
        rows = np.arange(u * p.tile_tokens, (u + 1) * p.tile_tokens)
        out[rows] = A.recipe_attention(qo, ko, vo, rows, sm_scale=0.2, bn=16, kv_valid=p.kv_valid,
                                       key_blocks=S.key_blocks_for_tile(p, u, 16),
                                       quantize_p=False, fp64_core=True)
    real_rows = p.perm >= 0
    assert np.allclose(out[real_rows], ref[real_rows], rtol=2e-7, atol=1e-7)


def test_sta_full_window_is_dense_bitwise_and_radius_zero_is_per_tile():
    grid, tile = (4, 8, 8), (2, 4, 4)
    p_full = S.plan(grid, grid, tile, (9, 9, 9))
    p_zero = S.plan(grid, grid, tile, (1, 1, 1))
    n = p_full.n_tokens
    rng = np.random.default_rng(19)
    q, k, v = (rng.standard_normal((n, 32)).astype(np.float32) for _ in range(3))
    qo, ko, vo, *_ = _ops(q, k, v, blk=p_full.tile_tokens)
    dense = A.recipe_attention(qo, ko, vo, np.arange(n), sm_scale=0.2, bn=16)
    tt = p_full.tile_tokens
    for u in range(p_full.n_tiles):
        rows = np.arange(u * tt, (u + 1) * tt)
        sta = A.recipe_attention(qo, ko, vo, rows, sm_scale=0.2, bn=16,
                                 key_blocks=S.key_blocks_for_tile(p_full, u, 16))
        assert np.array_equal(sta, dense[rows])
        zero = A.recipe_attention(qo, ko, vo, rows, sm_scale=0.2, bn=16,
                                  key_blocks=S.key_blocks_for_tile(p_zero, u, 16))
        # the same tile attended on its own, as a separate small problem
        sub = slice(u * tt, (u + 1) * tt)
        qs = A.Operand("fp8_block", qo.codes[sub], qo.scales[u:u + 1], tt)
        ks = A.Operand("fp8_block", ko.codes[sub], ko.scales[u:u + 1], tt)
        vs = A.Operand("fp8_channel", vo.codes[sub], vo.scales)
        alone = A.recipe_attention(qs, ks, vs, np.arange(tt), sm_scale=0.2, bn=16)
        assert np.array_equal(zero, alone)


@pytest.mark.parametrize("tau", [1, 3, 8])
@pytest.mark.parametrize("recipe", ["fp8", "mxfp4"])
def test_lazy_rescale_core_equals_brute_force(recipe, tau):
    """A rescale threshold tau > 0 only delays the change of reference
    maximum, which the normaliser and the accumulator share: with P not
    quantised the online softmax still equals the brute force exactly."""
    q, k, v = _rand(160, 64, 12, 2.0)
    k = k * np.linspace(0.5, 2.5, 160, dtype=np.float32)[:, None]   # maxima keep rising
    qo, ko, vo, qh, kh, vh = _ops(q, k, v, recipe=recipe)
    sm = 1 / np.sqrt(64)
    o = A.recipe_attention(qo, ko, vo, np.arange(160), sm_scale=sm, bn=16, quantize_p=False,
                           fp64_core=True, tau=tau)
    assert np.allclose(o, A.brute_force(qh, kh, vh, sm), rtol=2e-7, atol=1e-7)


def test_lazy_rescale_worked_case():
    """Two one-key tiles with logits 0 and 1.5 (log2 units), V = identity rows.
    tau = 0 and tau = 1: the reference maximum moves to 1.5, every P~ is exact
    (448 and 224 are E4M3 values), the output is the exact softmax.
    tau = 2: the reference stays at 0, P = (1, 2^1.5), P~ = E4M3(112 P) =
    (112, 320) (316.8 rounds to 320 on the E4M3 grid), so
    O = (112, 320) / 112 / (1 + 2^1.5)."""
    d = 32
    q = np.zeros((1, d), np.float32); q[0, 0] = 1.0
    k = np.zeros((2, d), np.float32); k[1, 0] = 1.0
    v = np.zeros((2, d), np.float32); v[0, 0] = 1.0; v[1, 1] = 1.0
    qo, ko, vo, *_ = _ops(q, k, v, blk=2)
    sm = 1.5 / A.LOG2E
    w = 2.0 ** -1.5
    exact = np.array([w / (1 + w), 1 / (1 + w)])
    for tau in (0, 1):
        o = A.recipe_attention(qo, ko, vo, [0], sm_scale=sm, bn=1, tau=tau)[0]
        assert np.allclose(o[:2], exact, rtol=1e-6), tau
    o = A.recipe_attention(qo, ko, vo, [0], sm_scale=sm, bn=1, tau=2)[0]
    p1 = float(np.float32(2.0 ** 1.5))
    assert np.allclose(o[:2], np.array([112.0, 320.0]) / 112.0 / (1 + p1), rtol=1e-6)
    assert np.all(o[2:] == 0)


def test_lazy_rescale_tau_zero_is_the_default():
    q, k, v = _rand(96, 64, 13, 2.0)
    qo, ko, vo, *_ = _ops(q, k, v)
    a = A.recipe_attention(qo, ko, vo, np.arange(96), sm_scale=0.125, bn=16)
    b = A.recipe_attention(qo, ko, vo, np.arange(96), sm_scale=0.125, bn=16, tau=0)
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        A.recipe_attention(qo, ko, vo, [0], sm_scale=0.125, bn=16, tau=1.5)


def _ops_fp4v(q, k, v):
    qo, ko, _, qh, kh, _ = _ops(q, k, v, recipe="mxfp4")
    vc, ve = Q.mxfp4_token_quantize(v)
    return qo, ko, A.Operand("mxfp4_tokens", vc, ve), qh, kh, Q.mxfp4_token_dequantize(vc, ve)


def test_fp4_p_requantisation_worked_group():
    """The MX rule on P: group maximum 1.0 -> e = -2, P / 2^e = (4, 1.2, 0.2)
    rounds to the E2M1 values (4, 1, 0), so P~ = (1, 0.25, 0); a group whose
    maximum is 0.3 has e = floor(log2 0.3) - 2 = -4, 0.3 * 16 = 4.8 -> 4, P~ = 0.25."""
    p = np.zeros((1, 64), np.float32)
    p[0, :3] = [1.0, 0.3, 0.05]
    p[0, 32] = 0.3
    pq = A.mx_requantize_p(p)
    assert np.array_equal(pq[0, :3], [1.0, 0.25, 0.0])
    assert pq[0, 32] == 0.25 and np.count_nonzero(pq) == 3


def test_fp4_pv_core_equals_brute_force_on_dequantised_v():
    q, k, v = _rand(200, 128, 14, 2.0)
    qo, ko, vo, qh, kh, vh = _ops_fp4v(q, k, v)
    sm = 1 / np.sqrt(128)
    o = A.recipe_attention(qo, ko, vo, np.arange(200), sm_scale=sm, bn=64, quantize_p=False,
                           fp64_core=True)
    assert np.allclose(o, A.brute_force(qh, kh, vh, sm), rtol=2e-7, atol=1e-7)


def test_fp4_pv_exact_special_cases():
    """P~ is exact when every P is 1 (equal keys: O = mean of V^ rows) and when
    one logit dominates (P = 1 for it, the rest round to 0 within its group
    and give empty groups elsewhere: O = that V^ row)."""
    rng = np.random.default_rng(15)
    n, d = 96, 128
    q = rng.standard_normal((n, d)).astype(np.float32)
    k = np.repeat(rng.standard_normal((1, d)).astype(np.float32), n, axis=0)
    v = rng.standard_normal((n, d)).astype(np.float32)
    qo, ko, vo, _, _, vh = _ops_fp4v(q, k, v)
    o = A.recipe_attention(qo, ko, vo, np.arange(4), sm_scale=0.1, bn=64)
    assert np.allclose(o, vh.mean(axis=0)[None, :], rtol=1e-6, atol=1e-6)
    k2 = np.zeros((n, d), np.float32)
    k2[50] = q[0] * 50.0                           # a logit ~ 50 sqrt(d) above the others
    qo, ko, vo, _, _, vh = _ops_fp4v(q, k2, v)
    o = A.recipe_attention(qo, ko, vo, [0], sm_scale=1 / np.sqrt(d), bn=64)
    assert np.allclose(o[0], vh[50], rtol=1e-6, atol=1e-6)
