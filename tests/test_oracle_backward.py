"""Pins for the oracle's attention backward pass and for the forward row
statistic LSE it consumes: central finite differences of an independently
written softmax attention, torch autograd in float64, and the invariants the
softmax fixes (gradient rows of dS sum to zero, so sum_j dK_j = 0; sum_j dV_j
= sum_i dO_i), plus the degenerate cases (one key, masked keys)."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import attention as A
from oracle import backward as G
from oracle import quant as Q


def _fwd(q, k, v, sm, mask=None):
    """softmax(q k^T sm) v and log2-sum-exp rows, float64, via scipy."""
    s = (q @ k.T) * sm
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    return softmax(s, axis=1) @ v, logsumexp(s, axis=1) / np.log(2.0)


def _loss(q, k, v, do, sm, mask=None):
    return float((_fwd(q, k, v, sm, mask)[0] * do).sum())


def _tiny(n, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)) for _ in range(4)]


def test_backward_equals_central_differences():
    q, k, v, do = _tiny(6, 5, 30)
    sm = 0.7
    o, lse = _fwd(q, k, v, sm)
    dq, dk, dv = G.backward_core(q, k, v, o, do, lse, sm)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, sm)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, sm)) / (2 * h)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-8), name


def test_backward_equals_torch_autograd_with_masks():
    n, d = 40, 16
    q, k, v, do = _tiny(n, d, 31)
    valid = np.ones(n, bool)
    valid[[3, 17, 39]] = False
    mask = np.tri(n, dtype=bool) & valid[None, :]
    mask[0, 0] = True            # keep row 0 alive (its only key is key 0)
    sm = 0.25
    o, lse = _fwd(q, k, v, sm, mask)
    dq, dk, dv = G.backward_core(q, k, v, o, do, lse, sm, mask)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    s = (tq @ tk.T) * sm
    s = s.masked_fill(~torch.tensor(mask), float("-inf"))
    out = torch.softmax(s, dim=1) @ tv
    out.backward(torch.tensor(do))
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    # masked keys receive no gradient
    assert np.all(dk[~valid] == 0) and np.all(dv[~valid] == 0)


def test_backward_invariants():
    n, d = 64, 32
    q, k, v, do = _tiny(n, d, 32)
    sm = 0.3
    o, lse = _fwd(q, k, v, sm)
    dq, dk, dv = G.backward_core(q, k, v, o, do, lse, sm)
    # a shift of every key by the same vector leaves every softmax row unchanged
    assert np.abs(dk.sum(axis=0)).max() < 1e-10
    # every softmax row sums to one
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-10)
    # causal: query 0 sees only key 0, whose weight is 1 whatever q0 is
    mask = np.tri(n, dtype=bool)
    o, lse = _fwd(q, k, v, sm, mask)
    dq, dk, dv = G.backward_core(q, k, v, o, do, lse, sm, mask)
    assert np.abs(dq[0]).max() < 1e-12
    assert np.allclose(dv[n - 1], do[n - 1] * softmax(q[n - 1] @ k.T * sm)[n - 1], atol=1e-12)


def test_single_token():
    q, k, v, do = _tiny(1, 8, 33)
    o, lse = _fwd(q, k, v, 0.5)
    dq, dk, dv = G.backward_core(q, k, v, o, do, lse, 0.5)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.allclose(dv, do, atol=1e-12)


@pytest.mark.parametrize("recipe", ["fp8", "mxfp4", "mxfp4_pv"])
def test_quantised_operands_use_the_dequantised_values(recipe):
    """attention_backward on quantised Operands equals autograd of the exact
    attention over the values the quantisers' own dequantisers return, with
    the forward recipe's LSE (P unquantised, float64 core)."""
    rng = np.random.default_rng(34)
    n, d = 96, 128
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) * 1.5 for _ in range(3))
    do = rng.standard_normal((n, d))
    if recipe == "fp8":
        qc, qs = Q.fp8_block_quantize(q, 32)
        kc, ks = Q.fp8_block_quantize(k, 32)
        qo, ko = A.Operand("fp8_block", qc, qs, 32), A.Operand("fp8_block", kc, ks, 32)
        qh, kh = Q.fp8_block_dequantize(qc, qs, 32), Q.fp8_block_dequantize(kc, ks, 32)
    else:
        qc, qe = Q.mxfp4_quantize(q)
        kc, ke = Q.mxfp4_quantize(k)
        qo, ko = A.Operand("mxfp4", qc, qe), A.Operand("mxfp4", kc, ke)
        qh, kh = Q.mxfp4_dequantize(qc, qe), Q.mxfp4_dequantize(kc, ke)
    if recipe == "mxfp4_pv":
        vc, ve = Q.mxfp4_token_quantize(v)
        vo, vh = A.Operand("mxfp4_tokens", vc, ve), Q.mxfp4_token_dequantize(vc, ve)
    else:
        vc, vs = Q.fp8_channel_quantize(v)
        vo, vh = A.Operand("fp8_channel", vc, vs), Q.fp8_channel_dequantize(vc, vs)
    sm = 1 / np.sqrt(d)
    o, lse = A.recipe_attention(qo, ko, vo, np.arange(n), sm_scale=sm, bn=64, causal=True,
                                quantize_p=False, fp64_core=True, return_lse=True)
    dq, dk, dv = G.attention_backward(qo, ko, vo, o, do, lse, sm_scale=sm, causal=True)
    tq, tk, tv = (torch.tensor(np.asarray(a, np.float64), requires_grad=True) for a in (qh, kh, vh))
    s = ((tq @ tk.T) * sm).masked_fill(~torch.tensor(np.tri(n, dtype=bool)), float("-inf"))
    (torch.softmax(s, dim=1) @ tv).backward(torch.tensor(do))
    scale = max(np.abs(tq.grad.numpy()).max(), 1e-30)
    # o and lse are float32, so agreement is at float32 level
    assert np.abs(dq - tq.grad.numpy()).max() < 1e-5 * scale
    assert np.abs(dk - tk.grad.numpy()).max() < 1e-5 * max(np.abs(tk.grad.numpy()).max(), 1e-30)
    assert np.abs(dv - tv.grad.numpy()).max() < 1e-5 * max(np.abs(tv.grad.numpy()).max(), 1e-30)


@pytest.mark.parametrize("tau", [0, 3])
def test_forward_lse_is_the_log2_sum_of_exponentials(tau):
    """LSE_i = log2 sum_j 2^(S_ij) of the recipe's scores, whatever tau did to
    the reference maximum (returned in float32, so equal to float32 rounding)."""
    rng = np.random.default_rng(35)
    n, d = 150, 64
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) * 2.0 for _ in range(3))
    qc, qs = Q.fp8_block_quantize(q, 64)
    kc, ks = Q.fp8_block_quantize(k, 64)
    vc, vs = Q.fp8_channel_quantize(v)
    qo, ko = A.Operand("fp8_block", qc, qs, 64), A.Operand("fp8_block", kc, ks, 64)
    vo = A.Operand("fp8_channel", vc, vs)
    qh, kh = Q.fp8_block_dequantize(qc, qs, 64), Q.fp8_block_dequantize(kc, ks, 64)
    sm = 0.125
    mask = np.tri(n, dtype=bool)
    want = logsumexp(np.where(mask, qh.astype(np.float64) @ kh.T.astype(np.float64) * sm, -np.inf),
                     axis=1) / np.log(2.0)
    _, lse64 = A.recipe_attention(qo, ko, vo, np.arange(n), sm_scale=sm, bn=64, causal=True,
                                  fp64_core=True, tau=tau, return_lse=True)
    assert np.abs(lse64 - want).max() < 1e-5 * np.abs(want).max() + 1e-6
    _, lse32 = A.recipe_attention(qo, ko, vo, np.arange(n), sm_scale=sm, bn=64, causal=True,
                                  tau=tau, return_lse=True)
    assert np.abs(lse32 - want).max() < 1e-5
    # a row without a valid key has LSE -inf
    _, lse_m = A.recipe_attention(qo, ko, vo, np.arange(4), sm_scale=sm, bn=64,
                                  kv_valid=np.zeros(n, np.uint8), return_lse=True)
    assert np.all(np.isneginf(lse_m))


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_gradients_equal_the_full_ones(causal):
    n, d = 70, 16
    q, k, v, do = _tiny(n, d, 36)
    valid = np.ones(n, bool)
    valid[[5, 44]] = False
    mask = valid[None, :] & (np.tri(n, dtype=bool) if causal else True)
    o, lse = _fwd(q, k, v, 0.4, mask)
    full = G.backward_core(q, k, v, o, do, lse, 0.4, mask)
    rows, cols = np.array([0, 3, 44, 69]), np.array([0, 5, 17, 69])
    dq, dk, dv = G.backward_sampled(q, k, v, o, do, lse, 0.4, rows, cols, causal=causal,
                                    kv_valid=valid)
    assert np.allclose(dq, full[0][rows], rtol=1e-12, atol=1e-14)
    assert np.allclose(dk, full[1][cols], rtol=1e-12, atol=1e-14)
    assert np.allclose(dv, full[2][cols], rtol=1e-12, atol=1e-14)
