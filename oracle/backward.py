"""Attention backward pass (test infrastructure: only the tests, the smoke
check and the CPU baseline of the benchmark may use this module).

Sources: "FA4极速LLM：10分钟搞定20倍内存直降！", FA4 co-design list (the
backward pass and its intermediates S, P, dP, dS, dQ); FPSAttention page
("FP8量化与稀疏性协同加速视频扩散模型"), introduction: the FP8 quantisation is
training-aware, so gradients flow through the quantised attention.

Reading.  The pages define no gradient for the quantisers, so the plainest
one is taken: quantisation passes gradients straight through.  The gradient
is that of O = softmax(S) V^ with S = Q^ K^T * sm_scale over the
dequantised operands Q^, K^, V^ the forward pass used, evaluated with the
forward's row statistic LSE (log2 units, P_ij = 2^(S_ij log2(e) - LSE_i))
and the forward's output O:
    P   = 2^(S log2(e) - LSE)           (0 for masked keys)
    dV^ = P^T dO
    dP  = dO V^^T
    D_i = sum_c dO_ic O_ic
    dS  = P * (dP - D)
    dQ^ = sm_scale dS K^
    dK^ = sm_scale dS^T Q^
With an exact forward (O = P V^, LSE = log2 sum_j 2^(S_ij log2 e)) these are
the exact derivatives of sum(dO * O); the recipe's forward differs from that
only by its rounding.  Everything here is float64.
"""
import numpy as np

from .attention import LOG2E, _decoded, _v_decoded


def dequantized(op):
    """All token rows of a quantised operand as float64 values (the scales
    applied): Q^ / K^ for 'fp8_block' and 'mxfp4', V^ for 'fp8_channel' and
    'mxfp4_tokens'."""
    n = op.codes.shape[0]
    rows = np.arange(n)
    if op.kind in ("fp8_block", "mxfp4"):
        vals, div = _decoded(op, rows)
        return vals / div[:, None]
    vals = _v_decoded(op, rows)
    if op.kind == "fp8_channel":
        vals = vals / op.scales.astype(np.float64)[None, :]
    return vals


def backward_core(qh, kh, vh, o, do, lse, sm_scale, mask=None):
    """(dQ, dK, dV) in float64 from dequantised operands [N, d], the forward
    output o [Nq, d], the upstream gradient do [Nq, d] and lse [Nq] (log2
    units); mask[i, j] False removes key j for query i."""
    qh, kh, vh, o, do = (np.asarray(a, dtype=np.float64) for a in (qh, kh, vh, o, do))
    lse = np.asarray(lse, dtype=np.float64)
    s = (qh @ kh.T) * (sm_scale * LOG2E)
    ok = np.isfinite(lse)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.exp2(s - np.where(ok, lse, 0.0)[:, None])
    p = np.where(ok[:, None], p, 0.0)
    if mask is not None:
        p = np.where(mask, p, 0.0)
    dv = p.T @ do
    dp = do @ vh.T
    dd = (do * o).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = sm_scale * (ds @ kh)
    dk = sm_scale * (ds.T @ qh)
    return dq, dk, dv


def attention_backward(q, k, v, o, do, lse, *, sm_scale, causal=False, kv_valid=None):
    """Gradients with respect to the dequantised Q^, K^, V^ of one (batch,
    head) (Operand objects of attention.py), all N token rows."""
    qh, kh, vh = dequantized(q), dequantized(k), dequantized(v)
    n = qh.shape[0]
    mask = np.ones((n, n), dtype=bool)
    if causal:
        mask &= np.tri(n, dtype=bool)
    if kv_valid is not None:
        mask &= np.asarray(kv_valid, dtype=bool)[None, :]
    return backward_core(qh, kh, vh, o, do, lse, sm_scale, mask)


def backward_sampled(qh, kh, vh, o, do, lse, sm_scale, rows, cols, causal=False, kv_valid=None):
    """The same gradients evaluated only where they are sampled: dQ for the
    query rows `rows` and dK, dV for the keys `cols` (float64), from
    dequantised operands [N, d], the forward output o and lse of every row
    and the upstream gradient do [N, d].  Each sampled row (key) uses all keys
    (queries), so the cost is linear in N per sample."""
    qh, kh, vh, o, do = (np.asarray(a, dtype=np.float64) for a in (qh, kh, vh, o, do))
    lse = np.asarray(lse, dtype=np.float64)
    rows, cols = np.asarray(rows, np.int64), np.asarray(cols, np.int64)
    n = qh.shape[0]
    kvalid = np.ones(n, bool) if kv_valid is None else np.asarray(kv_valid, bool)
    ok = np.isfinite(lse)
    dd = (do * o).sum(axis=1)

    def probs(s, ri, ci):
        m = ok[ri][:, None] & kvalid[ci][None, :]
        if causal:
            m &= ci[None, :] <= ri[:, None]
        with np.errstate(invalid="ignore", over="ignore"):
            p = np.exp2(s - np.where(ok[ri], lse[ri], 0.0)[:, None])
        return np.where(m, p, 0.0)

    allq = np.arange(n)
    # rows: dQ_i = sm sum_j P_ij (dP_ij - D_i) K^_j
    p = probs((qh[rows] @ kh.T) * (sm_scale * LOG2E), rows, allq)
    ds = p * (do[rows] @ vh.T - dd[rows][:, None])
    dq = sm_scale * (ds @ kh)
    # keys: dK_j = sm sum_i dS_ij Q^_i, dV_j = sum_i P_ij dO_i
    p = probs((qh @ kh[cols].T) * (sm_scale * LOG2E), allq, cols)
    ds = p * (do @ vh[cols].T - dd[:, None])
    dk = sm_scale * (ds.T @ qh)
    dv = p.T @ do
    return dq, dk, dv
