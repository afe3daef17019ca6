"""Attention: the staged-precision online-softmax recipe and an fp64 brute
force (test infrastructure).

Definition [FV §2.1]: Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V.
FlashAttention [FA4, FlashAttention section]: the keys are visited tile by tile
and the softmax is normalised while it is computed (online softmax), so no
N x N matrix is kept.  [FA4, co-design list: conditional softmax rescaling]
the running output is rescaled only when the running maximum crosses a
threshold.  With threshold tau = 0 (the default recipe) the reference maximum
follows every rise and a skipped rescale is a factor of exactly 1.  With
tau > 0 (log2 units, an integer) the reference maximum moves only when a row
maximum exceeds it by more than tau, so P may reach 2^tau; P is then
quantised with the scale 448 / 2^tau, which keeps it inside the E4M3 range.
[FPS §3.1] P is quantised per tensor to FP8 with the fixed scale 1/448:
P~ = E4M3(448 * P) and P ~= P~ / 448 (tau = 0).

Recipe, one query row i of one (batch, head), key tiles of BN keys visited in
ascending order (for sliding-tile attention: the tiles of the query's window
list in ascending order; causal: keys j <= i; padded keys masked):
  m = -inf, l = 0, acc = 0, rho = 448 / 2^tau
  per tile:
    S_j   = fl32( (sum_k dec(qQ_ik) dec(qK_jk)) / (s_Q(i) s_K(j)) * sm_scale * log2(e) )
            (MXFP4: the per-32 scales 2^(eQ+eK) sit inside the sum);
            masked keys get S_j = -inf; a tile without a valid key is skipped
    c     = max(m, max_j S_j)
    m'    = c if c > fl32(m + tau) else m   (tau = 0: m' = c)
    alpha = 2^(m - m')  (1 when m' == m)
    P_j   = fl32(2^(S_j - m'))                      (so 0 <= P_j <= 2^tau)
    l     = alpha l + sum_j P_j                      (P before quantisation)
    P~_j  = E4M3(fl32(rho P_j))
    acc_c = alpha acc_c + sum_j dec(P~_j) dec(qV_jc) (float64)
    m     = m'
  O_ic = fl32(acc_c / l / rho / s_V(c)); a row with no valid key gives 0.
(The comparison c > m + tau decides whether the reference moves; it is made
in float32, as in the kernel.)

FP4 P.V [FV §1, FP4 attention; FP4G §1, MX micro-scaling]: with V in MXFP4
along tokens (kind 'mxfp4_tokens'), P is requantised to MXFP4 as well, per
query row and per group of 32 consecutive keys of the tile, by the same MX
rule as Q and K:
    e_g   = clamp(floor(log2 max_{j in g} P_j) - 2, -127, 127)  (-127 if all 0)
    P~_j  = E2M1(fl32(P_j 2^-e_g)) 2^e_g
    acc_c = alpha acc_c + sum_j P~_j V^_jc, V^ = E2M1 code * 2^e_V
    O_ic  = fl32(acc_c / l)   (the scales are inside P~ and V^)
The products of decoded FP8 codes are exact in float64 and so are their sums
at these lengths, so a float64 matrix product serves as the exact sum.
"""
import numpy as np

from .formats import e4m3_decode, e4m3_encode, e2m1_decode, e2m1_encode, f32_unbiased_exponent

LOG2E = 1.4426950408889634


class Operand:
    """One quantised (batch, head) operand in the kernel's token order.

    kind 'fp8_block':   codes [N, d] uint8 E4M3, scales [ceil(N/blk)] float32
    kind 'mxfp4':       codes [N, d] uint8 4-bit E2M1, scales [N, d/32] uint8 E8M0
    kind 'fp8_channel': codes [N, d] uint8 E4M3, scales [d] float32
    kind 'mxfp4_tokens' (V for FP4 P.V): codes [N, d] uint8 4-bit E2M1,
                        scales [N/32, d] uint8 E8M0 (per channel, 32 tokens)
    """

    def __init__(self, kind, codes, scales, blk=None):
        self.kind, self.codes, self.scales, self.blk = kind, codes, scales, blk


def _decoded(op, rows):
    """Decoded values (float64) of the given token rows, and the per-row
    divisor (float64, 1 for MXFP4 whose scales are applied inside)."""
    if op.kind == "fp8_block":
        vals = e4m3_decode(op.codes[rows])
        div = op.scales[rows // op.blk].astype(np.float64)
        return vals, div
    if op.kind == "mxfp4":
        vals = e2m1_decode(op.codes[rows])
        d = vals.shape[-1]
        sc = np.ldexp(1.0, op.scales[rows].astype(np.int64) - 127)
        vals = (vals.reshape(len(rows), d // 32, 32) * sc[..., None]).reshape(len(rows), d)
        return vals, np.ones(len(rows))
    raise ValueError(op.kind)


def _v_decoded(v, cols):
    """V values (float64) of the given token rows; for FP8 V without the
    per-channel scale (the recipe divides by it at the end)."""
    if v.kind == "mxfp4_tokens":
        sc = np.ldexp(1.0, v.scales[cols // 32].astype(np.int64) - 127)
        return e2m1_decode(v.codes[cols]) * sc
    return e4m3_decode(v.codes[cols])


def mx_requantize_p(p):
    """MXFP4 requantisation of P (rows x keys, float32, keys in groups of 32
    from the first column): the MX rule per row and group; returns the
    dequantised values P~ (float64)."""
    p = np.asarray(p, dtype=np.float32)
    out = np.zeros(p.shape)
    for g0 in range(0, p.shape[1], 32):
        pg = p[:, g0:g0 + 32]
        amax = pg.max(axis=1)
        e = np.clip(f32_unbiased_exponent(np.where(amax > 0, amax, 1.0)) - 2, -127, 127)
        e = np.where(amax > 0, e, -127)
        scaled = (pg.astype(np.float64) * np.ldexp(1.0, -e)[:, None]).astype(np.float32)
        out[:, g0:g0 + 32] = e2m1_decode(e2m1_encode(scaled)) * np.ldexp(1.0, e)[:, None]
    return out


def scores(q, k, qrows, kcols, sm_scale, fp64_core=False):
    """S' for the given query rows x key columns (log2 domain), float32
    (float64 when fp64_core)."""
    qv, qdiv = _decoded(q, qrows)
    kv, kdiv = _decoded(k, kcols)
    s = (qv @ kv.T) / (qdiv[:, None] * kdiv[None, :]) * (sm_scale * LOG2E)
    return s if fp64_core else s.astype(np.float32)


def recipe_attention(q, k, v, rows, *, sm_scale, bn, causal=False, kv_valid=None,
                     key_blocks=None, quantize_p=True, fp64_core=False, tau=0, return_lse=False):
    """Output rows O[rows, :] (float32) of one (batch, head).

    return_lse: also return the row statistic LSE_i = m_i + log2(l_i)
    (float32, log2 units of S; -inf for a row without a valid key), which
    gives the softmax row as P_ij = 2^(S_ij - LSE_i) for the backward pass.

    key_blocks: None (all BN-key tiles 0..ceil(N/BN)-1) or an ascending list of
    key-tile start indices shared by every row in `rows`.
    tau: rescale threshold (integer, log2 units; 0 = the eager recipe).
    quantize_p=False / fp64_core=True switch parts of the recipe off so that
    tests can pin the online-softmax core against the brute force.
    """
    if int(tau) != tau or tau < 0:
        raise ValueError("tau must be a non-negative integer")
    fp4_pv = v.kind == "mxfp4_tokens"
    if fp4_pv and bn % 32:
        raise ValueError("FP4 P.V needs key tiles of whole 32-key groups")
    p_scale = 1.0 if fp4_pv else 448.0 * 2.0 ** -int(tau)
    rows = np.asarray(rows, dtype=np.int64)
    n, d = k.codes.shape
    r = len(rows)
    ftype = np.float64 if fp64_core else np.float32
    m = np.full(r, -np.inf, dtype=ftype)
    l = np.zeros(r)
    acc = np.zeros((r, d))
    if key_blocks is None:
        key_blocks = range(0, n, bn)
    for t0 in key_blocks:
        cols = np.arange(t0, min(n, t0 + bn))
        s = scores(q, k, rows, cols, sm_scale, fp64_core)
        valid = np.ones((r, len(cols)), dtype=bool)
        if kv_valid is not None:
            valid &= kv_valid[cols][None, :].astype(bool)
        if causal:
            valid &= cols[None, :] <= rows[:, None]
        s = np.where(valid, s, -np.inf).astype(ftype)
        tmax = s.max(axis=1)
        has = valid.any(axis=1)
        cand = np.where(has, np.maximum(m, tmax), m).astype(ftype)
        moves = cand > (m + ftype(tau)).astype(ftype)     # -inf + tau stays -inf
        m_new = np.where(moves, cand, m).astype(ftype)
        with np.errstate(invalid="ignore"):
            alpha = np.where(m_new == m, 1.0,
                             np.exp2(m.astype(np.float64) - m_new.astype(np.float64)))
            p = np.exp2(s.astype(np.float64) - m_new.astype(np.float64)[:, None])
        p = np.where(valid, p, 0.0)
        if not fp64_core:
            p = p.astype(np.float32)
        l = alpha * l + p.astype(np.float64).sum(axis=1)
        if not quantize_p:
            pq = p_scale * p.astype(np.float64)
        elif fp4_pv:
            pq = mx_requantize_p(p)
        else:
            pq = e4m3_decode(e4m3_encode(np.float32(p_scale) * p.astype(np.float32)))
        acc = alpha[:, None] * acc + pq @ _v_decoded(v, cols)
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        if fp4_pv:
            o = acc / l[:, None]
        else:
            o = acc / l[:, None] / p_scale / v.scales.astype(np.float64)[None, :]
    o = np.where((l > 0)[:, None], o, 0.0)
    if return_lse:
        with np.errstate(divide="ignore", invalid="ignore"):
            lse = np.where(l > 0, m.astype(np.float64) + np.log2(l), -np.inf)
        return o.astype(np.float32), lse.astype(np.float32)
    return o.astype(np.float32)


def brute_force(q, k, v, sm_scale, mask=None):
    """softmax(q k^T * sm_scale) v in float64 with the natural exponential;
    mask[i, j] False removes key j for query i; a fully masked row gives 0."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s = (q @ k.T) * sm_scale
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    ok = np.isfinite(mx[:, 0])
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.exp(s - mx)
    den = e.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (e @ v) / den
    return np.where(ok[:, None], o, 0.0)
