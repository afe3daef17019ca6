"""GPU parity of the forward's row statistic LSE and of the attention backward
pass against the oracle, through the C ABI.

The backward takes the forward's O and LSE as inputs; the parity test feeds
both sides the oracle's forward (computed from the same host inputs), so the
comparison sees the backward's own arithmetic only.  The forward's O and LSE
have their own parity tests.

Gate for the gradients, element by element, from the backward's arithmetic:
its products take P, dS and dO / s_V rounded to bf16 (8 significant bits:
relative error at most u = 2^-8) and sum in fp32.  To first order, with
A = |dO| |V^|^T,
    |err dQ| <= sm u (P A + |dS|) |K^|,   |err dK| <= sm u (P A + |dS|)^T |Q^|,
    |err dV| <= 2 u P^T |dO|
(P A: dP's error through dS = P (dP - D), which cancels; |dS|: dS's own
rounding; P and dO rounded for dV).  The test allows twice that plus 1e-6 of
the tensor's largest element for the fp32 sums, and a mean-abs error of at
most 1e-3 of the largest element.  A wrong index, sign or scale gives errors
of the order of the gradient, far above these bounds (u times sums of
absolute terms)."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import backward as OB
from tests.helpers import oracle_operands

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8
GRAD_MEAN = 1e-3


def _inputs(B, H, N, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    qkv = [(rng.standard_normal((B, H, N, d)) * scale).astype(np.float32) for _ in range(3)]
    for h in range(H):
        ch = rng.permutation(d)[:4]
        for t in range(2):
            qkv[t][:, h, :, ch] *= rng.lognormal(0, 1.5, 4).astype(np.float32)[:, None, None]
    ts = [torch.from_numpy(a).to(torch.bfloat16) for a in qkv]
    do = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32))
    return [t.float().numpy() for t in ts], ts, do


def _quantize(lib, dev, recipe, blk):
    if recipe == "fp8":
        q = lib.quantize(dev[0], "fp8_block", blk)
        k = lib.quantize(dev[1], "fp8_block", blk)
    else:
        q = lib.quantize(dev[0], "mxfp4")
        k = lib.quantize(dev[1], "mxfp4")
    v = lib.quantize(dev[2], "mxfp4_v" if recipe == "mxfp4_pv" else "fp8_channel")
    return q, k, v


def _oracle_lse(x, recipe, blk, causal, sm, bn, kv_valid=None, tau=0):
    q, k, v = x
    B, H, N, d = q.shape
    ops = oracle_operands(q, k, v, recipe, blk)
    o = np.zeros((B, H, N, d), np.float32)
    lse = np.zeros((B, H, N), np.float32)
    for b in range(B):
        for h in range(H):
            qo, ko, vo = ops[b][h]
            o[b, h], lse[b, h] = OA.recipe_attention(qo, ko, vo, np.arange(N), sm_scale=sm, bn=bn,
                                                     causal=causal, kv_valid=kv_valid, tau=tau,
                                                     return_lse=True)
    return ops, o, lse


def _check_lse(got, ref, what):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), what + ": rows without keys differ"
    assert np.all(got[~fin] == ref[~fin])
    err = np.abs(got[fin].astype(np.float64) - ref[fin])
    bound = 1e-4 + 1e-6 * np.abs(ref[fin])
    assert np.all(err <= bound), "%s: LSE error %.3g" % (what, err.max())


@pytest.mark.parametrize("case", [
    dict(N=1000, recipe="fp8", blk=128, causal=False, tau=0),    # ping-pong kernel
    dict(N=700, recipe="fp8", blk=64, causal=True, tau=0),       # 4-wave kernel
    dict(N=520, recipe="mxfp4", causal=False, tau=0),
    dict(N=450, recipe="mxfp4_pv", causal=True, tau=0),
    dict(N=600, recipe="fp8", blk=128, causal=False, tau=4),
    dict(N=384, recipe="mxfp4", causal=True, tau=3),
])
def test_forward_lse_parity(gpu_lib, case):
    B, H, d = 1, 2, 128
    x, ts, _ = _inputs(B, H, case["N"], d, 60)
    blk = case.get("blk", 32)
    q, k, v = _quantize(gpu_lib, [t.cuda() for t in ts], case["recipe"], blk)
    out, lse = gpu_lib.attention_dense(q, k, v, causal=case["causal"], tau=case["tau"], lse=True)
    torch.cuda.synchronize()
    mode = 1 if case["causal"] else 0
    _, bn = gpu_lib.attention_info("fp8_block" if case["recipe"] == "fp8" else "mxfp4", d, mode)
    _, _, ref = _oracle_lse(x, case["recipe"], blk, case["causal"], 1 / np.sqrt(d), bn, tau=case["tau"])
    _check_lse(lse.cpu().numpy(), ref, str(case))


def test_forward_lse_masked_rows(gpu_lib):
    """Every key masked: LSE is -inf and O is 0."""
    B, H, N, d = 1, 1, 256, 128
    _, ts, _ = _inputs(B, H, N, d, 61)
    q, k, v = _quantize(gpu_lib, [t.cuda() for t in ts], "fp8", 64)
    kvv = torch.zeros(N, dtype=torch.uint8, device="cuda")
    out, lse = gpu_lib.attention_dense(q, k, v, kv_valid=kvv, lse=True)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lse)) and torch.all(out == 0)


def _error_bounds(qo, ko, vo, o, do, lse, sm, mask):
    """First-order bounds of the backward's bf16 roundings (module docstring)."""
    qh, kh, vh = OB.dequantized(qo), OB.dequantized(ko), OB.dequantized(vo)
    s = (qh @ kh.T) * (sm * OA.LOG2E)
    ok = np.isfinite(lse)
    p = np.where(ok[:, None] & mask, np.exp2(s - np.where(ok, lse, 0.0)[:, None]), 0.0)
    dp = do @ vh.T
    ds = p * (dp - (do * o).sum(axis=1)[:, None])
    a = np.abs(do) @ np.abs(vh).T
    w = p * a + np.abs(ds)
    return (sm * U_BF16 * (w @ np.abs(kh)), sm * U_BF16 * (w.T @ np.abs(qh)),
            2 * U_BF16 * (p.T @ np.abs(do)))


def _grads_close(got, ref, bounds, what):
    for name, g, r, e in zip("qkv", got, ref, bounds):
        g = g.astype(np.float64)
        assert np.all(np.isfinite(g)), "%s d%s: non-finite" % (what, name)
        scale = np.abs(r).max()
        err = np.abs(g - r)
        lim = 2 * e + 1e-6 * scale
        worst = np.unravel_index(np.argmax(err - lim), err.shape)
        assert np.all(err <= lim), "%s d%s: error %.3g at %s over its bound %.3g (max|ref| %.3g)" % (
            what, name, err[worst], worst, lim[worst], scale)
        assert err.mean() <= GRAD_MEAN * scale, "%s d%s: mean-abs %.3g" % (what, name, err.mean())
        print("%s d%s: max err/bound %.3f, max-abs %.3g of max|ref| %.3g" % (
            what, name, (err / lim).max(), err.max(), scale))


@pytest.mark.parametrize("case", [
    dict(N=300, recipe="fp8", blk=64, causal=False, dodt=torch.float32),
    dict(N=520, recipe="fp8", blk=128, causal=True, dodt=torch.bfloat16),
    dict(N=384, recipe="mxfp4", causal=False, dodt=torch.bfloat16),
    dict(N=450, recipe="mxfp4_pv", causal=True, dodt=torch.float32),
    dict(N=200, recipe="fp8", blk=32, causal=False, dodt=torch.float32, mask=True),
    dict(N=130, recipe="mxfp4", causal=True, dodt=torch.float32, mask=True),
])
def test_backward_parity(gpu_lib, case):
    B, H, d = 1, 2, 128
    N = case["N"]
    x, ts, do = _inputs(B, H, N, d, 62)
    do = do.to(case["dodt"])
    blk = case.get("blk", 32)
    kv_valid = None
    if case.get("mask"):
        kv_valid = np.ones(N, np.uint8)
        kv_valid[np.random.default_rng(63).permutation(N)[: N // 5]] = 0
        kv_valid[0] = 1
    print("backward case", case, flush=True)
    sm = 1 / np.sqrt(d)
    mode = 1 if case["causal"] else 0
    _, bn = gpu_lib.attention_info("fp8_block" if case["recipe"] == "fp8" else "mxfp4", d, mode)
    ops, o_ref, lse_ref = _oracle_lse(x, case["recipe"], blk, case["causal"], sm, bn, kv_valid)

    q, k, v = _quantize(gpu_lib, [t.cuda() for t in ts], case["recipe"], blk)
    kvv = torch.from_numpy(kv_valid).cuda() if kv_valid is not None else None
    dq, dk, dv = gpu_lib.attention_backward(q, k, v, torch.from_numpy(o_ref).cuda(), do.cuda(),
                                            torch.from_numpy(lse_ref).cuda(), causal=case["causal"],
                                            kv_valid=kvv)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in (dq, dk, dv)]

    do_h = do.float().numpy().astype(np.float64)
    mask = np.ones((N, N), bool)
    if case["causal"]:
        mask &= np.tri(N, dtype=bool)
    if kv_valid is not None:
        mask &= kv_valid.astype(bool)[None, :]
    for b in range(B):
        for h in range(H):
            qo, ko, vo = ops[b][h]
            ref = OB.attention_backward(qo, ko, vo, o_ref[b, h], do_h[b, h], lse_ref[b, h], sm_scale=sm,
                                        causal=case["causal"], kv_valid=kv_valid)
            bounds = _error_bounds(qo, ko, vo, o_ref[b, h].astype(np.float64), do_h[b, h],
                                   lse_ref[b, h].astype(np.float64), sm, mask)
            _grads_close([g[b, h] for g in got], ref, bounds, "%s h%d" % (case, h))


def test_backward_deterministic(gpu_lib):
    B, H, N, d = 1, 2, 384, 128
    _, ts, do = _inputs(B, H, N, d, 64)
    q, k, v = _quantize(gpu_lib, [t.cuda() for t in ts], "fp8", 128)
    out, lse = gpu_lib.attention_dense(q, k, v, causal=True, lse=True)
    g1 = gpu_lib.attention_backward(q, k, v, out, do.cuda(), lse, causal=True)
    g2 = gpu_lib.attention_backward(q, k, v, out, do.cuda(), lse, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_batch_and_strided_views(gpu_lib):
    """B = 2, H = 3 with O, dO and the gradient buffers passed as [B, N, H, d]
    tensors viewed as [B, H, N, d] (token stride H*d): every (b, h) matches
    the oracle under the element-wise gate, and the gradients land in the
    caller's strided layout."""
    B, H, N, d = 2, 3, 200, 128
    x, ts, do = _inputs(B, H, N, d, 65)
    sm = 1 / np.sqrt(d)
    _, bn = gpu_lib.attention_info("fp8_block", d, 0)
    ops, o_ref, lse_ref = _oracle_lse(x, "fp8", 64, False, sm, bn)
    q, k, v = _quantize(gpu_lib, [t.cuda() for t in ts], "fp8", 64)
    o_bnhd = torch.from_numpy(np.ascontiguousarray(o_ref.transpose(0, 2, 1, 3))).cuda()
    do_bnhd = do.permute(0, 2, 1, 3).contiguous().to(torch.bfloat16).cuda()
    grads = tuple(torch.full((B, N, H, d), float("nan"), device="cuda").permute(0, 2, 1, 3)
                  for _ in range(3))
    dq, dk, dv = gpu_lib.attention_backward(q, k, v, o_bnhd.permute(0, 2, 1, 3), do_bnhd.permute(0, 2, 1, 3),
                                            torch.from_numpy(lse_ref).cuda(), grads=grads)
    torch.cuda.synchronize()
    assert dq.stride() == (N * H * d, d, H * d, 1)
    got = [t.cpu().numpy() for t in (dq, dk, dv)]
    do_h = do_bnhd.permute(0, 2, 1, 3).float().cpu().numpy().astype(np.float64)
    mask = np.ones((N, N), bool)
    for b in range(B):
        for h in range(H):
            qo, ko, vo = ops[b][h]
            ref = OB.attention_backward(qo, ko, vo, o_ref[b, h], do_h[b, h], lse_ref[b, h], sm_scale=sm)
            bounds = _error_bounds(qo, ko, vo, o_ref[b, h].astype(np.float64), do_h[b, h],
                                   lse_ref[b, h].astype(np.float64), sm, mask)
            _grads_close([g[b, h] for g in got], ref, bounds, "b%d h%d" % (b, h))


@pytest.mark.parametrize("sm", [0.02, 0.25])
def test_backward_custom_softmax_scale(gpu_lib, sm):
    """The backward with a softmax scale other than 1/sqrt(d), against the
    oracle with the same scale (forward O and LSE from the oracle)."""
    B, H, N, d = 1, 2, 330, 128
    x, ts, do = _inputs(B, H, N, d, 66)
    _, bn = gpu_lib.attention_info("fp8_block", d, 1)
    ops, o_ref, lse_ref = _oracle_lse(x, "fp8", 64, True, sm, bn)
    q, k, v = _quantize(gpu_lib, [t.cuda() for t in ts], "fp8", 64)
    dq, dk, dv = gpu_lib.attention_backward(q, k, v, torch.from_numpy(o_ref).cuda(), do.cuda(),
                                            torch.from_numpy(lse_ref).cuda(), causal=True, sm_scale=sm)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in (dq, dk, dv)]
    do_h = do.numpy().astype(np.float64)
    mask = np.tri(N, dtype=bool)
    for h in range(H):
        qo, ko, vo = ops[0][h]
        ref = OB.attention_backward(qo, ko, vo, o_ref[0, h], do_h[0, h], lse_ref[0, h], sm_scale=sm, causal=True)
        bounds = _error_bounds(qo, ko, vo, o_ref[0, h].astype(np.float64), do_h[0, h],
                               lse_ref[0, h].astype(np.float64), sm, mask)
        _grads_close([g[0, h] for g in got], ref, bounds, "sm %g h%d" % (sm, h))


@pytest.mark.parametrize("case", [
    dict(grid=(2, 32, 32), real=(2, 30, 29), tile=(2, 8, 8), H=2, recipe="fp8", blk=None),
    # (6, 8, 8) tiles of 384 tokens, as the sliding-tile workloads use: a
    # workgroup's 128 keys or queries are a third of a window tile
    dict(grid=(6, 16, 24), real=(5, 15, 22), tile=(6, 8, 8), H=1, recipe="fp8", blk=None),
    # FP8 blocks of 16 tokens: the Q and K scales vary inside a 32-token step
    dict(grid=(2, 32, 32), real=(2, 30, 29), tile=(2, 8, 8), H=1, recipe="fp8", blk=16),
    dict(grid=(6, 16, 24), real=(5, 15, 22), tile=(6, 8, 8), H=1, recipe="mxfp4", blk=None),
], ids=["fp8_tile128", "fp8_tile384", "fp8_blk16", "mxfp4_tile384"])
def test_sta_backward_parity(gpu_lib, case):
    """Backward of sliding-tile attention (pab_attention_sta_backward) on a
    padded grid with window (1, 3, 3), so a tile sees at most 9 of the others.
    Both sides take the oracle's per-tile forward (kernel token order); the
    reference is the oracle backward with the token-level mask "tile of j in
    the window of the tile of i, and key j valid", under the element-wise
    gate.  FP8 scale blocks are one tile unless the case sets blk."""
    from oracle import sta as OS
    grid, real, tile, window = case["grid"], case["real"], case["tile"], (1, 3, 3)
    hp = gpu_lib.sta_plan(grid, real, tile, window)
    dp = gpu_lib.DevicePlan(hp)
    op = OS.plan(grid, real, tile, window)
    B, H, N, d, tt = 1, case["H"], hp.n_tokens, 128, hp.tile_tokens
    recipe, blk = case["recipe"], case["blk"] or hp.tile_tokens
    x, ts, do = _inputs(B, H, N, d, 67)
    sm = 1 / np.sqrt(d)
    _, bn = gpu_lib.attention_info("mxfp4" if recipe == "mxfp4" else "fp8_block", d, 2)
    ops = oracle_operands(*x, recipe, blk)
    o_ref = np.zeros((B, H, N, d), np.float32)
    lse_ref = np.zeros((B, H, N), np.float32)
    for h in range(H):
        qo, ko, vo = ops[0][h]
        for u in range(op.n_tiles):
            rows = np.arange(u * tt, (u + 1) * tt)
            o_ref[0, h, rows], lse_ref[0, h, rows] = OA.recipe_attention(
                qo, ko, vo, rows, sm_scale=sm, bn=bn, kv_valid=op.kv_valid,
                key_blocks=OS.key_blocks_for_tile(op, u, bn), return_lse=True)
    tiles_of = np.arange(N) // tt
    see = np.zeros((op.n_tiles, op.n_tiles), bool)
    for u in range(op.n_tiles):
        see[u, op.win_idx[op.win_off[u]:op.win_off[u + 1]]] = True
    assert np.array_equal(see, see.T) and not see.all()
    mask = see[tiles_of][:, tiles_of] & op.kv_valid.astype(bool)[None, :]
    q, k, v = _quantize(gpu_lib, [t.cuda() for t in ts], recipe, blk)
    print("sta backward %s: %d tiles of %d tokens, %d pairs, N = %d" % (
        recipe, op.n_tiles, tt, int(see.sum()), N), flush=True)
    dq, dk, dv = gpu_lib.attention_sta_backward(q, k, v, dp, torch.from_numpy(o_ref).cuda(), do.cuda(),
                                                torch.from_numpy(lse_ref).cuda())
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in (dq, dk, dv)]
    do_h = do.numpy().astype(np.float64)
    for h in range(H):
        qo, ko, vo = ops[0][h]
        qh, kh, vh = OB.dequantized(qo), OB.dequantized(ko), OB.dequantized(vo)
        ref = OB.backward_core(qh, kh, vh, o_ref[0, h], do_h[0, h], lse_ref[0, h], sm, mask)
        bounds = _error_bounds(qo, ko, vo, o_ref[0, h].astype(np.float64), do_h[0, h],
                               lse_ref[0, h].astype(np.float64), sm, mask)
        _grads_close([g[0, h] for g in got], ref, bounds, "sta %s h%d" % (recipe, h))
