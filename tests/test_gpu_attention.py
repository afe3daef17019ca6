"""GPU parity of the fused attention kernel against the oracle recipe at the
kernel's KV tile size, through the C ABI: small shapes spanning several tiles
and ragged tails, causal, MXFP4, key padding, output permutation and
sliding-tile windows."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import sta as OS
from tests.helpers import assert_close, oracle_operands

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, seed, dtype=torch.bfloat16, outliers=True, scale=1.0):
    rng = np.random.default_rng(seed)
    qkv = [(rng.standard_normal((B, H, N, d)) * scale).astype(np.float32) for _ in range(3)]
    if outliers:
        for h in range(H):
            ch = rng.permutation(d)[:4]
            for t in range(2):
                qkv[t][:, h, :, ch] *= rng.lognormal(0, 1.5, 4).astype(np.float32)[:, None, None]
    ts = [torch.from_numpy(a).to(dtype) for a in qkv]
    return [t.float().numpy() for t in ts], ts


def _run_dense(lib, ts, recipe, blk, causal, sm_scale=None, kv_valid=None, tau=0):
    dev = [t.cuda() for t in ts]
    if recipe == "fp8":
        q = lib.quantize(dev[0], "fp8_block", blk)
        k = lib.quantize(dev[1], "fp8_block", blk)
    else:
        q = lib.quantize(dev[0], "mxfp4")
        k = lib.quantize(dev[1], "mxfp4")
    v = lib.quantize(dev[2], "fp8_channel")
    kvv = torch.from_numpy(kv_valid).cuda() if kv_valid is not None else None
    out = lib.attention_dense(q, k, v, causal=causal, sm_scale=sm_scale, kv_valid=kvv, tau=tau)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle_dense(x, recipe, blk, causal, sm_scale, bn, kv_valid=None, rows=None, tau=0):
    q, k, v = x
    B, H, N, d = q.shape
    ops = oracle_operands(q, k, v, recipe, blk)
    out = np.zeros((B, H, N, d), np.float32)
    rows = np.arange(N) if rows is None else rows
    for b in range(B):
        for h in range(H):
            qo, ko, vo = ops[b][h]
            out[b, h, rows] = OA.recipe_attention(qo, ko, vo, rows, sm_scale=sm_scale, bn=bn,
                                                  causal=causal, kv_valid=kv_valid, tau=tau)
    return out


@pytest.mark.parametrize("case", [
    dict(B=1, H=2, N=256, d=64, recipe="fp8", blk=64, causal=False, dtype=torch.float32, outl=False),
    dict(B=1, H=2, N=1000, d=128, recipe="fp8", blk=128, causal=False, dtype=torch.bfloat16, outl=True),
    dict(B=2, H=1, N=700, d=128, recipe="fp8", blk=128, causal=True, dtype=torch.bfloat16, outl=True),
    dict(B=1, H=2, N=520, d=128, recipe="mxfp4", blk=None, causal=False, dtype=torch.bfloat16, outl=True),
    dict(B=1, H=1, N=300, d=64, recipe="fp8", blk=32, causal=True, dtype=torch.float32, outl=False),
    dict(B=1, H=2, N=384, d=128, recipe="fp8", blk=384, causal=False, dtype=torch.bfloat16, outl=True),
], ids=["tiny_d64", "ragged_d128", "causal", "mxfp4", "causal_blk32_d64", "blk384"])
def test_dense_parity(gpu_lib, case):
    print("dense parity", case, flush=True)
    x, ts = _inputs(case["B"], case["H"], case["N"], case["d"], 31 + case["N"], case["dtype"],
                    case["outl"])
    bm, bn = gpu_lib.attention_info("mxfp4" if case["recipe"] == "mxfp4" else "fp8_block",
                                    case["d"], 1 if case["causal"] else 0)
    sm = 1 / np.sqrt(case["d"])
    got = _run_dense(gpu_lib, ts, case["recipe"], case["blk"], case["causal"])
    ref = _oracle_dense(x, case["recipe"], case["blk"], case["causal"], sm, bn)
    mx, mean = assert_close(got, ref, str(case))
    print("  max-abs %.3g mean-abs %.3g" % (mx, mean))


@pytest.mark.parametrize("N", [1, 33, 65, 129, 257])
@pytest.mark.parametrize("recipe,d,causal", [("fp8", 128, False), ("fp8", 128, True), ("fp8", 64, False),
                                             ("mxfp4", 128, False), ("mxfp4", 128, True)])
def test_short_sequences(gpu_lib, N, recipe, d, causal):
    """Token counts of one, and just past a key step or a query tile: the
    last tile's rows past N are neither computed into nor stored (every
    output element is written, none past the tensor)."""
    print("short", N, recipe, d, causal, flush=True)
    x, ts = _inputs(1, 2, N, d, 700 + N, torch.bfloat16, True)
    _, bn = gpu_lib.attention_info("mxfp4" if recipe == "mxfp4" else "fp8_block", d, 1 if causal else 0)
    blk = 64 if recipe == "fp8" else None
    dev = [t.cuda() for t in ts]
    qr = "fp8_block" if recipe == "fp8" else "mxfp4"
    q, k = (gpu_lib.quantize(t, qr, blk) for t in dev[:2])
    v = gpu_lib.quantize(dev[2], "fp8_channel")
    out = torch.full((1, 2, N, d), float("nan"), device="cuda")
    gpu_lib.attention_dense(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.isnan(got).any()
    ref = _oracle_dense(x, recipe, blk, causal, 1 / np.sqrt(d), bn)
    assert_close(got, ref, "short N=%d %s d=%d causal=%s" % (N, recipe, d, causal))


@pytest.mark.parametrize("tau", [2, 8])
@pytest.mark.parametrize("case", [
    dict(recipe="fp8", d=128, N=1000, causal=False, blk=128),
    dict(recipe="mxfp4", d=128, N=1000, causal=False, blk=None),
    dict(recipe="fp8", d=128, N=700, causal=True, blk=128),
    dict(recipe="fp8", d=64, N=520, causal=False, blk=64),
], ids=["fp8_dense", "mxfp4_dense", "fp8_causal", "fp8_d64"])
def test_rescale_threshold_parity(gpu_lib, case, tau):
    """Softmax rescale threshold tau > 0 against the oracle with the same tau.
    Key magnitudes ramp up along the sequence, so row maxima keep rising by
    amounts on both sides of tau."""
    print("rescale threshold", tau, case, flush=True)
    N, d = case["N"], case["d"]
    x, _ = _inputs(1, 2, N, d, 60 + N, torch.float32, True)
    x[1] = x[1] * np.linspace(0.3, 3.0, N, dtype=np.float32)[None, None, :, None]
    ts = [torch.from_numpy(a).to(torch.bfloat16) for a in x]
    x = [t.float().numpy() for t in ts]
    _, bn = gpu_lib.attention_info("mxfp4" if case["recipe"] == "mxfp4" else "fp8_block", d,
                                   1 if case["causal"] else 0)
    got = _run_dense(gpu_lib, ts, case["recipe"], case["blk"], case["causal"], tau=tau)
    ref = _oracle_dense(x, case["recipe"], case["blk"], case["causal"], 1 / np.sqrt(d), bn, tau=tau)
    mx, mean = assert_close(got, ref, "tau %d %s" % (tau, case))
    print("  max-abs %.3g mean-abs %.3g" % (mx, mean))
    eager = _run_dense(gpu_lib, ts, case["recipe"], case["blk"], case["causal"], tau=0)
    assert not np.array_equal(got, eager), "tau had no effect"


def test_key_padding_mask(gpu_lib):
    x, ts = _inputs(1, 2, 600, 128, 5, torch.bfloat16, True)
    valid = np.ones(600, np.uint8)
    valid[[0, 1, 130, 131, 599]] = 0
    valid[256:384] = 0                       # one whole key tile masked
    got = _run_dense(gpu_lib, ts, "fp8", 128, False, kv_valid=valid)
    _, bn = gpu_lib.attention_info("fp8_block", 128, 0)
    ref = _oracle_dense(x, "fp8", 128, False, 1 / np.sqrt(128), bn, kv_valid=valid)
    assert_close(got, ref, "kv_valid")


def test_deterministic(gpu_lib):
    _, ts = _inputs(1, 2, 900, 128, 6, torch.bfloat16, True)
    a = _run_dense(gpu_lib, ts, "fp8", 128, False)
    for _ in range(3):
        assert np.array_equal(a, _run_dense(gpu_lib, ts, "fp8", 128, False))


def _sta_setup(lib, grid, real, tile, window, H=2, seed=40, outl=True):
    hp = lib.sta_plan(grid, real, tile, window)
    op = OS.plan(grid, real, tile, window)
    assert np.array_equal(hp.perm, op.perm) and np.array_equal(hp.win_idx, op.win_idx)
    n_real = int(np.prod(real))
    x, ts = _inputs(1, H, n_real, 128, seed, torch.bfloat16, outl)
    return hp, op, x, ts


def _run_sta(lib, hp, ts, window_plan=None, dense=False, tau=0, steps=False):
    dp = lib.DevicePlan(hp if window_plan is None else window_plan)
    dev = [t.cuda() for t in ts]
    q = lib.quantize(dev[0], "fp8_block", hp.tile_tokens, perm=dp.perm, n_out=dp.n_tokens)
    k = lib.quantize(dev[1], "fp8_block", hp.tile_tokens, perm=dp.perm, n_out=dp.n_tokens)
    v = lib.quantize(dev[2], "fp8_channel", perm=dp.perm, n_out=dp.n_tokens)
    if dense:
        out = lib.attention_dense(q, k, v, kv_valid=dp.kv_valid, out_perm=dp.perm, n_out=dp.n_real,
                                  tau=tau)
    else:
        out = lib.attention_sta(q, k, v, dp, tau=tau, steps=steps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("window,tau", [((3, 3, 3), 0), ((1, 3, 5), 0), ((3, 3, 3), 4)])
def test_sta_parity_with_padding(gpu_lib, window, tau):
    grid, real, tile = (6, 16, 32), (5, 15, 30), (2, 8, 8)
    hp, op, x, ts = _sta_setup(gpu_lib, grid, real, tile, window)
    got = _run_sta(gpu_lib, hp, ts, tau=tau)
    _, bn = gpu_lib.attention_info("fp8_block", 128, 2)
    xk = [OS.gather_tokens(a, op.perm) for a in x]
    ops = oracle_operands(*xk, "fp8", op.tile_tokens)
    ref = np.zeros_like(got)
    tt = op.tile_tokens
    for h in range(2):
        qo, ko, vo = ops[0][h]
        for u in range(op.n_tiles):
            rows = np.arange(u * tt, (u + 1) * tt)
            o = OA.recipe_attention(qo, ko, vo, rows, sm_scale=1 / np.sqrt(128), bn=bn,
                                    kv_valid=op.kv_valid,
                                    key_blocks=OS.key_blocks_for_tile(op, u, bn), tau=tau)
            keep = op.perm[rows] >= 0
            ref[0, h, op.perm[rows][keep]] = o[keep]
    assert_close(got, ref, "sta %s" % (window,))
    # window lists in BN-key steps without the padding steps: the same bits
    # (the last frame of every tile in the last tile row is padding here)
    assert np.array_equal(_run_sta(gpu_lib, hp, ts, tau=tau, steps=True), got)


@pytest.mark.parametrize("steps", [False, True])
def test_sta_head_dim_64(gpu_lib, steps):
    """Sliding-tile FP8 attention with d = 64 on a padded grid (the 4-wave
    kernel's d = 64 instance), window lists in tiles and in key steps."""
    grid, real, tile, window = (4, 16, 16), (3, 14, 16), (2, 8, 8), (1, 3, 3)
    hp = gpu_lib.sta_plan(grid, real, tile, window)
    op = OS.plan(grid, real, tile, window)
    dp = gpu_lib.DevicePlan(hp)
    n_real = int(np.prod(real))
    x, ts = _inputs(1, 2, n_real, 64, 45, torch.bfloat16, True)
    dev = [t.cuda() for t in ts]
    q = gpu_lib.quantize(dev[0], "fp8_block", hp.tile_tokens, perm=dp.perm, n_out=dp.n_tokens)
    k = gpu_lib.quantize(dev[1], "fp8_block", hp.tile_tokens, perm=dp.perm, n_out=dp.n_tokens)
    v = gpu_lib.quantize(dev[2], "fp8_channel", perm=dp.perm, n_out=dp.n_tokens)
    got = gpu_lib.attention_sta(q, k, v, dp, steps=steps)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    _, bn = gpu_lib.attention_info("fp8_block", 64, 2)
    xk = [OS.gather_tokens(a, op.perm) for a in x]
    ops = oracle_operands(*xk, "fp8", op.tile_tokens)
    ref = np.full_like(got, np.nan)
    tt = op.tile_tokens
    for h in range(2):
        qo, ko, vo = ops[0][h]
        for u in range(op.n_tiles):
            rows = np.arange(u * tt, (u + 1) * tt)
            keep = op.perm[rows] >= 0
            if not keep.any():
                continue
            o = OA.recipe_attention(qo, ko, vo, rows[keep], sm_scale=1 / np.sqrt(64), bn=bn,
                                    kv_valid=op.kv_valid, key_blocks=OS.key_blocks_for_tile(op, u, bn))
            ref[0, h, op.perm[rows][keep]] = o
    assert_close(got, ref, "sta d=64 steps=%s" % steps)


@pytest.mark.parametrize("recipe", ["fp8", "mxfp4"])
def test_sta_batch_of_two(gpu_lib, recipe):
    """Sliding-tile attention with B = 2 on a padded grid: every (b, h) slice
    matches the oracle, in the caller's token order and through strided output
    (the kernel's batch and head offsets of inputs, outputs and the row
    statistic)."""
    grid, real, tile, window = (4, 16, 16), (3, 15, 13), (2, 8, 8), (1, 3, 3)
    hp = gpu_lib.sta_plan(grid, real, tile, window)
    op = OS.plan(grid, real, tile, window)
    dp = gpu_lib.DevicePlan(hp)
    n_real = int(np.prod(real))
    B, H = 2, 2
    x, ts = _inputs(B, H, n_real, 128, 44, torch.bfloat16, True)
    dev = [t.cuda() for t in ts]
    blk = hp.tile_tokens if recipe == "fp8" else None
    qr = "fp8_block" if recipe == "fp8" else "mxfp4"
    q = gpu_lib.quantize(dev[0], qr, blk, perm=dp.perm, n_out=dp.n_tokens, operand=False)
    k = gpu_lib.quantize(dev[1], qr, blk, perm=dp.perm, n_out=dp.n_tokens)
    v = gpu_lib.quantize(dev[2], "fp8_channel", perm=dp.perm, n_out=dp.n_tokens)
    buf = torch.full((B, n_real, H, 128), float("nan"), device="cuda")
    got = gpu_lib.attention_sta(q, k, v, dp, out=buf.permute(0, 2, 1, 3), steps=True)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    _, bn = gpu_lib.attention_info(qr, 128, 2)
    xk = [OS.gather_tokens(a, op.perm) for a in x]
    ops = oracle_operands(*xk, recipe, op.tile_tokens)
    ref = np.full_like(got, np.nan)
    tt = op.tile_tokens
    for b in range(B):
        for h in range(H):
            qo, ko, vo = ops[b][h]
            for u in range(op.n_tiles):
                rows = np.arange(u * tt, (u + 1) * tt)
                keep = op.perm[rows] >= 0
                if not keep.any():
                    continue
                o = OA.recipe_attention(qo, ko, vo, rows[keep], sm_scale=1 / np.sqrt(128), bn=bn,
                                        kv_valid=op.kv_valid, key_blocks=OS.key_blocks_for_tile(op, u, bn))
                ref[b, h, op.perm[rows][keep]] = o
    assert not np.isnan(got).any()
    assert_close(got, ref, "sta B=2 %s" % recipe)


@pytest.mark.parametrize("grid,real,tile,window", [
    ((8, 16, 24), (7, 15, 22), (4, 8, 8), (3, 3, 3)),          # 256-token tiles
    ((6, 32, 32), (5, 30, 31), (6, 16, 16), (1, 3, 3)),        # 1536-token tiles
])
def test_sta_tile_variants(gpu_lib, grid, real, tile, window):
    """Other tile shapes of the sliding-tile schedule (the FPSAttention page,
    tile-size ablation): per-tile FP8 scales over 256 and 1536 tokens, padded
    grids; 96 sampled query rows per tile (first, last and seeded ones)."""
    hp, op, x, ts = _sta_setup(gpu_lib, grid, real, tile, window, seed=43)
    got = _run_sta(gpu_lib, hp, ts)
    _, bn = gpu_lib.attention_info("fp8_block", 128, 2)
    xk = [OS.gather_tokens(a, op.perm) for a in x]
    ops = oracle_operands(*xk, "fp8", op.tile_tokens)
    tt = op.tile_tokens
    rng = np.random.default_rng(7)
    checked = 0
    for h in range(2):
        qo, ko, vo = ops[0][h]
        for u in range(op.n_tiles):
            rows = np.unique(np.concatenate([[0, tt - 1], rng.choice(tt, 94, replace=False)])) + u * tt
            rows = rows[op.perm[rows] >= 0]
            if rows.size == 0:
                continue
            o = OA.recipe_attention(qo, ko, vo, rows, sm_scale=1 / np.sqrt(128), bn=bn,
                                    kv_valid=op.kv_valid,
                                    key_blocks=OS.key_blocks_for_tile(op, u, bn))
            assert_close(got[0, h, op.perm[rows]], o, "sta tile %s head %d tile %d" % (tile, h, u))
            checked += rows.size
    assert checked > 0


def test_sta_full_window_equals_dense_bitwise(gpu_lib):
    grid, real, tile = (4, 16, 16), (4, 13, 16), (2, 8, 8)
    hp, op, x, ts = _sta_setup(gpu_lib, grid, real, tile, (9, 9, 9), seed=41)
    sta = _run_sta(gpu_lib, hp, ts)
    dense = _run_sta(gpu_lib, hp, ts, dense=True)
    assert np.array_equal(sta, dense)


def test_nonfinite_count(gpu_lib):
    x = torch.zeros(1000, device="cuda")
    x[[3, 500, 999]] = torch.tensor([float("nan"), float("inf"), -float("inf")], device="cuda")
    assert int(gpu_lib.count_nonfinite(x).item()) == 3


def _run_fp4pv(lib, ts, causal=False, tau=0, plan=None):
    dev = [t.cuda() for t in ts]
    perm = plan.perm if plan is not None else None
    n_out = plan.n_tokens if plan is not None else None
    q = lib.quantize(dev[0], "mxfp4", None, perm, n_out)
    k = lib.quantize(dev[1], "mxfp4", None, perm, n_out)
    v = lib.quantize(dev[2], "mxfp4_v", None, perm, n_out)
    if plan is not None:
        out = lib.attention_sta(q, k, v, plan, tau=tau)
    else:
        out = lib.attention_dense(q, k, v, causal=causal, tau=tau)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("case", [
    dict(N=1000, causal=False, tau=0),
    dict(N=700, causal=True, tau=0),
    dict(N=520, causal=False, tau=4),
], ids=["dense", "causal", "tau4"])
def test_fp4_pv_parity(gpu_lib, case):
    """FP4 P.V (MXFP4 Q/K, V in MXFP4 along tokens, P requantised per 32 keys)
    against the oracle recipe, every output element."""
    print("fp4 p.v", case, flush=True)
    N = case["N"]
    x, ts = _inputs(1, 2, N, 128, 80 + N, torch.bfloat16, True)
    got = _run_fp4pv(gpu_lib, ts, case["causal"], case["tau"])
    _, bn = gpu_lib.attention_info("mxfp4", 128, 1 if case["causal"] else 0)
    ops = oracle_operands(*x, "mxfp4_pv", None)
    ref = np.zeros_like(got)
    for h in range(2):
        qo, ko, vo = ops[0][h]
        ref[0, h] = OA.recipe_attention(qo, ko, vo, np.arange(N), sm_scale=1 / np.sqrt(128), bn=bn,
                                        causal=case["causal"], tau=case["tau"])
    mx, mean = assert_close(got, ref, "fp4 p.v %s" % case)
    print("  max-abs %.3g mean-abs %.3g" % (mx, mean))


def test_fp4_pv_sta(gpu_lib):
    grid, real, tile, window = (6, 16, 32), (5, 15, 30), (2, 8, 8), (3, 3, 3)
    hp, op, x, ts = _sta_setup(gpu_lib, grid, real, tile, window, seed=44)
    dp = gpu_lib.DevicePlan(hp)
    got = _run_fp4pv(gpu_lib, ts, plan=dp)
    _, bn = gpu_lib.attention_info("mxfp4", 128, 2)
    xk = [OS.gather_tokens(a, op.perm) for a in x]
    ops = oracle_operands(*xk, "mxfp4_pv", None)
    ref = np.zeros_like(got)
    tt = op.tile_tokens
    for h in range(2):
        qo, ko, vo = ops[0][h]
        for u in range(op.n_tiles):
            rows = np.arange(u * tt, (u + 1) * tt)
            o = OA.recipe_attention(qo, ko, vo, rows, sm_scale=1 / np.sqrt(128), bn=bn,
                                    kv_valid=op.kv_valid, key_blocks=OS.key_blocks_for_tile(op, u, bn))
            keep = op.perm[rows] >= 0
            ref[0, h, op.perm[rows][keep]] = o[keep]
    mx, mean = assert_close(got, ref, "fp4 p.v sta")
    print("  max-abs %.3g mean-abs %.3g" % (mx, mean))


@pytest.mark.parametrize("case", [
    dict(recipe="fp8", d=128, blk=128),   # ping-pong kernel
    dict(recipe="mxfp4", d=128, blk=32),  # 4-wave kernel
    dict(recipe="fp8", d=64, blk=64),
])
def test_dense_key_tiles_equal_dense(gpu_lib, case):
    """Visiting only the key tiles that hold a valid key gives the dense result
    bit for bit (a tile without a valid key leaves the online softmax as it
    is); a query block stored nowhere is skipped without touching the rest."""
    B, H, N, d = 1, 2, 1000, case["d"]
    x, ts = _inputs(B, H, N, d, 70)
    dev = [t.cuda() for t in ts]
    if case["recipe"] == "fp8":
        q = gpu_lib.quantize(dev[0], "fp8_block", case["blk"])
        k = gpu_lib.quantize(dev[1], "fp8_block", case["blk"])
    else:
        q = gpu_lib.quantize(dev[0], "mxfp4")
        k = gpu_lib.quantize(dev[1], "mxfp4")
    v = gpu_lib.quantize(dev[2], "fp8_channel")
    bn = gpu_lib.attention_info("fp8_block" if case["recipe"] == "fp8" else "mxfp4", d, 0)[1]
    kv = np.ones(N, np.uint8)
    for t in (0, 2, 5, 6, 15):                     # whole tiles of padding (15: the ragged tail)
        kv[t * bn:(t + 1) * bn] = 0
    kv[np.random.default_rng(71).permutation(N)[:50]] = 0
    perm = np.arange(N, dtype=np.int32)
    perm[256:384] = -1                             # a query block stored nowhere
    tiles = gpu_lib.key_tiles(kv)
    assert 0 not in tiles and 15 not in tiles and len(tiles) == -(-N // bn) - 5
    kvd, permd, tilesd = (torch.from_numpy(a).cuda() for a in (kv, perm, tiles))
    ref = torch.zeros((B, H, N, d), dtype=torch.float32, device="cuda")
    got = torch.zeros_like(ref)
    gpu_lib.attention_dense(q, k, v, kv_valid=kvd, out_perm=permd, out=ref)
    gpu_lib.attention_dense(q, k, v, kv_valid=kvd, out_perm=permd, out=got, key_tiles=tilesd)
    ref_l, ref_lse = gpu_lib.attention_dense(q, k, v, kv_valid=kvd, lse=True)
    got_l, got_lse = gpu_lib.attention_dense(q, k, v, kv_valid=kvd, lse=True, key_tiles=tilesd)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.all(got[:, :, 256:384] == 0)
    assert torch.equal(got_l, ref_l) and torch.equal(got_lse, ref_lse)


@pytest.mark.parametrize("recipe,causal,sm", [("fp8", False, 0.3), ("fp8", True, 0.02), ("mxfp4", False, 0.15)])
def test_custom_softmax_scale(gpu_lib, recipe, causal, sm):
    """A softmax scale other than 1/sqrt(d) (the scaling_factor argument of the
    FastVideo call, §5.2) reaches the kernel and matches the oracle with the
    same scale."""
    print("softmax scale", recipe, causal, sm, flush=True)
    N, d = 520, 128
    x, ts = _inputs(1, 2, N, d, 95, torch.bfloat16, True)
    blk = 128 if recipe == "fp8" else None
    _, bn = gpu_lib.attention_info("mxfp4" if recipe == "mxfp4" else "fp8_block", d, 1 if causal else 0)
    got = _run_dense(gpu_lib, ts, recipe, blk, causal, sm_scale=sm)
    ref = _oracle_dense(x, recipe, blk, causal, sm, bn)
    mx, mean = assert_close(got, ref, "sm_scale %g" % sm)
    default = _oracle_dense(x, recipe, blk, causal, 1 / np.sqrt(d), bn)
    assert np.abs(default - ref).max() > 100 * mx     # the scale changes the result
    print("  max-abs %.3g mean-abs %.3g" % (mx, mean))
