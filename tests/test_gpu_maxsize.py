"""Attention at the largest token count the library accepts per head,
N = 2^22 (pab_attention_dense returns PAB_UNSUPPORTED above it).  At this size
every 32-bit offset and buffer size in the kernels is at its largest.

The oracle cannot compute rows one by one at this size, so the inputs are
built so that the method's result has a closed form that holds at any size:
 * every key row is the same bf16 vector, so after quantisation (FP8 per
   block or MXFP4) every score of a query row has the same value S;
 * the online softmax then gives P = 2^(S c - m) = 1 for every visible key,
   P~ = E4M3(448 P) = 448 exactly (the fixed P scale of 1/448, FPSAttention
   §3.1), and l = the number of visible keys, so O is the mean of the
   dequantised V over the visible keys;
 * V takes values in {+-0.5, +-1, +-2} with a 2 in every channel, so the
   per-channel scale is 448 / 2 = 224 and every V * 224 (112, 224 or 448) is an
   E4M3 value: the dequantised V equals V.
Hence O_i = (1/N) sum_j V_j (dense) or (1/(i+1)) sum_{j<=i} V_j (causal),
computed on the host in float64.  The kernel accumulates in fp32 over 65536
key tiles; the bound on that rounding is far inside the 1e-2 max-abs and
1e-3 mean-abs gate.  The quantised K and V codes are checked against the
oracle's encoders."""
import numpy as np
import pytest
import torch

from oracle import formats as OF
from oracle import quant as OQ
from tests.helpers import MAX_ABS, MEAN_ABS, vt_to_tokens

pytestmark = pytest.mark.gpu

N = 1 << 22
D = 128
V_TABLE = np.array([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0])


@pytest.fixture(scope="module")
def inputs():
    rng = np.random.default_rng(2022)
    idx = rng.integers(0, len(V_TABLE), (N, D), dtype=np.int8)
    idx[0] = len(V_TABLE) - 1                         # a 2 in every channel
    k_row = rng.standard_normal(D).astype(np.float32)
    k_row[rng.permutation(D)[:4]] *= 8.0              # outlier channels
    gen = torch.Generator(device="cuda").manual_seed(2022)
    q = torch.randn((1, 1, N, D), generator=gen, device="cuda").to(torch.bfloat16)
    k_row_t = torch.from_numpy(k_row).to(torch.bfloat16)
    k = k_row_t.cuda().view(1, 1, 1, D).expand(1, 1, N, D)   # token stride 0
    table = torch.tensor(V_TABLE, dtype=torch.bfloat16, device="cuda")
    v = table[torch.from_numpy(idx).cuda().long()].view(1, 1, N, D)
    # float64 sums of V over token chunks, then prefix sums
    chunk = 1 << 18
    sums = np.stack([V_TABLE[idx[c:c + chunk]].sum(axis=0) for c in range(0, N, chunk)])
    return dict(idx=idx, k_row=k_row_t.float().numpy(), q=q, k=k, v=v, chunk=chunk, sums=sums)


def _check_output(out, x, causal, what):
    idx, chunk, sums = x["idx"], x["chunk"], x["sums"]
    worst, total = 0.0, 0.0
    before = np.zeros(D)
    for n, c in enumerate(range(0, N, chunk)):
        got = out[0, 0, c:c + chunk].cpu().numpy().astype(np.float64)
        if causal:
            ref = (before + np.cumsum(V_TABLE[idx[c:c + chunk]], axis=0)) / np.arange(c + 1, c + chunk + 1)[:, None]
        else:
            ref = np.broadcast_to(sums.sum(axis=0) / N, got.shape)
        before = before + sums[n]
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        total += float(err.sum())
    mean = total / (N * D)
    print("%s: N = %d, max-abs %.3g, mean-abs %.3g" % (what, N, worst, mean), flush=True)
    assert worst <= MAX_ABS and mean <= MEAN_ABS, (what, worst, mean)


def _check_v_codes(vq, x):
    """Scale 224 in every channel and codes equal to the oracle's E4M3 encoding
    of V * 224."""
    assert torch.all(vq.scales == 224.0)
    codes = vt_to_tokens(vq.codes[0, 0].cpu().numpy(), N)            # [N, d]
    enc = OF.e4m3_encode(V_TABLE * 224.0)
    assert np.array_equal(codes, enc[x["idx"]])


@pytest.mark.parametrize("recipe,causal", [("fp8", False), ("fp8", True), ("mxfp4", False)])
def test_maximum_tokens_per_head(gpu_lib, inputs, recipe, causal):
    print("max-size case", recipe, "causal" if causal else "dense", flush=True)
    x = inputs
    if recipe == "fp8":
        qq = gpu_lib.quantize(x["q"], "fp8_block", 128)
        kq = gpu_lib.quantize(x["k"], "fp8_block", 128)
        kc, ks = OQ.fp8_block_quantize(np.tile(x["k_row"], (128, 1)), 128)
        assert np.array_equal(kq.codes[0, 0, :128].cpu().numpy(), kc)
        assert np.array_equal(kq.codes[0, 0, N - 128:].cpu().numpy(), kc)
        assert torch.all(kq.scales == float(ks[0]))
    else:
        qq = gpu_lib.quantize(x["q"], "mxfp4")
        kq = gpu_lib.quantize(x["k"], "mxfp4")
        kc, ke = OQ.mxfp4_quantize(x["k_row"][None, :])
        kc = OF.e2m1_pack(kc)                          # two codes per byte, low nibble first
        assert np.array_equal(kq.codes[0, 0, :1].cpu().numpy(), kc)
        assert np.array_equal(kq.codes[0, 0, N - 1:].cpu().numpy(), kc)
        assert np.array_equal(kq.scales[0, 0, N - 1:].cpu().numpy(), ke)
    vq = gpu_lib.quantize(x["v"], "fp8_channel")
    _check_v_codes(vq, x)
    out = gpu_lib.attention_dense(qq, kq, vq, causal=causal)
    torch.cuda.synchronize()
    _check_output(out, x, causal, "%s %s" % (recipe, "causal" if causal else "dense"))


NB = 1 << 20     # the largest tokens per head of pab_attention_backward
SAMPLES = 64


@pytest.mark.timeout(600)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_maximum_tokens_per_head(gpu_lib, causal):
    """The backward at N = 2^20 (its limit), FP8 recipe.  The same
    construction (equal keys, exactly quantised V) gives the forward in closed
    form: row i sees n_i keys (N, or i + 1 causal) with one score s_i, so
    O_i = mean of V over them and LSE_i = s_i + log2(n_i).  Both sides take
    these O and LSE; the oracle's gradients of sampled rows and keys
    (backward_sampled) are the reference, under the gate of the other backward
    tests: each element within twice the first-order bound of the library's
    bf16 roundings.  dQ is zero in exact arithmetic here (equal keys make the
    softmax flat in Q), so its mean-abs error is held to the bound alone."""
    from oracle import attention as OA
    from oracle import backward as OB
    from tests.fullsize import sampled_bounds
    print("max-size backward", "causal" if causal else "dense", flush=True)
    n, d = NB, D
    rng = np.random.default_rng(2020 + int(causal))
    q = torch.from_numpy(rng.standard_normal((n, d)).astype(np.float32)).to(torch.bfloat16)
    k_row = torch.from_numpy(rng.standard_normal(d).astype(np.float32)).to(torch.bfloat16)
    idx = rng.integers(0, len(V_TABLE), (n, d), dtype=np.int8)
    idx[0] = len(V_TABLE) - 1
    do = torch.from_numpy(rng.standard_normal((n, d)).astype(np.float32)).to(torch.bfloat16)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, SAMPLES, replace=False)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, SAMPLES, replace=False)]))

    # oracle operands and the closed-form forward
    qc, qs = OQ.fp8_block_quantize(q.float().numpy(), 128)
    kc, ks = OQ.fp8_block_quantize(np.tile(k_row.float().numpy(), (128, 1)), 128)
    qh = OB.dequantized(OA.Operand("fp8_block", qc, qs, 128))
    kh = np.tile(OB.dequantized(OA.Operand("fp8_block", kc, ks, 128))[0], (n, 1))
    vh = V_TABLE[idx]
    sm = 1.0 / np.sqrt(d)
    cnt = np.arange(1, n + 1, dtype=np.float64) if causal else np.full(n, float(n))
    o = np.ascontiguousarray(np.cumsum(vh, axis=0) / cnt[:, None] if causal else
                             np.broadcast_to(vh.mean(axis=0), (n, d)), dtype=np.float32)
    lse = ((qh @ kh[0]) * (sm * OA.LOG2E) + np.log2(cnt)).astype(np.float32)

    dev = torch.device("cuda:0")
    qq = gpu_lib.quantize(q.view(1, 1, n, d).to(dev), "fp8_block", 128)
    kq = gpu_lib.quantize(k_row.to(dev).view(1, 1, 1, d).expand(1, 1, n, d), "fp8_block", 128)
    table = torch.tensor(V_TABLE, dtype=torch.bfloat16, device=dev)
    vq = gpu_lib.quantize(table[torch.from_numpy(idx).to(dev).long()].view(1, 1, n, d), "fp8_channel")
    blocks = np.unique(rows // 128)
    got_qc = qq.codes[0, 0].cpu().numpy()
    for b in blocks:
        assert np.array_equal(got_qc[128 * b:128 * b + 128], qc[128 * b:128 * b + 128])
    assert np.array_equal(qq.scales[0, 0, :n // 128].cpu().numpy(), qs)
    dq, dk, dv = gpu_lib.attention_backward(
        qq, kq, vq, torch.from_numpy(o).view(1, 1, n, d).to(dev), do.view(1, 1, n, d).to(dev),
        torch.from_numpy(lse).view(1, 1, n).to(dev), causal=causal)
    torch.cuda.synchronize()
    print("  gpu backward done", flush=True)

    do64 = do.float().numpy().astype(np.float64)
    ref = OB.backward_sampled(qh, kh, vh, o, do64, lse, sm, rows, cols, causal=causal)
    bounds = sampled_bounds(qh, kh, vh, o, do64, lse, sm, rows, cols, causal)
    got = (dq[0, 0, rows].cpu().numpy(), dk[0, 0, cols].cpu().numpy(), dv[0, 0, cols].cpu().numpy())
    for nm, g, r, b in zip("qkv", got, ref, bounds):
        assert np.all(np.isfinite(g)), "d%s: non-finite" % nm
        err = np.abs(g.astype(np.float64) - r)
        scale = np.abs(r).max()
        lim = 2 * b + 1e-6 * scale
        print("  d%s: max err/bound %.3f, max-abs %.3g of max|ref| %.3g" % (
            nm, (err / lim).max(), err.max(), scale), flush=True)
        assert np.all(err <= lim), "d%s" % nm
        assert err.mean() <= 1e-3 * (scale if nm != "q" else 2 * b.max())
