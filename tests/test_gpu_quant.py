"""GPU parity of the quantizer kernels: codes and scales bit-exact against the
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import formats as OF
from oracle import quant as OQ
from oracle import sta as OS
from tests.helpers import vt_to_tokens

pytestmark = pytest.mark.gpu


def _inputs(shape, seed, dtype, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        ch = rng.permutation(shape[-1])[:4]
        x[..., ch] *= rng.lognormal(0, 1.5, 4).astype(np.float32)
    t = torch.from_numpy(x).to(dtype)
    return t.float().numpy(), t


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,H,N,d,blk", [(1, 2, 256, 64, 64), (1, 3, 1000, 128, 128),
                                          (2, 2, 200, 128, 384), (1, 1, 77, 64, 16),
                                          (1, 2, 3500, 128, 1536), (1, 1, 700, 64, 2048)])
def test_fp8_block_bit_exact(gpu_lib, dtype, B, H, N, d, blk):
    print("fp8_block", B, H, N, d, blk, dtype, flush=True)
    x, xt = _inputs((B, H, N, d), 100 + N, dtype)
    qt = gpu_lib.quantize(xt.cuda(), "fp8_block", blk)
    torch.cuda.synchronize()
    codes, scales = OQ.fp8_block_quantize(x, blk)
    g_codes = qt.codes.cpu().numpy()
    g_scales = qt.scales.cpu().numpy()
    nb = -(-N // blk)
    assert np.array_equal(g_scales[..., :nb], scales)
    assert np.all(g_scales[..., nb:] == 1.0)
    assert np.array_equal(g_codes[..., :N, :], codes)
    assert np.all(g_codes[..., N:, :] == 0)
    # the bf16 operand copy holds the exact value of every code
    vals = qt.operand.float().cpu().numpy()
    assert np.array_equal(vals, OF.e4m3_decode(g_codes).astype(np.float32))


def test_fp8_block_strided_packed_qkv(gpu_lib):
    B, N, H, d = 2, 300, 3, 128
    x, xt = _inputs((B, N, 3, H, d), 7, torch.bfloat16)
    dev = xt.cuda()
    k_view = dev[:, :, 1].permute(0, 2, 1, 3)           # [B, H, N, d], strided
    qt = gpu_lib.quantize(k_view, "fp8_block", 128)
    torch.cuda.synchronize()
    codes, scales = OQ.fp8_block_quantize(np.ascontiguousarray(x[:, :, 1].transpose(0, 2, 1, 3)), 128)
    assert np.array_equal(qt.scales.cpu().numpy()[..., :3], scales)
    assert np.array_equal(qt.codes.cpu().numpy()[..., :N, :], codes)


def test_fp8_block_token_gather(gpu_lib):
    p = OS.plan((4, 16, 16), (3, 15, 16), (2, 8, 8), (3, 3, 3))
    n_real = 3 * 15 * 16
    x, xt = _inputs((1, 2, n_real, 128), 8, torch.bfloat16)
    perm = torch.from_numpy(p.perm).cuda()
    qt = gpu_lib.quantize(xt.cuda(), "fp8_block", 128, perm=perm, n_out=p.n_tokens)
    torch.cuda.synchronize()
    xk = OS.gather_tokens(x, p.perm)
    codes, scales = OQ.fp8_block_quantize(xk, 128)
    assert np.array_equal(qt.scales.cpu().numpy(), scales)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,H,N,d", [(1, 2, 256, 64), (1, 3, 1000, 128), (2, 2, 130, 128)])
def test_fp8_channel_bit_exact(gpu_lib, dtype, B, H, N, d):
    print("fp8_channel", B, H, N, d, dtype, flush=True)
    x, xt = _inputs((B, H, N, d), 200 + N, dtype)
    qt = gpu_lib.quantize(xt.cuda(), "fp8_channel")
    torch.cuda.synchronize()
    codes, scales = OQ.fp8_channel_quantize(x)
    assert np.array_equal(qt.scales.cpu().numpy(), scales)
    vt = qt.codes.cpu().numpy()
    assert vt.shape == (B, H, d, gpu_lib.token_alloc(N))
    assert np.array_equal(vt_to_tokens(vt, N), codes)
    full = vt_to_tokens(vt, vt.shape[-1])
    assert np.all(full[..., N:, :] == 0)


def test_fp8_channel_token_gather(gpu_lib):
    p = OS.plan((4, 16, 16), (3, 15, 16), (2, 8, 8), (3, 3, 3))
    n_real = 3 * 15 * 16
    x, xt = _inputs((1, 2, n_real, 128), 9, torch.bfloat16)
    qt = gpu_lib.quantize(xt.cuda(), "fp8_channel", perm=torch.from_numpy(p.perm).cuda(),
                          n_out=p.n_tokens)
    torch.cuda.synchronize()
    codes, scales = OQ.fp8_channel_quantize(OS.gather_tokens(x, p.perm))
    assert np.array_equal(qt.scales.cpu().numpy(), scales)
    assert np.array_equal(vt_to_tokens(qt.codes.cpu().numpy(), p.n_tokens), codes)


def _mx_special_values(n_rows):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((1, 1, n_rows, 128)) *
         np.exp2(rng.uniform(-30, 30, (1, 1, n_rows, 4))).repeat(32, -1)).astype(np.float32)
    x[0, 0, 0, :32] = 0.0                                   # zero group
    x[0, 0, 1, :32] = 1.75                                  # clipped to 1.5
    x[0, 0, 2, :32] = np.float32(2.0 ** -130)               # subnormal amax
    x[0, 0, 2, 1] = -np.float32(2.0 ** -140)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    x[0, 0, 3, :32] = np.tile(np.concatenate([ties, -ties]), 2)   # amax 6 -> e = 0
    x[0, 0, 4, 32:64] = np.float32(3e38)                    # huge
    return x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mxfp4_bit_exact(gpu_lib, dtype):
    x = _mx_special_values(300)
    xt = torch.from_numpy(x).to(dtype)
    x = xt.float().numpy()
    qt = gpu_lib.quantize(xt.cuda(), "mxfp4")
    torch.cuda.synchronize()
    codes, e8 = OQ.mxfp4_quantize(x)
    assert np.array_equal(qt.scales.cpu().numpy()[..., :300, :], e8)
    assert np.array_equal(OF.e2m1_unpack(qt.codes.cpu().numpy())[..., :300, :], codes)


def _exhaustive_chunk(lo_bits, hi_bits, step=1):
    """Every `step`-th float32 bit pattern in [lo_bits, hi_bits) laid out as
    blocks of 16 tokens x 128 channels whose first element is 448, so each
    block's scale is exactly 1 and the codes are the plain E4M3 conversion."""
    pats = np.arange(lo_bits, hi_bits, step, dtype=np.uint32).view(np.float32)
    per = 16 * 128 - 1
    nblk = -(-len(pats) // per)
    buf = np.zeros(nblk * per, np.float32)
    buf[:len(pats)] = pats
    buf = buf.reshape(nblk, per)
    blocks = np.concatenate([np.full((nblk, 1), 448.0, np.float32), buf], axis=1)
    return blocks.reshape(1, 1, nblk * 16, 128), len(pats)


@pytest.mark.parametrize("lo,hi,step", [
    (0.0, 2.0 ** -16, 251),           # +-0, float32 subnormals and tiny normals, sampled
    (2.0 ** -16, 2.0 ** -12, 1),      # below the E4M3 grid: round to +-0 (0x80 for negatives)
    (2.0 ** -12, 2.0 ** -4, 1), (2.0 ** -4, 2.0 ** 2, 1), (2.0 ** 2, 448.0, 1)])
def test_fp8_conversion_exhaustive_binades(gpu_lib, lo, hi, step):
    """Device conversion against the oracle encoder for every float32 in [lo, hi)
    (every `step`-th bit pattern) and its negative; the negatives of values that
    round to zero must give the code of -0 (0x80)."""
    lo_b = int(np.float32(lo).view(np.uint32))
    hi_b = int(np.float32(hi).view(np.uint32))
    for sign in (1.0, -1.0):
        x, n = _exhaustive_chunk(lo_b, hi_b, step)
        if sign < 0 and lo == 0.0:
            assert np.signbit(np.float32(sign) * x.reshape(-1)[1])      # -0.0 is among the inputs
        x *= np.float32(sign)
        x[..., ::16, 0] = 448.0
        print("exhaustive", lo, hi, sign, n, flush=True)
        qt = gpu_lib.quantize(torch.from_numpy(x).cuda(), "fp8_block", 16)
        torch.cuda.synchronize()
        assert np.all(qt.scales.cpu().numpy() == 1.0)
        got = qt.codes.cpu().numpy().reshape(-1)[:x.size]
        want = OF.e4m3_encode(x.reshape(-1))
        bad = np.nonzero(got != want)[0]
        assert len(bad) == 0, "first mismatch: x=%r got %02x want %02x" % (
            x.reshape(-1)[bad[0]], got[bad[0]], want[bad[0]])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N", [256, 300, 1000])
def test_mxfp4_v_bit_exact(gpu_lib, dtype, N):
    """V in MXFP4 along tokens (FP4 P.V): codes and E8M0 scales equal the
    oracle's bit for bit after undoing the documented layout (transposed, slot
    order of the FP4 P.V operand, interleaved channels); padding slots are
    zero codes."""
    from tests.helpers import v4_codes_to_tokens, v4_scales_to_channels
    x, t = _inputs((1, 2, N, 128), 70 + N, dtype, True)
    x[0, 1, 5:9] *= 1000.0                       # a group with a large exponent
    t = torch.from_numpy(x).to(dtype)
    x = t.float().numpy()
    qt = gpu_lib.quantize(t.cuda(), "mxfp4_v")
    na = gpu_lib.token_alloc(N)
    codes = qt.codes.cpu().numpy()
    scales = qt.scales.cpu().numpy()
    assert codes.shape == (1, 2, 128, na // 2) and scales.shape == (1, 2, na // 32, 128)
    for h in range(2):
        rc, re = OQ.mxfp4_token_quantize(x[0, h])
        got = v4_codes_to_tokens(codes[0, h], na)
        assert np.array_equal(got[:N], rc), "codes differ, head %d" % h
        assert not got[N:].any(), "padding codes not zero"
        gs = v4_scales_to_channels(scales[0, h])
        assert np.array_equal(gs[:re.shape[0]], re), "scales differ, head %d" % h
