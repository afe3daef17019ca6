"""GPU tests of the one-call Python API (precision_attention_block_amd.api):
it quantises and attends through the C ABI and matches the oracle recipe; a
packed qkv tensor passed as three strided views gives the same result as
contiguous inputs; sliding-tile attention through a device plan matches the
oracle; check_finite raises when the device count reports a non-finite
output."""
import numpy as np
import pytest
import torch

from tests.helpers import assert_close, oracle_sta
from tests.test_gpu_attention import _inputs, _oracle_dense

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("recipe,causal", [("fp8", False), ("fp8", True), ("mxfp4", False)])
def test_attention_matches_oracle(gpu_lib, recipe, causal):
    from precision_attention_block_amd import api
    x, ts = _inputs(1, 2, 640, 128, 77, torch.bfloat16, True)
    got = api.attention(*(t.cuda() for t in ts), recipe=recipe, block_tokens=128,
                        causal=causal).cpu().numpy()
    mode = 1 if causal else 0
    _, bn = gpu_lib.attention_info("mxfp4" if recipe == "mxfp4" else "fp8_block", 128, mode)
    ref = _oracle_dense(x, recipe, 128 if recipe == "fp8" else None, causal, 1 / np.sqrt(128), bn)
    assert_close(got, ref, "api %s causal=%s" % (recipe, causal))


def test_packed_qkv_views_equal_contiguous(gpu_lib):
    from precision_attention_block_amd import api
    B, N, H, d = 1, 384, 2, 128
    rng = np.random.default_rng(3)
    qkv = torch.from_numpy(rng.standard_normal((B, N, 3, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    views = [qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)]        # [B, H, N, d], strided
    a = api.attention(*views).cpu().numpy()
    b = api.attention(*(t.contiguous() for t in views)).cpu().numpy()
    assert np.array_equal(a, b)


def test_sta_through_device_plan(gpu_lib):
    from precision_attention_block_amd import api
    grid, real, tile, window = (4, 16, 16), (3, 15, 16), (2, 8, 8), (1, 3, 3)
    hp = gpu_lib.sta_plan(grid, real, tile, window)
    dp = gpu_lib.DevicePlan(hp, "cuda")
    n_real = int(np.prod(real))
    x, ts = _inputs(1, 2, n_real, 128, 91, torch.bfloat16, True)
    got = api.attention(*(t.cuda() for t in ts), recipe="fp8", block_tokens=None, sta=dp).cpu().numpy()
    _, bn = gpu_lib.attention_info("fp8_block", 128, 2)
    ref = oracle_sta(x, grid, real, tile, window, hp.tile_tokens, bn, 1 / np.sqrt(128))
    assert_close(got, ref, "api sta")


def test_check_finite_raises(gpu_lib, monkeypatch):
    from precision_attention_block_amd import api
    _, ts = _inputs(1, 1, 256, 128, 5, torch.float32, False)
    q, k, v = (t.cuda() for t in ts)
    api.attention(q, k, v, check_finite=True)             # finite output: no error
    # with finite inputs (the contract) every code is finite, so a valid call
    # never produces a non-finite output; the fallback signal is exercised by
    # making the device count report one
    monkeypatch.setattr(api.B, "count_nonfinite", lambda out: torch.ones(1, dtype=torch.int32))
    with pytest.raises(FloatingPointError):
        api.attention(q, k, v, check_finite=True)


@pytest.mark.parametrize("recipe,causal", [("fp8", True), ("mxfp4", False)])
def test_autograd_uses_the_library_backward(gpu_lib, recipe, causal):
    """attention_autograd's gradients are exactly those of a direct
    pab_attention_backward call on the same quantised operands."""
    from precision_attention_block_amd import api
    rng = np.random.default_rng(80)
    B, H, N, d = 1, 2, 300, 128
    q, k, v = (torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(torch.bfloat16)
               .cuda().requires_grad_() for _ in range(3))
    dout = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).cuda()
    out = api.attention_autograd(q, k, v, recipe=recipe, block_tokens=64, causal=causal)
    out.backward(dout)
    qq, kq, vq = api.quantize_qkv(q.detach(), k.detach(), v.detach(), recipe, 64, q_operand=True)
    o2, lse = gpu_lib.attention_dense(qq, kq, vq, causal=causal, lse=True)
    grads = gpu_lib.attention_backward(qq, kq, vq, o2, dout, lse, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for g, ref in zip((q.grad, k.grad, v.grad), grads):
        assert g.dtype == torch.bfloat16 and torch.equal(g, ref.to(torch.bfloat16))


@pytest.mark.parametrize("shape", [(1, 2, 0, 128), (0, 2, 256, 128), (1, 0, 256, 128)])
@pytest.mark.parametrize("recipe", ["fp8", "mxfp4", "mxfp4_pv"])
def test_empty_inputs(gpu_lib, shape, recipe):
    """An empty batch, head or token axis gives empty outputs and gradients
    (the library launches nothing), and the device stays usable."""
    from precision_attention_block_amd import api
    print("empty case", shape, recipe, flush=True)
    q, k, v = (torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    out = api.attention(q, k, v, recipe=recipe, block_tokens=128)
    assert out.shape == shape and out.dtype == torch.float32
    qq, kq, vq = api.quantize_qkv(q, k, v, recipe, 128)
    o, lse = gpu_lib.attention_dense(qq, kq, vq, causal=True, lse=True)
    assert o.shape == shape and lse.shape == shape[:3]
    grads = gpu_lib.attention_backward(qq, kq, vq, o, torch.zeros(shape, device="cuda"), lse)
    assert all(g.shape == shape for g in grads)
    torch.cuda.synchronize()
    x = torch.randn(1, 1, 256, 128, device="cuda")
    assert torch.all(torch.isfinite(api.attention(x, x, x)))


@pytest.mark.parametrize("recipe,causal", [("fp8", False), ("fp8", True), ("mxfp4", False)])
def test_strided_output_equals_contiguous(gpu_lib, recipe, causal):
    """O written into a caller's [B, N, H, d] buffer viewed as [B, H, N, d]
    (token stride H*d) equals the contiguous output bit for bit, and every
    element of the caller's buffer (filled with NaN first) is written."""
    from precision_attention_block_amd import api
    B, H, N, d = 2, 3, 520, 128
    _, ts = _inputs(B, H, N, d, 91, torch.bfloat16, True)
    qq, kq, vq = api.quantize_qkv(*(t.cuda() for t in ts), recipe, 128)
    ref = gpu_lib.attention_dense(qq, kq, vq, causal=causal)
    buf = torch.full((B, N, H, d), float("nan"), device="cuda")
    got = gpu_lib.attention_dense(qq, kq, vq, causal=causal, out=buf.permute(0, 2, 1, 3))
    torch.cuda.synchronize()
    assert got.stride() == (N * H * d, d, H * d, 1)
    assert torch.equal(got, ref)
    assert not torch.isnan(buf).any()


def test_sta_kernel_order_output_on_a_padded_grid(gpu_lib):
    """attention_sta without the output permutation returns every token slot
    of the padded grid in the kernel's tile-major order; its real rows equal
    the caller-order output bit for bit."""
    from precision_attention_block_amd import api
    grid, real, tile, window = (4, 16, 16), (3, 15, 16), (2, 8, 8), (1, 3, 3)
    hp = gpu_lib.sta_plan(grid, real, tile, window)
    dp = gpu_lib.DevicePlan(hp, "cuda")
    _, ts = _inputs(1, 2, int(np.prod(real)), 128, 92, torch.bfloat16, True)
    qq, kq, vq = api.quantize_qkv(*(t.cuda() for t in ts), "fp8", hp.tile_tokens, dp.perm, hp.n_tokens)
    caller = gpu_lib.attention_sta(qq, kq, vq, dp)
    kernel = gpu_lib.attention_sta(qq, kq, vq, dp, use_out_perm=False)
    torch.cuda.synchronize()
    assert kernel.shape[2] == hp.n_tokens > caller.shape[2] == hp.n_real
    perm = dp.perm.cpu().numpy()
    live = np.nonzero(perm >= 0)[0]
    assert torch.equal(kernel[:, :, live].cpu(), caller[:, :, perm[live]].cpu())


@pytest.mark.parametrize("d,causal", [(128, False), (128, True), (64, False)])
def test_fp8_forward_needs_no_q_operand(gpu_lib, d, causal):
    """The forward decodes Q's E4M3 codes in registers: a Q view without its
    bf16 operand copy is accepted and gives the output of a view with it, bit
    for bit (ping-pong kernel for dense d = 128, 4-wave kernel otherwise)."""
    x, ts = _inputs(1, 2, 700, d, 41, torch.bfloat16, True)
    q, k, v = (t.cuda() for t in ts)
    kq = gpu_lib.quantize(k, "fp8_block", 64)
    vq = gpu_lib.quantize(v, "fp8_channel")
    with_op = gpu_lib.quantize(q, "fp8_block", 64)
    without = gpu_lib.quantize(q, "fp8_block", 64, operand=False)
    assert without.operand is None and with_op.operand is not None
    assert torch.equal(with_op.codes, without.codes) and torch.equal(with_op.scales, without.scales)
    a = gpu_lib.attention_dense(with_op, kq, vq, causal=causal)
    b = gpu_lib.attention_dense(without, kq, vq, causal=causal)
    assert torch.equal(a, b)
    _, bn = gpu_lib.attention_info("fp8_block", d, 1 if causal else 0)
    ref = _oracle_dense(x, "fp8", 64, causal, 1 / np.sqrt(d), bn)
    assert_close(b.cpu().numpy(), ref, "no Q operand d=%d causal=%s" % (d, causal))


@pytest.mark.parametrize("recipe", ["fp8", "mxfp4"])
def test_sta_result_does_not_depend_on_the_tile_order(gpu_lib, recipe):
    """The plan's tile order only decides when each query tile's workgroups
    run: issuing the tiles in reverse or in index order gives the same output
    and row statistic, bit for bit."""
    from precision_attention_block_amd import api
    grid, real, tile, window = (4, 16, 24), (3, 15, 22), (2, 8, 8), (1, 3, 3)
    hp = gpu_lib.sta_plan(grid, real, tile, window)
    dp = gpu_lib.DevicePlan(hp, "cuda")
    _, ts = _inputs(1, 2, int(np.prod(real)), 128, 93, torch.bfloat16, True)
    qq, kq, vq = api.quantize_qkv(*(t.cuda() for t in ts), recipe, hp.tile_tokens, dp.perm, hp.n_tokens)
    ref, ref_lse = gpu_lib.attention_sta(qq, kq, vq, dp, lse=True)
    plan_order = dp.lpt.clone()
    for order in (plan_order.flip(0), torch.arange(hp.n_tiles, dtype=torch.int32, device="cuda")):
        dp.lpt = order.contiguous()
        for steps in (False, True):
            out, lse = gpu_lib.attention_sta(qq, kq, vq, dp, lse=True, steps=steps)
            torch.cuda.synchronize()
            assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    dp.lpt = plan_order
