"""Guard bands around every device buffer the library writes: each output,
the backward's workspace and the gradients are views into a larger buffer
whose 4 KiB before and after hold a known byte pattern; after the call that
pattern must be intact.  Ragged token counts (N = 700), every recipe and every
kernel family (quantisers, ping-pong and 4-wave forward, sliding-tile on a
padded grid, backward with a caller workspace and without one), so that a
write past the end of a tile, a row or a buffer shows up here even where the
values it leaves would not."""
import ctypes

import numpy as np
import pytest
import torch

from tests.test_gpu_attention import _inputs

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """`nbytes` of device memory with GUARD bytes of PATTERN on both sides."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        self.raw = torch.full((self.n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")

    def view(self, dtype, shape):
        return self.raw[GUARD:GUARD + self.n].view(dtype).view(shape)

    def ptr(self):
        return self.raw.data_ptr() + GUARD

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.raw[:GUARD] == PATTERN).all()) and bool((self.raw[GUARD + self.n:] == PATTERN).all())


def _quantize(lib, x, recipe, blk, perm=None, n_out=None, operand=True):
    """pab_quantize into guarded buffers; returns (QTensor, guards)."""
    B, H, N, d = x.shape
    n_out = N if n_out is None else n_out
    na = lib.token_alloc(n_out)
    if recipe == "fp8_block":
        sizes = (B * H * na * d, B * H * (-(-na // blk)) * 4)
    elif recipe == "fp8_channel":
        sizes = (B * H * d * na, B * H * d * 4)
    elif recipe == "mxfp4":
        sizes = (B * H * na * d // 2, B * H * na * d // 32)
    else:
        sizes = (B * H * d * na // 2, B * H * (na // 32) * d)
    codes, scales = Guarded(sizes[0]), Guarded(sizes[1])
    op = Guarded(B * H * na * d * 2) if recipe == "fp8_block" and operand else None
    dt = lib.PAB_BF16 if x.dtype == torch.bfloat16 else lib.PAB_F32
    st = lib.lib().pab_quantize(ctypes.c_void_p(x.data_ptr()), dt, lib._i64(x.shape), lib._i64(x.stride()),
                                lib.RECIPES[recipe], int(blk or 0),
                                ctypes.c_void_p(perm.data_ptr() if perm is not None else 0), n_out,
                                ctypes.c_void_p(codes.ptr()), ctypes.c_void_p(scales.ptr()),
                                ctypes.c_void_p(op.ptr() if op is not None else 0), lib._stream(x.device))
    lib._check(st, "pab_quantize")
    sdt = torch.float32 if recipe.startswith("fp8") else torch.uint8
    qt = lib.QTensor(codes.view(torch.uint8, (-1,)), scales.view(sdt, (-1,)), recipe,
                     blk if recipe == "fp8_block" else 0, B, H, n_out, d,
                     op.view(torch.bfloat16, (-1,)) if op is not None else None)
    return qt, [g for g in (codes, scales, op) if g is not None]


def _operands(lib, ts, recipe, blk, perm=None, n_out=None, q_operand=True):
    q, k, v = (t.cuda() for t in ts)
    if recipe == "fp8":
        qq, g1 = _quantize(lib, q, "fp8_block", blk, perm, n_out, q_operand)
        kq, g2 = _quantize(lib, k, "fp8_block", blk, perm, n_out)
    else:
        qq, g1 = _quantize(lib, q, "mxfp4", None, perm, n_out)
        kq, g2 = _quantize(lib, k, "mxfp4", None, perm, n_out)
    vq, g3 = _quantize(lib, v, "mxfp4_v" if recipe == "mxfp4_pv" else "fp8_channel", None, perm, n_out)
    return (qq, kq, vq), g1 + g2 + g3


@pytest.mark.parametrize("recipe,d,causal", [("fp8", 128, False), ("fp8", 128, True), ("fp8", 64, False),
                                             ("mxfp4", 128, False), ("mxfp4_pv", 128, True)])
def test_forward_and_backward_stay_inside_their_buffers(gpu_lib, recipe, d, causal):
    print("guard bands", recipe, d, causal, flush=True)
    B, H, N = 1, 2, 700
    _, ts = _inputs(B, H, N, d, 50 + d, torch.bfloat16, True)
    (qq, kq, vq), guards = _operands(gpu_lib, ts, recipe, 64, q_operand=d == 128)
    out = Guarded(B * H * N * d * 4)
    lse = Guarded(B * H * N * 4)
    o, l = gpu_lib.attention_dense(qq, kq, vq, causal=causal, out=out.view(torch.float32, (B, H, N, d)),
                                   lse=lse.view(torch.float32, (B, H, N)))
    guards += [out, lse]
    if d == 128:
        dout = torch.randn((B, H, N, d), device="cuda")
        ws = Guarded(gpu_lib.backward_workspace_bytes(B, H, N, d))
        grads = [Guarded(B * H * N * d * 4) for _ in range(3)]
        gpu_lib.attention_backward(qq, kq, vq, o, dout, l, causal=causal,
                                   workspace=ws.view(torch.uint8, (-1,)),
                                   grads=tuple(g.view(torch.float32, (B, H, N, d)) for g in grads))
        grads2 = [Guarded(B * H * N * d * 4) for _ in range(3)]
        gpu_lib.attention_backward_noalloc(qq, kq, vq, o, dout, l, causal=causal,
                                           grads=tuple(g.view(torch.float32, (B, H, N, d)) for g in grads2))
        guards += [ws] + grads + grads2
    for i, g in enumerate(guards):
        assert g.intact(), "guard band %d of %d overwritten" % (i, len(guards))


@pytest.mark.parametrize("recipe", ["fp8", "mxfp4"])
def test_sliding_tile_stays_inside_its_buffers(gpu_lib, recipe):
    grid, real, tile, window = (4, 16, 24), (3, 15, 22), (2, 8, 8), (1, 3, 3)
    hp = gpu_lib.sta_plan(grid, real, tile, window)
    dp = gpu_lib.DevicePlan(hp, "cuda")
    n_real, d = int(np.prod(real)), 128
    _, ts = _inputs(1, 2, n_real, d, 51, torch.bfloat16, True)
    (qq, kq, vq), guards = _operands(gpu_lib, ts, recipe, hp.tile_tokens, dp.perm, hp.n_tokens)
    for steps in (False, True):
        out = Guarded(2 * n_real * d * 4)
        lse = Guarded(2 * hp.n_tokens * 4)
        gpu_lib.attention_sta(qq, kq, vq, dp, out=out.view(torch.float32, (1, 2, n_real, d)),
                              lse=lse.view(torch.float32, (1, 2, hp.n_tokens)), steps=steps)
        guards += [out, lse]
    # the backward works in the kernel's token order on every token slot
    o, l = gpu_lib.attention_sta(qq, kq, vq, dp, use_out_perm=False, lse=True)
    ws = Guarded(gpu_lib.backward_workspace_bytes(1, 2, hp.n_tokens, d))
    grads = [Guarded(2 * hp.n_tokens * d * 4) for _ in range(3)]
    gpu_lib.attention_sta_backward(qq, kq, vq, dp, o, torch.randn_like(o), l, workspace=ws.view(torch.uint8, (-1,)),
                                   grads=tuple(g.view(torch.float32, (1, 2, hp.n_tokens, d)) for g in grads))
    guards += [ws] + grads
    for i, g in enumerate(guards):
        assert g.intact(), "guard band %d of %d overwritten" % (i, len(guards))
