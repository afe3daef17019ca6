"""One-call attention on unquantised inputs: quantise Q, K, V with the staged
recipe and run the fused kernel (all on the device through libpab).

The FastVideo FP4 article (wmrh.cn, §5.2) calls its kernel as
fp4_attention(qkv, mask, head_dim, scaling_factor); its §8.2 falls back to
standard attention when the output holds NaN/Inf.  `check_finite=True` runs
the library's non-finite count and raises, so that the caller can fall back;
this module itself never computes attention another way."""
from . import binding as B


def quantize_qkv(q, k, v, recipe="fp8", block_tokens=128, perm=None, n_out=None,
                 q_operand=False):
    """recipe: "fp8" (Q/K FP8 per block), "mxfp4" (Q/K MXFP4) or "mxfp4_pv"
    (Q/K MXFP4 and V MXFP4 along tokens: both products in FP4).
    q_operand: also write Q's bf16 operand copy (FP8), which the backward
    reads; the forward decodes Q's codes itself."""
    if recipe == "fp8":
        qq = B.quantize(q, "fp8_block", block_tokens, perm, n_out, operand=q_operand)
        kq = B.quantize(k, "fp8_block", block_tokens, perm, n_out)
    elif recipe in ("mxfp4", "mxfp4_pv"):
        qq = B.quantize(q, "mxfp4", None, perm, n_out)
        kq = B.quantize(k, "mxfp4", None, perm, n_out)
    else:
        raise ValueError(recipe)
    vq = B.quantize(v, "mxfp4_v" if recipe == "mxfp4_pv" else "fp8_channel", None, perm, n_out)
    return qq, kq, vq


def attention(q, k, v, recipe="fp8", block_tokens=None, causal=False, sm_scale=None, sta=None,
              check_finite=False, tau=0):
    """q, k, v: CUDA tensors [B, H, N, d] (float32 or bfloat16, any strides with
    unit channel stride; a packed qkv [B, N, 3, H, d] can be passed as three
    permuted views).  sta: None, or a binding.DevicePlan for sliding-tile
    attention over tokens given in raster order of the plan's real grid.
    block_tokens: tokens per FP8 Q/K scale block; None gives one scale per 3D
    tile on the sliding-tile path (the FPSAttention page, §2.3 and §3.1: one
    tile serves both the quantisation and the sparsity) and 128 tokens on the
    dense path.
    tau: softmax rescale threshold (0 = rescale on every rise of the maximum).
    Returns float32 [B, H, N, d]."""
    if sta is None:
        qq, kq, vq = quantize_qkv(q, k, v, recipe, 128 if block_tokens is None else block_tokens)
        out = B.attention_dense(qq, kq, vq, causal=causal, sm_scale=sm_scale, tau=tau)
    else:
        if causal:
            raise ValueError("sliding-tile attention has no causal mask")
        qq, kq, vq = quantize_qkv(q, k, v, recipe, sta.tile_tokens if block_tokens is None
                                  else block_tokens, sta.perm, sta.n_tokens)
        out = B.attention_sta(qq, kq, vq, sta, sm_scale=sm_scale, tau=tau)
    if check_finite:
        bad = int(B.count_nonfinite(out).item())
        if bad:
            raise FloatingPointError("attention output holds %d non-finite values" % bad)
    return out


def _attention_function():
    import torch

    class QuantizedAttention(torch.autograd.Function):
        """Dense or causal attention on quantised operands with the gradient of
        pab_attention_backward: the quantisers pass gradients straight through
        (training-aware quantisation, the FPSAttention page's introduction).
        The forward keeps the quantised operands, O and the row statistic for
        the backward; d = 128."""

        @staticmethod
        def forward(ctx, q, k, v, recipe, block_tokens, causal, sm_scale):
            qq, kq, vq = quantize_qkv(q, k, v, recipe, block_tokens, q_operand=True)
            out, lse = B.attention_dense(qq, kq, vq, causal=causal, sm_scale=sm_scale, lse=True)
            ctx.ops = (qq, kq, vq)
            ctx.causal, ctx.sm_scale = causal, sm_scale
            ctx.dtypes = (q.dtype, k.dtype, v.dtype)
            ctx.save_for_backward(out, lse)
            return out

        @staticmethod
        def backward(ctx, dout):
            out, lse = ctx.saved_tensors
            if dout.dtype not in (torch.float32, torch.bfloat16):
                dout = dout.float()
            if dout.stride(-1) != 1:
                dout = dout.contiguous()
            dq, dk, dv = B.attention_backward(*ctx.ops, out, dout, lse, causal=ctx.causal,
                                              sm_scale=ctx.sm_scale)
            dq, dk, dv = (g.to(t) for g, t in zip((dq, dk, dv), ctx.dtypes))
            return dq, dk, dv, None, None, None, None

    return QuantizedAttention


_QA = None


def attention_autograd(q, k, v, recipe="fp8", block_tokens=128, causal=False, sm_scale=None):
    """attention() as a differentiable op for training: q, k, v CUDA tensors
    [B, H, N, 128] (float32 or bfloat16); the backward runs
    pab_attention_backward (gradients with respect to the dequantised
    operands, passed straight through the quantisers)."""
    global _QA
    if _QA is None:
        _QA = _attention_function()
    return _QA.apply(q, k, v, recipe, block_tokens, causal, sm_scale)
