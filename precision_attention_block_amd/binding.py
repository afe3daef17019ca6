"""Thin ctypes binding of libpab (include/pab.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels of libpab.so.  PyTorch provides device memory and the current stream.
Importing this module fails loudly when the library has not been built; there
is no fallback path.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpab.so")

PAB_OK, PAB_INVALID_ARG, PAB_UNSUPPORTED, PAB_HIP_ERROR = 0, 1, 2, 3
PAB_F32, PAB_BF16 = 0, 1
RECIPES = {"fp8_block": 0, "fp8_channel": 1, "mxfp4": 2, "mxfp4_v": 3}
TOKEN_ALIGN = 128

EXPORTS = [
    "pab_abi_version", "pab_status_str", "pab_last_hip_error", "pab_token_alloc",
    "pab_attention_info", "pab_quantize", "pab_attention_dense", "pab_attention_sta",
    "pab_sta_plan", "pab_count_nonfinite", "pab_attention_backward_workspace",
    "pab_attention_backward", "pab_attention_sta_backward", "pab_attention_dense_tiles", "pab_key_tiles",
    "pab_attention_sta_steps", "pab_sta_steps", "pab_attention_backward_noalloc",
]


class PabError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib().pab_status_str(status).decode()
        if status == PAB_HIP_ERROR:
            msg += " (hipError %d)" % _lib().pab_last_hip_error()
        super().__init__("%s: %s" % (where, msg))


class QView(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("operand", ctypes.c_void_p),
                ("recipe", ctypes.c_int), ("block_tokens", ctypes.c_int),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64)]


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libpab.so is not built (run precision_attention_block_amd.build): "
                              + LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        vp = ctypes.c_void_p
        L.pab_abi_version.restype = ctypes.c_int
        L.pab_status_str.restype = ctypes.c_char_p
        L.pab_status_str.argtypes = [ctypes.c_int]
        L.pab_last_hip_error.restype = ctypes.c_int
        L.pab_token_alloc.restype = ctypes.c_int64
        L.pab_token_alloc.argtypes = [ctypes.c_int64]
        L.pab_attention_info.restype = ctypes.c_int
        L.pab_attention_info.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        L.pab_quantize.restype = ctypes.c_int
        L.pab_quantize.argtypes = [vp, ctypes.c_int, i64p, i64p, ctypes.c_int, ctypes.c_int, vp,
                                   ctypes.c_int64, vp, vp, vp, vp]
        L.pab_attention_dense.restype = ctypes.c_int
        L.pab_attention_dense.argtypes = [ctypes.POINTER(QView)] * 3 + [
            ctypes.c_int, ctypes.c_float, ctypes.c_int, vp, vp, ctypes.c_int64, vp, i64p, vp, vp]
        L.pab_attention_sta.restype = ctypes.c_int
        L.pab_attention_sta.argtypes = [ctypes.POINTER(QView)] * 3 + [
            ctypes.c_float, ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp,
            ctypes.c_int64, vp, i64p, vp, vp]
        L.pab_attention_dense_tiles.restype = ctypes.c_int
        L.pab_attention_dense_tiles.argtypes = [ctypes.POINTER(QView)] * 3 + [
            ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp, vp, ctypes.c_int64, vp, i64p, vp, vp]
        L.pab_attention_sta_steps.restype = ctypes.c_int
        L.pab_attention_sta_steps.argtypes = list(L.pab_attention_sta.argtypes)
        L.pab_sta_steps.restype = ctypes.c_int
        L.pab_sta_steps.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int64, ctypes.c_int,
                                    vp, vp, i64p]
        L.pab_key_tiles.restype = ctypes.c_int
        L.pab_key_tiles.argtypes = [vp, ctypes.c_int64, ctypes.c_int, vp, i64p]
        L.pab_attention_backward_workspace.restype = ctypes.c_int64
        L.pab_attention_backward_workspace.argtypes = [ctypes.c_int64] * 4
        L.pab_attention_backward.restype = ctypes.c_int
        L.pab_attention_backward.argtypes = [ctypes.POINTER(QView)] * 3 + [
            ctypes.c_int, ctypes.c_float, vp, vp, i64p, vp, ctypes.c_int, i64p, vp, vp, vp, vp,
            i64p, vp, ctypes.c_int64, vp]
        L.pab_attention_backward_noalloc.restype = ctypes.c_int
        L.pab_attention_backward_noalloc.argtypes = [ctypes.POINTER(QView)] * 3 + [
            ctypes.c_int, ctypes.c_float, vp, vp, i64p, vp, ctypes.c_int, i64p, vp, vp, vp, vp,
            i64p, vp]
        L.pab_attention_sta_backward.restype = ctypes.c_int
        L.pab_attention_sta_backward.argtypes = [ctypes.POINTER(QView)] * 3 + [
            ctypes.c_float, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp, i64p, vp, ctypes.c_int, i64p,
            vp, vp, vp, vp, i64p, vp, ctypes.c_int64, vp]
        ip = ctypes.POINTER(ctypes.c_int)
        L.pab_sta_plan.restype = ctypes.c_int
        L.pab_sta_plan.argtypes = [ip, ip, ip, ip, vp, vp, vp, vp, vp, vp, i64p, i64p, i64p]
        L.pab_count_nonfinite.restype = ctypes.c_int
        L.pab_count_nonfinite.argtypes = [vp, ctypes.c_int64, vp, vp]
        _L = L
    return _L


def lib():
    return _lib()


def _check(status, where):
    if status != PAB_OK:
        raise PabError(status, where)


def _i64(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def token_alloc(n):
    return int(_lib().pab_token_alloc(int(n)))


def attention_info(recipe, d, mode):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(_lib().pab_attention_info(RECIPES[recipe], int(d), int(mode), ctypes.byref(bm),
                                     ctypes.byref(bn)), "pab_attention_info")
    return bm.value, bn.value


class QTensor:
    """A quantised operand in the library's layouts (device tensors)."""

    def __init__(self, codes, scales, recipe, block_tokens, B, H, N, d, operand=None):
        self.codes, self.scales, self.recipe, self.operand = codes, scales, recipe, operand
        self.block_tokens, self.B, self.H, self.N, self.d = block_tokens, B, H, N, d

    def view(self):
        return QView(self.codes.data_ptr(), self.scales.data_ptr(),
                     self.operand.data_ptr() if self.operand is not None else None,
                     RECIPES[self.recipe], int(self.block_tokens or 0), self.B, self.H, self.N,
                     self.d)


def quantize(x, recipe, block_tokens=None, perm=None, n_out=None, operand=True):
    """Quantise x (CUDA tensor [B, H, N, d], float32 or bfloat16, innermost
    stride 1) with one recipe; perm (int32 CUDA [n_out]) gathers tokens.
    For fp8_block, operand=True also writes the bf16 operand copy that the
    attention kernel reads."""
    import torch
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    B, H, N, d = x.shape
    n_out = N if n_out is None else int(n_out)
    na = token_alloc(n_out)
    dev = x.device
    op = None
    if recipe == "fp8_block":
        if block_tokens is None:
            raise ValueError("fp8_block needs block_tokens")
        codes = torch.empty((B, H, na, d), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, -(-na // block_tokens)), dtype=torch.float32, device=dev)
        if operand:
            op = torch.empty((B, H, na, d), dtype=torch.bfloat16, device=dev)
    elif recipe == "fp8_channel":
        codes = torch.empty((B, H, d, na), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    elif recipe == "mxfp4":
        codes = torch.empty((B, H, na, d // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, na, d // 32), dtype=torch.uint8, device=dev)
    elif recipe == "mxfp4_v":
        codes = torch.empty((B, H, d, na // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, na // 32, d), dtype=torch.uint8, device=dev)
    else:
        raise ValueError(recipe)
    if x.dtype == torch.float32:
        dt = PAB_F32
    elif x.dtype == torch.bfloat16:
        dt = PAB_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    if perm is not None and (perm.dtype != torch.int32 or not perm.is_cuda):
        raise TypeError("perm must be an int32 device tensor")
    st = _lib().pab_quantize(ctypes.c_void_p(x.data_ptr()), dt, _i64(x.shape), _i64(x.stride()),
                             RECIPES[recipe], int(block_tokens or 0),
                             ctypes.c_void_p(perm.data_ptr() if perm is not None else 0), n_out,
                             ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                             ctypes.c_void_p(op.data_ptr() if op is not None else 0), _stream(dev))
    _check(st, "pab_quantize")
    return QTensor(codes, scales, recipe, block_tokens if recipe == "fp8_block" else 0,
                   B, H, n_out, d, op)


def _out_tensor(q, n_out, out):
    import torch
    if out is None:
        out = torch.empty((q.B, q.H, n_out, q.d), dtype=torch.float32, device=q.codes.device)
    return out


def _lse_tensor(q, lse):
    import torch
    if lse is True:
        return torch.empty((q.B, q.H, q.N), dtype=torch.float32, device=q.codes.device)
    return None if lse is None or lse is False else lse


def key_tiles(kv_valid_host):
    """Ascending indices (int32 numpy) of the key tiles of kv_valid (host uint8
    numpy) that hold a valid key (pab_key_tiles)."""
    kv = np.ascontiguousarray(kv_valid_host, dtype=np.uint8)
    bn = attention_info("fp8_block", 128, 0)[1]
    cnt = ctypes.c_int64()
    _check(_lib().pab_key_tiles(kv.ctypes.data, kv.size, bn, None, ctypes.byref(cnt)), "pab_key_tiles")
    out = np.zeros(max(cnt.value, 1), np.int32)
    _check(_lib().pab_key_tiles(kv.ctypes.data, kv.size, bn, out.ctypes.data, ctypes.byref(cnt)),
           "pab_key_tiles")
    return out[:cnt.value]


def attention_dense(q, k, v, causal=False, sm_scale=None, kv_valid=None, out_perm=None,
                    n_out=None, out=None, tau=0, lse=None, key_tiles=None):
    """O = softmax(Q K^T sm_scale) V on quantised operands; returns float32
    [B, H, n_out, d] (n_out defaults to N).  tau: softmax rescale threshold
    (see pab_attention_dense).  lse: None, True (allocate) or a float32
    [B, H, N] tensor for the row statistic; when given, returns (O, lse).
    key_tiles: int32 device tensor of the key tiles to visit (non-causal, with
    kv_valid masking every other key; pab_attention_dense_tiles)."""
    n_out = q.N if n_out is None else int(n_out)
    out = _out_tensor(q, n_out, out)
    lse_t = _lse_tensor(q, lse)
    if key_tiles is not None:
        if causal or kv_valid is None:
            raise ValueError("key_tiles needs a non-causal call with kv_valid")
        qv, kv, vv = q.view(), k.view(), v.view()
        st = _lib().pab_attention_dense_tiles(
            ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), float(sm_scale or 0.0), int(tau),
            ctypes.c_void_p(key_tiles.data_ptr()), int(key_tiles.numel()),
            ctypes.c_void_p(kv_valid.data_ptr()),
            ctypes.c_void_p(out_perm.data_ptr() if out_perm is not None else 0), n_out,
            ctypes.c_void_p(out.data_ptr()), _i64(out.stride()),
            ctypes.c_void_p(lse_t.data_ptr() if lse_t is not None else 0), _stream(out.device))
        _check(st, "pab_attention_dense_tiles")
        return (out, lse_t) if lse_t is not None else out
    qv, kv, vv = q.view(), k.view(), v.view()
    st = _lib().pab_attention_dense(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), int(bool(causal)),
        float(sm_scale or 0.0), int(tau),
        ctypes.c_void_p(kv_valid.data_ptr() if kv_valid is not None else 0),
        ctypes.c_void_p(out_perm.data_ptr() if out_perm is not None else 0), n_out,
        ctypes.c_void_p(out.data_ptr()), _i64(out.stride()),
        ctypes.c_void_p(lse_t.data_ptr() if lse_t is not None else 0), _stream(out.device))
    _check(st, "pab_attention_dense")
    return (out, lse_t) if lse_t is not None else out


def attention_sta(q, k, v, plan, sm_scale=None, use_kv_valid=True, use_out_perm=True, n_out=None,
                  out=None, tau=0, lse=None, steps=False):
    """Sliding-tile attention with a DevicePlan (see sta_plan / DevicePlan);
    lse as in attention_dense.  steps: walk the plan's BN-key step lists,
    which leave out the steps without a valid key (pab_attention_sta_steps;
    same result, less work on a padded grid)."""
    if n_out is None:   # caller order: the real tokens; kernel order: every token slot
        n_out = plan.n_real if use_out_perm else q.N
    n_out = int(n_out)
    out = _out_tensor(q, n_out, out)
    lse_t = _lse_tensor(q, lse)
    qv, kv, vv = q.view(), k.view(), v.view()
    fn = _lib().pab_attention_sta_steps if steps else _lib().pab_attention_sta
    off, idx = (plan.step_off, plan.step_idx) if steps else (plan.win_off, plan.win_idx)
    st = fn(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), float(sm_scale or 0.0), int(tau),
        ctypes.c_void_p(off.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
        ctypes.c_void_p(plan.lpt.data_ptr()), int(plan.n_tiles), int(plan.tile_tokens),
        ctypes.c_void_p(plan.kv_valid.data_ptr() if use_kv_valid else 0),
        ctypes.c_void_p(plan.perm.data_ptr() if use_out_perm else 0), n_out,
        ctypes.c_void_p(out.data_ptr()), _i64(out.stride()),
        ctypes.c_void_p(lse_t.data_ptr() if lse_t is not None else 0), _stream(out.device))
    _check(st, "pab_attention_sta_steps" if steps else "pab_attention_sta")
    return (out, lse_t) if lse_t is not None else out


def backward_workspace_bytes(B, H, N, d):
    return int(_lib().pab_attention_backward_workspace(int(B), int(H), int(N), int(d)))


def attention_backward(q, k, v, out, dout, lse, causal=False, sm_scale=None, kv_valid=None,
                       workspace=None, grads=None):
    """Gradients (dQ, dK, dV), float32 [B, H, N, d], with respect to the
    dequantised operands of attention_dense (quantisers pass gradients
    straight through; see pab_attention_backward).  out and lse come from the
    forward (called without out_perm); dout is float32 or bfloat16."""
    import torch
    dev = out.device
    if workspace is None:
        workspace = torch.empty(backward_workspace_bytes(q.B, q.H, q.N, q.d), dtype=torch.uint8,
                                device=dev)
    if grads is None:
        grads = tuple(torch.empty((q.B, q.H, q.N, q.d), dtype=torch.float32, device=dev)
                      for _ in range(3))
    dq, dk, dv = grads
    if dk.stride() != dq.stride() or dv.stride() != dq.stride():
        raise ValueError("dq, dk and dv must share strides")
    dt = {torch.float32: PAB_F32, torch.bfloat16: PAB_BF16}[dout.dtype]
    qv, kv, vv = q.view(), k.view(), v.view()
    st = _lib().pab_attention_backward(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), int(bool(causal)),
        float(sm_scale or 0.0), ctypes.c_void_p(kv_valid.data_ptr() if kv_valid is not None else 0),
        ctypes.c_void_p(out.data_ptr()), _i64(out.stride()), ctypes.c_void_p(dout.data_ptr()), dt,
        _i64(dout.stride()), ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(dq.data_ptr()),
        ctypes.c_void_p(dk.data_ptr()), ctypes.c_void_p(dv.data_ptr()), _i64(dq.stride()),
        ctypes.c_void_p(workspace.data_ptr()), int(workspace.numel()), _stream(dev))
    _check(st, "pab_attention_backward")
    return dq, dk, dv


NOALLOC_SCRATCH_BYTES = 32 << 20


def attention_backward_noalloc(q, k, v, out, dout, lse, causal=False, sm_scale=None,
                               kv_valid=None, grads=None):
    """attention_backward without a workspace argument: the library takes it
    from its own device array (pab_attention_backward_noalloc); the gradient
    buffers are the caller's (allocated here when `grads` is None)."""
    import torch
    dev = out.device
    if grads is None:
        grads = tuple(torch.empty((q.B, q.H, q.N, q.d), dtype=torch.float32, device=dev)
                      for _ in range(3))
    dq, dk, dv = grads
    if dk.stride() != dq.stride() or dv.stride() != dq.stride():
        raise ValueError("dq, dk and dv must share strides")
    dt = {torch.float32: PAB_F32, torch.bfloat16: PAB_BF16}[dout.dtype]
    qv, kv, vv = q.view(), k.view(), v.view()
    st = _lib().pab_attention_backward_noalloc(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), int(bool(causal)),
        float(sm_scale or 0.0), ctypes.c_void_p(kv_valid.data_ptr() if kv_valid is not None else 0),
        ctypes.c_void_p(out.data_ptr()), _i64(out.stride()), ctypes.c_void_p(dout.data_ptr()), dt,
        _i64(dout.stride()), ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(dq.data_ptr()),
        ctypes.c_void_p(dk.data_ptr()), ctypes.c_void_p(dv.data_ptr()), _i64(dq.stride()),
        _stream(dev))
    _check(st, "pab_attention_backward_noalloc")
    return dq, dk, dv


def attention_sta_backward(q, k, v, plan, out, dout, lse, sm_scale=None, use_kv_valid=True,
                           workspace=None, grads=None):
    """Gradients (dQ, dK, dV) of attention_sta (a DevicePlan), float32
    [B, H, N, d] in the kernel's tile-major token order; out and lse come from
    attention_sta called with use_out_perm=False (pab_attention_sta_backward)."""
    import torch
    dev = out.device
    if workspace is None:
        workspace = torch.empty(backward_workspace_bytes(q.B, q.H, q.N, q.d), dtype=torch.uint8,
                                device=dev)
    if grads is None:
        grads = tuple(torch.empty((q.B, q.H, q.N, q.d), dtype=torch.float32, device=dev)
                      for _ in range(3))
    dq, dk, dv = grads
    if dk.stride() != dq.stride() or dv.stride() != dq.stride():
        raise ValueError("dq, dk and dv must share strides")
    dt = {torch.float32: PAB_F32, torch.bfloat16: PAB_BF16}[dout.dtype]
    qv, kv, vv = q.view(), k.view(), v.view()
    st = _lib().pab_attention_sta_backward(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), float(sm_scale or 0.0),
        ctypes.c_void_p(plan.win_off.data_ptr()), ctypes.c_void_p(plan.win_idx.data_ptr()),
        int(plan.n_tiles), int(plan.tile_tokens),
        ctypes.c_void_p(plan.kv_valid.data_ptr() if use_kv_valid else 0),
        ctypes.c_void_p(out.data_ptr()), _i64(out.stride()), ctypes.c_void_p(dout.data_ptr()), dt,
        _i64(dout.stride()), ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(dq.data_ptr()),
        ctypes.c_void_p(dk.data_ptr()), ctypes.c_void_p(dv.data_ptr()), _i64(dq.stride()),
        ctypes.c_void_p(workspace.data_ptr()), int(workspace.numel()), _stream(dev))
    _check(st, "pab_attention_sta_backward")
    return dq, dk, dv


def sta_steps(hp):
    """BN-key step lists (step_off, step_idx) of a HostPlan's windows, without
    the steps that hold no valid key (pab_sta_steps)."""
    bn = attention_info("fp8_block", 128, 0)[1]
    wo = np.ascontiguousarray(hp.win_off, np.int32)
    wi = np.ascontiguousarray(hp.win_idx, np.int32)
    kv = np.ascontiguousarray(hp.kv_valid, np.uint8)
    cnt = ctypes.c_int64()
    args = (wo.ctypes.data, wi.ctypes.data, int(hp.n_tiles), int(hp.tile_tokens), kv.ctypes.data,
            kv.size, bn)
    _check(_lib().pab_sta_steps(*args, None, None, ctypes.byref(cnt)), "pab_sta_steps")
    off = np.zeros(int(hp.n_tiles) + 1, np.int32)
    idx = np.zeros(max(cnt.value, 1), np.int32)
    _check(_lib().pab_sta_steps(*args, off.ctypes.data, idx.ctypes.data, ctypes.byref(cnt)),
           "pab_sta_steps")
    return off, idx


class HostPlan:
    pass


def sta_plan(grid, real_grid, tile, window):
    """Runs the native planner; returns numpy arrays (perm, inv_perm, kv_valid,
    win_off, win_idx, lpt) and sizes."""
    L = _lib()
    c3 = lambda v: (ctypes.c_int * 3)(*[int(x) for x in v])
    g, rg, t, w = c3(grid), c3(real_grid), c3(tile), c3(window)
    nt, nti, npr = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(L.pab_sta_plan(g, rg, t, w, None, None, None, None, None, None, ctypes.byref(nt),
                          ctypes.byref(nti), ctypes.byref(npr)), "pab_sta_plan")
    n_real = int(np.prod(real_grid))
    p = HostPlan()
    p.perm = np.empty(nt.value, np.int32)
    p.inv_perm = np.empty(n_real, np.int32)
    p.kv_valid = np.empty(nt.value, np.uint8)
    p.win_off = np.empty(nti.value + 1, np.int32)
    p.win_idx = np.empty(npr.value, np.int32)
    p.lpt = np.empty(nti.value, np.int32)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    _check(L.pab_sta_plan(g, rg, t, w, ptr(p.perm), ptr(p.inv_perm), ptr(p.kv_valid),
                          ptr(p.win_off), ptr(p.win_idx), ptr(p.lpt), ctypes.byref(nt),
                          ctypes.byref(nti), ctypes.byref(npr)), "pab_sta_plan")
    p.n_tokens, p.n_tiles, p.n_pairs = nt.value, nti.value, npr.value
    p.tile_tokens = int(np.prod(tile))
    p.n_real = n_real
    return p


class DevicePlan:
    """A HostPlan's arrays copied to the device."""

    def __init__(self, hp, device="cuda"):
        import torch
        for name in ("perm", "inv_perm", "kv_valid", "win_off", "win_idx", "lpt"):
            setattr(self, name, torch.from_numpy(getattr(hp, name)).to(device))
        # key tiles holding a valid key, for dense attention on the padded grid,
        # and the window lists in BN-key steps without the padding steps
        self.key_tiles = torch.from_numpy(key_tiles(hp.kv_valid)).to(device)
        so, si = sta_steps(hp)
        self.step_off, self.step_idx = (torch.from_numpy(a).to(device) for a in (so, si))
        self.n_tokens, self.n_tiles, self.n_pairs = hp.n_tokens, hp.n_tiles, hp.n_pairs
        self.tile_tokens, self.n_real = hp.tile_tokens, hp.n_real


def count_nonfinite(x):
    import torch
    cnt = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(_lib().pab_count_nonfinite(ctypes.c_void_p(x.data_ptr()), x.numel(),
                                      ctypes.c_void_p(cnt.data_ptr()), _stream(x.device)),
           "pab_count_nonfinite")
    return cnt
