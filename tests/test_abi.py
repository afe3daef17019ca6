"""CPU tests of the C ABI library: it loads, exports every symbol the header
declares, its planner matches the oracle planner, and argument validation
rejects bad calls before touching a device (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import sta as OS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from precision_attention_block_amd import binding
    binding.lib()
    return binding


def test_exports_every_declared_symbol(B):
    header = open(os.path.join(ROOT, "include", "pab.h")).read()
    declared = set(re.findall(r"\b(pab_[a-z_]+)\s*\(", header))
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert hasattr(B.lib(), name), name
    assert B.lib().pab_abi_version() == 9


def test_probe_library_exports_its_header():
    """libpab_probe.so (the matrix-instruction probe the GPU tests use) loads
    and exports what include/pab_probe.h declares."""
    header = open(os.path.join(ROOT, "include", "pab_probe.h")).read()
    declared = set(re.findall(r"\b(pab_[a-z0-9_]+)\s*\(", header))
    assert declared == {"pab_probe_mfma_e4m3"}
    L = ctypes.CDLL(os.path.join(ROOT, "precision_attention_block_amd", "libpab_probe.so"))
    for name in declared:
        assert hasattr(L, name), name
    f = ctypes.c_void_p(4096)
    L.pab_probe_mfma_e4m3.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
    assert L.pab_probe_mfma_e4m3(f, f, f, 2, None) == 1                      # unknown kind
    assert L.pab_probe_mfma_e4m3(f, ctypes.c_void_p(4100), f, 0, None) == 1  # misaligned


def test_token_alloc_and_info(B):
    assert B.token_alloc(1) == 128 and B.token_alloc(128) == 128 and B.token_alloc(129) == 256
    assert B.token_alloc(0) == 0 and B.token_alloc(-7) == 0
    assert B.token_alloc(2 ** 63 - 1) == -1                 # rounding up would overflow
    assert B.backward_workspace_bytes(1, 1, 2 ** 62, 128) == -1
    assert B.backward_workspace_bytes(2 ** 40, 2 ** 40, 128, 128) == -1
    assert B.attention_info("fp8_block", 128, 0) == (256, 64)
    assert B.attention_info("fp8_block", 128, 1) == (128, 64)
    assert B.attention_info("fp8_block", 128, 2) == (128, 64)
    assert B.attention_info("fp8_block", 128, 3) == (128, 64)   # listed key steps: 4-wave kernel
    assert B.attention_info("fp8_block", 64, 0) == (128, 64)
    assert B.attention_info("mxfp4", 128, 0) == (128, 64)
    assert B.attention_info("mxfp4", 128, 1)[1] == 64
    with pytest.raises(B.PabError):
        B.attention_info("mxfp4", 64, 0)
    with pytest.raises(B.PabError):
        B.attention_info("fp8_block", 96, 0)


@pytest.mark.parametrize("grid,real,tile,window", [
    ((12, 48, 80), (12, 48, 80), (6, 8, 8), (3, 3, 3)),
    ((24, 48, 80), (21, 45, 80), (6, 8, 8), (3, 5, 5)),
    ((4, 8, 8), (3, 7, 8), (2, 4, 4), (1, 3, 5)),
    ((6, 16, 32), (5, 15, 30), (2, 8, 8), (9, 9, 9)),
])
def test_native_planner_matches_oracle(B, grid, real, tile, window):
    hp = B.sta_plan(grid, real, tile, window)
    op = OS.plan(grid, real, tile, window)
    assert np.array_equal(hp.perm, op.perm)
    assert np.array_equal(hp.kv_valid, op.kv_valid)
    assert np.array_equal(hp.win_off, op.win_off)
    assert np.array_equal(hp.win_idx, op.win_idx)
    assert np.array_equal(hp.lpt, op.lpt)
    ok = op.perm >= 0
    assert np.array_equal(hp.inv_perm[op.perm[ok]], np.nonzero(ok)[0])


def _st(B, name, *args):
    return getattr(B.lib(), name)(*args)


def test_quantize_validation_without_device(B):
    L = B.lib()
    shape = B._i64([1, 2, 256, 128])
    strides = B._i64([2 * 256 * 128, 256 * 128, 128, 1])
    fake = ctypes.c_void_p(4096)          # aligned, never dereferenced: validation fails first
    null = ctypes.c_void_p(0)
    q = lambda *a: L.pab_quantize(*a)
    # null input / outputs
    assert q(null, 1, shape, strides, 0, 128, null, 256, fake, fake, fake, null) == B.PAB_INVALID_ARG
    assert q(fake, 1, shape, strides, 0, 128, null, 256, null, fake, fake, null) == B.PAB_INVALID_ARG
    # bad dtype, recipe, block, n_out, strides, alignment, unsupported d
    assert q(fake, 7, shape, strides, 0, 128, null, 256, fake, fake, fake, null) == B.PAB_INVALID_ARG
    assert q(fake, 1, shape, strides, 9, 128, null, 256, fake, fake, null, null) == B.PAB_INVALID_ARG
    assert q(fake, 1, shape, strides, 0, 100, null, 256, fake, fake, fake, null) == B.PAB_INVALID_ARG
    assert q(fake, 1, shape, strides, 0, 16400, null, 256, fake, fake, fake, null) == B.PAB_INVALID_ARG
    assert q(fake, 1, shape, strides, 0, 128, null, 300, fake, fake, fake, null) == B.PAB_INVALID_ARG
    bad_str = B._i64([2 * 256 * 128, 256 * 128, 128, 2])
    assert q(fake, 1, shape, bad_str, 0, 128, null, 256, fake, fake, fake, null) == B.PAB_INVALID_ARG
    odd_str = B._i64([2 * 256 * 128, 256 * 128, 130, 1])
    assert q(fake, 1, shape, odd_str, 0, 128, null, 256, fake, fake, fake, null) == B.PAB_INVALID_ARG
    assert q(ctypes.c_void_p(4098), 1, shape, strides, 0, 128, null, 256, fake, fake, fake, null) \
        == B.PAB_INVALID_ARG
    shape96 = B._i64([1, 2, 256, 96])
    assert q(fake, 1, shape96, strides, 0, 128, null, 256, fake, fake, fake, null) == B.PAB_UNSUPPORTED
    shape64 = B._i64([1, 2, 256, 64])
    assert q(fake, 1, shape64, strides, 2, 0, null, 256, fake, fake, null, null) == B.PAB_UNSUPPORTED
    # an operand copy is only defined for the FP8 block recipe
    assert q(fake, 1, shape, strides, 1, 0, null, 256, fake, fake, fake, null) == B.PAB_INVALID_ARG
    assert L.pab_last_hip_error() == 0


def test_attention_validation_without_device(B):
    L = B.lib()
    fake = 4096
    mk = lambda recipe, n=256, d=128, blk=128, op=fake: B.QView(fake, fake, op, recipe, blk, 1, 2, n, d)
    qv, kv, vv = mk(0), mk(0), mk(1)
    out_str = B._i64([2 * 256 * 128, 256 * 128, 128, 1])
    null = ctypes.c_void_p(0)
    f = ctypes.c_void_p(fake)
    dense = lambda q, k, v, strides=out_str, n_out=256, sm=0.0, tau=0, lse=null: L.pab_attention_dense(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, sm, tau, null, null, n_out, f, strides,
        lse, null)
    assert dense(qv, kv, mk(0)) == B.PAB_INVALID_ARG          # V with the Q/K recipe
    assert dense(qv, mk(2), vv) == B.PAB_INVALID_ARG          # mixed Q/K recipes
    assert dense(qv, mk(0, n=300), vv) == B.PAB_INVALID_ARG   # shape mismatch
    assert dense(qv, mk(0, op=0), vv) == B.PAB_INVALID_ARG    # FP8 K without operand copy
    assert dense(mk(0, op=fake + 2), kv, vv) == B.PAB_INVALID_ARG   # misaligned Q operand copy
    assert dense(mk(0, d=96), mk(0, d=96), mk(1, d=96)) == B.PAB_UNSUPPORTED
    assert dense(qv, kv, vv, n_out=100) == B.PAB_INVALID_ARG  # output too small
    assert dense(qv, kv, vv, sm=float("nan")) == B.PAB_INVALID_ARG
    assert dense(qv, kv, vv, tau=-1) == B.PAB_INVALID_ARG     # rescale threshold out of range
    assert dense(qv, kv, vv, tau=9) == B.PAB_INVALID_ARG
    bad = B._i64([2 * 256 * 128, 256 * 128, 130, 1])
    assert dense(qv, kv, vv, strides=bad) == B.PAB_INVALID_ARG
    assert dense(qv, kv, vv, lse=ctypes.c_void_p(fake + 2)) == B.PAB_INVALID_ARG   # misaligned lse
    sta = L.pab_attention_sta(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), 0.0, 0, f, f, f,
                              2, 100, null, null, 256, f, out_str, null, null)
    assert sta == B.PAB_INVALID_ARG                           # tile not a multiple of 128
    sta = L.pab_attention_sta(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), 0.0, 0, f, f, f,
                              3, 128, null, null, 256, f, out_str, null, null)
    assert sta == B.PAB_INVALID_ARG                           # tiles do not cover N
    sta = L.pab_attention_sta(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), 0.0, 12, f, f, f,
                              2, 128, null, null, 256, f, out_str, null, null)
    assert sta == B.PAB_INVALID_ARG                           # rescale threshold out of range
    assert L.pab_last_hip_error() == 0


def test_backward_validation_without_device(B):
    L = B.lib()
    fake = 4096
    mk = lambda recipe, n=256, d=128, blk=128, op=fake: B.QView(fake, fake, op, recipe, blk, 1, 2, n, d)
    qv, kv, vv = mk(0), mk(0), mk(1)
    st = B._i64([2 * 256 * 128, 256 * 128, 128, 1])
    null = ctypes.c_void_p(0)
    f = ctypes.c_void_p(fake)
    need = L.pab_attention_backward_workspace(1, 2, 256, 128)
    # seven bf16 [BH, n_alloc, d] arrays, four float32 [BH, n_alloc], one float32 [n_alloc]
    assert need == 7 * 2 * 256 * 128 * 2 + 4 * 2 * 256 * 4 + 256 * 4
    assert L.pab_attention_backward_workspace(0, 2, 256, 128) == 0      # empty
    assert L.pab_attention_backward_workspace(-1, 2, 256, 128) < 0

    def bwd(q=qv, k=kv, v=vv, ws=fake * 16, nbytes=need, dt=B.PAB_F32, lse=f, gstr=st, dstr=st):
        return L.pab_attention_backward(
            ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, 0.0, null, f, st, f, dt, dstr,
            lse, f, f, f, gstr, ctypes.c_void_p(ws), nbytes, null)
    assert bwd(nbytes=need - 1) == B.PAB_INVALID_ARG                 # workspace too small
    assert bwd(ws=fake * 16 + 64) == B.PAB_INVALID_ARG                # workspace not 256-aligned
    assert bwd(lse=null) == B.PAB_INVALID_ARG
    assert bwd(dt=7) == B.PAB_INVALID_ARG                             # unknown dO dtype
    assert bwd(gstr=B._i64([2 * 256 * 128, 256 * 128, 130, 1])) == B.PAB_INVALID_ARG
    assert bwd(dt=B.PAB_BF16, dstr=B._i64([2 * 256 * 128, 256 * 128, 132, 1])) == B.PAB_INVALID_ARG
    assert bwd(q=mk(0, d=64), k=mk(0, d=64), v=mk(1, d=64)) == B.PAB_UNSUPPORTED
    assert bwd(k=mk(2)) == B.PAB_INVALID_ARG                          # mixed Q/K recipes
    assert bwd(q=mk(0, op=0)) == B.PAB_INVALID_ARG                    # FP8 Q without operand copy
    assert L.pab_last_hip_error() == 0


def test_backward_noalloc_validation_without_device(B):
    """pab_attention_backward_noalloc checks its size limit and every argument
    before it touches a device."""
    L = B.lib()
    fake = 4096
    mk = lambda recipe, n=256, h=2, op=fake: B.QView(fake, fake, op, recipe, 128, 1, h, n, 128)
    st = B._i64([2 * 256 * 128, 256 * 128, 128, 1])
    null = ctypes.c_void_p(0)
    f = ctypes.c_void_p(fake)

    def call(q, k, v, lse=f):
        return L.pab_attention_backward_noalloc(
            ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, 0.0, null, f, st, f, B.PAB_F32, st,
            lse, f, f, f, st, null)
    # the workspace of H = 64 heads of 8192 tokens is far above the array's 32 MiB
    big = [mk(0, 8192, 64), mk(0, 8192, 64), mk(1, 8192, 64)]
    assert L.pab_attention_backward_workspace(1, 64, 8192, 128) > B.NOALLOC_SCRATCH_BYTES
    assert call(*big) == B.PAB_UNSUPPORTED
    assert call(mk(0), mk(0), mk(1), lse=null) == B.PAB_INVALID_ARG
    assert call(mk(0, op=0), mk(0), mk(1)) == B.PAB_INVALID_ARG       # FP8 Q without operand copy
    assert call(mk(0), mk(2), mk(1)) == B.PAB_INVALID_ARG             # mixed Q/K recipes
    assert L.pab_last_hip_error() == 0
    header = open(os.path.join(ROOT, "include", "pab.h")).read()
    assert "#define PAB_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)" in header
    assert B.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_key_tiles_helper(B):
    """pab_key_tiles lists the BN-key tiles holding a nonzero byte."""
    rng = np.random.default_rng(3)
    bn = B.attention_info("fp8_block", 128, 0)[1]
    for n in (1, 64, 65, 1000, 4096 + 17):
        kv = (rng.random(n) < 0.3).astype(np.uint8)
        kv[: min(n, 2 * bn)] = 0                 # two empty tiles at the front
        want = [t for t in range(-(-n // bn)) if kv[t * bn:(t + 1) * bn].any()]
        assert list(B.key_tiles(kv)) == want
    L = B.lib()
    cnt = ctypes.c_int64()
    kv = np.ones(10, np.uint8)
    assert L.pab_key_tiles(kv.ctypes.data, 10, bn + 1, None, ctypes.byref(cnt)) == B.PAB_INVALID_ARG
    assert L.pab_key_tiles(None, 10, bn, None, ctypes.byref(cnt)) == B.PAB_INVALID_ARG


def test_dense_tiles_validation_without_device(B):
    L = B.lib()
    fake = 4096
    mk = lambda recipe, n=256, d=128, blk=128, op=fake: B.QView(fake, fake, op, recipe, blk, 1, 2, n, d)
    qv, kv, vv = mk(0), mk(0), mk(1)
    st = B._i64([2 * 256 * 128, 256 * 128, 128, 1])
    null = ctypes.c_void_p(0)
    f = ctypes.c_void_p(fake)
    call = lambda tiles=f, n_tiles=2, kvv=f: L.pab_attention_dense_tiles(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), 0.0, 0, tiles, n_tiles, kvv, null, 256,
        f, st, null, null)
    assert call(tiles=null) == B.PAB_INVALID_ARG
    assert call(kvv=null) == B.PAB_INVALID_ARG                 # skipped keys must be masked
    assert call(n_tiles=0) == B.PAB_INVALID_ARG
    assert call(n_tiles=5) == B.PAB_INVALID_ARG                # more tiles than N holds
    assert L.pab_last_hip_error() == 0


def test_sta_steps_helper(B):
    """pab_sta_steps expands each window into its BN-key steps, ascending, and
    drops the steps without a valid key."""
    bn = B.attention_info("fp8_block", 128, 0)[1]
    hp = B.sta_plan((8, 16, 16), (7, 13, 16), (4, 8, 8), (3, 3, 3))
    off, idx = B.sta_steps(hp)
    spt = hp.tile_tokens // bn
    for u in range(hp.n_tiles):
        want = [w * spt + s for w in hp.win_idx[hp.win_off[u]:hp.win_off[u + 1]] for s in range(spt)
                if hp.kv_valid[(w * spt + s) * bn:(w * spt + s + 1) * bn].any()]
        assert list(idx[off[u]:off[u + 1]]) == want
    assert off[-1] < len(hp.win_idx) * spt        # the padded grid loses some steps
    L = B.lib()
    cnt = ctypes.c_int64()
    wo, wi = hp.win_off.copy(), hp.win_idx.copy()
    wi[0] = hp.n_tiles                               # window tile out of range
    assert L.pab_sta_steps(wo.ctypes.data, wi.ctypes.data, hp.n_tiles, hp.tile_tokens, None,
                           hp.n_tokens, bn, None, None, ctypes.byref(cnt)) == B.PAB_INVALID_ARG


def test_planner_validation(B):
    L = B.lib()
    c3 = lambda v: (ctypes.c_int * 3)(*v)
    n = ctypes.c_int64()
    assert L.pab_sta_plan(c3((12, 48, 80)), c3((12, 48, 80)), c3((5, 8, 8)), c3((3, 3, 3)),
                          None, None, None, None, None, None, ctypes.byref(n), None, None) \
        == B.PAB_INVALID_ARG                                  # grid not a multiple of tile
    assert L.pab_sta_plan(c3((12, 48, 80)), c3((13, 48, 80)), c3((6, 8, 8)), c3((3, 3, 3)),
                          None, None, None, None, None, None, ctypes.byref(n), None, None) \
        == B.PAB_INVALID_ARG                                  # real grid larger than grid


def test_empty_inputs_are_no_ops_without_device(B):
    """B, H or N equal to 0: OK with NULL pointers, nothing launched (the calls
    would fault on a NULL pointer otherwise); negative sizes are invalid."""
    L = B.lib()
    null = ctypes.c_void_p(0)
    st = B._i64([0, 0, 0, 1])
    for shape, n_out in (([1, 2, 0, 128], 0), ([0, 2, 256, 128], 256), ([1, 0, 256, 128], 256)):
        assert L.pab_quantize(null, 1, B._i64(shape), st, 0, 128, null, n_out, null, null, null,
                              null) == B.PAB_OK
    assert L.pab_quantize(null, 1, B._i64([1, 2, 0, 128]), st, 0, 128, null, 5, null, null, null,
                          null) == B.PAB_INVALID_ARG                  # n_out != N without perm
    assert L.pab_quantize(null, 1, B._i64([1, -1, 4, 128]), st, 0, 128, null, 4, null, null, null,
                          null) == B.PAB_INVALID_ARG
    mk = lambda recipe, B_=1, H=2, n=0: B.QView(0, 0, 0, recipe, 128, B_, H, n, 128)
    out_str = B._i64([0, 0, 128, 1])
    for b_, h, n in ((1, 2, 0), (0, 2, 256), (1, 0, 256)):
        q, k, v = mk(0, b_, h, n), mk(0, b_, h, n), mk(1, b_, h, n)
        assert L.pab_attention_dense(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 1, 0.0, 0,
                                     null, null, n, null, out_str, null, null) == B.PAB_OK
        assert L.pab_attention_backward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, 0.0,
                                        null, null, out_str, null, 0, out_str, null, null, null,
                                        null, out_str, null, 0, null) == B.PAB_OK
        assert B.backward_workspace_bytes(b_, h, n, 128) == 0
    q, k, v = mk(0, n=0), mk(0, n=4), mk(1, n=0)           # sizes disagree: not an empty call
    assert L.pab_attention_dense(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, 0.0, 0, null,
                                 null, 0, null, out_str, null, null) == B.PAB_INVALID_ARG
    q = mk(0, n=-1)
    assert L.pab_attention_dense(ctypes.byref(q), ctypes.byref(q), ctypes.byref(mk(1, n=-1)), 0, 0.0,
                                 0, null, null, 0, null, out_str, null, null) == B.PAB_INVALID_ARG
    assert B.backward_workspace_bytes(1, 2, -1, 128) == -1
    assert L.pab_last_hip_error() == 0


def test_size_limits_without_device(B):
    """Sizes past the device's grid limits or the kernels' 32-bit buffer
    offsets are PAB_UNSUPPORTED before any launch; the largest allowed sizes
    pass validation (checked with a NULL output, which is then rejected)."""
    L = B.lib()
    fake = ctypes.c_void_p(4096)
    null = ctypes.c_void_p(0)

    def quant(b, h, n, blk=128):
        return L.pab_quantize(fake, 1, B._i64([b, h, n, 128]), B._i64([0, 0, 128, 1]), 0, blk, null,
                              n, fake, fake, fake, null)
    # every call here fails validation: block 100 is invalid, checked after the limits
    assert quant(1, 65537, 128, blk=100) == B.PAB_UNSUPPORTED        # grid y
    assert quant(1, 65536, 128, blk=100) == B.PAB_INVALID_ARG
    assert quant(1, 1, (1 << 27) + 1, blk=100) == B.PAB_UNSUPPORTED
    assert quant(1, 1, 1 << 27, blk=100) == B.PAB_INVALID_ARG
    assert quant(1, 1, 1 << 31) == B.PAB_UNSUPPORTED

    def dense(b, h, n, out=fake):
        mk = lambda recipe: B.QView(4096, 4096, 4096, recipe, 128, b, h, n, 128)
        q, k, v = mk(0), mk(0), mk(1)
        return L.pab_attention_dense(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, 0.0, 0,
                                     null, null, n, out, B._i64([0, 0, 128, 1]), null, null)
    assert dense(1, 1, (1 << 22) + 1) == B.PAB_UNSUPPORTED           # per-head descriptor bytes
    assert dense(1, 1, 1 << 22, out=null) == B.PAB_INVALID_ARG       # allowed size, NULL output
    assert dense(1 << 9, 1, 1 << 22) == B.PAB_UNSUPPORTED            # B*H*n_alloc = 2^31
    assert dense(1, (1 << 9) - 1, 1 << 22, out=null) == B.PAB_INVALID_ARG
    assert dense(1, (1 << 24) + 1, 128) == B.PAB_UNSUPPORTED
    mk = lambda recipe: B.QView(4096, 4096, 4096, recipe, 128, 1, 65537, 256, 128)
    q, k, v = mk(0), mk(0), mk(1)
    st = B._i64([0, 0, 128, 1])
    assert L.pab_attention_backward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, 0.0, null,
                                    fake, st, fake, 0, st, fake, fake, fake, fake, st,
                                    ctypes.c_void_p(4096 * 256), 1 << 40, null) == B.PAB_UNSUPPORTED
    assert L.pab_last_hip_error() == 0


def test_sta_backward_validation_without_device(B):
    """pab_attention_sta_backward rejects bad window arguments before any
    launch; the rest of its validation is pab_attention_backward's."""
    L = B.lib()
    fake = 4096
    mk = lambda recipe: B.QView(fake, fake, fake, recipe, 128, 1, 2, 256, 128)
    qv, kv, vv = mk(0), mk(0), mk(1)
    st = B._i64([2 * 256 * 128, 256 * 128, 128, 1])
    null = ctypes.c_void_p(0)
    f = ctypes.c_void_p(fake)
    need = L.pab_attention_backward_workspace(1, 2, 256, 128)

    def sta(win_off=f, win_idx=f, n_tiles=2, tile=128, nbytes=need):
        return L.pab_attention_sta_backward(
            ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), 0.0, win_off, win_idx, n_tiles, tile,
            null, f, st, f, B.PAB_F32, st, f, f, f, f, st, ctypes.c_void_p(fake * 16), nbytes, null)
    assert sta(win_off=null) == B.PAB_INVALID_ARG
    assert sta(win_idx=ctypes.c_void_p(fake + 2)) == B.PAB_INVALID_ARG      # misaligned list
    assert sta(tile=100) == B.PAB_INVALID_ARG                               # not a multiple of 128
    assert sta(n_tiles=3) == B.PAB_INVALID_ARG                              # tiles do not cover N
    assert sta(nbytes=need - 1) == B.PAB_INVALID_ARG                        # workspace too small
    assert L.pab_last_hip_error() == 0
