"""How the gfx950 matrix instructions accumulate E4M3 products, through
libpab_probe (include/pab_probe.h): one 32x32x64 product D = C + A B^T.

The FP8 recipe asks for S = Q K^T from the exact products of the quantised
values with fp32 accumulation (FPSAttention page, §3.1; the recipe's oracle
sums the products exactly).  These cases show that the FP8 matrix instruction
(v_mfma_scale_f32_32x32x64_f8f6f4) does not do that, and that the bf16
instruction on the exact bf16 values of the same codes does, which is why the
attention kernel computes the FP8 recipe's S on the bf16 instruction:

* the FP8 instruction sums each group of 8 consecutive products in fixed
  point about 13 bits below the group's largest product, then adds the group
  sums and C in fp32: 448 - 448 + 2^-6 inside one group gives 0, 448^2 -
  448^2 + 14 gives 8, and 448 + 2^-9 loses the 2^-9 wherever the -448 that
  cancels the 448 sits;
* on quantised rows with outlier channels its error reaches 1e-4 of
  sum |q k|, which exponentiated logits of sharp rows turn into output
  errors above the 1e-2 gate; the bf16 instruction stays at fp32 rounding.

The expected values are this hardware's measured results; exact values come
from float64 sums of the decoded codes.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as OQ

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "precision_attention_block_amd", "libpab_probe.so")
DEC = F.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
FP8_MFMA, BF16_MFMA = 0, 1


def _enc(x):
    return int(F.e4m3_encode(np.asarray([x], np.float32))[0])


@pytest.fixture(scope="module")
def probe(gpu_lib):
    if not os.path.exists(PROBE):
        pytest.fail("libpab_probe.so is not built (run precision_attention_block_amd.build)")
    L = ctypes.CDLL(PROBE)
    L.pab_probe_mfma_e4m3.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
    L.pab_probe_mfma_e4m3.restype = ctypes.c_int

    def run(a, b, c, kind):
        A = torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()
        Bm = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).cuda()
        C = torch.from_numpy(np.ascontiguousarray(c, np.float32)).cuda()
        assert L.pab_probe_mfma_e4m3(A.data_ptr(), Bm.data_ptr(), C.data_ptr(), kind, None) == 0
        torch.cuda.synchronize()
        return C.cpu().numpy().astype(np.float64)
    return run


def _exact(a, b, c):
    return c.astype(np.float64) + DEC[a] @ DEC[b].T


def _rows(entries, b_val=1.0):
    """A has one case per row (a list of (k, value) products); B is b_val
    everywhere, so D[r, j] = sum of row r's values times b_val."""
    a = np.zeros((32, 64), np.uint8)
    for r, row in enumerate(entries):
        for k, x in row:
            a[r, k] = _enc(x)
    return a, np.full((32, 64), _enc(b_val), np.uint8)


# (products as (k, value), B value, measured FP8-instruction result)
CASES = [
    ([(0, 448.0), (1, -448.0), (2, 2.0 ** -5)], 1.0, 2.0 ** -5),    # 13 bits below 2^8 survive
    ([(0, 448.0), (1, -448.0), (2, 2.0 ** -6)], 1.0, 0.0),          # one bit further: lost
    ([(0, 448.0), (1, -448.0), (8, 2.0 ** -9)], 1.0, 2.0 ** -9),    # small product in another group
    ([(0, 448.0), (63, -448.0), (40, 2.0 ** -9)], 1.0, 2.0 ** -9),  # 448 alone in its group
    ([(0, 448.0), (1, 2.0 ** -9), (40, -448.0)], 1.0, 0.0),         # 448 + 2^-9 share a group
    ([(0, 448.0), (1, -448.0), (2, 2.0 ** -5)], 448.0, 8.0),        # 448^2 - 448^2 + 14 -> 8
    ([(0, 448.0), (1, -448.0), (2, 2.0 ** -2)], 448.0, 112.0),      # + 112: a multiple of 8
]


def test_fp8_instruction_truncates_inside_groups_of_8(probe):
    entries = [e for e, bv, _ in CASES]
    for bv in sorted({bv for _, bv, _ in CASES}):
        a, b = _rows([e if cb == bv else [] for e, cb, _ in CASES], bv)
        c = np.zeros((32, 32), np.float32)
        fp8 = probe(a, b, c, FP8_MFMA)
        bf16 = probe(a, b, c, BF16_MFMA)
        ex = _exact(a, b, c)
        for r, (e, cb, want) in enumerate(CASES):
            if cb != bv:
                continue
            assert np.all(fp8[r] == want), (e, fp8[r, 0], want)
            assert np.all(bf16[r] == ex[r]), (e, bf16[r, 0], ex[r, 0])     # exact on bf16
    assert len(entries) == len(CASES)


def test_accumulator_input_adds_in_fp32(probe):
    """C enters in fp32 on both instructions: 200704 + 1 is exact, and
    200704 + 2^-7 rounds to 200704 (half an fp32 ulp, ties to even)."""
    a, b = _rows([[(5, 1.0)], [(5, 2.0 ** -6)], [(5, 2.0 ** -7)]])
    c = np.full((32, 32), 200704.0, np.float32)
    for kind in (FP8_MFMA, BF16_MFMA):
        d = probe(a, b, c, kind)
        assert d[0, 0] == 200705.0 and d[1, 0] == 200704.0 + 2.0 ** -6 and d[2, 0] == 200704.0


def test_quantised_outlier_rows(probe):
    """Quantised N(0,1) rows with four outlier channels (lognormal(0, 1.5)
    gains, 128-token FP8 blocks): the bf16 instruction is exact to fp32
    rounding, the FP8 one is off by more than 1e-5 of sum |q k|."""
    rng = np.random.default_rng(5)
    worst = {FP8_MFMA: 0.0, BF16_MFMA: 0.0}
    for _ in range(3):
        q = rng.standard_normal((128, 64)).astype(np.float32)
        k = rng.standard_normal((128, 64)).astype(np.float32)
        ch = rng.permutation(64)[:4]
        q[:, ch] *= rng.lognormal(0, 1.5, 4).astype(np.float32)
        k[:, ch] *= rng.lognormal(0, 1.5, 4).astype(np.float32)
        a = OQ.fp8_block_quantize(q, 128)[0][:32]
        b = OQ.fp8_block_quantize(k, 128)[0][:32]
        c = np.zeros((32, 32), np.float32)
        ex = _exact(a, b, c)
        mag = np.abs(DEC[a]) @ np.abs(DEC[b]).T
        for kind in worst:
            worst[kind] = max(worst[kind], float((np.abs(probe(a, b, c, kind) - ex) / mag).max()))
    print("max |err| / sum |q k|: FP8 instruction %.3g, bf16 instruction %.3g"
          % (worst[FP8_MFMA], worst[BF16_MFMA]))
    assert worst[BF16_MFMA] < 2.0 ** -22
    assert worst[FP8_MFMA] > 1e-5
