"""The denoising-step-aware schedule on the GPU: one step of each phase
(coarse blocks + sparse window, fine blocks + dense window, intermediate
blocks + medium window) matches the oracle run with that phase's settings."""
import numpy as np
import pytest
import torch

from tests.helpers import assert_close, oracle_sta
from tests.test_gpu_attention import _inputs

pytestmark = pytest.mark.gpu


def test_one_step_per_phase(gpu_lib):
    from precision_attention_block_amd import schedule as S
    grid, real, tile = (4, 16, 24), (3, 15, 22), (2, 8, 8)
    sch = S.DenoisingSchedule(10, grid, real, tile,
                              early=S.Phase(384, (1, 1, 1)), middle=S.Phase(64, S.FULL),
                              late=S.Phase(128, (3, 3, 3)))
    x, ts = _inputs(1, 2, int(np.prod(real)), 128, 123, torch.bfloat16, True)
    q, k, v = (t.cuda() for t in ts)
    _, bn = gpu_lib.attention_info("fp8_block", 128, 2)
    for t in (1, 5, 10):
        ph = sch.phase(t)
        got = sch.attention(q, k, v, t).cpu().numpy()
        ref = oracle_sta(x, grid, real, tile, sch.window_tiles(ph.window), ph.block_tokens, bn,
                         1 / np.sqrt(128))
        assert_close(got, ref, "step %d %s" % (t, ph))
    assert len(sch._plans) == 3
