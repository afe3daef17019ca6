"""Host logic of the denoising-step-aware schedule (no GPU): phase
boundaries at alpha1 * D and alpha2 * D, steps counted from 1, the dense
window resolved to the whole grid ("FP8量化与稀疏性协同加速视频扩散模型", §3.2)."""
import pytest

from precision_attention_block_amd import schedule as S


def test_phases_of_a_50_step_run():
    sch = S.DenoisingSchedule(50, (24, 48, 80), (21, 45, 80), (6, 8, 8))
    got = [sch.phase(t) for t in range(1, 51)]
    assert got[:10] == [S.COARSE] * 10                      # t <= 0.2 D
    assert got[10:35] == [S.FINE] * 25                      # 0.2 D < t <= 0.7 D
    assert got[35:] == [S.INTERMEDIATE] * 15                # t > 0.7 D


def test_uneven_thresholds_and_custom_phases():
    a, b, c = S.Phase(256, (1, 1, 1)), S.Phase(64, S.FULL), S.Phase(128, (3, 3, 3))
    sch = S.DenoisingSchedule(7, (4, 16, 16), (3, 15, 16), (2, 8, 8), 0.3, 0.5, a, b, c)
    # t1 = 2.1, t2 = 3.5
    assert [sch.phase(t) for t in range(1, 8)] == [a, a, b, c, c, c, c]


def test_dense_window_covers_the_grid_and_bad_input():
    sch = S.DenoisingSchedule(10, (24, 48, 80), (21, 45, 80), (6, 8, 8))
    assert sch.window_tiles(S.FULL) == (9, 13, 21)          # radius >= tiles - 1 on every axis
    assert sch.window_tiles((3, 5, 5)) == (3, 5, 5)
    with pytest.raises(ValueError):
        sch.phase(0)
    with pytest.raises(ValueError):
        sch.phase(11)
    with pytest.raises(ValueError):
        S.DenoisingSchedule(10, (4, 8, 8), (4, 8, 8), (2, 4, 4), 0.8, 0.5)
