"""The V-Smooth step schedule (VC-Attention paper §3.4 and Appendix A):
grouping and demeaning on the first quarter of the denoising steps, the
permutation recomputed every 4 steps inside that window and reused in
between, plain FP8 ExpCast attention afterwards.  Host logic only."""
import pytest

import bit_fp8_attention_amd as vc


def _plan(n):
    return [vc.vsmooth_schedule(n, s) for s in range(n)]


def test_wan_40_steps_regroups_at_0_4_8():
    p = _plan(40)
    assert [s for s, m in enumerate(p) if m == "group"] == [0, 4, 8]
    assert [s for s, m in enumerate(p) if m != "plain"] == list(range(10))  # window ceil(40 / 4)


def test_longcat_50_steps_regroups_at_0_4_8_12():
    p = _plan(50)
    assert [s for s, m in enumerate(p) if m == "group"] == [0, 4, 8, 12]
    assert sum(m != "plain" for m in p) == 13


def test_minimax_8_steps_has_a_two_step_window():
    assert _plan(8) == ["group", "reuse"] + ["plain"] * 6


def test_schedule_rejects_bad_arguments():
    for args in [(0, 0), (10, 10), (10, -1), (10, 0, 0)]:
        with pytest.raises(ValueError):
            vc.vsmooth_schedule(*args)
