"""Timestep policy decisions (host logic, no GPU)."""
import pytest

from image_diffusion_dits_amd.policy import StepPolicy


def test_first_tenth_of_the_steps_is_dense():
    p = StepPolicy(50)
    sch = p.schedule()
    assert p.n_dense == 5
    assert sch[:5] == ["dense"] * 5 and sch[5:] == ["predict"] * 45


@pytest.mark.parametrize("n,frac,want", [(30, 0.1, 3), (7, 0.1, 1), (1, 0.1, 1),
                                         (10, 0.0, 0), (10, 1.0, 10), (25, 0.2, 5)])
def test_dense_count_is_the_fraction_rounded_up(n, frac, want):
    assert StepPolicy(n, dense_fraction=frac).n_dense == want


def test_mask_refresh_cadence():
    p = StepPolicy(12, dense_fraction=0.25, refresh_every=3)
    assert p.schedule() == ["dense"] * 3 + ["predict", "reuse", "reuse"] * 3


@pytest.mark.parametrize("kw", [dict(n_steps=0), dict(n_steps=5, dense_fraction=1.5),
                                dict(n_steps=5, sparsity_pct=100),
                                dict(n_steps=5, refresh_every=0)])
def test_invalid_policies_are_rejected(kw):
    with pytest.raises(ValueError):
        StepPolicy(**kw)


def test_steps_outside_the_run_are_rejected():
    p = StepPolicy(4)
    with pytest.raises(ValueError):
        p.mode(4)
    with pytest.raises(ValueError):
        p.mode(-1)
