"""Host logic of the training-step integration: which kind of step each training step is
(notes "INSTANT: ...", 整体框架: calibration every N_t steps, compression in between)."""
from types import SimpleNamespace

import pytest

torch = pytest.importorskip("torch")


def _modes(N_t, N_cal, generation, steps):
    from rank_compressed_backprop_amd.linear import InstantLinear
    fake = SimpleNamespace(N_t=N_t, N_cal=N_cal, generation=generation)
    return [InstantLinear.mode_of_step(fake, s) for s in range(steps)]


def test_window_schedule():
    assert _modes(5, 2, 1, 10) == ["calibrate", "finalize", "compress", "compress", "compress"] * 2
    assert _modes(4, 1, 3, 8) == ["finalize", "compress", "compress", "compress"] * 2
    # N_cal = N_t: every step calibrates, the last of each window finalizes
    assert _modes(3, 3, 1, 6) == ["calibrate", "calibrate", "finalize"] * 2


def test_no_projections_yet_means_exact_backward():
    assert _modes(5, 2, 0, 5) == ["calibrate", "finalize", "exact", "exact", "exact"]
