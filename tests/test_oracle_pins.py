"""The oracle against its pins (CPU only). See ``oracle_pins.py`` for what
each pin rests on."""
import numpy as np
import pytest

import oracle as oracle_pkg

from . import oracle_pins as pins
from . import workloads as wl


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle, pin):
    pin(oracle)


def test_segments_pin():
    pins.pin_segments(oracle_pkg.build_segments)


def test_tiny_config_runs(oracle):
    w = wl.tiny()
    y = oracle.sgmv(wl.storage(w.Y), wl.storage(w.X), wl.storage(w.A_pool), wl.storage(w.B_pool),
                    w.seg_start, w.seg_adapter, w.alpha)
    assert y.shape == (8, 256) and np.all(np.isfinite(y)) and np.any(y != 0)


def test_rejects_out_of_pool_ids(oracle):
    w = wl.tiny()
    bad = w.seg_adapter.copy()
    bad[1] = 4
    with pytest.raises(ValueError):
        oracle.shrink(wl.storage(w.X), wl.storage(w.A_pool), w.seg_start, bad)


def test_openmp_rows_bitwise(oracle, monkeypatch):
    """Rows are independent, so any thread count gives the same bits."""
    rng = np.random.Generator(np.random.PCG64(21))
    w = wl.random_case(rng, max_M=16, max_seg=6)
    a = oracle.sgmv(wl.storage(w.Y), wl.storage(w.X), wl.storage(w.A_pool), wl.storage(w.B_pool),
                    w.seg_start, w.seg_adapter, w.alpha)
    b = oracle.sgmv(wl.storage(w.Y), wl.storage(w.X), wl.storage(w.A_pool), wl.storage(w.B_pool),
                    w.seg_start, w.seg_adapter, w.alpha)
    assert np.array_equal(a, b)
