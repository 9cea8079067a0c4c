"""The fp64 oracle against its pins (CPU only; no GPU, no HIP library)."""

import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__[4:])
def test_pin(orc, pin):
    pin(orc)


def test_threads_do_not_change_results(orc):
    import numpy as np
    r = np.random.default_rng(0)
    x = r.normal(0, 3, (37, 211))
    t = r.integers(0, 211, 37)
    g = r.normal(0, 1, 37)
    orc.set_threads(1)
    a = orc.logp_bwd(x, t, g), orc.entropy_bwd(x, g, 30.0)
    orc.set_threads(4)
    b = orc.logp_bwd(x, t, g), orc.entropy_bwd(x, g, 30.0)
    orc.set_threads(1)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
