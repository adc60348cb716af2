"""The fp64 oracle against its pins (CPU only)."""
import math
import random

import pytest

import oracle
from oracle import pyref
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle.load_library()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_online_softmax_equals_batch_softmax():
    """Lab 00 of the phase: the online softmax equals the batch softmax."""
    rnd = random.Random(1)
    for n in (1, 2, 5, 16, 33):
        xs = [rnd.gauss(0.0, 3.0) for _ in range(n)]
        want = pyref.batch_softmax(xs)
        for block in range(1, n + 1):
            got = pyref.online_softmax(xs, block)
            assert max(abs(a - b) for a, b in zip(got, want)) < 1e-15
            assert abs(math.fsum(got) - 1.0) < 1e-14


def test_online_softmax_handles_huge_logits():
    """Subtracting the running max keeps exp() finite for large scores."""
    xs = [1000.0, 999.0, -1000.0, 998.0]
    got = pyref.online_softmax(xs, 1)
    want = pyref.batch_softmax(xs)
    assert all(math.isfinite(x) for x in got)
    assert max(abs(a - b) for a, b in zip(got, want)) < 1e-15


def test_oracle_rejects_bad_arguments(lib):
    import numpy as np
    q = np.zeros((1, 3, 4, 8), np.uint16)
    k = np.zeros((1, 2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.oracle_fwd(q, k, k, scale=1.0, dtype="f16", lib=lib)
    with pytest.raises(TypeError):
        oracle.oracle_fwd(q.astype(np.float64), k, k, scale=1.0, dtype="f16", lib=lib)


def test_oracle_empty_sequence(lib):
    import numpy as np
    q = np.zeros((1, 2, 0, 8), np.uint16)
    o, lse = oracle.oracle_fwd(q, q, q, scale=1.0, dtype="f16", lib=lib)
    assert o.shape == (1, 2, 0, 8) and lse.shape == (1, 2, 0)
