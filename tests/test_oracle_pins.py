"""The float64 oracle against what the pages and mathematics fix."""

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_oracle_pool_equals_the_oracle():
    """Spreading a batch over worker processes changes nothing, bit for bit."""
    import numpy as np

    import oracle
    from oracle_pool import oracle_batch
    from oracle_pins import scattered, small_batch
    b = small_batch(5, [1, 17, 40, 3, 100, 64, 7], 8, 2, 64, spare=3)
    kc, vc = scattered(oracle, b)
    want = oracle.decode(b.q, kc, vc, b.block_tables, b.context_lens, b.scale)
    got = oracle_batch("decode", b.q, kc, vc, b.block_tables, b.context_lens, b.scale, procs=3)
    assert np.isfinite(want).all() and np.array_equal(got, want)
