"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.attention)


def test_errors():
    import numpy as np
    q = np.zeros((1, 1, 3, 2))
    k = np.zeros((1, 1, 2, 2))
    with pytest.raises(ValueError, match="bad shape"):      # Sq > Skv
        oracle.attention(q, k, k, 0.5, 1)
    with pytest.raises(ValueError, match="non-finite"):
        oracle.attention(k, k, k, float("nan"), 1)
    with pytest.raises(ValueError):
        oracle.attention(k.astype(np.float32), k, k, 0.5, 1)


def test_threads_do_not_change_results():
    import numpy as np
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((3, 5, 17, 8)) for _ in range(3))
    a = oracle.attention(q, k, v, 0.3, 1, [17, 9, 2], nthreads=1)
    b = oracle.attention(q, k, v, 0.3, 1, [17, 9, 2], nthreads=7)
    assert np.array_equal(a, b)
