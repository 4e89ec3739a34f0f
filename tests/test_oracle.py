"""The CPU oracle against its pins (formats, exact arithmetic, closed forms)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_exact_tiny_all_shapes(oracle_lib):
    """Brute force over M in {1,2,7,16,33}, N in {1,16,17,64}, K in {16,32,48,256}."""
    pins.pin_exact_tiny(oracle_lib)


def test_thread_count_invariance(oracle_lib):
    import numpy as np
    import oracle
    codes, scales, xb = pins.tiny_inputs(3, 37, 128, 4)
    y1, S1 = oracle.proj(codes, scales, 0.3, xb, nthreads=1, lib=oracle_lib)
    y8, S8 = oracle.proj(codes, scales, 0.3, xb, nthreads=8, lib=oracle_lib)
    assert np.array_equal(y1, y8) and np.array_equal(S1, S8)


def test_rejects_bad_arguments(oracle_lib):
    import numpy as np
    import oracle
    codes = np.zeros((4, 8), np.uint8)
    scales = np.zeros((4, 1), np.uint8)
    x = np.zeros((1, 16), np.uint16)
    with pytest.raises(ValueError):
        oracle.proj_rows(codes, scales, 1.0, x, rows=[4], lib=oracle_lib)
