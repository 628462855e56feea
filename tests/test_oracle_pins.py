"""The oracle against what the pages and the mathematics fix (CPU only)."""

import pytest

from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()


def test_rejects_bad_inputs():
    import numpy as np

    import oracle

    with pytest.raises(ValueError):
        oracle.quantize_sym(np.ones((2, 96), dtype=np.float16), 64)   # in % group != 0
    with pytest.raises(ValueError):
        oracle.quantize_sym(np.array([[np.inf, 0.0]], dtype=np.float16), 2)
    with pytest.raises(TypeError):
        oracle.quantize_sym(np.ones((2, 64), dtype=np.float32), 32)
    with pytest.raises(ValueError):
        oracle.quantize_asym(np.array([[np.nan, 0.0]], dtype=np.float16), 2)
