"""The CPU oracle against its pins (closed forms, brute force, invariants,
library special cases, an independent PyTorch formulation)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_rejects_bad_shapes():
    bad = [
        oracle.OracleConfig(1, 9, 8, 4, 1, 2, 1),   # H not divisible by n_win
        oracle.OracleConfig(1, 8, 9, 4, 1, 2, 1),   # W not divisible by n_win
        oracle.OracleConfig(1, 8, 8, 6, 4, 2, 1),   # C not divisible by heads
        oracle.OracleConfig(0, 8, 8, 4, 1, 2, 1),   # empty batch
    ]
    import numpy as np
    for cfg in bad:
        x = np.zeros((max(cfg.batch, 1), cfg.height, cfg.width, cfg.channels))
        with pytest.raises(ValueError):
            oracle.region_means(cfg, x)
