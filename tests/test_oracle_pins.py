"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_bad_arguments(orc):
    import numpy as np
    import oracle
    with pytest.raises(TypeError):
        orc.gemm("max_plus", np.zeros((2, 2), np.float64), np.zeros((2, 2), np.float64))
    with pytest.raises(oracle.OracleError):
        orc.permute(np.zeros((2, 3), np.float32), (0, 0))
    with pytest.raises(oracle.OracleError):
        orc.diag_gather("max_plus", np.zeros((2, 3), np.float32), "ii", "i")
    with pytest.raises(oracle.OracleError):
        orc.contract_pair("ij,jk,kl->il", "max_plus", np.zeros((2, 3), np.float32),
                          np.zeros((3, 4), np.float32))
