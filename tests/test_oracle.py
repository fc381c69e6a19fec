"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins


def _fn(q, k, v, scale, causal, valid_len=None, rows=None, keep_mask=None, add_mask=None):
    return oracle.attn_fwd(q, k, v, scale, causal, valid_len, rows=rows, threads=2,
                           keep_mask=keep_mask, add_mask=add_mask)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS + oracle_pins.MASK_PINS,
                         ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_fn)


def test_rejects_bad_arguments():
    q = np.zeros((1, 3, 4, 2))
    k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, k, k, 1.0, False)   # Hq % Hkv != 0
    q = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, k, k, 1.0, False, rows=np.array([8], np.int64))  # row out of range


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 4, 33, 8))
    k = rng.standard_normal((2, 2, 33, 8))
    v = rng.standard_normal((2, 2, 33, 8))
    vl = np.array([20, 33], np.int32)
    O1, L1 = oracle.attn_fwd(q, k, v, 0.3, True, vl, threads=1)
    O4, L4 = oracle.attn_fwd(q, k, v, 0.3, True, vl, threads=4)
    np.testing.assert_array_equal(O1, O4)
    np.testing.assert_array_equal(L1, L4)



def _bwd(q, k, v, dout, scale, causal, valid_len=None, **mask):
    return oracle.attn_bwd(q, k, v, dout, scale, causal, valid_len, threads=2, **mask)


@pytest.mark.parametrize("pin", oracle_pins.BWD_PINS + oracle_pins.BWD_MASK_PINS,
                         ids=lambda p: p.__name__)
def test_bwd_pin(pin):
    pin(_bwd, _fn)
