"""The fp64 oracle against facts other than itself (see oracle_pins.py)."""

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.attention_fwd)


def test_oracle_row_subset_matches_full():
    from fa_inputs import make_qkv, sample_rows
    import numpy as np
    q, k, v = make_qkv(1, 2, 700, 64, "bf16", 30)
    rows = sample_rows(700, head=5, tail=5, stride=37)
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, causal, 0.125)
        o_r, lse_r = oracle.attention_fwd(q, k, v, causal, 0.125, rows=rows)
        assert np.array_equal(o_r, o[:, :, rows]) and np.array_equal(lse_r, lse[:, :, rows])


def test_oracle_rejects_bad_arguments():
    import numpy as np
    z = np.zeros((1, 1, 4, 8), np.float32)
    with pytest.raises(RuntimeError):
        oracle.attention_fwd(z, z, z, False, 1.0, rows=[4])
    with pytest.raises(RuntimeError):
        oracle.attention_fwd(z, z, z, False, 1.0, tile_n=-1)
