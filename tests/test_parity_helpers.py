"""The parity checks themselves (tests/gpu_util.py) reject what they must, on
the CPU: a NaN code where the oracle saturates to 448, a code two steps away,
a changed q_pe lane; and accept one code step and signed zeros."""

import numpy as np
import pytest

from gpu_util import assert_e4m3_parity

N = 512


def _ref(rng):
    out = rng.integers(0, 256, (2, 3, N + 64), dtype=np.uint8)
    out[(out & 0x7F) == 0x7F] = 0x7E  # no NaN in the reference's projection
    out[0, 0, 5] = 0x7E                # +448
    out[1, 2, 9] = 0xFE                # -448
    out[0, 1, 7] = 0x00                # +0
    return {"out": out}


def test_e4m3_parity_accepts_one_step_and_signed_zero():
    ref = _ref(np.random.default_rng(3))
    got = ref["out"].copy()
    got[0, 1, 7] = 0x80                # -0 for +0
    got[0, 0, 5] = 0x7D                # one step below 448
    assert assert_e4m3_parity(got, ref)["max_code_dist"] <= 1


@pytest.mark.parametrize("where,code", [((0, 0, 5), 0x7F), ((1, 2, 9), 0xFF), ((0, 2, 11), 0x7F)])
def test_e4m3_parity_rejects_nan_for_a_finite_code(where, code):
    ref = _ref(np.random.default_rng(3))
    got = ref["out"].copy()
    got[where] = code
    with pytest.raises(AssertionError, match="NaN"):
        assert_e4m3_parity(got, ref)


def test_e4m3_parity_rejects_two_steps_and_q_pe_change():
    ref = _ref(np.random.default_rng(3))
    ref["out"][1, 1, 100] = 0x14
    got = ref["out"].copy()
    got[1, 1, 100] = 0x12              # two code steps away
    with pytest.raises(AssertionError, match="distance"):
        assert_e4m3_parity(got, ref)
    got = ref["out"].copy()
    got[0, 0, N + 3] ^= 1              # one q_pe bit
    with pytest.raises(AssertionError, match="q_pe"):
        assert_e4m3_parity(got, ref)
