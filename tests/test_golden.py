"""The stored c0 fixture (written by tests/golden/make_golden.py from the
oracle alone) still matches the generator and the oracle."""

from pathlib import Path

import numpy as np

from golden.make_golden import c0_fixture_text

GOLDEN = Path(__file__).resolve().parent / "golden" / "c0_h8_m1_bf16.txt"


def load_c0():
    lines = [l for l in GOLDEN.read_text().splitlines() if l and not l.startswith("#")]
    digest = lines[0].split()[1]
    out = np.array([[int(t, 16) for t in l.split()] for l in lines[1:]], np.uint16)[None]
    return digest, out


def test_c0_golden_unchanged():
    assert GOLDEN.read_text() == c0_fixture_text()
    digest, out = load_c0()
    assert out.shape == (1, 8, 576)
