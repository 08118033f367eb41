"""Writes the golden fixtures in this folder. It calls only the CPU oracle
(and the shared seeded input generator); nothing here comes from the HIP path.

Fixture ``c0_h8_m1_bf16.txt``: the smallest decode case, H = 8 heads, M = 1
token, BF16 weights and output, inputs drawn by ``workloads.make_inputs`` with
seed 1000 (shapes from sparkinfer PR #75 "[GG] Add BF16 MLA query projection
and assembly", section "What", with the nope width 128). The file stores the
sha256 of the input bytes (so a drift of the generator is visible) and the
oracle's [1,8,576] output as hex bf16 patterns, one head per line.

Run: python tests/golden/make_golden.py
"""

import hashlib
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
sys.path.insert(0, str(HERE.parents[1]))

import oracle  # noqa: E402
from workloads import SEED, WEIGHT_BF16, make_inputs  # noqa: E402


def input_digest(inp) -> str:
    h = hashlib.sha256()
    for a in (inp.q_nope, inp.w, inp.q_pe):
        h.update(a.tobytes())
    return h.hexdigest()


def c0_fixture_text() -> str:
    inp = make_inputs(SEED["c0"], H=8, weight_format=WEIGHT_BF16, M_draw=1)
    out = oracle.mla_query(inp.q_nope, inp.q_pe, inp.w, diagnostics=False)["out"]
    lines = ["# c0: H=8 M=1 BF16 weights, BF16 output, seed 1000; written by make_golden.py (oracle only)",
             f"inputs_sha256 {input_digest(inp)}"]
    for h in range(8):
        lines.append(" ".join(f"{int(v):04x}" for v in out[0, h]))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    (HERE / "c0_h8_m1_bf16.txt").write_text(c0_fixture_text())
    print("wrote", HERE / "c0_h8_m1_bf16.txt")
