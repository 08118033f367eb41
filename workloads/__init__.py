"""Seeded synthetic inputs for the fused MLA decode query projection.

Shared by the tests, the smoke check and the benchmark; both the CPU oracle
and the HIP path consume exactly these bytes. This module holds none of the
method's arithmetic: it draws random numbers with numpy's PCG64 and turns
them into bf16 / E4M3 bit patterns with torch's own CPU casts (library
conversions, round-to-nearest-even), and E8M0 scale bytes as plain integers.

Shapes and distributions follow the pages' per-rank decode shapes: heads
H in {8, 11, 16} (TP8, TP6 with 66 padded heads, TP4 of a 64-head model),
M = 1..32 tokens, nope dim K = 128, latent N = 512, rope R = 64
(sparkinfer PR #75 "[GG] Add BF16 MLA query projection and assembly",
sections "What" and "Validation"; vLLM PR #174 "[GG] Fuse MXFP8 and BF16 MLA
query assembly", sections "What" and "Layout and topology behavior"). The
pages measure live serving of trained checkpoints; these synthetic tensors
stand in for them.

Recipe (all draws from ``numpy.random.Generator(PCG64(seed))`` in this order):
  1. q_nope  ~ N(0, 1), fp32, then bf16                      [M_draw, H, K]
  2. BF16 W  ~ N(0, 1/sqrt(K)) (standard deviation), bf16      [H, K, N]
     MXFP8 W: payload ~ N(0, 1/sqrt(K)) cast to E4M3FN       [H, K, N]
              then scale exponent e ~ U{-8..0}, byte 127 + e   [H, K, N/32]
  3. q_pe    ~ N(0, 1), fp32, then bf16                       [M_draw, H, R]
The M sweep draws at ``M_draw`` (default 32) and a call with M tokens uses
the first M rows, so one seed serves every M of a sweep.
"""

from __future__ import annotations

import dataclasses

import numpy as np

K_NOPE, N_LATENT, R_ROPE, MX_BLOCK = 128, 512, 64, 32
WEIGHT_BF16, WEIGHT_MXFP8 = 0, 1
OUT_BF16, OUT_E4M3 = 0, 1

# Seeds of the named workloads: 1000 + workload index.
SEED = {"c0": 1000, "c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004}


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _e4m3_bits(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


@dataclasses.dataclass
class Inputs:
    """Host bit patterns of one weight set plus a token batch."""

    q_nope: np.ndarray  # uint16 [M,H,K]
    q_pe: np.ndarray  # uint16 [M,H,R]
    w: np.ndarray  # uint16 [H,K,N] (bf16) or uint8 [H,K,N] (E4M3)
    w_scales: np.ndarray | None  # uint8 [H,K,N/32] or None
    weight_format: int
    seed: int

    @property
    def M(self):
        return self.q_nope.shape[0]

    @property
    def H(self):
        return self.q_nope.shape[1]

    def take(self, M: int) -> "Inputs":
        """The first M tokens of the batch (same weights)."""
        if not 0 <= M <= self.M:
            raise ValueError(f"M={M} outside 0..{self.M}")
        return dataclasses.replace(self, q_nope=self.q_nope[:M].copy(), q_pe=self.q_pe[:M].copy())


def make_inputs(seed: int, H: int, weight_format: int, M_draw: int = 32, K: int = K_NOPE,
                N: int = N_LATENT, R: int = R_ROPE) -> Inputs:
    """Draw one seeded input set (see the module docstring for the recipe)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((M_draw, H, K), dtype=np.float32)
    std = np.float32(1.0 / np.sqrt(K))
    if weight_format == WEIGHT_BF16:
        w = _bf16_bits(rng.standard_normal((H, K, N), dtype=np.float32) * std)
        s = None
    elif weight_format == WEIGHT_MXFP8:
        w = _e4m3_bits(rng.standard_normal((H, K, N), dtype=np.float32) * std)
        s = (127 + rng.integers(-8, 1, size=(H, K, N // MX_BLOCK))).astype(np.uint8)
    else:
        raise ValueError(f"unknown weight format {weight_format}")
    pe = rng.standard_normal((M_draw, H, R), dtype=np.float32)
    return Inputs(q_nope=_bf16_bits(q), q_pe=_bf16_bits(pe), w=w, w_scales=s,
                  weight_format=weight_format, seed=seed)


def bf16_bits(x) -> np.ndarray:
    """fp32 values -> bf16 bit patterns via torch's cast (for hand-built inputs)."""
    return _bf16_bits(np.asarray(x, np.float32))


def e4m3_bits(x) -> np.ndarray:
    """fp32 values -> E4M3FN codes via torch's cast (for hand-built inputs)."""
    return _e4m3_bits(np.asarray(x, np.float32))


def algorithmic_bytes(M: int, H: int, weight_format: int, out_dtype: int, K: int = K_NOPE,
                      N: int = N_LATENT, R: int = R_ROPE) -> int:
    """Bytes one call must move, each counted once: weights (+ E8M0 scales),
    q_nope, q_pe, the [M,H,N+R] output, and the 4-byte q_scale for E4M3 output."""
    wb = H * K * N * (2 if weight_format == WEIGHT_BF16 else 1)
    sb = H * K * (N // MX_BLOCK) if weight_format == WEIGHT_MXFP8 else 0
    ob = M * H * (N + R) * (2 if out_dtype == OUT_BF16 else 1)
    return wb + sb + M * H * K * 2 + M * H * R * 2 + ob + (4 if out_dtype == OUT_E4M3 else 0)
