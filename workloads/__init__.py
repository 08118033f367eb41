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

Dense MLA decode attention (``make_attn_inputs``): M sequences with one query
each and ragged cached lengths, a paged latent cache of 576-wide rows (512
latent, then 64 rotary) and a block table that scatters each sequence's pages
over the pool in random order (so page indices run high and out of order; the
vLLM page's serving check covers high cache-page indices). Recipe, in order:
  1. q   ~ N(0, q_std), fp32, then bf16                       [M, H, 576]
  2. kv  ~ N(0, kv_std), fp32, then bf16                      [num_pages, P, 576]
  3. a permutation of the num_pages physical pages; sequence m takes the next
     ceil(T_m / P) of them in order; unused table entries are -1.
softmax_scale defaults to 1/sqrt(192) (128 nope + 64 rope dims per head). The
pages' serving runs (4096-token outputs, 64k contexts) stand in as lengths.
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


D_ROW = N_LATENT + R_ROPE
ATTN_PAGE = 64
PARTIAL_BF16, PARTIAL_FP32 = 0, 1


@dataclasses.dataclass
class AttnInputs:
    """Host bit patterns of one decode-attention batch."""

    q: np.ndarray  # uint16 [M,H,576]
    kv: np.ndarray  # uint16 [num_pages,P,576]
    block_table: np.ndarray  # int32 [M,max_blocks], -1 where unused
    seq_lens: np.ndarray  # int32 [M]
    softmax_scale: float
    seed: int

    @property
    def M(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def page_size(self):
        return self.kv.shape[1]


def make_attn_inputs(seed: int, H: int, seq_lens, page_size: int = ATTN_PAGE, spare_pages: int = 2,
                     max_blocks: int | None = None, q_std: float = 1.0, kv_std: float = 1.0,
                     softmax_scale: float = 192.0 ** -0.5) -> AttnInputs:
    """Draw one seeded decode-attention batch (recipe in the module docstring)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(seq_lens, np.int64)
    M = lens.shape[0]
    blocks = (lens + page_size - 1) // page_size
    total = int(blocks.sum())
    num_pages = total + spare_pages
    if max_blocks is None:
        max_blocks = max(int(blocks.max()) if M else 0, 1)
    q = _bf16_bits(rng.standard_normal((M, H, D_ROW), dtype=np.float32) * np.float32(q_std))
    kv = np.empty((num_pages, page_size, D_ROW), np.uint16)
    step = max(1, (1 << 24) // (page_size * D_ROW))  # draw in slabs of about 16M values
    for p0 in range(0, num_pages, step):
        p1 = min(num_pages, p0 + step)
        kv[p0:p1] = _bf16_bits(rng.standard_normal((p1 - p0, page_size, D_ROW), dtype=np.float32)
                               * np.float32(kv_std))
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((M, max_blocks), -1, np.int32)
    nxt = 0
    for m in range(M):
        b = int(blocks[m])
        table[m, :b] = perm[nxt:nxt + b]
        nxt += b
    return AttnInputs(q=q, kv=kv, block_table=table, seq_lens=lens.astype(np.int32),
                      softmax_scale=float(softmax_scale), seed=seed)


def attn_algorithmic_bytes(seq_lens, H: int, page_size: int = ATTN_PAGE) -> int:
    """Bytes one attention call must move, each counted once: every cached row
    of every sequence (576 bf16), the queries, the block-table entries in use,
    the sequence lengths and the bf16 [M,H,512] output. Split partials are
    the implementation's own traffic and are not counted."""
    lens = np.asarray(seq_lens, np.int64)
    M = lens.shape[0]
    blocks = int(((lens + page_size - 1) // page_size).sum())
    return int(lens.sum()) * D_ROW * 2 + M * H * D_ROW * 2 + blocks * 4 + M * 4 + M * H * N_LATENT * 2
