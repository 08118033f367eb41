"""GPU parity of dense MLA decode attention with split partials
(mlaq_attn_run) against the oracle's split procedure with the same split
count and partial dtype (b12x PR #441 "Allow FP32 split partials in prepared
dense MLA": partials in BF16 or FP32, BF16 output; its validation checks
error against a higher-precision reference, graph replay and high cache-page
indices).

Bar, per output element, with o the oracle's merged result before the final
rounding (double), vabs = sum_t p_t |v_t|, smag = max_t scale sum_d |q_d k_td|
and u = 2^-24, gamma_n = n u / (1 - n u):
  |gpu - o| <= ulp_bf16(o)                          final bf16 rounding
             + max_s ulp_store(o_s)                 partial storage (a rounding flip)
             + (2^-8 + 4 eps + 4 gamma_T') vabs     bf16 P (2^-9, doubled), score and
                                                    accumulation errors
             + 4 dlse vmax + 2^-20 max|o|           merge weights and fp32 merge
with eps = 2 (gamma_576 + 2^-22) smag + 2^-21 the relative error of one
softmax weight (fp32 score product, scale rounding, exp2), T' = T + 2 tiles
+ 8, dlse = 2^-20 (1 + |lse|) + 2 gamma_T' + eps, vmax = max |v|. The
partials read back from the workspace meet the same bar per range, and per
call rel-L2 ||gpu - o|| / ||o|| <= 4e-3.
"""

import math

import numpy as np
import pytest
import torch

import mla_decode_query_amd as mq
import oracle
from gpu_util import (BF16P, FP32P, assert_attn_parity, attn_oracle_run as oracle_run, dev_bf16, out_bits,
                      read_partials, ulp_bf16)
from workloads import make_attn_inputs

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mq.library()


class Dev:
    """Device copies of one AttnInputs."""

    def __init__(self, inp, kv=None, table=None):
        self.q = dev_bf16(inp.q)
        self.kv = dev_bf16(inp.kv) if kv is None else kv
        self.bt = torch.from_numpy(inp.block_table if table is None else table).cuda()
        self.sl = torch.from_numpy(inp.seq_lens).cuda()
        self.M, self.H = inp.M, inp.H


def run_attn(d, scale, S, pd, q=None, with_ws=False):
    """One call; returns out bits, lse and (optionally) the workspace tensor."""
    out = torch.empty((d.M, d.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((d.M, d.H), dtype=torch.float32, device="cuda")
    n = mq.mlaq_attn_workspace_size(d.M, d.H, S, pd)
    ws = torch.empty((n,), dtype=torch.uint8, device="cuda") if n else None
    mq.mlaq_attn_run(d.q if q is None else q, d.kv, d.bt, d.sl, out, scale, S, pd, ws, lse)
    torch.cuda.synchronize()
    res = (out_bits(out), lse.cpu().numpy().astype(np.float64))
    return res + (ws,) if with_ws else res


_cache = {}


def cached_inputs(seed, H, lens, P=64, **kw):
    key = (seed, H, tuple(lens), P, tuple(sorted(kw.items())))
    if key not in _cache:
        _cache[key] = make_attn_inputs(seed, H, lens, page_size=P, **kw)
    return _cache[key]


RAGGED = [1, 63, 64, 65, 200, 0, 1000, 129]


@pytest.mark.parametrize("pd", [BF16P, FP32P])
@pytest.mark.parametrize("H", [8, 11, 16])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_attn_parity_ragged(pd, H, S):
    inp = cached_inputs(8000 + H, H, RAGGED)
    d = Dev(inp)
    gpu, lse, ws = run_attn(d, inp.softmax_scale, S, pd, with_ws=True)
    assert_attn_parity(gpu, lse, oracle_run(inp, S, pd), inp, S, pd, f"ragged H={H} S={S} pd={pd}", ws)


@pytest.mark.parametrize("H,P,lens", [(1, 64, [300, 7, 64]), (5, 16, [300, 7, 64, 0]), (16, 1, [70, 3]),
                                      (13, 128, [500, 129, 1]), (16, 48, [333, 97])])
def test_attn_heads_and_page_sizes(H, P, lens):
    inp = cached_inputs(8100 + H + P, H, lens, P=P)
    d = Dev(inp)
    for S, pd in ((1, BF16P), (4, BF16P), (4, FP32P)):
        gpu, lse, ws = run_attn(d, inp.softmax_scale, S, pd, with_ws=True)
        assert_attn_parity(gpu, lse, oracle_run(inp, S, pd), inp, S, pd, f"H={H} P={P} S={S} pd={pd}", ws)


def test_attn_decode_batch_full_size():
    """The measured workload: 32 sequences of 4096 cached tokens, 16 heads,
    the library's split count; both partial dtypes. Against the exact split
    partials (over 4 M values), FP32 partials err at least 4x less than BF16
    ones: they keep the softmax weights to 16 bits in the value product and
    store fp32, where BF16 partials round both to bf16."""
    H, M, T = 16, 32, 4096
    inp = cached_inputs(8200, H, [T] * M)
    d = Dev(inp)
    S = mq.mlaq_attn_num_splits(M, T)
    assert S >= 2
    exact = oracle_run(inp, S, oracle.PARTIAL_EXACT)
    perr = {}
    for pd in (BF16P, FP32P):
        gpu, lse, ws = run_attn(d, inp.softmax_scale, S, pd, with_ws=True)
        assert_attn_parity(gpu, lse, oracle_run(inp, S, pd), inp, S, pd, f"full size pd={pd}", ws)
        part, _ = read_partials(ws, M, H, S, pd)
        perr[pd] = np.linalg.norm(part - exact["part"]) / np.linalg.norm(exact["part"])
    assert perr[FP32P] < 0.25 * perr[BF16P], f"partial errors fp32 {perr[FP32P]} vs bf16 {perr[BF16P]}"
    print(f"relative L2 error of the partials against exact ones: fp32 {perr[FP32P]:.3e}, bf16 {perr[BF16P]:.3e}")


def test_attn_long_context():
    """One 65,536-token sequence (the pages' 64k-context decode), 16 heads."""
    H, T = 16, 65536
    inp = cached_inputs(8300, H, [T])
    d = Dev(inp)
    for S in (mq.mlaq_attn_num_splits(1, T), 1):
        gpu, lse, ws = run_attn(d, inp.softmax_scale, S, BF16P, with_ws=True)
        assert_attn_parity(gpu, lse, oracle_run(inp, S, BF16P), inp, S, BF16P, f"64k S={S}", ws)


@pytest.mark.parametrize("S", [1, 2, 5])
@pytest.mark.parametrize("pd", [BF16P, FP32P])
def test_attn_structured_bit_exact(S, pd):
    """q = 0 with every cached row equal: every weight is exactly 1 and every
    partial and the output are that row. A single token gives its row."""
    H = 16
    inp = make_attn_inputs(8400, H, [256, 64, 1, 77])
    inp.q[:2] = 0
    row = inp.kv[inp.block_table[0, 0], 5].copy()
    for m in range(2):
        for b in range(int(math.ceil(inp.seq_lens[m] / 64))):
            inp.kv[inp.block_table[m, b]] = row
    gpu, _ = run_attn(Dev(inp), inp.softmax_scale, S, pd)
    assert np.array_equal(gpu[:2], np.broadcast_to(row[:512], (2, H, 512))), "constant rows"
    assert np.array_equal(gpu[2], np.broadcast_to(inp.kv[inp.block_table[2, 0], 0, :512], (H, 512))), "T = 1"
    ref = oracle_run(inp, S, pd)
    assert np.array_equal(gpu[:3], ref["out"][:3])


def test_attn_rising_and_falling_scores():
    """Cached rows scaled page by page by powers of two (x1, x2, x4, x8 in a
    fixed pattern; exact in bf16, both key and value), so that along each
    range the scores' running maximum rises by less than 8 (log2 units) on
    some tiles and by far more on others, and falls back in between: the
    rescaling of the running sums and outputs is taken mid-range, at several
    split counts and both partial dtypes."""
    H = 16
    inp = make_attn_inputs(8450, H, [4096, 1000, 300])
    pattern = [0, 1, 0, 2, 0, 0, 3, 1]
    for m in range(inp.M):
        for b in range(int(math.ceil(inp.seq_lens[m] / 64))):
            page = inp.kv[inp.block_table[m, b]]
            normal = ((page >> 7) & 0xFF) > 0
            page[normal] += np.uint16(pattern[b % 8] << 7)
    d = Dev(inp)
    for S, pd in ((1, BF16P), (4, BF16P), (4, FP32P), (16, BF16P)):
        gpu, lse, ws = run_attn(d, inp.softmax_scale, S, pd, with_ws=True)
        assert_attn_parity(gpu, lse, oracle_run(inp, S, pd), inp, S, pd, f"scaled pages S={S} pd={pd}", ws)


def test_attn_high_page_indices():
    """A 4.4 GB cache pool (byte offsets past 2^32) with the sequences' pages
    placed at its top end."""
    H = 16
    inp = cached_inputs(8500, H, [1000, 64, 333])
    n_pool = 60000
    pool = torch.zeros((n_pool, 64, 576), dtype=torch.bfloat16, device="cuda")
    used = np.unique(inp.block_table[inp.block_table >= 0])
    remap = {int(p): n_pool - 1 - i for i, p in enumerate(used)}
    for p, hp in remap.items():
        pool[hp] = dev_bf16(inp.kv[p])
    table = np.where(inp.block_table >= 0, np.vectorize(lambda x: remap.get(int(x), -1))(inp.block_table), -1)
    d = Dev(inp, kv=pool, table=table.astype(np.int32))
    for S, pd in ((1, BF16P), (6, FP32P)):
        gpu, lse = run_attn(d, inp.softmax_scale, S, pd)
        assert_attn_parity(gpu, lse, oracle_run(inp, S, pd), inp, S, pd, f"high pages S={S}")
    del pool
    torch.cuda.empty_cache()


def test_attn_strided_query():
    """q inside the fused query's pitched workspace (640-element head pitch),
    and a head-major [H,M,576] q passed as a transposed view."""
    H = 11
    inp = cached_inputs(8600, H, [130, 64, 7])
    d = Dev(inp)
    ref = oracle_run(inp, 3, BF16P)
    ws = torch.zeros((inp.M, H, 640), dtype=torch.bfloat16, device="cuda")
    ws[:, :, :576] = d.q
    gpu, lse = run_attn(d, inp.softmax_scale, 3, BF16P, q=ws[:, :, :576])
    assert_attn_parity(gpu, lse, ref, inp, 3, BF16P, "pitched q")
    qhm = d.q.transpose(0, 1).contiguous()
    gpu2, _ = run_attn(d, inp.softmax_scale, 3, BF16P, q=qhm.transpose(0, 1))
    assert np.array_equal(gpu2, gpu), "head-major q view"


def test_attn_device_values_are_clamped():
    """A sequence length past the block table's capacity acts as the capacity;
    table entries past the live blocks are never used."""
    H = 8
    inp = make_attn_inputs(8700, H, [128, 100], max_blocks=3)
    inp.block_table[1, 2] = inp.block_table[0, 0]  # a live page for the clamped tail
    d = Dev(inp)
    sl = inp.seq_lens.copy()
    sl[1] = 10 ** 6
    d.sl = torch.from_numpy(sl).cuda()
    got, lse = run_attn(d, inp.softmax_scale, 2, BF16P)
    inp.seq_lens = np.array([128, 3 * 64], np.int32)  # what the library must have used
    assert_attn_parity(got, lse, oracle_run(inp, 2, BF16P), inp, 2, BF16P, "clamped length")
    wide = make_attn_inputs(8701, H, [128, 100], max_blocks=6)
    d = Dev(wide)
    base, _ = run_attn(d, wide.softmax_scale, 2, BF16P)
    table = wide.block_table.copy()
    table[table < 0] = 2 ** 30
    d.bt = torch.from_numpy(table).cuda()
    again, _ = run_attn(d, wide.softmax_scale, 2, BF16P)
    assert np.array_equal(again, base)


def test_attn_guard_bytes_and_determinism():
    H = 16
    inp = cached_inputs(8800, H, [500, 3, 0, 64])
    d = Dev(inp)
    S, pd = 4, FP32P
    n = inp.M * H * 512
    buf = torch.full((4096 + n + 4096,), 0x5A5A, dtype=torch.int16, device="cuda")
    out = buf[4096:4096 + n].view(torch.bfloat16).view(inp.M, H, 512)
    need = mq.mlaq_attn_workspace_size(inp.M, H, S, pd)
    wsbuf = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    mq.mlaq_attn_run(d.q, d.kv, d.bt, d.sl, out, inp.softmax_scale, S, pd, wsbuf[:need])
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:4096] == 0x5A5A) and np.all(host[4096 + n:] == 0x5A5A), "out guard bytes"
    assert np.all(wsbuf[need:].cpu().numpy() == 0xA5), "workspace tail"
    first = out_bits(out)
    again, _ = run_attn(d, inp.softmax_scale, S, pd)
    assert np.array_equal(first, again)


def test_attn_graph_replay_with_mutated_inputs():
    """Capture split + merge once; change q, the cache and the lengths in
    place; each replay matches an eager call bit for bit and the oracle."""
    H, S, pd = 16, 4, BF16P
    mq.mlaq_attn_prewarm(pd)
    lens0 = [700, 64, 5]
    pool = 40

    def spare(lens):
        return pool - sum((x + 63) // 64 for x in lens)

    inp = make_attn_inputs(8900, H, lens0, max_blocks=16, spare_pages=spare(lens0))
    d = Dev(inp)
    out = torch.empty((inp.M, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((mq.mlaq_attn_workspace_size(inp.M, H, S, pd),), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st, capture_error_mode="global"):
            mq.mlaq_attn_run(d.q, d.kv, d.bt, d.sl, out, inp.softmax_scale, S, pd, ws)
    torch.cuda.synchronize()
    for seed, lens in ((8900, lens0), (8901, [1000, 1, 333]), (8902, [64, 0, 1024])):
        cur = make_attn_inputs(seed, H, lens, max_blocks=16, spare_pages=spare(lens))
        d.q.copy_(dev_bf16(cur.q))
        d.kv.copy_(dev_bf16(cur.kv))
        d.bt.copy_(torch.from_numpy(cur.block_table))
        d.sl.copy_(torch.from_numpy(cur.seq_lens))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_bits(out)
        eager, lse = run_attn(d, cur.softmax_scale, S, pd)
        assert np.array_equal(got, eager), f"replay {seed} differs from eager"
        assert_attn_parity(got, lse, oracle_run(cur, S, pd), cur, S, pd, f"replay {seed}")


def test_attn_two_streams_at_once():
    """Two calls in flight together on two streams, each with its own
    workspace: the library keeps no state between calls, so each result is
    bit-identical to the same call made alone."""
    H = 16
    a_inp = cached_inputs(8910, H, [1500, 300, 64, 9])
    b_inp = cached_inputs(8911, H, [2000, 7, 640])
    da, db = Dev(a_inp), Dev(b_inp)
    alone_a, _ = run_attn(da, a_inp.softmax_scale, 6, BF16P)
    alone_b, _ = run_attn(db, b_inp.softmax_scale, 3, FP32P)
    outs, wss = [], []
    for d, S, pd in ((da, 6, BF16P), (db, 3, FP32P)):
        outs.append(torch.empty((d.M, H, 512), dtype=torch.bfloat16, device="cuda"))
        wss.append(torch.empty((mq.mlaq_attn_workspace_size(d.M, H, S, pd),), dtype=torch.uint8, device="cuda"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            mq.mlaq_attn_run(da.q, da.kv, da.bt, da.sl, outs[0], a_inp.softmax_scale, 6, BF16P, wss[0])
        with torch.cuda.stream(s2):
            mq.mlaq_attn_run(db.q, db.kv, db.bt, db.sl, outs[1], b_inp.softmax_scale, 3, FP32P, wss[1])
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(outs[0]), alone_a)
        assert np.array_equal(out_bits(outs[1]), alone_b)


def test_attn_can_implement_and_split_heuristic():
    assert mq.mlaq_attn_can_implement(16, 64, 16)
    assert mq.mlaq_attn_can_implement(11, 1, 256, mq.MLAQ_PARTIAL_FP32)
    assert not mq.mlaq_attn_can_implement(17, 64, 16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert mq.mlaq_attn_num_splits(32, 4096) == min(2 * cus // 32, 16)
    assert mq.mlaq_attn_num_splits(1, 65536) == min(2 * cus, 256)
    assert mq.mlaq_attn_num_splits(4 * cus, 65536) == 1
    assert mq.mlaq_attn_num_splits(32, 10) == 1


def test_attn_many_short_sequences():
    """1024 sequences of 0..200 tokens (grid and merge grid at scale)."""
    H = 16
    lens = [int(x) for x in np.random.Generator(np.random.PCG64(8950)).integers(0, 201, 1024)]
    inp = make_attn_inputs(8951, H, lens)
    d = Dev(inp)
    for S, pd in ((1, BF16P), (3, FP32P)):
        gpu, lse = run_attn(d, inp.softmax_scale, S, pd)
        assert_attn_parity(gpu, lse, oracle_run(inp, S, pd), inp, S, pd, f"1024 sequences S={S}")


# (M, H, S) per merge instantiation: the merge kernel takes QN column parts
# (the smallest power of two with 32 QN >= S, doubled while M H QN < 256, at
# most 16) and R ranges per thread (the smallest power of two with
# 4 QN R >= S); these 19 shapes give every reachable (QN, R).
MERGE_SHAPES = [
    (16, 16, 3), (16, 16, 7), (16, 16, 16), (16, 16, 32),     # QN 1, R 1/2/4/8
    (8, 16, 5), (8, 16, 12), (8, 16, 30), (8, 16, 64),        # QN 2
    (4, 16, 16), (4, 16, 20), (4, 16, 50), (4, 16, 128),      # QN 4
    (2, 16, 2), (2, 16, 33), (2, 16, 100), (2, 16, 256),      # QN 8
    (1, 16, 2), (1, 16, 100), (1, 16, 200),                   # QN 16
]


@pytest.mark.parametrize("M,H,S", MERGE_SHAPES)
def test_attn_merge_shapes(M, H, S):
    """Every merge instantiation against the oracle's split procedure: ragged
    lengths near 64 S tokens (most ranges full, the last ones short or
    empty), BF16 partials, and FP32 partials for the larger split counts."""
    lens = [max(1, min(64 * S, 6000) - 37 * i) for i in range(M)]
    inp = cached_inputs(8970 + M + S, H, lens)
    d = Dev(inp)
    for pd in ((BF16P, FP32P) if S >= 64 else (BF16P,)):
        gpu, lse, ws = run_attn(d, inp.softmax_scale, S, pd, with_ws=True)
        assert_attn_parity(gpu, lse, oracle_run(inp, S, pd), inp, S, pd, f"merge M={M} H={H} S={S} pd={pd}", ws)


def test_attn_bad_device_values_give_clamped_results():
    """Negative lengths act as 0 (zeros, lse = -inf); live block-table entries
    below 0 or past the pool read page 0 or the last page, exactly as the
    oracle does on the clamped table."""
    H = 8
    inp = make_attn_inputs(8960, H, [150, 90, 40])
    n_pages = inp.kv.shape[0]
    table = inp.block_table.copy()
    table[0, 1] = -7
    table[1, 0] = n_pages + 5
    sl = inp.seq_lens.copy()
    sl[2] = -5
    d = Dev(inp, table=table)
    d.sl = torch.from_numpy(sl).cuda()
    got, lse = run_attn(d, inp.softmax_scale, 2, BF16P)
    clamped = make_attn_inputs(8960, H, [150, 90, 40])
    clamped.block_table = np.clip(table, 0, n_pages - 1).astype(np.int32)
    clamped.block_table[2] = -1
    clamped.seq_lens = np.array([150, 90, 0], np.int32)
    assert_attn_parity(got, lse, oracle_run(clamped, 2, BF16P), clamped, 2, BF16P, "clamped table")
