"""GPU test of the allocation-free attention entry point
(mlaq_attn_run_noalloc): its partials live in the library's device scratch
array instead of a caller workspace, and its output must be the output of
mlaq_attn_run (caller workspace) on the same inputs, bit for bit, and within
the oracle's parity bar. Two calls in a row on one device, the second with a
smaller input (fewer sequences, heads and splits, the other partial dtype),
so the second call runs over what the first left in the array; then a
one-split call (no scratch used) and a graph replay of the entry point."""

import numpy as np
import pytest
import torch

import mla_decode_query_amd as mq
from gpu_util import BF16P, FP32P, assert_attn_parity, attn_oracle_run, dev_bf16, out_bits
from workloads import make_attn_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mq.library()


class Dev:
    def __init__(self, inp):
        self.q = dev_bf16(inp.q)
        self.kv = dev_bf16(inp.kv)
        self.bt = torch.from_numpy(inp.block_table).cuda()
        self.sl = torch.from_numpy(inp.seq_lens).cuda()
        self.M, self.H = inp.M, inp.H


def _with_workspace(d, scale, S, pd):
    out = torch.empty((d.M, d.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((d.M, d.H), dtype=torch.float32, device="cuda")
    n = mq.mlaq_attn_workspace_size(d.M, d.H, S, pd)
    ws = torch.empty((n,), dtype=torch.uint8, device="cuda") if n else None
    mq.mlaq_attn_run(d.q, d.kv, d.bt, d.sl, out, scale, S, pd, ws, lse)
    torch.cuda.synchronize()
    return out_bits(out), lse.cpu().numpy()


def _noalloc(d, scale, S, pd):
    out = torch.empty((d.M, d.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((d.M, d.H), dtype=torch.float32, device="cuda")
    mq.mlaq_attn_run_noalloc(d.q, d.kv, d.bt, d.sl, out, scale, S, pd, lse)
    torch.cuda.synchronize()
    return out_bits(out), lse.cpu().numpy()


CASES = [
    # (seed, H, lengths, splits, partial dtype): the second is smaller in every dimension.
    (7101, 16, [1000, 4096, 63, 0, 129, 2000, 64, 1], 8, BF16P),
    (7102, 8, [70, 1, 300], 3, FP32P),
]


def test_noalloc_matches_workspace_entry_point_twice_in_a_row():
    inputs = [make_attn_inputs(seed, H, lens) for seed, H, lens, _, _ in CASES]
    devs = [Dev(inp) for inp in inputs]
    # Both calls first, back to back on the array, then the comparisons.
    got = [_noalloc(d, inp.softmax_scale, S, pd) for d, inp, (_, _, _, S, pd) in zip(devs, inputs, CASES)]
    for (seed, H, lens, S, pd), d, inp, (g_out, g_lse) in zip(CASES, devs, inputs, got):
        w_out, w_lse = _with_workspace(d, inp.softmax_scale, S, pd)
        assert np.array_equal(g_out, w_out), f"seed {seed}: output differs from mlaq_attn_run"
        assert np.array_equal(g_lse.view(np.uint32), w_lse.view(np.uint32)), f"seed {seed}: lse differs"
        ref = attn_oracle_run(inp, S, pd)
        assert_attn_parity(g_out, g_lse.astype(np.float64), ref, inp, S, pd, f"noalloc seed {seed}")


def test_noalloc_one_split_and_repeat_after_larger_call():
    # One split writes the output directly (no scratch); then the larger plan
    # again, after the array holds the smaller call's partials.
    seed, H, lens, S, pd = CASES[1]
    inp = make_attn_inputs(seed, H, lens)
    d = Dev(inp)
    assert np.array_equal(_noalloc(d, inp.softmax_scale, 1, pd)[0], _with_workspace(d, inp.softmax_scale, 1, pd)[0])
    seed, H, lens, S, pd = CASES[0]
    inp = make_attn_inputs(seed, H, lens)
    d = Dev(inp)
    a = _noalloc(d, inp.softmax_scale, S, pd)
    b = _with_workspace(d, inp.softmax_scale, S, pd)
    assert np.array_equal(a[0], b[0])


def test_noalloc_graph_replay():
    seed, H, lens, S, pd = CASES[0]
    inp = make_attn_inputs(seed, H, lens)
    d = Dev(inp)
    want = _with_workspace(d, inp.softmax_scale, S, pd)[0]
    out = torch.empty((d.M, d.H, 512), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        mq.mlaq_attn_run_noalloc(d.q, d.kv, d.bt, d.sl, out, inp.softmax_scale, S, pd, None, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mq.mlaq_attn_run_noalloc(d.q, d.kv, d.bt, d.sl, out, inp.softmax_scale, S, pd, None, s)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), want), f"replay {rep}"


def test_noalloc_rejects_a_plan_beyond_the_array():
    inp = make_attn_inputs(7103, 16, [64] * 40)
    d = Dev(inp)
    out = torch.empty((d.M, d.H, 512), dtype=torch.bfloat16, device="cuda")
    assert mq.mlaq_attn_workspace_size(40, 16, 64, FP32P) > mq.MLAQ_ATTN_SCRATCH_BYTES
    with pytest.raises(mq.MlaqError, match="bytes of scratch"):
        mq.mlaq_attn_run_noalloc(d.q, d.kv, d.bt, d.sl, out, inp.softmax_scale, 64, FP32P)
