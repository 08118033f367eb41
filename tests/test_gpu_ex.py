"""GPU parity of mlaq_run_ex: the GLM nope width K = 192 (sparkinfer PR #75
"[GG] Add BF16 MLA query projection and assembly", section "What") and
strided views -- a head-major q_nope (the page's [H,M,K] batch view) and
pitched output workspaces (its "Validation" section lists pitched outputs;
vLLM PR #174 "[GG] Fuse MXFP8 and BF16 MLA query assembly", "Layout and
topology behavior", writes straight into the attention backend's workspace).
Same parity bar as tests/test_gpu_parity.py; the oracle always gets contiguous
copies."""

import numpy as np
import pytest
import torch

import mla_decode_query_amd as mq
import oracle
from gpu_util import assert_bf16_parity, assert_e4m3_parity, dev_bf16, dev_u8, out_bits, run_oracle
from workloads import SEED, WEIGHT_BF16, WEIGHT_MXFP8, bf16_bits, make_inputs

pytestmark = pytest.mark.gpu

BF16, E4M3 = mq.MLAQ_OUT_BF16, mq.MLAQ_OUT_E4M3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mq.library()


_cache = {}


def inputs(seed, H, wf, K):
    key = (seed, H, wf, K)
    if key not in _cache:
        _cache[key] = make_inputs(seed, H=H, weight_format=wf, M_draw=32, K=K)
    return _cache[key]


def weights(inp):
    if inp.weight_format == WEIGHT_BF16:
        return dev_bf16(inp.w), None
    return dev_u8(inp.w), dev_u8(inp.w_scales)


def run_contiguous(inp, od, qs=None):
    w, s = weights(inp)
    q, pe = dev_bf16(inp.q_nope), dev_bf16(inp.q_pe)
    out = torch.empty((inp.M, inp.H, mq.ROW), dtype=torch.bfloat16 if od == BF16 else torch.uint8, device="cuda")
    qt = None if qs is None else torch.tensor([qs], dtype=torch.float32, device="cuda")
    mq.mlaq_run_ex(q, pe, w, s, qt, out, inp.weight_format, od)
    torch.cuda.synchronize()
    return out_bits(out)


@pytest.mark.parametrize("wf", [WEIGHT_BF16, WEIGHT_MXFP8])
@pytest.mark.parametrize("H", [8, 11, 16])
@pytest.mark.parametrize("M", [1, 4, 6, 17, 32])
def test_k192_bf16_out(wf, H, M):
    inp = inputs(SEED["c1"] + 100, H, wf, 192).take(M)
    assert_bf16_parity(run_contiguous(inp, BF16), run_oracle(inp, BF16), f"K=192 wf={wf} H={H} M={M}")


@pytest.mark.parametrize("wf", [WEIGHT_BF16, WEIGHT_MXFP8])
@pytest.mark.parametrize("H", [8, 16])
@pytest.mark.parametrize("M", [1, 9, 32])
def test_k192_e4m3_out(wf, H, M):
    inp = inputs(SEED["c4"] + 100, H, wf, 192).take(M)
    base = run_oracle(inp, BF16)
    qs = oracle.qscale_from_result(base["acc"], inp.q_pe)
    assert_e4m3_parity(run_contiguous(inp, E4M3, qs), run_oracle(inp, E4M3, qs), f"K=192 e4m3 wf={wf} H={H} M={M}")


@pytest.mark.parametrize("M", [9, 32])
def test_k192_structured_bit_exact(M):
    """Identity weights (W[h,k,n] = 1 iff n = k + 64 (h mod 5)) and the all-ones
    MXFP8 payload with E8M0 bytes 127 - ((h+k+j) mod 9): exact in any order
    (M = 9: one token tile, whose waves hold three k-blocks each)."""
    H, K = 16, 192
    rng = np.random.Generator(np.random.PCG64(901))
    q = bf16_bits(rng.standard_normal((M, H, K), dtype=np.float32))
    pe = bf16_bits(rng.standard_normal((M, H, 64), dtype=np.float32))
    w = np.zeros((H, K, 512), np.uint16)
    for h in range(H):
        w[h, np.arange(K), np.arange(K) + 64 * (h % 5)] = 0x3F80

    class I:
        pass

    a = I()
    a.q_nope, a.q_pe, a.w, a.w_scales, a.weight_format, a.M, a.H = q, pe, w, None, WEIGHT_BF16, M, H
    assert np.array_equal(run_contiguous(a, BF16), run_oracle(a, BF16)["out"])
    b = I()
    hh, kk, jj = np.meshgrid(np.arange(H), np.arange(K), np.arange(16), indexing="ij")
    qk = bf16_bits(np.array([2.0 ** -(k % 4) for k in range(K)], np.float32))
    b.q_nope = np.broadcast_to(qk, (M, H, K)).copy()
    b.q_pe, b.w, b.w_scales = pe, np.full((H, K, 512), 0x38, np.uint8), (127 - (hh + kk + jj) % 9).astype(np.uint8)
    b.weight_format, b.M, b.H = WEIGHT_MXFP8, M, H
    assert np.array_equal(run_contiguous(b, BF16), run_oracle(b, BF16)["out"])


@pytest.mark.parametrize("K", [128, 192])
@pytest.mark.parametrize("wf,od,M", [(WEIGHT_BF16, BF16, 1), (WEIGHT_BF16, E4M3, 17), (WEIGHT_MXFP8, BF16, 32),
                                     (WEIGHT_MXFP8, E4M3, 6)])
@pytest.mark.parametrize("out_layout", ["token_major_pitched", "head_major_pitched"])
def test_head_major_q_and_pitched_out(K, wf, od, M, out_layout):
    """q_nope and q_pe stored head-major ([H,M,*] storage, passed as transposed
    views); the output written into a wider workspace (row pitch 640 elements,
    token- or head-major). Padding and everything outside the rows stay
    untouched."""
    H = 11
    inp = inputs(SEED["c2"] + 200, H, wf, K).take(M)
    q_hm = dev_bf16(np.ascontiguousarray(inp.q_nope.transpose(1, 0, 2)))  # [H,M,K] storage
    pe_hm = dev_bf16(np.ascontiguousarray(inp.q_pe.transpose(1, 0, 2)))
    q, pe = q_hm.transpose(0, 1), pe_hm.transpose(0, 1)  # [M,H,*] views
    w, s = weights(inp)
    dt = torch.bfloat16 if od == BF16 else torch.uint8
    pitch = 640
    if out_layout == "token_major_pitched":
        ws = torch.full((M, H, pitch), 0, dtype=dt, device="cuda")
        out = ws[:, :, :mq.ROW]
    else:
        ws = torch.full((H, M, pitch), 0, dtype=dt, device="cuda")
        out = ws.transpose(0, 1)[:, :, :mq.ROW]
    canary = 0x5A5A if od == BF16 else 0x5A
    (ws.view(torch.int16) if od == BF16 else ws).fill_(canary)
    qs_val = 0.03 if od == E4M3 else None
    qs = None if qs_val is None else torch.tensor([qs_val], dtype=torch.float32, device="cuda")
    mq.mlaq_run_ex(q, pe, w, s, qs, out, wf, od)
    torch.cuda.synchronize()
    got = out_bits(out.contiguous())
    ref = run_oracle(inp, od, qs_val)
    if od == BF16:
        assert_bf16_parity(got, ref, f"strided K={K}")
    else:
        assert_e4m3_parity(got, ref, f"strided K={K}")
    pad = out_bits(ws[..., mq.ROW:].contiguous())
    assert np.all(pad == canary), "pitch padding was written"


def test_ex_and_run_agree_bitwise():
    """K = 128, contiguous: both entry points launch the same kernel."""
    inp = inputs(SEED["c1"], 16, WEIGHT_MXFP8, 128).take(20)
    w, s = weights(inp)
    q, pe = dev_bf16(inp.q_nope), dev_bf16(inp.q_pe)
    qs = torch.tensor([0.02], dtype=torch.float32, device="cuda")
    o1 = torch.empty((20, 16, mq.ROW), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    mq.mlaq_run(q, pe, w, s, qs, o1, WEIGHT_MXFP8, E4M3)
    mq.mlaq_run_ex(q, pe, w, s, qs, o2, WEIGHT_MXFP8, E4M3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_k192_graph_replay_with_strided_views():
    """Capture mlaq_run_ex (K = 192, head-major q, pitched out) once; change the
    inputs in place and replay; each replay matches the oracle and an eager call."""
    H, M, K, wf = 8, 4, 192, WEIGHT_BF16
    mq.mlaq_prewarm(H, [M], wf, BF16)
    first = make_inputs(3000, H=H, weight_format=wf, M_draw=M, K=K)
    q_hm = dev_bf16(np.ascontiguousarray(first.q_nope.transpose(1, 0, 2)))
    pe = dev_bf16(first.q_pe)
    w, _ = weights(first)
    ws = torch.zeros((M, H, 640), dtype=torch.bfloat16, device="cuda")
    out = ws[:, :, :mq.ROW]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st, capture_error_mode="global"):
            mq.mlaq_run_ex(q_hm.transpose(0, 1), pe, w, None, None, out, wf, BF16)
    torch.cuda.synchronize()
    for rep, seed in enumerate([3000, 3001, 3002]):
        cur = make_inputs(seed, H=H, weight_format=wf, M_draw=M, K=K)
        q_hm.copy_(dev_bf16(np.ascontiguousarray(cur.q_nope.transpose(1, 0, 2))))
        pe.copy_(dev_bf16(cur.q_pe))
        w.copy_(dev_bf16(cur.w))
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_bits(out.contiguous())
        assert_bf16_parity(got, run_oracle(cur, BF16), f"replay {rep}")
        ws2 = torch.zeros_like(ws)
        mq.mlaq_run_ex(q_hm.transpose(0, 1), pe, w, None, None, ws2[:, :, :mq.ROW], wf, BF16)
        torch.cuda.synchronize()
        assert torch.equal(ws2, ws)


@pytest.mark.parametrize("K", [128, 192])
@pytest.mark.parametrize("od", [BF16, E4M3])
@pytest.mark.parametrize("wf", [WEIGHT_BF16, WEIGHT_MXFP8])
def test_stream_cache_hint(wf, od, K):
    """MLAQ_CACHE_STREAM (nontemporal weight loads and output stores for BF16
    weights; the ordinary kernels for MXFP8) changes timing only: every head
    count and both token tiles give the oracle's parity and the bits of the
    default hint, into a pitched output whose padding stays untouched."""
    qs_val = 0.03
    for H in (8, 11, 16):
        for M in (1, 9, 17, 32):
            inp = inputs(SEED["c2"] + 7, H, wf, K).take(M)
            w, s = weights(inp)
            q, pe = dev_bf16(inp.q_nope), dev_bf16(inp.q_pe)
            qt = None if od == BF16 else torch.tensor([qs_val], dtype=torch.float32, device="cuda")
            dt = torch.bfloat16 if od == BF16 else torch.uint8
            canary = 0x5A5A if od == BF16 else 0x5A
            outs = []
            for hint in (mq.MLAQ_CACHE_DEFAULT, mq.MLAQ_CACHE_STREAM):
                ws = torch.full((M, H, 640), canary, dtype=torch.int16 if od == BF16 else torch.uint8,
                                device="cuda").view(dt)
                mq.mlaq_run_ex(q, pe, w, s, qt, ws[:, :, :mq.ROW], wf, od, cache_hint=hint)
                outs.append(ws)
            torch.cuda.synchronize()
            tag = f"stream hint wf={wf} od={od} K={K} H={H} M={M}"
            assert torch.equal(outs[0], outs[1]), tag + ": differs from the default hint"
            got = out_bits(outs[1][:, :, :mq.ROW].contiguous())
            if od == BF16:
                assert_bf16_parity(got, run_oracle(inp, od), tag)
            else:
                assert_e4m3_parity(got, run_oracle(inp, od, qs_val), tag)
            pad = out_bits(outs[1][:, :, mq.ROW:].contiguous())
            assert np.all(pad == canary), tag + ": pitch padding was written"


def test_stream_hint_output_seen_by_the_next_kernel():
    """The nontemporal stores of the streaming kernels are visible to the next
    kernel on the stream: a graph of fused calls (BF16 weights, streaming
    hint), each followed at once by a copy kernel reading the fresh output,
    replayed with new inputs; every copy equals the oracle's result."""
    H, M = 16, 32
    first = inputs(SEED["c1"] + 11, H, WEIGHT_BF16, 128)
    q, pe = dev_bf16(first.q_nope), dev_bf16(first.q_pe)
    w, _ = weights(first)
    qs = torch.tensor([0.02], dtype=torch.float32, device="cuda")
    outs = [torch.empty((M, H, mq.ROW), dtype=torch.uint8, device="cuda") for _ in range(2)]
    seen = [torch.empty_like(o) for o in outs]
    mq.mlaq_prewarm(H, [M], WEIGHT_BF16, E4M3)
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st, capture_error_mode="global"):
            for o, s in zip(outs, seen):
                mq.mlaq_run_ex(q, pe, w, None, qs, o, WEIGHT_BF16, E4M3, cache_hint=mq.MLAQ_CACHE_STREAM)
                s.copy_(o)
    torch.cuda.synchronize()
    for rep, seed in enumerate([SEED["c1"] + 12, SEED["c1"] + 13, SEED["c1"] + 12]):
        cur = make_inputs(seed, H=H, weight_format=WEIGHT_BF16, M_draw=M)
        q.copy_(dev_bf16(cur.q_nope))
        pe.copy_(dev_bf16(cur.q_pe))
        w.copy_(dev_bf16(cur.w))
        for o, s in zip(outs, seen):
            o.fill_(0xAA)
            s.fill_(0x55)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = run_oracle(cur, E4M3, 0.02)
        for i, s in enumerate(seen):
            assert_e4m3_parity(out_bits(s), ref, f"replay {rep}, consumer copy {i}")
