"""GPU parity of the V up-projection (mlaq_uv_run) against the oracle:
out[m,h,v] = bf16(sum_c x[m,h,c] W_UV[h,v,c]), c < 512, v < 128. Seeded inputs
(x ~ N(0,1) bf16, W_UV ~ N(0, 1/sqrt(512)) bf16 or E4M3 with E8M0 exponents
U{-8..0}) for H = 8/11/16 and M = 1..32, structured cases bit-exact, output
canaries, graph replay with mutated inputs. Bar: |gpu - acc| <= 2 ulp_bf16(acc)
+ 2 gamma_512 sum|x w| per element, rel-L2 <= 4e-3."""

import numpy as np
import pytest
import torch

import mla_decode_query_amd as mq
import oracle
from gpu_util import assert_uv_parity, dev_bf16, dev_u8, out_bits
from workloads import WEIGHT_BF16, WEIGHT_MXFP8, bf16_bits, e4m3_bits

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mq.library()


def uv_inputs(seed, H, wf, M=32):
    """Seeded UV inputs (the recipe of workloads.make_inputs, with the latent
    as the reduction axis): x, then W_UV (payload then scales)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = bf16_bits(rng.standard_normal((M, H, 512), dtype=np.float32))
    std = np.float32(512 ** -0.5)
    if wf == WEIGHT_BF16:
        return x, bf16_bits(rng.standard_normal((H, 128, 512), dtype=np.float32) * std), None
    w = e4m3_bits(rng.standard_normal((H, 128, 512), dtype=np.float32) * std)
    s = (127 + rng.integers(-8, 1, size=(H, 128, 16))).astype(np.uint8)
    return x, w, s


def run_uv(x, w, s, wf, out=None):
    xd = dev_bf16(x)
    wd = dev_bf16(w) if wf == WEIGHT_BF16 else dev_u8(w)
    sd = None if s is None else dev_u8(s)
    if out is None:
        out = torch.empty((x.shape[0], x.shape[1], 128), dtype=torch.bfloat16, device="cuda")
    mq.mlaq_uv_run(xd, wd, sd, out, wf)
    torch.cuda.synchronize()
    return out_bits(out)


_cache = {}


@pytest.mark.parametrize("wf", [WEIGHT_BF16, WEIGHT_MXFP8])
@pytest.mark.parametrize("H", [8, 11, 16])
@pytest.mark.parametrize("M", [1, 2, 5, 8, 16, 17, 31, 32])
def test_uv_parity(wf, H, M):
    key = (wf, H)
    if key not in _cache:
        _cache[key] = uv_inputs(5000 + 10 * H + wf, H, wf)
    x, w, s = _cache[key]
    x = x[:M].copy()
    ref = oracle.uv_projection(x, w, s, weight_format=wf)
    assert_uv_parity(run_uv(x, w, s, wf), ref, f"uv wf={wf} H={H} M={M}")


@pytest.mark.parametrize("M", [1, 32])
def test_uv_structured_bit_exact(M):
    H = 16
    rng = np.random.Generator(np.random.PCG64(77))
    x = bf16_bits(rng.standard_normal((M, H, 512), dtype=np.float32))
    w = np.zeros((H, 128, 512), np.uint16)
    for h in range(H):
        w[h, np.arange(128), np.arange(128) + 128 * (h % 4)] = 0x3F80
    assert np.array_equal(run_uv(x, w, None, WEIGHT_BF16), oracle.uv_projection(x, w)["out"])
    # all-ones E4M3 payload, E8M0 bytes 127 - ((h+v+j) mod 9), x = 2^-(c mod 4): exact sums
    w8 = np.full((H, 128, 512), 0x38, np.uint8)
    hh, vv, jj = np.meshgrid(np.arange(H), np.arange(128), np.arange(16), indexing="ij")
    s8 = (127 - (hh + vv + jj) % 9).astype(np.uint8)
    xk = bf16_bits(np.array([2.0 ** -(c % 4) for c in range(512)], np.float32))
    xs = np.broadcast_to(xk, (M, H, 512)).copy()
    assert np.array_equal(run_uv(xs, w8, s8, WEIGHT_MXFP8),
                          oracle.uv_projection(xs, w8, s8, weight_format=WEIGHT_MXFP8)["out"])


def test_uv_e4m3_decode_exhaustive():
    """Every E4M3 code through a one-hot x (x[c0] = 1): out[v] is the exact
    bf16 of decode(code) * 2^(S-127) for the code placed at (v, c0)."""
    H, M, c0 = 16, 1, 37
    w = np.zeros((H, 128, 512), np.uint8)
    s = np.full((H, 128, 16), 127, np.uint8)
    for h in range(H):
        w[h, :, c0] = np.arange(128, dtype=np.uint8) + (128 if h % 2 else 0)
        s[h, :, c0 // 32] = [119, 121, 123, 125, 127, 129, 10, 246][h % 8]
    x = np.zeros((M, H, 512), np.uint16)
    x[:, :, c0] = 0x3F80
    gpu = run_uv(x, w, s, WEIGHT_MXFP8)
    ref = oracle.uv_projection(x, w, s, weight_format=WEIGHT_MXFP8)["out"]
    nan_ref = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    nan_gpu = ((gpu & 0x7F80) == 0x7F80) & ((gpu & 0x7F) != 0)
    assert np.array_equal(nan_ref, nan_gpu)
    assert np.array_equal(gpu[~nan_ref], ref[~nan_ref])


def test_uv_guard_bytes_and_determinism():
    H, M = 11, 7
    x, w, s = uv_inputs(6001, H, WEIGHT_MXFP8, M=M)
    n = M * H * 128
    buf = torch.full((4096 + n + 4096,), 0x5A5A, dtype=torch.int16, device="cuda")
    out = buf[4096:4096 + n].view(torch.bfloat16).view(M, H, 128)
    a = run_uv(x, w, s, WEIGHT_MXFP8, out=out)
    host = buf.cpu().numpy()
    assert np.all(host[:4096] == 0x5A5A) and np.all(host[4096 + n:] == 0x5A5A)
    assert np.array_equal(run_uv(x, w, s, WEIGHT_MXFP8), a)
    assert_uv_parity(a, oracle.uv_projection(x, w, s, weight_format=WEIGHT_MXFP8), "guard")


def test_uv_graph_replay_with_mutated_inputs():
    H, M, wf = 16, 8, WEIGHT_BF16
    mq.mlaq_uv_prewarm(H, [M], wf)
    x0, w0, _ = uv_inputs(7000, H, wf, M=M)
    xd, wd = dev_bf16(x0), dev_bf16(w0)
    out = torch.empty((M, H, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st, capture_error_mode="global"):
            mq.mlaq_uv_run(xd, wd, None, out, wf)
    torch.cuda.synchronize()
    for seed in (7000, 7001, 7002):
        x, w, _ = uv_inputs(seed, H, wf, M=M)
        xd.copy_(dev_bf16(x))
        wd.copy_(dev_bf16(w))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_uv_parity(out_bits(out), oracle.uv_projection(x, w), f"replay {seed}")


def test_uv_can_implement_on_device():
    assert mq.mlaq_uv_can_implement(16, 32, weight_format=WEIGHT_MXFP8)
    assert mq.mlaq_uv_can_implement(11, 1, weight_format=WEIGHT_BF16)
    assert not mq.mlaq_uv_can_implement(16, 32, v_dim=64)


@pytest.mark.parametrize("wf", [WEIGHT_BF16, WEIGHT_MXFP8])
def test_uv_stream_cache_hint(wf):
    """mlaq_uv_run_ex accepts MLAQ_CACHE_STREAM (the UV kernels ignore the
    hint) and gives the oracle's parity and the bits of the default hint for
    every head count and both token tiles, leaving the bytes past the output
    untouched."""
    for H in (8, 11, 16):
        x_all, w, s = uv_inputs(5100 + 10 * H + wf, H, wf)
        wd = dev_bf16(w) if wf == WEIGHT_BF16 else dev_u8(w)
        sd = None if s is None else dev_u8(s)
        for M in (1, 9, 17, 32):
            x = x_all[:M].copy()
            xd = dev_bf16(x)
            outs = []
            for hint in (mq.MLAQ_CACHE_DEFAULT, mq.MLAQ_CACHE_STREAM):
                buf = torch.full((M * H * 128 + 64,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                out = buf[:M * H * 128].view(M, H, 128)
                mq.mlaq_uv_run_ex(xd, wd, sd, out, wf, cache_hint=hint)
                outs.append(buf)
            torch.cuda.synchronize()
            tag = f"uv stream hint wf={wf} H={H} M={M}"
            assert torch.equal(outs[0], outs[1]), tag + ": differs from the default hint"
            got = out_bits(outs[1][:M * H * 128].view(M, H, 128))
            assert_uv_parity(got, oracle.uv_projection(x, w, s, weight_format=wf), tag)
            assert np.all(out_bits(outs[1][M * H * 128:]) == 0x5A5A), tag + ": wrote past the output"


def test_uv_stream_hint_in_a_graph_with_a_consumer():
    """Two UV calls passed the streaming hint, captured in one graph, each followed at once
    by a copy kernel reading its output; replays with new x and W_UV in place
    match the oracle in every copy."""
    H, M, wf = 11, 32, WEIGHT_BF16
    mq.mlaq_uv_prewarm(H, [M], wf)
    x0, w0, _ = uv_inputs(7100, H, wf, M=M)
    xd, wd = dev_bf16(x0), dev_bf16(w0)
    outs = [torch.empty((M, H, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    seen = [torch.empty_like(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st, capture_error_mode="global"):
            for o, s in zip(outs, seen):
                mq.mlaq_uv_run_ex(xd, wd, None, o, wf, cache_hint=mq.MLAQ_CACHE_STREAM)
                s.copy_(o)
    torch.cuda.synchronize()
    for seed in (7101, 7102, 7101):
        x, w, _ = uv_inputs(seed, H, wf, M=M)
        xd.copy_(dev_bf16(x))
        wd.copy_(dev_bf16(w))
        for o, s in zip(outs, seen):
            o.zero_()
            s.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.uv_projection(x, w)
        for i, s in enumerate(seen):
            assert_uv_parity(out_bits(s), ref, f"replay {seed}, consumer copy {i}")
