"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Workloads: c0 (H=8, M=1, BF16), c1 (H=16, BF16, every M in 1..32), c2
(H=11, BF16, odd M), c3 (H=16, MXFP8, every M in 1..32), E4M3 output for both
weight formats with q_scale = amax/448 from the oracle, and the 64-layer
decode-step layer shape (H=16, M=32, E4M3 out) in the launch configuration the
benchmark times. Structured inputs whose result is known exactly are compared
bit for bit.
"""

import numpy as np
import pytest
import torch

import mla_decode_query_amd as mq
import oracle
from gpu_util import (assert_bf16_parity, assert_e4m3_parity, dev_bf16, dev_u8, new_out, out_bits, run_gpu,
                      run_oracle, to_device)
from workloads import SEED, WEIGHT_BF16, WEIGHT_MXFP8, bf16_bits, make_inputs

pytestmark = pytest.mark.gpu

BF16, E4M3 = mq.MLAQ_OUT_BF16, mq.MLAQ_OUT_E4M3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected gfx950, got {name}"
    mq.library()


_cache = {}


def inputs(cfg, H, wf):
    key = (cfg, H, wf)
    if key not in _cache:
        _cache[key] = make_inputs(SEED[cfg], H=H, weight_format=wf, M_draw=32)
    return _cache[key]


# ----------------------------------------------------------------------------
# Seeded workloads vs the oracle
# ----------------------------------------------------------------------------

def test_c0_matches_oracle_and_golden():
    from test_golden import load_c0

    inp = make_inputs(SEED["c0"], H=8, weight_format=WEIGHT_BF16, M_draw=1)
    gpu = run_gpu(inp, BF16)
    ref = run_oracle(inp, BF16)
    stats = assert_bf16_parity(gpu, ref, "c0")
    _, golden = load_c0()
    assert np.array_equal(ref["out"], golden)
    print("c0", stats)


@pytest.mark.parametrize("M", range(1, 33))
def test_c1_bf16_h16(M):
    inp = inputs("c1", 16, WEIGHT_BF16).take(M)
    assert_bf16_parity(run_gpu(inp, BF16), run_oracle(inp, BF16), f"c1 M={M}")


@pytest.mark.parametrize("M", [1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 32])
def test_c2_bf16_h11(M):
    inp = inputs("c2", 11, WEIGHT_BF16).take(M)
    assert_bf16_parity(run_gpu(inp, BF16), run_oracle(inp, BF16), f"c2 M={M}")


@pytest.mark.parametrize("H", [8, 11])
@pytest.mark.parametrize("M", [1, 4, 6, 17, 32])
def test_bf16_other_heads(H, M):
    inp = inputs("c0", H, WEIGHT_BF16).take(M)
    assert_bf16_parity(run_gpu(inp, BF16), run_oracle(inp, BF16), f"H={H} M={M}")


@pytest.mark.parametrize("M", range(1, 33))
def test_c3_mxfp8_h16(M):
    inp = inputs("c3", 16, WEIGHT_MXFP8).take(M)
    assert_bf16_parity(run_gpu(inp, BF16), run_oracle(inp, BF16), f"c3 M={M}")


@pytest.mark.parametrize("H", [8, 11])
@pytest.mark.parametrize("M", [1, 9, 32])
def test_mxfp8_other_heads(H, M):
    inp = inputs("c3", H, WEIGHT_MXFP8).take(M)
    assert_bf16_parity(run_gpu(inp, BF16), run_oracle(inp, BF16), f"mxfp8 H={H} M={M}")


@pytest.mark.parametrize("wf", [WEIGHT_BF16, WEIGHT_MXFP8])
@pytest.mark.parametrize("H", [8, 11, 16])
@pytest.mark.parametrize("M", [1, 6, 16, 17, 32])
def test_e4m3_output(wf, H, M):
    inp = inputs("c4", H, wf).take(M)
    base = run_oracle(inp, BF16)
    qs = oracle.qscale_from_result(base["acc"], inp.q_pe)
    ref = run_oracle(inp, E4M3, qs)
    assert_e4m3_parity(run_gpu(inp, E4M3, qs), ref, f"e4m3 wf={wf} H={H} M={M}")


def test_decode_step_layer_shapes_full_compare():
    """The two layer kinds of the 64-layer decode step (H=16, M=32, E4M3 out),
    full size, in the benchmark's launch configuration, every element."""
    for wf in (WEIGHT_BF16, WEIGHT_MXFP8):
        inp = make_inputs(SEED["c4"], H=16, weight_format=wf, M_draw=32)
        base = run_oracle(inp, BF16)
        qs = oracle.qscale_from_result(base["acc"], inp.q_pe)
        stats = assert_e4m3_parity(run_gpu(inp, E4M3, qs), run_oracle(inp, E4M3, qs), f"c4 wf={wf}")
        assert stats["equal_frac"] > 0.99
        stats = assert_bf16_parity(run_gpu(inp, BF16), base, f"c4 bf16 wf={wf}")
        assert stats["max_ulp_well_conditioned"] <= 1.0, stats
        print(f"c4 wf={wf}", stats)


# ----------------------------------------------------------------------------
# Structured inputs with exactly known results: bit-exact
# ----------------------------------------------------------------------------

class _Inp:
    def __init__(self, q, pe, w, s, wf):
        self.q_nope, self.q_pe, self.w, self.w_scales, self.weight_format = q, pe, w, s, wf

    M = property(lambda self: self.q_nope.shape[0])
    H = property(lambda self: self.q_nope.shape[1])


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_bf16(rng, shape):
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@pytest.mark.parametrize("H", [8, 11, 16])
@pytest.mark.parametrize("M", [1, 16, 17, 32])
def test_identity_bf16_bit_exact(H, M):
    rng = _rng(500 + H + M)
    q, pe = _rand_bf16(rng, (M, H, 128)), _rand_bf16(rng, (M, H, 64))
    w = np.zeros((H, 128, 512), np.uint16)
    for h in range(H):
        w[h, np.arange(128), np.arange(128) + 128 * (h % 4)] = 0x3F80
    inp = _Inp(q, pe, w, None, WEIGHT_BF16)
    gpu, ref = run_gpu(inp, BF16), run_oracle(inp, BF16)
    assert np.array_equal(gpu, ref["out"])


@pytest.mark.parametrize("M", [1, 32])
def test_one_hot_bit_exact(M):
    H = 16
    rng = _rng(600 + M)
    q, pe = _rand_bf16(rng, (M, H, 128)), _rand_bf16(rng, (M, H, 64))
    w = np.zeros((H, 128, 512), np.uint16)
    for h in range(H):
        w[h, (3 * h + 1) % 128, (37 * h + 5) % 512] = bf16_bits(np.array([2.0 ** (h % 3 - 1)], np.float32))[0]
    inp = _Inp(q, pe, w, None, WEIGHT_BF16)
    assert np.array_equal(run_gpu(inp, BF16), run_oracle(inp, BF16)["out"])


@pytest.mark.parametrize("M", [1, 32])
def test_mxfp8_scale_closed_form_bit_exact(M):
    """All-ones payload with E8M0 bytes 127 - ((h+k+j) mod 9) and q = 2^-(k mod 4):
    every sum is an exact multiple of 2^-11, so any order gives the same bits."""
    H = 16
    w = np.full((H, 128, 512), 0x38, np.uint8)
    hh, kk, jj = np.meshgrid(np.arange(H), np.arange(128), np.arange(16), indexing="ij")
    s = (127 - (hh + kk + jj) % 9).astype(np.uint8)
    qk = bf16_bits(np.array([2.0 ** -(k % 4) for k in range(128)], np.float32))
    q = np.broadcast_to(qk, (M, H, 128)).copy()
    pe = _rand_bf16(_rng(7), (M, H, 64))
    inp = _Inp(q, pe, w, s, WEIGHT_MXFP8)
    assert np.array_equal(run_gpu(inp, BF16), run_oracle(inp, BF16)["out"])


def test_e4m3_decode_exhaustive():
    """Every E4M3 payload code under several scale bytes, read through a
    one-hot q: out[n] = bf16(decode(code) * 2^(S-127)) exactly (NaN codes give NaN)."""
    H, M = 16, 1
    w = np.zeros((H, 128, 512), np.uint8)
    s = np.full((H, 128, 16), 127, np.uint8)
    k0 = 5
    for h in range(H):
        w[h, k0, :256] = np.arange(256, dtype=np.uint8)
        w[h, k0, 256:] = np.arange(256, dtype=np.uint8)[::-1]
        s[h, k0, :] = [119, 120, 121, 122, 123, 124, 125, 126, 127, 128, 130, 110, 100, 10, 140, 246][h % 16]
    q = np.zeros((M, H, 128), np.uint16)
    q[:, :, k0] = 0x3F80
    pe = np.zeros((M, H, 64), np.uint16)
    inp = _Inp(q, pe, w, s, WEIGHT_MXFP8)
    gpu = run_gpu(inp, BF16)
    ref = run_oracle(inp, BF16)["out"]
    nan_ref = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    nan_gpu = ((gpu & 0x7F80) == 0x7F80) & ((gpu & 0x7F) != 0)
    assert np.array_equal(nan_ref, nan_gpu), "NaN payload codes not propagated"
    assert np.array_equal(gpu[~nan_ref], ref[~nan_ref])


def test_e4m3_decode_every_scale_byte():
    """Every E4M3 payload code under every one of the 256 scale bytes: the
    kernel passes the byte as the exponent field of the scaled convert's fp32
    operand. With a one-hot q = 1.0 the oracle's output is bf16(decode(code) *
    2^(S-127)). Inside the exact domain (bytes 10..246, where every nonzero
    decoded weight is a normal bf16 value) the GPU matches it bit for bit.
    Outside it (bytes 0..9 and 247..254) the bound the header states holds:
    the NaN pattern is the same, normal results are bit-exact, results in the
    bf16 subnormal range are within one subnormal step (2^-133) of the oracle's,
    and results past the bf16 range are infinities of the same sign (or finite
    values of at least 2^127). Byte 255 gives NaN. One byte per head, 16 heads
    per call."""
    H, M, k0 = 16, 1, 77
    q = np.zeros((M, H, 128), np.uint16)
    q[:, :, k0] = 0x3F80
    pe = np.zeros((M, H, 64), np.uint16)
    scale_bytes = list(range(256))
    seen_outside = 0
    for c0 in range(0, 256, H):
        chunk = scale_bytes[c0:c0 + H]
        w = np.zeros((H, 128, 512), np.uint8)
        s = np.full((H, 128, 16), 127, np.uint8)
        for h in range(H):
            w[h, k0, :256] = np.arange(256, dtype=np.uint8)
            w[h, k0, 256:] = np.arange(256, dtype=np.uint8)[::-1]
            s[h, k0, :] = chunk[h]
        inp = _Inp(q, pe, w, s, WEIGHT_MXFP8)
        gpu = run_gpu(inp, BF16)
        ref = run_oracle(inp, BF16)["out"]
        nan_ref = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
        nan_gpu = ((gpu & 0x7F80) == 0x7F80) & ((gpu & 0x7F) != 0)
        assert np.array_equal(nan_ref, nan_gpu), f"NaN pattern differs, scale bytes {chunk}"
        for h, b in enumerate(chunk):
            g, r, nr = gpu[0, h, :512], ref[0, h, :512], nan_ref[0, h, :512]
            if b == 255:
                assert nan_gpu[0, h, :512].all(), "scale byte 255 must give NaN"
                continue
            if 10 <= b <= 246:
                assert np.array_equal(g[~nr], r[~nr]), f"scale byte {b}: not bit-exact inside the exact domain"
                continue
            seen_outside += 1
            gv = oracle.bf16_to_f32(g[~nr]).astype(np.float64)
            rv = oracle.bf16_to_f32(r[~nr]).astype(np.float64)
            normal = (np.abs(rv) >= 2.0 ** -126) & np.isfinite(rv)
            assert np.array_equal(g[~nr][normal], r[~nr][normal]), f"scale byte {b}: normal results differ"
            sub = np.abs(rv) < 2.0 ** -126
            assert np.all(np.abs(gv[sub] - rv[sub]) <= 2.0 ** -133), f"scale byte {b}: subnormal beyond one step"
            over = ~np.isfinite(rv)
            assert np.all((np.sign(gv[over]) == np.sign(rv[over])) & (np.abs(gv[over]) >= 2.0 ** 127)), \
                f"scale byte {b}: overflow not an infinity of the same sign"
    assert seen_outside == 18


@pytest.mark.parametrize("q_scale", [
    1.0, 0.125, 3.0, 1.0 / 448, -0.75,
    # The edges of the range where the kernel clamps x to 448 |q_scale| and
    # divides with one FMA correction of x * RN(1/q_scale) (2^-90 <= |q_scale|
    # <= 2^118), and scales outside it (IEEE division there): a subnormal
    # scale whose reciprocal overflows, the smallest normal, scales whose
    # 448-multiple overflows, huge scales with subnormal reciprocals, zero,
    # inf and NaN.
    2.0 ** -90, 3 * 2.0 ** -95, -(2.0 ** 118), 1.25 * 2.0 ** 118, 1.5 * 2.0 ** 119, 3 * 2.0 ** -140,
    2.0 ** -126, 2.0 ** -127, 2.0 ** 126, 1.5 * 2.0 ** 127, 0.0, float("inf"), float("nan"),
])
def test_e4m3_encode_exhaustive_via_q_pe(q_scale):
    """All 65536 bf16 patterns through the q_pe lanes of E4M3 output:
    e4m3_satfinite(fp32(x) / q_scale), bit-exact against the oracle encoder
    (IEEE division), for every scale value the device may hold."""
    H, M = 16, 32
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = np.zeros((H, 128, 512), np.uint16)
    q = np.zeros((M, H, 128), np.uint16)
    for half in range(2):
        pe = pats[half * 32768:(half + 1) * 32768].reshape(M, H, 64)
        inp = _Inp(q, pe, w, None, WEIGHT_BF16)
        gpu = run_gpu(inp, E4M3, q_scale)
        with np.errstate(over="ignore", invalid="ignore", divide="ignore", under="ignore"):
            want = oracle.e4m3_encode(oracle.bf16_to_f32(pe) / np.float32(q_scale))
            zero = oracle.e4m3_encode(np.zeros(1, np.float32) / np.float32(q_scale))[0]  # projection lanes: +0
        nan = (want & 0x7F) == 0x7F
        assert np.array_equal((gpu[..., 512:] & 0x7F) == 0x7F, nan)
        assert np.array_equal(gpu[..., 512:][~nan], want[~nan])
        if (zero & 0x7F) == 0x7F:  # a NaN code; its sign bit is not fixed
            assert np.all((gpu[..., :512] & 0x7F) == 0x7F)
        else:
            assert np.all(gpu[..., :512] == zero)


def test_bf16_rounding_two_term_sums():
    """acc = a + b with exactly two nonzero products: exact in fp32 whatever the
    order, so the bf16 rounding (ties included) must match the oracle's bits."""
    H, M = 16, 32
    rng = _rng(77)
    a = rng.standard_normal((M, H)).astype(np.float32)
    a_b = bf16_bits(a)
    # b sits at the tie position (half a bf16 ulp of a) for half the lanes, else random small.
    ea = np.floor(np.log2(np.abs(oracle.bf16_to_f32(a_b)))).astype(np.int64)
    tie = np.ldexp(1.0, ea - 8) * np.where(rng.random((M, H)) < 0.5, 1, 3)
    small = np.ldexp(rng.random((M, H)), ea - rng.integers(7, 14, (M, H)))
    b = np.where(rng.random((M, H)) < 0.5, tie, small).astype(np.float32)
    b_b = bf16_bits(b)
    q = np.zeros((M, H, 128), np.uint16)
    q[:, :, 10], q[:, :, 90] = a_b, b_b
    w = np.zeros((H, 128, 512), np.uint16)
    w[:, 10, :] = 0x3F80
    w[:, 90, :] = 0x3F80
    pe = _rand_bf16(rng, (M, H, 64))
    inp = _Inp(q, pe, w, None, WEIGHT_BF16)
    assert np.array_equal(run_gpu(inp, BF16), run_oracle(inp, BF16)["out"])
    qs = 0.5
    assert np.array_equal(run_gpu(inp, E4M3, qs), run_oracle(inp, E4M3, qs)["out"])


def test_e4m3_rounds_to_bf16_first():
    """acc = 1 + 2^-4 + 2^-12: bf16 gives the E4M3 midpoint 1.0625, which goes
    to the even code 0x38; skipping the bf16 step would give 0x39."""
    H, M = 8, 4
    q = np.zeros((M, H, 128), np.uint16)
    q[:, :, 3] = bf16_bits(np.array([1.0625], np.float32))[0]
    q[:, :, 77] = bf16_bits(np.array([2.0 ** -12], np.float32))[0]
    w = np.zeros((H, 128, 512), np.uint16)
    w[:, 3, 200] = 0x3F80
    w[:, 77, 200] = 0x3F80
    pe = np.zeros((M, H, 64), np.uint16)
    inp = _Inp(q, pe, w, None, WEIGHT_BF16)
    gpu = run_gpu(inp, E4M3, 1.0)
    assert np.all(gpu[:, :, 200] == 0x38)
    assert np.array_equal(gpu, run_oracle(inp, E4M3, 1.0)["out"])


# ----------------------------------------------------------------------------
# Invariants, memory safety, determinism, graphs, gate and prewarm
# ----------------------------------------------------------------------------

def test_h11_equals_first_heads_of_h16_and_deterministic():
    inp16 = inputs("c1", 16, WEIGHT_BF16).take(32)
    sub = _Inp(inp16.q_nope[:, :11].copy(), inp16.q_pe[:, :11].copy(), inp16.w[:11].copy(), None, WEIGHT_BF16)
    a = run_gpu(inp16, BF16)
    assert np.array_equal(run_gpu(inp16, BF16), a), "two runs differ"
    assert np.array_equal(run_gpu(sub, BF16), a[:, :11])


@pytest.mark.parametrize("wf,od,M", [(WEIGHT_BF16, BF16, 1), (WEIGHT_BF16, E4M3, 32), (WEIGHT_MXFP8, BF16, 17),
                                     (WEIGHT_MXFP8, E4M3, 7)])
def test_output_guard_bytes_untouched(wf, od, M):
    """The output sits inside a larger buffer filled with a canary; only the
    [M,H,576] rows may change. Inputs are placed flush against the end of
    their allocations."""
    H = 11
    inp = inputs("c2" if wf == WEIGHT_BF16 else "c3", H, wf).take(M)
    esz = 2 if od == BF16 else 1
    nbytes = M * H * 576 * esz
    guard = 4096
    buf = torch.full((guard + nbytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    out = buf[guard:guard + nbytes]
    out = out.view(torch.bfloat16) if od == BF16 else out
    out = out.view(M, H, 576)

    def flush_end(t):
        raw = t.view(torch.uint8).reshape(-1)
        big = torch.zeros(raw.numel() + 4096, dtype=torch.uint8, device="cuda")
        big[-raw.numel():] = raw
        return big[-raw.numel():].view(t.dtype).view(t.shape)

    q, pe, w, s = (flush_end(t) if t is not None else None for t in to_device(inp))
    qs = None
    if od == E4M3:
        qs = flush_end(torch.tensor([0.05], dtype=torch.float32, device="cuda"))
    mq.mlaq_run(q, pe, w, s, qs, out, wf, od)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:guard] == 0xA5) and np.all(host[guard + nbytes:] == 0xA5)
    ref = run_oracle(inp, od, 0.05 if od == E4M3 else None)
    got = out_bits(out)
    if od == BF16:
        assert_bf16_parity(got, ref)
    else:
        assert_e4m3_parity(got, ref)


@pytest.mark.parametrize("wf,od", [(WEIGHT_BF16, BF16), (WEIGHT_MXFP8, E4M3)])
def test_graph_capture_replay_with_mutated_inputs(wf, od):
    """Capture once, then change the inputs in place (same pointers, new
    contents and a new q_scale value) and replay; every replay, with eager
    work and synchronizations in between, matches the oracle on the current
    inputs. Capture runs in global mode, so any host sync or allocation inside
    mlaq_run would fail it."""
    H, M = 16, 8
    mq.mlaq_prewarm(H, [M], wf, od)
    first = make_inputs(2000, H=H, weight_format=wf, M_draw=M)
    q, pe, w, s = to_device(first)
    qs = torch.tensor([0.02], dtype=torch.float32, device="cuda") if od == E4M3 else None
    out = new_out(M, H, od)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream, capture_error_mode="global"):
            mq.mlaq_run(q, pe, w, s, qs, out, wf, od)
    torch.cuda.synchronize()
    for rep, seed in enumerate([2000, 2001, 2002]):
        cur = make_inputs(seed, H=H, weight_format=wf, M_draw=M)
        nq, npe, nw, ns = to_device(cur)
        q.copy_(nq)
        pe.copy_(npe)
        w.copy_(nw)
        if s is not None:
            s.copy_(ns)
        scale = None
        if qs is not None:
            scale = 0.02 * (rep + 1)
            qs.fill_(scale)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_bits(out)
        ref = run_oracle(cur, od, scale)
        if od == BF16:
            assert_bf16_parity(got, ref, f"replay {rep}")
        else:
            assert_e4m3_parity(got, ref, f"replay {rep}")
        # eager call between replays gives the same bits as the replay
        out2 = new_out(M, H, od)
        mq.mlaq_run(q, pe, w, s, qs, out2, wf, od)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out2), got)


def test_can_implement_and_prewarm_on_device():
    for wf in (WEIGHT_BF16, WEIGHT_MXFP8):
        for od in (BF16, E4M3):
            assert mq.mlaq_can_implement(16, 32, weight_format=wf, out_dtype=od)
            assert mq.mlaq_can_implement(11, 1, weight_format=wf, out_dtype=od)
            assert not mq.mlaq_can_implement(12, 1, weight_format=wf, out_dtype=od)
            assert not mq.mlaq_can_implement(16, 33, weight_format=wf, out_dtype=od)
            assert mq.mlaq_can_implement(16, 8, nope_dim=192, weight_format=wf, out_dtype=od)
            assert not mq.mlaq_can_implement(16, 8, nope_dim=256, weight_format=wf, out_dtype=od)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        mq.mlaq_prewarm(16, [1, 2, 4, 8, 16, 32], WEIGHT_MXFP8, E4M3)
        mq.mlaq_prewarm(11, [1, 17], WEIGHT_BF16, BF16)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 >= free0 - (2 << 20), "prewarm retained device memory"
    with pytest.raises(mq.MlaqError) as e:
        mq.mlaq_prewarm(16, [0], WEIGHT_BF16, BF16)
    assert e.value.status == mq.MLAQ_ERR_UNSUPPORTED


def test_run_errors_on_device_leave_output_untouched():
    inp = inputs("c1", 16, WEIGHT_BF16).take(4)
    q, pe, w, _ = to_device(inp)
    out = torch.full((4, 16, 576), 7.0, dtype=torch.bfloat16, device="cuda")
    qs = torch.tensor([1.0], device="cuda")
    with pytest.raises(mq.MlaqError) as e:
        mq.mlaq_run(q, pe, w, None, qs, out, WEIGHT_BF16, BF16)  # BF16 output takes no scale
    assert e.value.status == mq.MLAQ_ERR_INVALID_ARG
    with pytest.raises(mq.MlaqError) as e:
        mq.mlaq_run(q, pe, w, None, None, out.view(torch.uint8)[:, :, :576].contiguous(), WEIGHT_BF16, E4M3)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    # M = 0 is an empty batch: accepted, nothing written.
    empty = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device="cuda")
    mq.mlaq_run(empty(0, 16, 128), empty(0, 16, 64), w, None, None, empty(0, 16, 576), WEIGHT_BF16, BF16)
