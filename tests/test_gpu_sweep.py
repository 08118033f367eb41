"""Seeded sweeps over the launch spaces of the fused query and of the dense
MLA decode attention.

Fused query, through mlaq_run_ex: each
case draws a head count (8, 11, 16), a token count (1..32), the nope width
(128 or 192), the weight format, the output type, the cache hint and strided
layouts for q_nope, q_pe and the output (token- or head-major storage with
padded rows and heads, sparkinfer PR #75 "[GG] Add BF16 MLA query projection
and assembly", "What" and "Validation": the [H,M,K] batch view and pitched
outputs), and checks the result against the oracle on contiguous copies.
Padding around the output rows must stay untouched. Same parity bar as
tests/test_gpu_parity.py.

Attention, through mlaq_attn_run (b12x PR #441 "Allow FP32 split partials in
prepared dense MLA": BF16 or FP32 partials, validation against a reference of
higher precision): each case draws the head count (1..16), the page size,
the batch, sequence lengths that mix empty, single-token, page-edge and long
sequences, the split count and the partial dtype, and checks the output, the
lse and the partials read back from the workspace against the oracle's split
procedure with the same split count and partial dtype (the bar of
tests/test_gpu_attn.py)."""

import numpy as np
import pytest
import torch

import mla_decode_query_amd as mq
from gpu_util import (BF16P, FP32P, assert_attn_parity, assert_bf16_parity, assert_e4m3_parity, attn_oracle_run,
                      dev_bf16, dev_u8, out_bits, run_oracle)
from workloads import WEIGHT_BF16, WEIGHT_MXFP8, make_attn_inputs, make_inputs

pytestmark = pytest.mark.gpu

BF16, E4M3 = mq.MLAQ_OUT_BF16, mq.MLAQ_OUT_E4M3
CASES = 40
ATTN_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mq.library()


def draw(i):
    """The i-th case's shape, formats and layouts (a fixed function of i)."""
    rng = np.random.default_rng(770_000 + i)
    return dict(
        H=int(rng.choice([8, 11, 16])), M=int(rng.integers(1, 33)), K=int(rng.choice([128, 192])),
        wf=int(rng.choice([WEIGHT_BF16, WEIGHT_MXFP8])), od=int(rng.choice([BF16, E4M3])),
        hint=int(rng.choice([mq.MLAQ_CACHE_DEFAULT, mq.MLAQ_CACHE_STREAM])),
        q_layout=str(rng.choice(["token", "head"])), q_pad=8 * int(rng.integers(0, 3)),
        q_extra_heads=int(rng.integers(0, 2)),
        pe_layout=str(rng.choice(["token", "head"])), pe_pad=8 * int(rng.integers(0, 3)),
        out_layout=str(rng.choice(["token", "head"])), out_pad=8 * int(rng.integers(0, 4)),
        q_scale=float(10.0 ** rng.uniform(-3.0, -0.5)), seed=int(rng.integers(1 << 30)))


def strided(host, layout, pad, extra_heads=0):
    """A [M,H,W] bf16 device view of host bits [M,H,W] whose storage is
    token-major [M, H + extra_heads, W + pad] or head-major [H + extra_heads,
    M, W + pad]; the padding holds a canary pattern."""
    M, H, W = host.shape
    if layout == "token":
        st = torch.full((M, H + extra_heads, W + pad), 0x3F80, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        view = st[:, :H, :W]
    else:
        st = torch.full((H + extra_heads, M, W + pad), 0x3F80, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        view = st.transpose(0, 1)[:, :H, :W]
    view.copy_(dev_bf16(host))
    return view


@pytest.mark.parametrize("i", range(CASES))
def test_random_launch(i):
    c = draw(i)
    H, M, K, wf, od = c["H"], c["M"], c["K"], c["wf"], c["od"]
    inp = make_inputs(c["seed"], H=H, weight_format=wf, M_draw=M, K=K)
    q = strided(inp.q_nope, c["q_layout"], c["q_pad"], c["q_extra_heads"])
    pe = strided(inp.q_pe, c["pe_layout"], c["pe_pad"])
    if wf == WEIGHT_BF16:
        w, s = dev_bf16(inp.w), None
    else:
        w, s = dev_u8(inp.w), dev_u8(inp.w_scales)
    dt = torch.bfloat16 if od == BF16 else torch.uint8
    width = mq.ROW + c["out_pad"]
    canary = 0x5A5A if od == BF16 else 0x5A
    if c["out_layout"] == "token":
        ws = torch.empty((M, H, width), dtype=dt, device="cuda")
        out = ws[:, :, :mq.ROW]
    else:
        ws = torch.empty((H, M, width), dtype=dt, device="cuda")
        out = ws.transpose(0, 1)[:, :, :mq.ROW]
    (ws.view(torch.int16) if od == BF16 else ws).fill_(canary)
    qs_val = c["q_scale"] if od == E4M3 else None
    qs = None if qs_val is None else torch.tensor([qs_val], dtype=torch.float32, device="cuda")
    what = f"case {i}: {c}"
    print(what, flush=True)
    mq.mlaq_run_ex(q, pe, w, s, qs, out, wf, od, cache_hint=c["hint"])
    torch.cuda.synchronize()
    got = out_bits(out.contiguous())
    ref = run_oracle(inp, od, qs_val)
    if od == BF16:
        assert_bf16_parity(got, ref, what)
    else:
        assert_e4m3_parity(got, ref, what)
    if c["out_pad"]:
        pad = out_bits(ws[..., mq.ROW:].contiguous())
        assert np.all(pad == canary), f"{what}: output padding was written"


def draw_attn(i):
    """The i-th attention case (a fixed function of i)."""
    rng = np.random.default_rng(880_000 + i)
    P = int(rng.choice([1, 8, 16, 48, 64, 128, 256]))
    M = int(rng.integers(1, 6))
    lens = []
    for _ in range(M):
        kind = rng.integers(0, 6)
        lens.append(int([0, 1, max(P - 1, 1), P, P + 1, int(rng.integers(2, 3000))][kind]))
    return dict(H=int(rng.integers(1, 17)), P=P, lens=lens, S=int(rng.choice([1, 2, 3, 5, 8, 16, 33])),
                pd=int(rng.choice([BF16P, FP32P])), seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("i", range(ATTN_CASES))
def test_random_attention(i):
    c = draw_attn(i)
    what = f"attention case {i}: {c}"
    print(what, flush=True)
    inp = make_attn_inputs(c["seed"], c["H"], c["lens"], page_size=c["P"])
    M, H, S, pd = inp.q.shape[0], c["H"], c["S"], c["pd"]
    q = dev_bf16(inp.q)
    kv = dev_bf16(inp.kv)
    bt = torch.from_numpy(inp.block_table).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    out = torch.empty((M, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((M, H), dtype=torch.float32, device="cuda")
    n = mq.mlaq_attn_workspace_size(M, H, S, pd)
    ws = torch.empty((n,), dtype=torch.uint8, device="cuda") if n else None
    mq.mlaq_attn_run(q, kv, bt, sl, out, inp.softmax_scale, S, pd, ws, lse)
    torch.cuda.synchronize()
    gpu, gpu_lse = out_bits(out), lse.cpu().numpy().astype(np.float64)
    assert_attn_parity(gpu, gpu_lse, attn_oracle_run(inp, S, pd), inp, S, pd, what, ws)
