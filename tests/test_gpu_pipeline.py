"""The three kernels chained as one MLA decode layer on the GPU: the fused
query projection (BF16 output, q_pe appended), dense MLA decode attention over
a paged latent cache, and the V up-projection of its output. Each stage is
checked against the oracle applied to the GPU's own input of that stage, with
that stage's bar (tests/gpu_util.py); the final output is also compared with
the all-oracle chain (the intermediate bf16 roundings may differ by an ulp, so
that comparison is statistical: rel-L2 <= 1e-2). The chain runs eagerly and
as one captured hipGraph, which must give the same bits.

Shapes: H = 16 heads (a 64-head model at TP4), M = 32 decode sequences with
ragged cached lengths, page 64, nope 128, latent 512, rope 64, value 128;
BF16 or MXFP8 weights for both projections."""

import numpy as np
import pytest
import torch

import mla_decode_query_amd as mq
import oracle
from gpu_util import (BF16P, assert_attn_parity, assert_bf16_parity, assert_uv_parity, attn_oracle_run, dev_bf16,
                      dev_u8, out_bits)
from workloads import WEIGHT_BF16, WEIGHT_MXFP8, bf16_bits, e4m3_bits, make_attn_inputs, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mq.library()


def uv_weights(seed, H, wf):
    rng = np.random.Generator(np.random.PCG64(seed))
    std = np.float32(512 ** -0.5)
    if wf == WEIGHT_BF16:
        return bf16_bits(rng.standard_normal((H, 128, 512), dtype=np.float32) * std), None
    w = e4m3_bits(rng.standard_normal((H, 128, 512), dtype=np.float32) * std)
    return w, (127 + rng.integers(-8, 1, size=(H, 128, 16))).astype(np.uint8)


class Layer:
    def __init__(self, wf, seed=9100):
        H, M = 16, 32
        lens = [int(x) for x in np.random.Generator(np.random.PCG64(seed)).integers(1, 1500, M)]
        lens[3], lens[7] = 64, 1
        self.wf, self.H, self.M = wf, H, M
        self.qin = make_inputs(seed, H=H, weight_format=wf, M_draw=M)
        self.attn = make_attn_inputs(seed + 1, H, lens)  # the cache, table and lengths (its q is replaced)
        self.wuv, self.suv = uv_weights(seed + 2, H, wf)
        self.S = 4

    def device(self):
        d = {"q_nope": dev_bf16(self.qin.q_nope), "q_pe": dev_bf16(self.qin.q_pe),
             "w": dev_bf16(self.qin.w) if self.wf == WEIGHT_BF16 else dev_u8(self.qin.w),
             "ws": None if self.qin.w_scales is None else dev_u8(self.qin.w_scales),
             "kv": dev_bf16(self.attn.kv), "bt": torch.from_numpy(self.attn.block_table).cuda(),
             "sl": torch.from_numpy(self.attn.seq_lens).cuda(),
             "wuv": dev_bf16(self.wuv) if self.wf == WEIGHT_BF16 else dev_u8(self.wuv),
             "suv": None if self.suv is None else dev_u8(self.suv)}
        d["q"] = torch.empty((self.M, self.H, mq.ROW), dtype=torch.bfloat16, device="cuda")
        d["x"] = torch.empty((self.M, self.H, 512), dtype=torch.bfloat16, device="cuda")
        d["out"] = torch.empty((self.M, self.H, 128), dtype=torch.bfloat16, device="cuda")
        d["lse"] = torch.empty((self.M, self.H), dtype=torch.float32, device="cuda")
        n = mq.mlaq_attn_workspace_size(self.M, self.H, self.S, BF16P)
        d["wsp"] = torch.empty((n,), dtype=torch.uint8, device="cuda")
        return d

    def enqueue(self, d):
        mq.mlaq_run(d["q_nope"], d["q_pe"], d["w"], d["ws"], None, d["q"], self.wf, mq.MLAQ_OUT_BF16)
        mq.mlaq_attn_run(d["q"], d["kv"], d["bt"], d["sl"], d["x"], self.attn.softmax_scale, self.S, BF16P, d["wsp"],
                         d["lse"])
        mq.mlaq_uv_run(d["x"], d["wuv"], d["suv"], d["out"], self.wf)


def attn_case(layer, q_bits):
    a = layer.attn
    return type(a)(q=q_bits, kv=a.kv, block_table=a.block_table, seq_lens=a.seq_lens,
                   softmax_scale=a.softmax_scale, seed=a.seed)


@pytest.mark.parametrize("wf", [WEIGHT_BF16, WEIGHT_MXFP8])
def test_decode_layer_stagewise_and_end_to_end(wf):
    L = Layer(wf)
    d = L.device()
    L.enqueue(d)
    torch.cuda.synchronize()
    q, x, out = out_bits(d["q"]), out_bits(d["x"]), out_bits(d["out"])
    # stage 1: the fused query
    ref_q = oracle.mla_query(L.qin.q_nope, L.qin.q_pe, L.qin.w, L.qin.w_scales, weight_format=wf)
    assert_bf16_parity(q, ref_q, "query stage")
    # stage 2: attention on the GPU's query
    case = attn_case(L, q)
    ref_x = attn_oracle_run(case, L.S, BF16P)
    assert_attn_parity(x, d["lse"].cpu().numpy().astype(np.float64), ref_x, case, L.S, BF16P, "attention stage")
    # stage 3: the UV projection of the GPU's attention output
    ref_out = oracle.uv_projection(x, L.wuv, L.suv, weight_format=wf)
    assert_uv_parity(out, ref_out, "UV stage")
    # end to end against the all-oracle chain
    chain_x = attn_oracle_run(attn_case(L, ref_q["out"]), L.S, BF16P)["out"]
    chain = oracle.uv_projection(chain_x, L.wuv, L.suv, weight_format=wf)["out"]
    got = oracle.bf16_to_f32(out).astype(np.float64)
    want = oracle.bf16_to_f32(chain).astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= 1e-2, f"end-to-end rel-L2 {rel}"


def test_decode_layer_graph_matches_eager():
    L = Layer(WEIGHT_MXFP8, seed=9200)
    mq.mlaq_prewarm(L.H, [L.M], WEIGHT_MXFP8, mq.MLAQ_OUT_BF16)
    mq.mlaq_uv_prewarm(L.H, [L.M], WEIGHT_MXFP8)
    mq.mlaq_attn_prewarm(BF16P)
    d = L.device()
    L.enqueue(d)
    torch.cuda.synchronize()
    eager = out_bits(d["out"])
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st, capture_error_mode="global"):
            L.enqueue(d)
    torch.cuda.synchronize()
    for _ in range(3):
        d["out"].zero_()
        d["x"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(d["out"]), eager)
