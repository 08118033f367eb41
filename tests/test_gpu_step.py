"""The decode step exactly as the benchmark builds and times it: bench.Layer
objects (layer l: BF16 W_UK_T for even l, MXFP8 for odd l, H = 16, M = 32,
E4M3 output, inputs seeded as in the benchmark), their weights in two device
copies, and bench.step_graph's one-hipGraph-per-copy capture. Every layer's
output of every replay is compared with the oracle, element by element, to
the E4M3 bar (code distance <= 1, q_pe lanes bit-exact).

The per-layer q_scale here is the oracle's amax/448 written into the
layer's device scalar (the benchmark computes it with torch from the same
inputs; the kernel reads whatever value the scalar holds). The first 8 of
the step's 64 layers keep the oracle's share of the run short; the launch
shape, the capture and the weight rotation are the benchmark's own."""

import numpy as np
import pytest
import torch

import bench
import mla_decode_query_amd as mq
import oracle
import workloads as wl
from gpu_util import assert_e4m3_parity, out_bits

pytestmark = pytest.mark.gpu

LAYERS = 8


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mq.library()


def test_decode_step_graph_as_benchmarked():
    layers = [bench.Layer(torch, mq, wl, i) for i in range(LAYERS)]
    copies = [[L.weights_on_device(torch, mq) for L in layers] for _ in range(2)]
    refs = []
    for i, L in enumerate(layers):
        inp = wl.make_inputs(wl.SEED["c4"] * 100 + i, H=bench.H, weight_format=L.wf, M_draw=bench.M_STEP)
        base = oracle.mla_query(inp.q_nope, inp.q_pe, inp.w, inp.w_scales, weight_format=L.wf,
                                out_dtype=mq.MLAQ_OUT_BF16)
        qs = oracle.qscale_from_result(base["acc"], inp.q_pe)
        L.qs.copy_(torch.tensor([qs], dtype=torch.float32))
        refs.append(oracle.mla_query(inp.q_nope, inp.q_pe, inp.w, inp.w_scales, qs, weight_format=L.wf,
                                     out_dtype=mq.MLAQ_OUT_E4M3))
    for wf in (mq.MLAQ_WEIGHT_BF16, mq.MLAQ_WEIGHT_MXFP8):
        mq.mlaq_prewarm(bench.H, [bench.M_STEP], wf, mq.MLAQ_OUT_E4M3)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graphs = [bench.step_graph(torch, mq, layers, copies[c], stream) for c in range(2)]
    torch.cuda.synchronize()
    for c in (0, 1, 0):
        for L in layers:
            L.out.fill_(0xAA)
        torch.cuda.synchronize()
        graphs[c].replay()
        torch.cuda.synchronize()
        for i, (L, ref) in enumerate(zip(layers, refs)):
            assert_e4m3_parity(out_bits(L.out), ref, f"step replay of copy {c}, layer {i}")
