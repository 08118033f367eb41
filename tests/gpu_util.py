"""Helpers of the GPU parity tests: move seeded host inputs to the device, run
the HIP path through the C ABI, and compare with the oracle to the parity bar.

Parity bar (per element, from the pages' rounding chain: fp32 accumulation in
an unspecified k order, then bf16, then optionally E4M3):
* BF16 projection lanes: |gpu - acc| <= 2 ulp_bf16(acc) + 2 gamma_128 sum|q w|,
  where acc is the oracle's fp32 accumulator and gamma_128 = 128 u / (1 - 128 u),
  u = 2^-24 (the classic bound for any summation order with one rounding per
  add, doubled to also cover a truncating accumulator); and per call
  rel-L2 = ||gpu - acc|| / ||acc|| <= 4e-3;
* E4M3 projection lanes: code-ordinal distance <= 1 (+0 and -0 coincide);
* q_pe lanes (a bit copy, or one correctly rounded division and an encode):
  bit-exact.
"""

from __future__ import annotations

import numpy as np
import torch

import mla_decode_query_amd as mq
import oracle

GAMMA_128 = (128 * 2.0 ** -24) / (1 - 128 * 2.0 ** -24)
N = 512


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def to_device(inp):
    """(q_nope, q_pe, w, w_scales) device tensors for a workloads.Inputs."""
    q = dev_bf16(inp.q_nope)
    pe = dev_bf16(inp.q_pe)
    if inp.weight_format == mq.MLAQ_WEIGHT_BF16:
        w, s = dev_bf16(inp.w), None
    else:
        w, s = dev_u8(inp.w), dev_u8(inp.w_scales)
    return q, pe, w, s


def new_out(M, H, out_dtype):
    if out_dtype == mq.MLAQ_OUT_BF16:
        return torch.empty((M, H, mq.ROW), dtype=torch.bfloat16, device="cuda")
    return torch.empty((M, H, mq.ROW), dtype=torch.uint8, device="cuda")


def out_bits(out: torch.Tensor) -> np.ndarray:
    t = out.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.view(torch.uint8).numpy().copy()


def run_gpu(inp, out_dtype, q_scale=None, out=None):
    """One mlaq_run on the device; returns the output bit patterns."""
    q, pe, w, s = to_device(inp)
    qs = None if q_scale is None else torch.tensor([q_scale], dtype=torch.float32, device="cuda")
    if out is None:
        out = new_out(inp.M, inp.H, out_dtype)
    mq.mlaq_run(q, pe, w, s, qs, out, inp.weight_format, out_dtype)
    torch.cuda.synchronize()
    return out_bits(out)


def run_oracle(inp, out_dtype, q_scale=None):
    return oracle.mla_query(inp.q_nope, inp.q_pe, inp.w, inp.w_scales, q_scale,
                            weight_format=inp.weight_format, out_dtype=out_dtype)


def ulp_bf16(x):
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))


def bf16_f64(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def assert_bf16_parity(gpu: np.ndarray, ref: dict, what: str = ""):
    """Projection lanes within the bound, q_pe lanes bit-exact. Returns stats."""
    assert gpu.shape == ref["out"].shape, (gpu.shape, ref["out"].shape)
    got = bf16_f64(gpu[..., :N])
    acc = ref["acc"].astype(np.float64)
    bound = 2 * ulp_bf16(acc) + 2 * GAMMA_128 * ref["s_abs"]
    err = np.abs(got - acc)
    bad = ~(err <= bound)  # NaN counts as bad
    if bad.any():
        idx = tuple(int(i) for i in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} projection lanes outside the bound; first {idx}: "
                             f"gpu {got[idx]!r} oracle acc {acc[idx]!r} bound {bound[idx]!r}")
    na = np.linalg.norm(acc)
    rel = float(np.linalg.norm(got - acc) / na) if na > 0 else float(np.linalg.norm(got))
    assert rel <= 4e-3, f"{what}: rel-L2 {rel}"
    pe_ok = np.array_equal(gpu[..., N:], ref["out"][..., N:])
    assert pe_ok, f"{what}: q_pe lanes differ"
    ulps = err / ulp_bf16(acc)
    # Where the order-dependent term is under a quarter ulp, the fp32 sums of
    # any order round to within one bf16 ulp of the oracle's accumulator.
    well = 2 * GAMMA_128 * ref["s_abs"] <= 0.25 * ulp_bf16(acc)
    return {"max_ulp": float(ulps.max()), "max_ulp_well_conditioned": float(ulps[well].max(initial=0.0)),
            "well_conditioned_frac": float(well.mean()), "rel_l2": rel,
            "bitwise_equal_frac": float(np.mean(gpu[..., :N] == ref["out"][..., :N]))}


def ordinal(codes):
    c = np.asarray(codes).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def assert_e4m3_parity(gpu: np.ndarray, ref: dict, what: str = ""):
    assert gpu.shape == ref["out"].shape
    d = np.abs(ordinal(gpu[..., :N]) - ordinal(ref["out"][..., :N]))
    assert d.max() <= 1, f"{what}: E4M3 code distance {int(d.max())} at {np.argwhere(d > 1)[0]}"
    assert np.array_equal(gpu[..., N:], ref["out"][..., N:]), f"{what}: q_pe lanes differ"
    return {"max_code_dist": int(d.max()), "equal_frac": float(np.mean(d == 0))}
