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


def is_e4m3_nan(codes):
    return (np.asarray(codes) & 0x7F) == 0x7F


def assert_e4m3_parity(gpu: np.ndarray, ref: dict, what: str = ""):
    """Projection lanes: NaN exactly where the oracle has NaN, elsewhere code
    ordinal distance <= 1 (the NaN codes 0x7F/0xFF sit next to +-448 in the
    ordinal, so they are matched first); q_pe lanes bit-exact."""
    assert gpu.shape == ref["out"].shape
    g, r = gpu[..., :N], ref["out"][..., :N]
    gn, rn = is_e4m3_nan(g), is_e4m3_nan(r)
    assert np.array_equal(gn, rn), f"{what}: E4M3 NaN codes differ at {np.argwhere(gn != rn)[0]}"
    d = np.where(gn, 0, np.abs(ordinal(g) - ordinal(r)))
    assert d.max() <= 1, f"{what}: E4M3 code distance {int(d.max())} at {np.argwhere(d > 1)[0]}"
    assert np.array_equal(gpu[..., N:], ref["out"][..., N:]), f"{what}: q_pe lanes differ"
    return {"max_code_dist": int(d.max()), "equal_frac": float(np.mean(d == 0))}


# --------------------------------------------------------------------------
# Dense MLA decode attention (bar stated in tests/test_gpu_attn.py)
# --------------------------------------------------------------------------

BF16P, FP32P = mq.MLAQ_PARTIAL_BF16, mq.MLAQ_PARTIAL_FP32
U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def ulp_f32(x):
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 23).astype(np.int64))


def read_partials(ws, M, H, S, pd):
    """Partials [M,S,H,512] and lse_s [M,S,H] from the documented workspace layout."""
    esz = 4 if pd == FP32P else 2
    nb = M * S * H * 512 * esz
    raw = ws.cpu().numpy()
    with np.errstate(invalid="ignore"):  # ranges with no tokens leave their partials unwritten
        return _decode_partials(raw, nb, M, H, S, pd)


def _decode_partials(raw, nb, M, H, S, pd):
    if pd == FP32P:
        part = raw[:nb].view(np.float32).astype(np.float64)
    else:
        part = oracle.bf16_to_f32(raw[:nb].view(np.uint16)).astype(np.float64)
    off = (nb + 255) // 256 * 256
    plse = raw[off:off + M * S * H * 4].view(np.float32).astype(np.float64)
    return part.reshape(M, S, H, 512), plse.reshape(M, S, H)


def attn_oracle_run(inp, S, pd):
    return oracle.attention(inp.q, inp.kv, inp.block_table, inp.seq_lens, softmax_scale=inp.softmax_scale,
                            num_splits=S, partial_dtype=pd, threads=16)


def _terms(inp, ref):
    T = inp.seq_lens.astype(np.float64)
    tprime = T + 2 * 64 + 8
    gT = np.array([gamma(t) for t in tprime])[:, None]
    eps = 2 * (gamma(576) + 2.0 ** -22) * ref["smag"] + 2.0 ** -21  # [M,H]
    vmax = float(np.max(np.abs(oracle.bf16_to_f32(inp.kv[..., :512]))))
    return gT, eps, vmax


def assert_attn_parity(gpu, gpu_lse, ref, inp, S, pd, what, ws=None):
    gT, eps, vmax = _terms(inp, ref)
    o = ref["o"]
    got = oracle.bf16_to_f32(gpu).astype(np.float64)
    live = inp.seq_lens > 0
    upart = np.zeros_like(o)
    lse_mag = np.abs(np.where(np.isfinite(ref["lse"]), ref["lse"], 0.0))
    if S > 1:
        ok = np.isfinite(ref["plse"])[..., None]
        ustore = ulp_bf16(ref["part"]) if pd == BF16P else ulp_f32(ref["part"])
        upart = np.max(np.where(ok, ustore, 0.0), axis=1)
        lse_mag = np.maximum(lse_mag, np.max(np.abs(np.where(np.isfinite(ref["plse"]), ref["plse"], 0.0)), axis=1))
    dlse = 2.0 ** -20 * (1 + lse_mag) + 2 * gT + eps  # [M,H]
    # The softmax weights enter the value product rounded to bf16 (2^-9,
    # doubled), or with FP32 partials as a bf16 pair hi + lo (16 bits).
    pterm = 2.0 ** -16 if (pd == FP32P and S > 1) else 2.0 ** -8
    bound = (ulp_bf16(o) + upart + (pterm + 4 * eps[..., None] + 4 * gT[..., None]) * ref["vabs"]
             + 4 * dlse[..., None] * vmax + 2.0 ** -20 * np.max(np.abs(o)))
    bad = ~(np.abs(got - o) <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs outside the bound, first {np.argwhere(bad)[0]}: "
                           f"gpu {got[bad][0]} oracle {o[bad][0]} bound {bound[bad][0]}")
    if live.any():
        rel = np.linalg.norm(got[live] - o[live]) / max(np.linalg.norm(o[live]), 1e-30)
        assert rel <= 4e-3, f"{what}: rel-L2 {rel}"
    # empty sequences: zeros and lse = -inf
    assert np.all(gpu[~live] == 0), f"{what}: empty sequences must give 0"
    assert np.all(np.isneginf(gpu_lse[~live])), f"{what}: empty sequences must give lse = -inf"
    lerr = np.abs(gpu_lse[live] - ref["lse"][live])
    assert np.all(lerr <= dlse[live]), f"{what}: lse off by {lerr.max()}"
    if ws is not None and S > 1:
        part, plse = read_partials(ws, inp.M, inp.H, S, pd)
        ok = np.isfinite(ref["plse"])
        assert np.array_equal(np.isneginf(plse), ~ok), f"{what}: empty ranges must store lse = -inf"
        ustore = ulp_bf16(ref["part"]) if pd == BF16P else ulp_f32(ref["part"])
        pb = ustore + (pterm + 4 * eps[:, None, :, None] + 4 * gT[:, :, None, None]) * ref["pvabs"]
        pbad = ok[..., None] & ~(np.abs(part - ref["part"]) <= pb)
        assert not pbad.any(), f"{what}: {int(pbad.sum())} partials outside the bound, first {np.argwhere(pbad)[0]}"
        lb = 2.0 ** -20 * (1 + np.abs(np.where(ok, ref["plse"], 0))) + 2 * gT[:, :, None] + eps[:, None, :]
        assert np.all(np.abs(plse[ok] - ref["plse"][ok]) <= lb[ok]), f"{what}: lse_s"




# --------------------------------------------------------------------------
# V up-projection (bar stated in tests/test_gpu_uv.py)
# --------------------------------------------------------------------------

GAMMA_512 = (512 * 2.0 ** -24) / (1 - 512 * 2.0 ** -24)


def assert_uv_parity(gpu, ref, what=""):
    got = oracle.bf16_to_f32(gpu).astype(np.float64)
    acc = ref["acc"].astype(np.float64)
    bound = 2 * ulp_bf16(acc) + 2 * GAMMA_512 * ref["s_abs"]
    bad = ~(np.abs(got - acc) <= bound)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside the bound, first {np.argwhere(bad)[0]}"
    rel = np.linalg.norm(got - acc) / np.linalg.norm(acc)
    assert rel <= 4e-3, f"{what}: rel-L2 {rel}"


