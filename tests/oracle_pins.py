"""Pins that tie the CPU oracle to facts outside itself.

Each ``check_*`` function raises AssertionError when the oracle (optionally a
specific build of it, ``lib``) disagrees with something the mathematics or an
independent library fixes:

* codecs against torch's own bf16 / float8_e4m3fn / float8_e8m0fnu casts and
  against values the OCP OFP8 and MX v1.0 specifications fix;
* the projection against layouts whose result is known exactly (identity,
  one-hot, all-ones with power-of-two E8M0 scales, exactly representable
  E4M3 outputs), against exact rational arithmetic on tiny shapes, and
  against invariants (power-of-two scaling, head permutation, zero input,
  head-count prefix, thread-count independence).

The same functions run on deliberately broken builds of the oracle
(tests/test_oracle_mutants.py) to show that each plausible mistake is caught.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import oracle
from workloads import K_NOPE, MX_BLOCK, N_LATENT, R_ROPE, bf16_bits, e4m3_bits

BF16_ONE = 0x3F80


def _f32(bits_u16):
    return oracle.bf16_to_f32(bits_u16)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_bf16(rng, shape, std=1.0):
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def _ulp_bf16(x):
    """Spacing of bf16 values at |x| (normal range; 2^-133 below it)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


# --------------------------------------------------------------------------
# Codecs
# --------------------------------------------------------------------------

def check_e4m3_decode(lib=None):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes, lib_path=lib)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref)), "NaN codes differ from torch float8_e4m3fn"
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin]), "E4M3 decode differs from torch float8_e4m3fn"
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))
    # OCP OFP8 anchors: 1.0, max normal 448, min normal 2^-6, min subnormal 2^-9, NaN.
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9 and ours[0x07] == 7 * 2.0 ** -9
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and np.sum(np.isnan(ours)) == 2


def check_e8m0_decode(lib=None):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e8m0_decode(codes, lib_path=lib)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255]), "E8M0 decode differs from torch float8_e8m0fnu"
    assert ours[127] == 1.0 and ours[120] == 2.0 ** -7 and ours[0] == 2.0 ** -127


def check_bf16_round(lib=None):
    rng = _rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # Half of them on exact ties (low 16 bits = 0x8000), which exercise the even rule.
    bits[::2] = (bits[::2] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ours = oracle.bf16_round(x, lib_path=lib)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref), "bf16 RNE differs from torch's cast"
    fixed = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000001,
                      0x80000000], np.uint32).view(np.float32)
    got = oracle.bf16_round(fixed, lib_path=lib)
    assert list(got) == [0x3F80, 0x3F82, 0x3F81, 0x7F80, 0xFF80, 0x0000, 0x8000], [hex(v) for v in got]
    nan = oracle.bf16_round(np.array([np.nan], np.float32), lib_path=lib)
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


def check_e4m3_encode(lib=None):
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8), lib_path=lib)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    # Round trip of every finite code.
    rt = oracle.e4m3_encode(dec[finite].astype(np.float32), lib_path=lib)
    assert np.array_equal(rt, finite), "E4M3 encode(decode(c)) != c"
    # Every midpoint between adjacent positive codes goes to the even code.
    pos = np.arange(0, 0x7E, dtype=np.int64)
    mids = ((dec[pos] + dec[pos + 1]) / 2).astype(np.float32)
    got = oracle.e4m3_encode(mids, lib_path=lib).astype(np.int64)
    want = np.where(pos % 2 == 0, pos, pos + 1)
    assert np.array_equal(got, want), "E4M3 ties are not resolved to the even code"
    got_neg = oracle.e4m3_encode(-mids, lib_path=lib).astype(np.int64)
    assert np.array_equal(got_neg, want | 0x80)
    # Against torch's cast on values inside the finite range (torch's cast is RNE there).
    rng = _rng(11)
    x = np.concatenate([
        rng.standard_normal(50_000).astype(np.float32) * np.float32(40.0),
        rng.standard_normal(50_000).astype(np.float32) * np.float32(0.01),
        np.ldexp(rng.random(20_000), -rng.integers(0, 12, 20_000)).astype(np.float32),
    ])
    x = x[np.abs(x) < 448.0]
    ours = oracle.e4m3_encode(x, lib_path=lib)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref), "E4M3 encode differs from torch's cast in range"
    # Saturation and specials (satfinite reading: everything past 448 -> 448).
    special = np.array([449.0, 463.9, 464.0, 470.0, 480.0, 1e9, np.inf, -np.inf, -500.0, 0.0,
                        -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 7.5 * 2.0 ** -9, 2.0 ** -11], np.float32)
    got = list(oracle.e4m3_encode(special, lib_path=lib))
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x00, 0x02,
                   0x08, 0x00], [hex(v) for v in got]
    nan = oracle.e4m3_encode(np.array([np.nan, -np.nan], np.float32), lib_path=lib)
    assert (int(nan[0]) & 0x7F) == 0x7F and (int(nan[1]) & 0x7F) == 0x7F


# --------------------------------------------------------------------------
# Projection: exact structured cases
# --------------------------------------------------------------------------

def _run(q, pe, w, s=None, q_scale=None, wf=0, od=0, lib=None, threads=1):
    return oracle.mla_query(q, pe, w, s, q_scale, weight_format=wf, out_dtype=od, threads=threads,
                            lib_path=lib)


def check_identity_bf16(lib=None, H=16, M=3):
    rng = _rng(21)
    q = _rand_bf16(rng, (M, H, K_NOPE))
    pe = _rand_bf16(rng, (M, H, R_ROPE))
    w = np.zeros((H, K_NOPE, N_LATENT), np.uint16)
    for h in range(H):
        w[h, np.arange(K_NOPE), np.arange(K_NOPE) + 128 * (h % 4)] = BF16_ONE
    out = _run(q, pe, w, lib=lib)["out"]
    want = np.zeros((M, H, N_LATENT + R_ROPE), np.uint16)
    for h in range(H):
        want[:, h, 128 * (h % 4):128 * (h % 4) + K_NOPE] = q[:, h, :]
    want[:, :, N_LATENT:] = pe
    assert np.array_equal(out, want), "identity weights do not reproduce q_nope / q_pe bit-exactly"


def check_identity_mxfp8(lib=None, H=16, M=2):
    rng = _rng(22)
    q = _rand_bf16(rng, (M, H, K_NOPE))
    pe = _rand_bf16(rng, (M, H, R_ROPE))
    w = np.zeros((H, K_NOPE, N_LATENT), np.uint8)
    s = np.zeros((H, K_NOPE, N_LATENT // MX_BLOCK), np.uint8)
    e = np.zeros((H, K_NOPE), np.int64)
    for h in range(H):
        for k in range(K_NOPE):
            n = k + 128 * (h % 4)
            w[h, k, n] = 0x38  # E4M3 1.0
            e[h, k] = (h + 3 * k) % 7 - 5
            s[h, k, :] = 127 + e[h, k]
    out = _run(q, pe, w, s, wf=1, lib=lib)["out"]
    want = np.zeros((M, H, N_LATENT + R_ROPE), np.uint16)
    for h in range(H):
        scaled = _f32(q[:, h, :]).astype(np.float64) * np.ldexp(1.0, e[h])[None, :]
        want[:, h, 128 * (h % 4):128 * (h % 4) + K_NOPE] = bf16_bits(scaled.astype(np.float32))
    want[:, :, N_LATENT:] = pe
    assert np.array_equal(out, want), "MXFP8 identity (1.0 x 2^e) not exact"


def check_one_hot(lib=None, H=11, M=4):
    rng = _rng(23)
    q = _rand_bf16(rng, (M, H, K_NOPE))
    pe = _rand_bf16(rng, (M, H, R_ROPE))
    w = np.zeros((H, K_NOPE, N_LATENT), np.uint16)
    k0 = [(3 * h + 1) % K_NOPE for h in range(H)]
    n0 = [(37 * h + 5) % N_LATENT for h in range(H)]
    p = [h % 3 - 1 for h in range(H)]
    for h in range(H):
        w[h, k0[h], n0[h]] = bf16_bits(np.array([2.0 ** p[h]], np.float32))[0]
    out = _run(q, pe, w, lib=lib)["out"]
    want = np.zeros((M, H, N_LATENT + R_ROPE), np.uint16)
    for h in range(H):
        v = _f32(q[:, h, k0[h]]).astype(np.float64) * 2.0 ** p[h]
        want[:, h, n0[h]] = bf16_bits(v.astype(np.float32))
    want[:, :, N_LATENT:] = pe
    assert np.array_equal(out, want), "one-hot weight lands in the wrong output lane"


def check_scale_closed_form(lib=None, H=16, M=2):
    """Payload 1.0 everywhere, E8M0 byte 127 - ((h+k+j) mod 9) for scale group j,
    q = 2^-(k mod 4): the sum is an integer number of 2^-11 units, exact in any order."""
    w = np.full((H, K_NOPE, N_LATENT), 0x38, np.uint8)
    hh, kk, jj = np.meshgrid(np.arange(H), np.arange(K_NOPE), np.arange(N_LATENT // MX_BLOCK),
                             indexing="ij")
    d = (hh + kk + jj) % 9
    s = (127 - d).astype(np.uint8)
    qk = np.array([2.0 ** -(k % 4) for k in range(K_NOPE)], np.float32)
    q = np.broadcast_to(bf16_bits(qk), (M, H, K_NOPE)).copy()
    pe = np.broadcast_to(bf16_bits(np.arange(R_ROPE, dtype=np.float32) - 7), (M, H, R_ROPE)).copy()
    out = _run(q, pe, w, s, wf=1, lib=lib)["out"]
    units = np.zeros((H, N_LATENT), np.int64)  # multiples of 2^-11
    for h in range(H):
        for n in range(N_LATENT):
            units[h, n] = sum(1 << (11 - (k % 4) - ((h + k + n // MX_BLOCK) % 9)) for k in range(K_NOPE))
    exact = (units.astype(np.float64) / 2048.0).astype(np.float32)  # exact: < 2^24 units
    want_proj = bf16_bits(exact)
    for m in range(M):
        assert np.array_equal(out[m, :, :N_LATENT], want_proj), "E8M0 scale applied to the wrong (k, n) group"
        assert np.array_equal(out[m, :, N_LATENT:], pe[m])


def check_e4m3_output(lib=None, H=8, M=3):
    """Identity weights and q chosen as E4M3 values times 2^p with q_scale = 2^p:
    every output code is known. One lane is pushed into (448, 480) to saturate."""
    p = -3
    rng = _rng(24)
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8), lib_path=lib)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes_q = rng.choice(finite, size=(M, H, K_NOPE))
    codes_pe = rng.choice(finite, size=(M, H, R_ROPE))
    q = bf16_bits((dec[codes_q] * 2.0 ** p).astype(np.float32))  # 4-bit values: exact in bf16
    pe = bf16_bits((dec[codes_pe] * 2.0 ** p).astype(np.float32))
    q[0, 0, 5] = bf16_bits(np.array([456.0 * 2.0 ** p], np.float32))[0]  # 456 is exact in bf16, above 448
    w = np.zeros((H, K_NOPE, N_LATENT), np.uint16)
    for h in range(H):
        w[h, np.arange(K_NOPE), np.arange(K_NOPE) + 128 * (h % 4)] = BF16_ONE
    out = _run(q, pe, w, q_scale=2.0 ** p, od=1, lib=lib)["out"]
    want = np.zeros((M, H, N_LATENT + R_ROPE), np.uint8)
    for h in range(H):
        want[:, h, 128 * (h % 4):128 * (h % 4) + K_NOPE] = codes_q[:, h, :]
    want[0, 0, 128 * 0 + 5] = 0x7E
    want[:, :, N_LATENT:] = codes_pe
    # +0 and -0 inputs: the projection of a -0 q lane through weight 1.0 is 0 + (-0) = +0.
    proj_zero = (want[:, :, :N_LATENT] == 0x80)
    want[:, :, :N_LATENT][proj_zero] = 0x00
    assert np.array_equal(out, want), "E4M3 output codes differ from the exactly known ones"


# --------------------------------------------------------------------------
# Projection: exact rational brute force and invariants
# --------------------------------------------------------------------------

GAMMA_128 = (128 * 2.0 ** -24) / (1 - 128 * 2.0 ** -24)


def check_brute_force(lib=None):
    """H, M in 1..3 with exact Fraction sums: the fp32 accumulator is within the
    standard recursive-summation bound gamma_K * sum|q w| of the exact value, and
    the bf16 result is within one bf16 ulp of it (equal unless near a tie)."""
    N, R = 64, 8
    for wf in (0, 1):
        for H in (1, 2, 3):
            for M in (1, 2, 3):
                rng = _rng(100 + 10 * H + M + 50 * wf)
                q = _rand_bf16(rng, (M, H, K_NOPE))
                pe = _rand_bf16(rng, (M, H, R))
                if wf == 0:
                    w = _rand_bf16(rng, (H, K_NOPE, N), std=K_NOPE ** -0.5)
                    s = None
                    wval = _f32(w).astype(np.float64)
                else:
                    w = e4m3_bits(rng.standard_normal((H, K_NOPE, N)).astype(np.float32) * 0.09)
                    s = (127 + rng.integers(-8, 1, (H, K_NOPE, N // MX_BLOCK))).astype(np.uint8)
                    dec = torch.from_numpy(w.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                    wval = dec * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(MX_BLOCK, axis=2)
                res = _run(q, pe, w, s, wf=wf, lib=lib)
                qv = _f32(q).astype(np.float64)
                mismatches = 0
                for m in range(M):
                    for h in range(H):
                        for n in range(N):
                            terms = [Fraction(qv[m, h, k]) * Fraction(wval[h, k, n]) for k in range(K_NOPE)]
                            exact = sum(terms, Fraction(0))
                            sabs = sum(abs(t) for t in terms)
                            acc = Fraction(float(res["acc"][m, h, n]))
                            assert abs(acc - exact) <= Fraction(GAMMA_128) * sabs, (wf, H, M, m, h, n)
                            assert abs(res["s_abs"][m, h, n] - float(sabs)) <= 1e-12 * float(sabs)
                            y = float(_f32(res["out"][m, h, n:n + 1])[0])
                            ex = float(exact)
                            err = abs(Fraction(y) - exact)
                            assert err <= Fraction(float(_ulp_bf16(ex))), (wf, H, M, m, h, n, y, ex)
                            if err > Fraction(float(_ulp_bf16(ex))) / 2:
                                mismatches += 1
                assert mismatches <= max(1, (M * H * N) // 100), mismatches
                assert np.array_equal(res["out"][:, :, N:], pe)


def check_invariants(lib=None):
    rng = _rng(31)
    H, M = 16, 5
    q = _rand_bf16(rng, (M, H, K_NOPE))
    pe = _rand_bf16(rng, (M, H, R_ROPE))
    w = _rand_bf16(rng, (H, K_NOPE, N_LATENT), std=K_NOPE ** -0.5)
    base = _run(q, pe, w, lib=lib)
    # Power-of-two scaling of q scales every accumulator exactly.
    q4 = bf16_bits(_f32(q) * np.float32(4.0))
    r4 = _run(q4, pe, w, lib=lib)
    assert np.array_equal(r4["acc"], base["acc"] * np.float32(4.0)), "2^p scaling not exact"
    # Permuting heads of (q, W, q_pe) permutes the output heads.
    perm = rng.permutation(H)
    rp = _run(q[:, perm], pe[:, perm], w[perm], lib=lib)
    assert np.array_equal(rp["out"], base["out"][:, perm]), "head permutation does not commute"
    # Zero q -> every projection lane is +0, whatever W holds.
    rz = _run(np.zeros_like(q), pe, w, lib=lib)
    assert not rz["out"][:, :, :N_LATENT].any(), "zero q does not give +0"
    # q_pe lanes do not depend on W.
    rw = _run(q, pe, np.zeros_like(w), lib=lib)
    assert np.array_equal(rw["out"][:, :, N_LATENT:], base["out"][:, :, N_LATENT:])
    # A prefix of heads (H = 11 of 16) gives the same heads' results.
    r11 = _run(q[:, :11], pe[:, :11], w[:11], lib=lib)
    assert np.array_equal(r11["out"], base["out"][:, :11]), "H=11 differs from the first 11 of H=16"
    # A prefix of tokens gives the same tokens' results.
    r3 = _run(q[:3], pe[:3], w, lib=lib)
    assert np.array_equal(r3["out"], base["out"][:3])
    # Thread count and repetition do not change a bit.
    rt = _run(q, pe, w, lib=lib, threads=8)
    assert np.array_equal(rt["out"], base["out"]) and np.array_equal(rt["acc"], base["acc"])
    assert np.array_equal(_run(q, pe, w, lib=lib)["out"], base["out"])
    # The fp32 accumulator stays within the summation bound of the fp64 sum.
    assert np.all(np.abs(base["acc"] - base["ref64"]) <= 2 * GAMMA_128 * base["s_abs"])


def _bf16_scalar(x):
    return int(bf16_bits(np.array([x], np.float32))[0])


def check_qscale(lib=None):
    """q_scale = amax / 448 over the layer's fp32 result: |projection accumulator|
    (before bf16 rounding) and |q_pe|, 1 when that is zero. The expected values
    below are exact quotients chosen so each one fails a different mistake."""
    q = lambda a, pe: oracle.qscale_from_result(np.asarray(a, np.float32), np.asarray(pe, np.uint16), lib_path=lib)
    rng = _rng(41)
    small = rng.uniform(-1.0, 1.0, (2, 16, N_LATENT)).astype(np.float32)
    pe_small = bf16_bits(rng.uniform(-1.0, 1.0, (2, 16, R_ROPE)).astype(np.float32))
    # The largest magnitude is a negative accumulator: 7 / 448 = 2^-6.
    acc = small.copy()
    acc[1, 5, 300] = -7.0
    assert q(acc, pe_small) == 2.0 ** -6, "amax must be taken over |acc|, negative values included"
    # The largest magnitude is a negative q_pe element: 14 / 448 = 2^-5.
    pe = pe_small.copy()
    pe[0, 9, 17] = _bf16_scalar(-14.0)
    assert q(small, pe) == 2.0 ** -5, "amax must include |q_pe|"
    pe[0, 9, 17] = _bf16_scalar(14.0)
    assert q(small, pe) == 2.0 ** -5
    # Projection all zero, q_pe not: 28 / 448 = 2^-4.
    pe = np.zeros_like(pe_small)
    pe[1, 0, 63] = _bf16_scalar(-28.0)
    assert q(np.zeros_like(small), pe) == 2.0 ** -4
    # q_pe all zero: the projection alone decides (a positive maximum, 896 / 448 = 2).
    acc = small.copy()
    acc[0, 0, 0] = 896.0
    assert q(acc, np.zeros_like(pe_small)) == 2.0
    # The fp32 accumulator, not its bf16 rounding: amax = 448 (1 + 2^-20) gives
    # 1 + 2^-20 exactly, where the bf16 value would give 1.
    acc = small.copy()
    acc[1, 15, 511] = np.float32(448.0 * (1.0 + 2.0 ** -20))
    assert q(acc, pe_small) == np.float32(1.0 + 2.0 ** -20), "amax must use the fp32 result before bf16"
    # Everything zero: 1 (not 0, which would divide by zero downstream).
    assert q(np.zeros_like(small), np.zeros_like(pe_small)) == 1.0
    # Random data at the step's scale: the fp32 quotient of the largest magnitude.
    acc = (rng.standard_normal((4, 16, N_LATENT)) * 3).astype(np.float32)
    pe = _rand_bf16(rng, (4, 16, R_ROPE))
    amax = max(float(np.max(np.abs(acc))), float(np.max(np.abs(_f32(pe)))))
    assert q(acc, pe) == np.float32(amax) / np.float32(448.0)


ALL_CHECKS = [check_e4m3_decode, check_e8m0_decode, check_bf16_round, check_e4m3_encode,
              check_identity_bf16, check_identity_mxfp8, check_one_hot, check_scale_closed_form,
              check_e4m3_output, check_brute_force, check_invariants, check_qscale]


def check_e4m3_double_rounding(lib=None):
    """E4M3 output rounds the projection to bf16 first. acc = 1 + 2^-4 + 2^-12 is
    above the E4M3 midpoint between 1.0 and 1.125, but its bf16 rounding is the
    midpoint itself, which then goes to the even code 0x38 (1.0)."""
    H, M = 8, 1
    q = np.zeros((M, H, K_NOPE), np.uint16)
    q[:, :, 3] = bf16_bits(np.float32(1.0625))
    q[:, :, 77] = bf16_bits(np.float32(2.0 ** -12))
    pe = np.zeros((M, H, R_ROPE), np.uint16)
    w = np.zeros((H, K_NOPE, N_LATENT), np.uint16)
    w[:, 3, 200] = BF16_ONE
    w[:, 77, 200] = BF16_ONE
    res = _run(q, pe, w, q_scale=1.0, od=1, lib=lib)
    assert float(res["acc"][0, 0, 200]) == 1.0625 + 2.0 ** -12
    assert np.all(res["out"][:, :, 200] == 0x38), "E4M3 output skipped the bf16 rounding step"
    assert not np.any(np.delete(res["out"][:, :, :N_LATENT], 200, axis=2))


ALL_CHECKS.insert(9, check_e4m3_double_rounding)


# --------------------------------------------------------------------------
# V up-projection oracle
# --------------------------------------------------------------------------

def check_uv_identity(lib=None, H=16, M=3):
    """W_UV[h,v,c] = 1 iff c = v + 128 (h mod 4): out[m,h,v] = x[m,h,v + 128 (h mod 4)]
    bit for bit (BF16 weights, and MXFP8 payload 1.0 with per-row 2^e scales)."""
    rng = _rng(51)
    x = _rand_bf16(rng, (M, H, 512))
    w = np.zeros((H, 128, 512), np.uint16)
    w8 = np.zeros((H, 128, 512), np.uint8)
    s8 = np.zeros((H, 128, 16), np.uint8)
    e = np.zeros((H, 128), np.int64)
    for h in range(H):
        v = np.arange(128)
        w[h, v, v + 128 * (h % 4)] = BF16_ONE
        w8[h, v, v + 128 * (h % 4)] = 0x38
        e[h] = (h + 3 * v) % 7 - 5
        s8[h] = (127 + e[h])[:, None]
    out = oracle.uv_projection(x, w, lib_path=lib)["out"]
    want = np.stack([x[:, h, 128 * (h % 4):128 * (h % 4) + 128] for h in range(H)], axis=1)
    assert np.array_equal(out, want), "UV identity weights do not select x bit-exactly"
    out8 = oracle.uv_projection(x, w8, s8, weight_format=1, lib_path=lib)["out"]
    want8 = np.stack([bf16_bits((_f32(want[:, h, :]).astype(np.float64) * np.ldexp(1.0, e[h])[None, :])
                                .astype(np.float32)) for h in range(H)], axis=1)
    assert np.array_equal(out8, want8), "UV MXFP8 identity (1.0 x 2^e) not exact"


def check_uv_scale_closed_form(lib=None, H=8, M=2):
    """Payload 1.0 everywhere, E8M0 byte 127 - ((h+v+j) mod 9) for latent group
    j = c/32, x = 2^-(c mod 4): an exact integer count of 2^-11 units."""
    w = np.full((H, 128, 512), 0x38, np.uint8)
    hh, vv, jj = np.meshgrid(np.arange(H), np.arange(128), np.arange(16), indexing="ij")
    s = (127 - (hh + vv + jj) % 9).astype(np.uint8)
    xk = np.array([2.0 ** -(c % 4) for c in range(512)], np.float32)
    x = np.broadcast_to(bf16_bits(xk), (M, H, 512)).copy()
    out = oracle.uv_projection(x, w, s, weight_format=1, lib_path=lib)["out"]
    units = np.zeros((H, 128), np.int64)
    for h in range(H):
        for v in range(128):
            units[h, v] = sum(1 << (11 - (c % 4) - ((h + v + c // 32) % 9)) for c in range(512))
    want = bf16_bits((units.astype(np.float64) / 2048.0).astype(np.float32))
    for m in range(M):
        assert np.array_equal(out[m], want), "UV E8M0 scale applied to the wrong (v, c) group"


GAMMA_512 = (512 * 2.0 ** -24) / (1 - 512 * 2.0 ** -24)


def check_uv_brute_force(lib=None):
    """H, M in 1..2, C = 64, V = 8: the fp32 accumulator within gamma_C * sum|x w|
    of the exact rational sum, the bf16 result within one ulp of it."""
    C, V = 64, 8
    gamma = (C * 2.0 ** -24) / (1 - C * 2.0 ** -24)
    for wf in (0, 1):
        for H in (1, 2):
            for M in (1, 2):
                rng = _rng(700 + 10 * H + M + 50 * wf)
                x = _rand_bf16(rng, (M, H, C))
                if wf == 0:
                    w = _rand_bf16(rng, (H, V, C), std=C ** -0.5)
                    s = None
                    wval = _f32(w).astype(np.float64)
                else:
                    w = e4m3_bits(rng.standard_normal((H, V, C)).astype(np.float32) * 0.1)
                    s = (127 + rng.integers(-8, 1, (H, V, C // MX_BLOCK))).astype(np.uint8)
                    dec = torch.from_numpy(w.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                    wval = dec * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(MX_BLOCK, axis=2)
                res = oracle.uv_projection(x, w, s, weight_format=wf, lib_path=lib)
                xv = _f32(x).astype(np.float64)
                for m in range(M):
                    for h in range(H):
                        for v in range(V):
                            terms = [Fraction(xv[m, h, c]) * Fraction(wval[h, v, c]) for c in range(C)]
                            exact = sum(terms, Fraction(0))
                            sabs = sum(abs(t) for t in terms)
                            acc = Fraction(float(res["acc"][m, h, v]))
                            assert abs(acc - exact) <= Fraction(gamma) * sabs, (wf, H, M, m, h, v)
                            y = float(_f32(res["out"][m, h, v:v + 1])[0])
                            assert abs(Fraction(y) - exact) <= Fraction(float(_ulp_bf16(float(exact)))), (m, h, v)


ALL_CHECKS.extend([check_uv_identity, check_uv_scale_closed_form, check_uv_brute_force])


# --------------------------------------------------------------------------
# Dense MLA decode attention with split partials
# --------------------------------------------------------------------------

def check_bf16_round_f64(lib=None):
    """double -> bf16 against an independent route: round to odd into fp32
    (truncate toward zero, set the last bit when inexact), then torch's fp32 ->
    bf16 cast. With 16 extra bits, round-to-odd followed by round-to-nearest
    gives the correctly rounded result (Boldo and Melquiond, "Emulation of FMA
    and correctly rounded sums: proved algorithms using rounding to odd").
    Midpoints and their double-precision neighbours, where a plain double ->
    fp32 -> bf16 route would round twice, are included."""
    rng = _rng(31)
    mags = np.ldexp(rng.random(20000) + 0.5, rng.integers(-140, 128, 20000))
    x = np.concatenate([mags * rng.choice([-1.0, 1.0], 20000), [0.0, -0.0, 1.0, -2.5]])
    # exact midpoints between neighbouring bf16 values and one double ulp either side
    lo = _f32(np.arange(0x3F80, 0x3FC0, dtype=np.uint16)).astype(np.float64)
    hi = _f32(np.arange(0x3F81, 0x3FC1, dtype=np.uint16)).astype(np.float64)
    mid = (lo + hi) / 2
    x = np.concatenate([x, mid, np.nextafter(mid, 0.0), np.nextafter(mid, 4.0), -mid,
                        [3.3895313892515355e38, 3.3961775292304957e38, 3.4e38, 1e300, 2.0 ** -133, 2.0 ** -134,
                         3 * 2.0 ** -135, 2.0 ** -140]])
    ours = oracle.bf16_round_f64(x, lib_path=lib)
    with np.errstate(over="ignore"):
        f = x.astype(np.float32)  # round to nearest
    f64 = f.astype(np.float64)
    over = np.abs(f64) > np.abs(x)
    f = np.where(over, np.nextafter(f, np.float32(0)), f)  # toward zero
    inexact = f.astype(np.float64) != x
    fb = f.view(np.uint32) | inexact.astype(np.uint32)  # round to odd
    fb = np.where(np.isinf(f), f.view(np.uint32), fb)
    ref = torch.from_numpy(fb.view(np.float32).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    big = np.abs(x) >= 3.3961775292304957e38  # past the last midpoint: infinity
    ref = np.where(big, np.where(x > 0, 0x7F80, 0xFF80), ref).astype(np.uint16)
    bad = ours != ref
    assert not bad.any(), f"double -> bf16 differs at {x[bad][:4]}: {ours[bad][:4]} vs {ref[bad][:4]}"


def _attn(inp, lib=None, **kw):
    return oracle.attention(inp.q, inp.kv, inp.block_table, inp.seq_lens,
                            softmax_scale=inp.softmax_scale, lib_path=lib, **kw)


def _gather(inp, m):
    """Rows of sequence m in token order, by numpy indexing (float64)."""
    T = int(inp.seq_lens[m])
    t = np.arange(T)
    pages = inp.block_table[m, t // inp.page_size]
    rows = inp.kv[pages, t % inp.page_size]
    return _f32(rows).astype(np.float64)


def _attn_case(seed, H, lens, P=64, **kw):
    from workloads import make_attn_inputs

    return make_attn_inputs(seed, H, lens, page_size=P, **kw)


def check_attn_against_sdpa(lib=None):
    """The unsplit definition against torch's scaled_dot_product_attention in
    float64 on the CPU (keys = whole 576-wide row, values = its first 512
    entries, shared by all heads), and lse against torch.logsumexp of the
    scores. Covers several pages per sequence, page size 16 and 64, and scores
    large enough that exp without the max shift would overflow."""
    for P, lens, qstd in ((64, [1, 70, 200, 129], 1.0), (16, [33, 5, 64], 1.0), (64, [90, 3], 40.0)):
        inp = _attn_case(1100 + P + len(lens), 5, lens, P=P, q_std=qstd)
        res = _attn(inp, lib)
        for m in range(inp.M):
            rows = _gather(inp, m)
            q = torch.from_numpy(_f32(inp.q[m]).astype(np.float64))  # [H,576]
            k = torch.from_numpy(rows)  # [T,576]
            v = torch.from_numpy(rows[:, :512].copy())
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[None, :, None, :], k[None, None].expand(1, inp.H, -1, -1),
                v[None, None].expand(1, inp.H, -1, -1), scale=inp.softmax_scale)[0, :, 0, :].numpy()
            got = res["o"][m]
            err = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
            assert err < 1e-11, f"P={P} m={m}: o differs from SDPA by {err}"
            lse_ref = torch.logsumexp(inp.softmax_scale * (q @ k.T), dim=1).numpy()
            assert np.allclose(res["lse"][m], lse_ref, rtol=1e-12, atol=1e-9), f"P={P} m={m}: lse"


def check_attn_closed_forms(lib=None):
    """q = 0: o is the plain mean of the values. T = 1: the value row itself,
    bit for bit. Two tokens: logistic weights. T = 0: o = 0, lse = -inf."""
    inp = _attn_case(1200, 3, [130, 1, 0])
    inp.q[0] = 0
    res = _attn(inp, lib)
    mean = _gather(inp, 0)[:, :512].mean(axis=0)
    assert np.allclose(res["o"][0], mean[None, :], rtol=1e-13, atol=1e-15), "q = 0 must average the values"
    t0 = inp.block_table[1, 0]
    assert np.array_equal(res["out"][1], np.broadcast_to(inp.kv[t0, 0, :512], (3, 512))), "T = 1 must copy"
    assert np.all(res["out"][2] == 0) and np.all(np.isneginf(res["lse"][2])), "T = 0"
    # two tokens, q one-hot at rotary dim 530: weights 1/(1 + e^-d), d = scale*a*(x1 - x0)
    two = _attn_case(1201, 2, [2])
    a, x0, x1 = 3.0, 0.5, -1.25
    two.q[:] = 0
    two.q[0, :, 530] = bf16_bits(np.array([a, 2 * a], np.float32))
    pg = two.block_table[0, 0]
    two.kv[pg, 0, 530], two.kv[pg, 1, 530] = bf16_bits(np.array([x0, x1], np.float32))
    res = _attn(two, lib)
    v = _gather(two, 0)[:, :512]
    for h, ah in enumerate((a, 2 * a)):
        d = two.softmax_scale * ah * (x1 - x0)
        w1 = 1.0 / (1.0 + np.exp(-d))
        assert np.allclose(res["o"][0, h], (1 - w1) * v[0] + w1 * v[1], rtol=1e-13, atol=1e-15), "two tokens"


def check_attn_splits(lib=None):
    """Merging exact split partials reproduces the unsplit result (the
    log-sum-exp identity) for any split count; the stored partials and their
    lse match an independent numpy evaluation of each 64-aligned range; FP32
    partials stay within fp32 rounding of the exact result; BF16 partials are
    the bf16 rounding of the exact partial, so one split gives the unsplit
    output bit for bit, and several move the result by at most a bf16 step."""
    inp = _attn_case(1300, 4, [200, 64, 1000, 65, 7])
    exact = _attn(inp, lib)
    for S in (1, 2, 3, 5, 64):
        r = _attn(inp, lib, num_splits=S, partial_dtype=oracle.PARTIAL_EXACT)
        assert np.allclose(r["o"], exact["o"], rtol=1e-12, atol=1e-14), f"S={S}: merge identity"
        assert np.allclose(r["lse"], exact["lse"], rtol=1e-12, atol=1e-12), f"S={S}: merged lse"
    # range boundaries: T = 200, S = 3 -> chunk 67 rounded up to 128: [0,128), [128,200), empty
    S = 3
    r = _attn(inp, lib, num_splits=S, partial_dtype=oracle.PARTIAL_EXACT)
    rows = _gather(inp, 0)
    q = _f32(inp.q[0]).astype(np.float64)
    sc = inp.softmax_scale * (q @ rows.T)  # [H,T]
    for s, (a, b) in enumerate(((0, 128), (128, 200))):
        seg = sc[:, a:b]
        mx = seg.max(axis=1, keepdims=True)
        e = np.exp(seg - mx)
        lse = mx[:, 0] + np.log(e.sum(axis=1))
        part = (e @ rows[a:b, :512]) / e.sum(axis=1, keepdims=True)
        assert np.allclose(r["plse"][0, s], lse, rtol=1e-12, atol=1e-12), f"range {s}: lse_s"
        assert np.allclose(r["part"][0, s], part, rtol=1e-12, atol=1e-14), f"range {s}: partial"
        pv = (e @ np.abs(rows[a:b, :512])) / e.sum(axis=1, keepdims=True)
        assert np.allclose(r["pvabs"][0, s], pv, rtol=1e-12, atol=1e-14), f"range {s}: sum p|v|"
    assert np.all(np.isneginf(r["plse"][0, 2])), "third range of T=200, S=3 is empty"
    # storage dtypes
    f32 = _attn(inp, lib, num_splits=5, partial_dtype=oracle.PARTIAL_FP32)
    scale = np.max(np.abs(exact["o"]))
    assert np.max(np.abs(f32["o"] - exact["o"])) <= 64 * 2.0 ** -24 * scale, "FP32 partials"
    assert np.array_equal(f32["part"], f32["part"].astype(np.float32).astype(np.float64)), "FP32 storage"
    ex5 = _attn(inp, lib, num_splits=5, partial_dtype=oracle.PARTIAL_EXACT)
    want_lse = ex5["plse"].astype(np.float32).astype(np.float64)
    assert np.array_equal(f32["plse"], want_lse), "lse_s is stored as the nearest fp32"
    b16 = _attn(inp, lib, num_splits=5, partial_dtype=oracle.PARTIAL_BF16)
    assert np.array_equal(b16["plse"], want_lse), "lse_s is fp32 with BF16 partials too"
    live = np.isfinite(ex5["plse"])[..., None] & np.ones_like(ex5["part"], bool)
    want = torch.from_numpy(ex5["part"][live].astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    close = np.abs(b16["part"][live] - ex5["part"][live]) <= _ulp_bf16(ex5["part"][live]) / 2 * (1 + 1e-9)
    assert close.all(), "BF16 partials must be the nearest bf16 of the exact partial"
    assert np.mean(b16["part"][live] == want) > 0.99, "BF16 partials"
    assert np.max(np.abs(b16["o"] - exact["o"])) <= 2.0 ** -8 * scale, "BF16 partials move o by < 1 step"
    assert np.max(np.abs(b16["o"] - exact["o"])) > 0, "BF16 partials must round"
    one = _attn(inp, lib, num_splits=1, partial_dtype=oracle.PARTIAL_BF16)
    assert np.array_equal(one["out"], exact["out"]), "one BF16 split = the unsplit bf16 output"


def check_attn_invariants(lib=None):
    """Moving a sequence's pages elsewhere in the pool, or changing the thread
    count, changes no output bit; each sequence and head is computed on its own
    (a batch gives the same bits as the sequences alone)."""
    inp = _attn_case(1400, 6, [300, 17, 128])
    base = _attn(inp, lib, num_splits=3)
    moved = _attn_case(1400, 6, [300, 17, 128])
    n = moved.kv.shape[0]
    perm = _rng(5).permutation(n)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(n)
    moved.kv = moved.kv[perm]
    moved.block_table = np.where(moved.block_table >= 0, inv[np.maximum(moved.block_table, 0)], -1).astype(np.int32)
    for kw in ({"num_splits": 3}, {"num_splits": 3, "threads": 1}):
        r = _attn(moved, lib, **kw)
        assert np.array_equal(r["out"], base["out"]) and np.array_equal(r["lse"], base["lse"]), f"pages moved {kw}"
    for m in range(inp.M):
        one = _attn_case(1400, 6, [300, 17, 128])
        one.q, one.block_table, one.seq_lens = one.q[m:m + 1], one.block_table[m:m + 1], one.seq_lens[m:m + 1]
        r = _attn(one, lib, num_splits=3)
        assert np.array_equal(r["out"][0], base["out"][m]), f"sequence {m} alone"
        r = _attn(dataclass_replace(one, q=one.q[:, 2:4].copy()), lib, num_splits=3)
        assert np.array_equal(r["out"][0], base["out"][m, 2:4]), f"heads 2..3 of sequence {m}"


def dataclass_replace(obj, **kw):
    import dataclasses

    return dataclasses.replace(obj, **kw)


ALL_CHECKS.extend([check_bf16_round_f64, check_attn_against_sdpa, check_attn_closed_forms, check_attn_splits,
                   check_attn_invariants])
