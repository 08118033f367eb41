"""CPU oracle for the fused MLA decode query projection and assembly.

TEST INFRASTRUCTURE ONLY. The product library and its Python binding never
import, load or call anything here; only ``tests/``, the smoke check and the
benchmark's CPU-baseline leg do. It shares no code with the HIP path.

The arithmetic lives in ``mlaq_oracle.c`` (plain C99, built with ``gcc -O2
-ffp-contract=off``); this module only builds it, loads it with ctypes and
marshals numpy arrays. What it computes, and the page passages it follows, are
stated at the top of ``mlaq_oracle.c``:

* per-head product ``q_nope[m,h,:] . W[h,:,n]`` with an fp32 accumulator in
  ascending k (sparkinfer PR #75 "[GG] Add BF16 MLA query projection and
  assembly", sections "What" and "Contract");
* bf16 round-to-nearest-even of the 512-wide projection, then, for E4M3
  output, ``e4m3_satfinite(fp32(y) / q_scale)`` (same page, "Contract");
* ``q_pe`` appended after the projection in the same 576-wide row (same page,
  "What"; vLLM PR #174 "[GG] Fuse MXFP8 and BF16 MLA query assembly",
  "What");
* MXFP8 weights decoded exactly as ``e4m3(P) * 2^(S - 127)`` with one E8M0
  scale per 32 contiguous n of each k row (sparkinfer PR #75, review thread on
  ``api.py``: scale factors along n, N-major weight).

* the V up-projection ``x[m,h,:] . W_UV[h,v,:]`` over the 512 latent values,
  fp32 accumulation, bf16 output (vLLM PR #174, "Layout and topology
  behavior" and "Safety scope and PR 173"; widths are readings);
* dense MLA decode attention over a paged latent cache, evaluated directly or
  through split partials stored as FP32 or BF16 and merged into a BF16 output
  (b12x PR #441 "Allow FP32 split partials in prepared dense MLA", commit
  text and "Behavior"), all in double.

Parity pins: every function here is checked against values the mathematics
or an independent library fixes (tests/oracle_pins.py, run by
tests/test_oracle_pins.py, and the planted mistakes of
tests/test_oracle_mutants.py); none is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SRC = _HERE / "mlaq_oracle.c"
LIB = _HERE / "libmlaq_oracle.so"

WEIGHT_BF16, WEIGHT_MXFP8 = 0, 1
OUT_BF16, OUT_E4M3 = 0, 1
MX_BLOCK = 32
PARTIAL_BF16, PARTIAL_FP32, PARTIAL_EXACT = 0, 1, 2
SPLIT_ALIGN = 64

GCC_FLAGS = ["-O2", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(out: Path | None = None, src: Path | None = None) -> Path:
    """Compile the oracle source (default ``mlaq_oracle.c``) with gcc into a
    shared library and return its path."""
    out = Path(out) if out is not None else LIB
    src = Path(src) if src is not None else SRC
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", *GCC_FLAGS, "-o", str(tmp), str(src), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def _load(path: Path | None = None):
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(str(path)))
    if _lib is None:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        _lib = _declare(ctypes.CDLL(str(LIB)))
    return _lib


def _declare(lib):
    P = ctypes.c_void_p
    lib.mlaq_oracle_run.restype = ctypes.c_int
    lib.mlaq_oracle_run.argtypes = [P, P, P, P, ctypes.c_float, P] + [ctypes.c_int] * 7 + [P, P, P, ctypes.c_int]
    lib.mlaq_oracle_uv_run.restype = ctypes.c_int
    lib.mlaq_oracle_uv_run.argtypes = [P, P, P, P] + [ctypes.c_int] * 5 + [P, P]
    lib.mlaq_oracle_attn_run.restype = ctypes.c_int
    lib.mlaq_oracle_attn_run.argtypes = ([P, P, P, P] + [ctypes.c_int] * 7 + [ctypes.c_double]
                                         + [ctypes.c_int] * 2 + [P] * 8 + [ctypes.c_int])
    lib.mlaq_oracle_qscale.restype = ctypes.c_float
    lib.mlaq_oracle_qscale.argtypes = [P, ctypes.c_size_t, P, ctypes.c_size_t]
    for name in ("mlaq_oracle_bf16_round", "mlaq_oracle_e4m3_encode", "mlaq_oracle_e4m3_decode",
                 "mlaq_oracle_e8m0_decode", "mlaq_oracle_bf16_round_f64"):
        fn = getattr(lib, name)
        fn.restype = None
        fn.argtypes = [P, P, ctypes.c_size_t]
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


class OracleError(RuntimeError):
    pass


def mla_query(q_nope, q_pe, w, w_scales=None, q_scale=None, *, weight_format=WEIGHT_BF16,
              out_dtype=OUT_BF16, threads=1, diagnostics=True, lib_path=None):
    """Run the oracle on host arrays.

    Arguments are numpy arrays of raw bit patterns: ``q_nope`` uint16 (bf16)
    ``[M,H,K]``, ``q_pe`` uint16 ``[M,H,R]``, ``w`` uint16 (bf16) or uint8
    (E4M3) ``[H,K,N]``, ``w_scales`` uint8 (E8M0) ``[H,K,N/32]`` for MXFP8.
    ``q_scale`` is a Python float (used only for E4M3 output).

    Returns a dict: ``out`` (uint16 or uint8 ``[M,H,N+R]``) and, with
    ``diagnostics``, ``acc`` (fp32 accumulators before rounding), ``s_abs``
    (fp64 sum of |q*w|) and ``ref64`` (fp64 sum of q*w), each ``[M,H,N]``.
    """
    lib = _load(lib_path)
    q_nope = _c(q_nope, np.uint16)
    q_pe = _c(q_pe, np.uint16)
    M, H, K = q_nope.shape
    R = q_pe.shape[2]
    if q_pe.shape[:2] != (M, H):
        raise OracleError("q_pe shape does not match q_nope")
    if weight_format == WEIGHT_BF16:
        w = _c(w, np.uint16)
        if w_scales is not None:
            raise OracleError("BF16 weights take no scales")
    else:
        w = _c(w, np.uint8)
        w_scales = _c(w_scales, np.uint8)
    Hw, Kw, N = w.shape
    if (Hw, Kw) != (H, K):
        raise OracleError("weight shape does not match q_nope")
    if weight_format == WEIGHT_MXFP8 and w_scales.shape != (H, K, N // MX_BLOCK):
        raise OracleError("scale shape must be [H,K,N/32]")
    if out_dtype == OUT_E4M3:
        if q_scale is None:
            raise OracleError("E4M3 output needs q_scale")
        out = np.zeros((M, H, N + R), np.uint8)
    else:
        out = np.zeros((M, H, N + R), np.uint16)
    acc = sabs = ref = None
    if diagnostics:
        acc = np.zeros((M, H, N), np.float32)
        sabs = np.zeros((M, H, N), np.float64)
        ref = np.zeros((M, H, N), np.float64)
    rc = lib.mlaq_oracle_run(_ptr(q_nope), _ptr(q_pe), _ptr(w), _ptr(w_scales),
                             float(q_scale if q_scale is not None else 1.0), _ptr(out),
                             M, H, K, N, R, int(weight_format), int(out_dtype),
                             _ptr(acc), _ptr(sabs), _ptr(ref), int(threads))
    if rc != 0:
        raise OracleError(f"mlaq_oracle_run failed with status {rc}")
    res = {"out": out}
    if diagnostics:
        res.update(acc=acc, s_abs=sabs, ref64=ref)
    return res


def uv_projection(x, w, w_scales=None, *, weight_format=WEIGHT_BF16, diagnostics=True, lib_path=None):
    """V up-projection on host arrays: ``x`` uint16 (bf16) ``[M,H,C]``, ``w``
    uint16 (bf16) or uint8 (E4M3) ``[H,V,C]`` (one latent row per value
    column), ``w_scales`` uint8 (E8M0) ``[H,V,C/32]`` for MXFP8. Returns
    ``out`` uint16 ``[M,H,V]`` and, with diagnostics, ``acc`` (fp32) and
    ``s_abs`` (fp64 sum of |x w|). The arithmetic is ``mlaq_oracle_uv_run``."""
    lib = _load(lib_path)
    x = _c(x, np.uint16)
    M, H, C = x.shape
    if weight_format == WEIGHT_BF16:
        w = _c(w, np.uint16)
        if w_scales is not None:
            raise OracleError("BF16 weights take no scales")
    else:
        w = _c(w, np.uint8)
        w_scales = _c(w_scales, np.uint8)
    Hw, V, Cw = w.shape
    if (Hw, Cw) != (H, C):
        raise OracleError("W_UV shape must be [H,V,C]")
    if weight_format == WEIGHT_MXFP8 and w_scales.shape != (H, V, C // MX_BLOCK):
        raise OracleError("scale shape must be [H,V,C/32]")
    out = np.zeros((M, H, V), np.uint16)
    acc = sabs = None
    if diagnostics:
        acc = np.zeros((M, H, V), np.float32)
        sabs = np.zeros((M, H, V), np.float64)
    rc = lib.mlaq_oracle_uv_run(_ptr(x), _ptr(w), _ptr(w_scales), _ptr(out), M, H, C, V, int(weight_format),
                                _ptr(acc), _ptr(sabs))
    if rc != 0:
        raise OracleError(f"mlaq_oracle_uv_run failed with status {rc}")
    res = {"out": out}
    if diagnostics:
        res.update(acc=acc, s_abs=sabs)
    return res


def attention(q, kv, block_table, seq_lens, *, softmax_scale, num_splits=0, partial_dtype=PARTIAL_BF16,
              dv=512, threads=8, diagnostics=True, lib_path=None):
    """Dense MLA decode attention over a paged latent cache, on host arrays.

    ``q`` uint16 (bf16) ``[M,H,D]``; ``kv`` uint16 ``[num_pages,P,D]`` (the
    first ``dv`` entries of a row are the value); ``block_table`` int32
    ``[M,max_blocks]``; ``seq_lens`` int32 ``[M]``. ``num_splits = 0``
    evaluates the definition; ``num_splits >= 1`` runs the split procedure with
    partials stored per ``partial_dtype``. The arithmetic is
    ``mlaq_oracle_attn_run``.

    Returns a dict: ``out`` (uint16 bf16 ``[M,H,dv]``) and, with
    ``diagnostics``, ``o`` (fp64 merged output before rounding), ``lse``
    (``[M,H]``), ``vabs`` (sum_t p_t |v_t|, ``[M,H,dv]``), ``smag`` (max_t of
    scale * sum_d |q_d kv_t[d]|, ``[M,H]``) and, when split, ``part``
    (``[M,S,H,dv]``) and ``plse`` (``[M,S,H]``), the stored partials, and
    ``pvabs`` (``[M,S,H,dv]``: sum_t p_t |v_t| within each range).
    """
    lib = _load(lib_path)
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    M, H, D = q.shape
    num_pages, P, Dk = kv.shape
    if Dk != D:
        raise OracleError("cache rows must have the query's width")
    if block_table.ndim != 2 or block_table.shape[0] != M or seq_lens.shape != (M,):
        raise OracleError("block_table must be [M,max_blocks] and seq_lens [M]")
    out = np.zeros((M, H, dv), np.uint16)
    o = lse = vabs = smag = part = plse = pvabs = None
    if diagnostics:
        o = np.zeros((M, H, dv), np.float64)
        lse = np.zeros((M, H), np.float64)
        vabs = np.zeros((M, H, dv), np.float64)
        smag = np.zeros((M, H), np.float64)
        if num_splits > 0:
            part = np.zeros((M, num_splits, H, dv), np.float64)
            plse = np.zeros((M, num_splits, H), np.float64)
            pvabs = np.zeros((M, num_splits, H, dv), np.float64)
    rc = lib.mlaq_oracle_attn_run(_ptr(q), _ptr(kv), _ptr(block_table), _ptr(seq_lens), M, H, D, int(dv), P,
                                  num_pages, block_table.shape[1], float(softmax_scale), int(num_splits),
                                  int(partial_dtype), _ptr(out), _ptr(o), _ptr(lse), _ptr(vabs), _ptr(smag),
                                  _ptr(part), _ptr(plse), _ptr(pvabs), int(threads))
    if rc != 0:
        raise OracleError(f"mlaq_oracle_attn_run failed with status {rc}")
    res = {"out": out}
    if diagnostics:
        res.update(o=o, lse=lse, vabs=vabs, smag=smag)
        if num_splits > 0:
            res.update(part=part, plse=plse, pvabs=pvabs)
    return res


def qscale_from_result(acc, q_pe, lib_path=None) -> float:
    """amax/448 over the fp32 projection and q_pe (1.0 when amax is 0)."""
    lib = _load(lib_path)
    acc = _c(acc, np.float32)
    q_pe = _c(q_pe, np.uint16)
    return float(lib.mlaq_oracle_qscale(_ptr(acc), acc.size, _ptr(q_pe), q_pe.size))


def _elementwise(name, arr, in_dtype, out_dtype, lib_path=None):
    lib = _load(lib_path)
    a = _c(arr, in_dtype)
    out = np.empty(a.shape, out_dtype)
    getattr(lib, name)(_ptr(a), _ptr(out), a.size)
    return out


def bf16_round(x, lib_path=None):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    return _elementwise("mlaq_oracle_bf16_round", x, np.float32, np.uint16, lib_path)


def bf16_round_f64(x, lib_path=None):
    """float64 array -> bf16 bit patterns (uint16), one round to nearest even."""
    return _elementwise("mlaq_oracle_bf16_round_f64", x, np.float64, np.uint16, lib_path)


def e4m3_encode(x, lib_path=None):
    """fp32 array -> E4M3FN codes (uint8), nearest-even, saturating to +-448."""
    return _elementwise("mlaq_oracle_e4m3_encode", x, np.float32, np.uint8, lib_path)


def e4m3_decode(codes, lib_path=None):
    """E4M3FN codes -> float64 values (NaN for 0x7F/0xFF)."""
    return _elementwise("mlaq_oracle_e4m3_decode", codes, np.uint8, np.float64, lib_path)


def e8m0_decode(codes, lib_path=None):
    """E8M0 bytes -> float64 2^(b-127) (NaN for 0xFF)."""
    return _elementwise("mlaq_oracle_e8m0_decode", codes, np.uint8, np.float64, lib_path)


def bf16_to_f32(bits):
    """Reinterpret bf16 bit patterns as float32 (a bit shift; not arithmetic)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
