"""CPU checks of the C-ABI boundary: libmlaq.so loads, exports every function
include/mlaq.h declares, agrees with the header's constants, and its host
logic (the pure capability gate, argument validation) gives the documented
status for each case. Only calls that return before any HIP call are made
here: invalid arguments are rejected first, so no kernel is ever launched."""

import ctypes
import re
from pathlib import Path

import pytest

import mla_decode_query_amd as mq
from mla_decode_query_amd import _build

HEADER = Path(__file__).resolve().parents[1] / "include" / "mlaq.h"


@pytest.fixture(scope="module")
def lib():
    if not mq.LIB_PATH.exists():
        _build.build()
    return mq.library()


def declared_functions():
    text = HEADER.read_text()
    return re.findall(r"^\s*(?:int|const char\s*\*)\s*(mlaq_\w+)\s*\(", text, re.M)


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == {"mlaq_plan_supported", "mlaq_can_implement", "mlaq_prewarm",
                                         "mlaq_run", "mlaq_last_error"}


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared in mlaq.h but not exported"


def test_python_constants_match_header():
    defines = dict(re.findall(r"#define\s+(MLAQ_\w+)\s+(\d+)", HEADER.read_text()))
    for name, value in defines.items():
        key = {"MLAQ_NOPE_DIM": "NOPE_DIM", "MLAQ_LATENT_DIM": "LATENT_DIM", "MLAQ_ROPE_DIM": "ROPE_DIM",
               "MLAQ_MAX_M": "MAX_M"}.get(name, name)
        assert getattr(mq, key) == int(value), name


OK, UNS, INV = mq.MLAQ_OK, mq.MLAQ_ERR_UNSUPPORTED, mq.MLAQ_ERR_INVALID_ARG


@pytest.mark.parametrize("wf", [0, 1])
@pytest.mark.parametrize("od", [0, 1])
@pytest.mark.parametrize("h", [8, 11, 16])
@pytest.mark.parametrize("m", [1, 17, 32])
def test_gate_accepts_supported_plans(lib, wf, od, h, m):
    assert mq.mlaq_plan_supported(h, m, weight_format=wf, out_dtype=od, arch="gfx950:sramecc+:xnack-") == OK
    assert mq.mlaq_plan_supported(h, m, weight_format=wf, out_dtype=od, arch="gfx950") == OK


@pytest.mark.parametrize("args,status,msg", [
    (dict(num_heads=12, max_m=1), UNS, "num_heads"),
    (dict(num_heads=4, max_m=1), UNS, "num_heads"),
    (dict(num_heads=16, max_m=0), UNS, "max_m"),
    (dict(num_heads=16, max_m=33), UNS, "max_m"),
    (dict(num_heads=16, max_m=4, nope_dim=192), UNS, "dims"),
    (dict(num_heads=16, max_m=4, latent_dim=256), UNS, "dims"),
    (dict(num_heads=16, max_m=4, rope_dim=32), UNS, "dims"),
    (dict(num_heads=16, max_m=4, arch="gfx942:sramecc+:xnack-"), UNS, "not gfx950"),
    (dict(num_heads=16, max_m=4, arch="gfx9500"), UNS, "not gfx950"),
    (dict(num_heads=16, max_m=4, arch="gfx90a"), UNS, "not gfx950"),
    (dict(num_heads=16, max_m=4, weight_format=2), INV, "weight_format"),
    (dict(num_heads=16, max_m=4, out_dtype=-1), INV, "out_dtype"),
    (dict(num_heads=16, max_m=4, arch=None), INV, "arch"),
])
def test_gate_rejects(lib, args, status, msg):
    assert mq.mlaq_plan_supported(**args) == status
    assert msg in mq.mlaq_last_error()


def test_gate_is_per_recipe(lib):
    # The BF16 recipe is decided by its own gate: an MXFP8-only condition
    # (latent width a multiple of 32) does not apply to it, and both recipes
    # reach the same verdict on the shapes they share.
    for wf in (0, 1):
        assert mq.mlaq_plan_supported(16, 8, weight_format=wf) == OK
    assert mq.mlaq_plan_supported(16, 8, latent_dim=500, weight_format=1) == UNS
    assert "multiple of 32" in mq.mlaq_last_error()
    assert mq.mlaq_plan_supported(16, 8, latent_dim=500, weight_format=0) == UNS
    assert "dims" in mq.mlaq_last_error()


A = 1 << 20  # a 16-byte-aligned fake address; never dereferenced by these cases


def run(lib, q=A, pe=2 * A, w=4 * A, s=None, qs=None, out=8 * A, M=4, H=16, wf=0, od=0):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mlaq_run(v(q), v(pe), v(w), v(s), v(qs), v(out), M, H, wf, od, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), INV, "non-NULL"),
    (dict(pe=None), INV, "non-NULL"),
    (dict(w=None), INV, "non-NULL"),
    (dict(out=None), INV, "non-NULL"),
    (dict(wf=1), INV, "need w_scales"),
    (dict(wf=0, s=16 * A), INV, "no w_scales"),
    (dict(od=1), INV, "needs q_scale"),
    (dict(od=0, qs=32 * A), INV, "no q_scale"),
    (dict(q=A + 8), INV, "16-byte aligned"),
    (dict(out=8 * A + 4), INV, "16-byte aligned"),
    (dict(od=1, qs=32 * A + 2), INV, "4-byte aligned"),
    (dict(out=A), INV, "overlaps"),
    (dict(out=2 * A + 64), INV, "overlaps"),
    (dict(out=4 * A - 16), INV, "overlaps"),
    (dict(wf=1, s=8 * A + 512), INV, "overlaps"),
    (dict(H=12), UNS, "H=12"),
    (dict(H=0), UNS, "H=0"),
    (dict(M=33), UNS, "M=33"),
    (dict(M=-1), UNS, "M=-1"),
    (dict(wf=3), INV, "weight_format"),
    (dict(od=7), INV, "out_dtype"),
])
def test_run_rejects_before_any_device_call(lib, kw, status, msg):
    assert run(lib, **kw) == status
    assert msg in mq.mlaq_last_error()


def test_run_with_no_tokens_is_a_noop(lib):
    # M = 0: nothing to read or write, so even NULL buffers are accepted.
    assert run(lib, q=None, pe=None, w=None, out=None, M=0) == OK
    assert mq.mlaq_last_error() == ""


def test_prewarm_rejects_bad_regimes_before_device(lib):
    assert lib.mlaq_prewarm(16, None, 3, 0, 0, 0) == INV
    assert lib.mlaq_prewarm(16, None, -1, 0, 0, 0) == INV
    assert lib.mlaq_prewarm(16, None, 0, 0, 0, 99) == INV  # device ordinal out of range
