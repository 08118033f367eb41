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
    return re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(mlaq_\w+)\s*\(", text, re.M)


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == {"mlaq_plan_supported", "mlaq_can_implement", "mlaq_prewarm",
                                         "mlaq_run", "mlaq_run_ex", "mlaq_last_error", "mlaq_uv_plan_supported",
                                         "mlaq_uv_can_implement", "mlaq_uv_prewarm", "mlaq_uv_run",
                                         "mlaq_uv_run_ex", "mlaq_attn_workspace_size", "mlaq_attn_num_splits",
                                         "mlaq_attn_plan_supported", "mlaq_attn_can_implement", "mlaq_attn_prewarm",
                                         "mlaq_attn_run", "mlaq_attn_run_noalloc"}


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared in mlaq.h but not exported"


def test_python_constants_match_header():
    defines = dict(re.findall(r"#define\s+(MLAQ_\w+)\s+(\d+)", HEADER.read_text()))
    for name, value in defines.items():
        key = {"MLAQ_NOPE_DIM": "NOPE_DIM", "MLAQ_NOPE_DIM_GLM": "NOPE_DIM_GLM", "MLAQ_LATENT_DIM": "LATENT_DIM",
               "MLAQ_ROPE_DIM": "ROPE_DIM", "MLAQ_MAX_M": "MAX_M", "MLAQ_V_DIM": "V_DIM"}.get(name, name)
        assert getattr(mq, key) == int(value), name


OK, UNS, INV = mq.MLAQ_OK, mq.MLAQ_ERR_UNSUPPORTED, mq.MLAQ_ERR_INVALID_ARG


@pytest.mark.parametrize("wf", [0, 1])
@pytest.mark.parametrize("od", [0, 1])
@pytest.mark.parametrize("h", [8, 11, 16])
@pytest.mark.parametrize("m", [1, 17, 32])
@pytest.mark.parametrize("k", [128, 192])
def test_gate_accepts_supported_plans(lib, wf, od, h, m, k):
    assert mq.mlaq_plan_supported(h, m, k, weight_format=wf, out_dtype=od, arch="gfx950:sramecc+:xnack-") == OK
    assert mq.mlaq_plan_supported(h, m, k, weight_format=wf, out_dtype=od, arch="gfx950") == OK


@pytest.mark.parametrize("args,status,msg", [
    (dict(num_heads=12, max_m=1), UNS, "num_heads"),
    (dict(num_heads=4, max_m=1), UNS, "num_heads"),
    (dict(num_heads=16, max_m=0), UNS, "max_m"),
    (dict(num_heads=16, max_m=33), UNS, "max_m"),
    (dict(num_heads=16, max_m=4, nope_dim=256), UNS, "dims"),
    (dict(num_heads=16, max_m=4, nope_dim=64), UNS, "dims"),
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


HEADER_PROBE = r"""
#include <stddef.h>
#include <stdio.h>
#include "mlaq.h"
int main(void) {
  printf("%zu", sizeof(mlaq_run_args));
#define F(x) printf(" %zu", offsetof(mlaq_run_args, x));
  F(q_nope) F(q_stride_m) F(q_stride_h) F(q_pe) F(pe_stride_m) F(pe_stride_h) F(w) F(w_scales) F(q_scale)
  F(out) F(out_stride_m) F(out_stride_h) F(M) F(H) F(nope_dim) F(weight_format) F(out_dtype) F(cache_hint)
  printf("\n");
  return 0;
}
"""


def test_run_args_layout_matches_header(tmp_path):
    """The binding's ctypes mirror has the C struct's size and field offsets
    (the header compiled by gcc as a C program)."""
    import subprocess

    src = tmp_path / "probe.c"
    src.write_text(HEADER_PROBE)
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", f"-I{HEADER.parent}", "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(mq.RunArgs)] + [getattr(mq.RunArgs, name).offset for name, _ in mq.RunArgs._fields_]
    assert got == want


def run_ex(lib, **kw):
    a = mq.RunArgs(A, 2048, 128, 2 * A, 1024, 64, 4 * A, None, None, 8 * A, 16 * 576, 576, 4, 16, 128, 0, 0)
    for k, v in kw.items():
        setattr(a, k, v)
    return lib.mlaq_run_ex(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(nope_dim=256), UNS, "nope_dim=256"),
    (dict(nope_dim=64), UNS, "nope_dim=64"),
    (dict(q_stride_m=-8), INV, "strides"),
    (dict(q_stride_h=100), INV, "strides"),
    (dict(pe_stride_h=4), INV, "strides"),
    (dict(out_stride_h=572), INV, "strides"),
    (dict(out_stride_h=1 << 24), INV, "strides"),
    (dict(q_stride_h=1 << 16), INV, "head strides"),   # head strides travel as 16-bit halves
    (dict(pe_stride_h=1 << 16), INV, "head strides"),
    (dict(out_stride_h=568), INV, "overlap"),          # rows of 576 elements would overlap
    (dict(out_stride_m=576 * 8), INV, "overlap"),      # m-major but tokens collide with heads
    (dict(out_stride_m=0, out_stride_h=576), INV, "overlap"),
    (dict(out=2 * A + 4096), INV, "overlaps an input"),
    (dict(q_nope=None), INV, "non-NULL"),
    (dict(w=4 * A + 8), INV, "16-byte aligned"),
    (dict(weight_format=1), INV, "need w_scales"),
    (dict(out_dtype=1), INV, "needs q_scale"),
    (dict(H=12), UNS, "H=12"),
    (dict(M=40), UNS, "M=40"),
    (dict(cache_hint=2), INV, "cache_hint 2"),
    (dict(cache_hint=-1), INV, "cache_hint -1"),
])
def test_run_ex_rejects_before_any_device_call(lib, kw, status, msg):
    assert run_ex(lib, **kw) == status
    assert msg in mq.mlaq_last_error()


def test_run_args_cache_hint_fills_tail_padding():
    """cache_hint sits in what was the struct's tail padding: the size is that
    of the fields before it rounded to 8 bytes, and a zero-initialised struct
    carries MLAQ_CACHE_DEFAULT."""
    assert ctypes.sizeof(mq.RunArgs) == 8 * 12 + 4 * 6
    assert mq.RunArgs.cache_hint.offset == 8 * 12 + 4 * 5
    assert mq.RunArgs().cache_hint == mq.MLAQ_CACHE_DEFAULT == 0
    assert mq.MLAQ_CACHE_STREAM == 1


def test_run_ex_null_args_and_empty_batch(lib):
    assert lib.mlaq_run_ex(None, None) == INV
    assert "NULL" in mq.mlaq_last_error()
    assert run_ex(lib, M=0, q_nope=None, out=None, nope_dim=192) == OK



@pytest.mark.parametrize("wf", [0, 1])
@pytest.mark.parametrize("h", [8, 11, 16])
@pytest.mark.parametrize("m", [1, 16, 32])
def test_uv_gate_accepts(lib, wf, h, m):
    assert mq.mlaq_uv_plan_supported(h, m, weight_format=wf) == OK


@pytest.mark.parametrize("args,status,msg", [
    (dict(num_heads=12, max_m=1), UNS, "num_heads"),
    (dict(num_heads=16, max_m=33), UNS, "max_m"),
    (dict(num_heads=16, max_m=4, latent_dim=576), UNS, "dims"),
    (dict(num_heads=16, max_m=4, v_dim=64), UNS, "dims"),
    (dict(num_heads=16, max_m=4, arch="gfx942"), UNS, "not gfx950"),
    (dict(num_heads=16, max_m=4, weight_format=5), INV, "weight_format"),
    (dict(num_heads=16, max_m=4, arch=None), INV, "arch"),
])
def test_uv_gate_rejects(lib, args, status, msg):
    assert mq.mlaq_uv_plan_supported(**args) == status
    assert msg in mq.mlaq_last_error()


def uv_run(lib, x=A, w=2 * A, s=None, out=4 * A, M=4, H=16, wf=0):
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.mlaq_uv_run(v(x), v(w), v(s), v(out), M, H, wf, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=None), INV, "non-NULL"),
    (dict(out=None), INV, "non-NULL"),
    (dict(wf=1), INV, "need w_uv_scales"),
    (dict(s=8 * A), INV, "no w_uv_scales"),
    (dict(x=A + 8), INV, "16-byte aligned"),
    (dict(out=2 * A + 256), INV, "overlaps"),
    (dict(H=7), UNS, "H=7"),
    (dict(M=33), UNS, "M=33"),
    (dict(wf=9), INV, "weight_format"),
])
def test_uv_run_rejects_before_any_device_call(lib, kw, status, msg):
    assert uv_run(lib, **kw) == status
    assert msg in mq.mlaq_last_error()


def test_uv_empty_batch_is_a_noop(lib):
    assert uv_run(lib, x=None, w=None, out=None, M=0) == OK


@pytest.mark.parametrize("hint", [2, -1, 7])
def test_uv_run_ex_rejects_unknown_cache_hint(lib, hint):
    v = ctypes.c_void_p
    assert lib.mlaq_uv_run_ex(v(A), v(2 * A), None, v(4 * A), 4, 16, 0, hint, None) == INV
    assert f"cache_hint {hint}" in mq.mlaq_last_error()


def test_uv_run_ex_default_hint_matches_uv_run_checks(lib):
    """Both entry points reject the same bad plan the same way (the hint is
    checked after the weight format, before anything else)."""
    v = ctypes.c_void_p
    for hint in (0, 1):
        assert lib.mlaq_uv_run_ex(v(A), v(2 * A), None, v(2 * A + 256), 4, 16, 0, hint, None) == INV
        assert "overlaps" in mq.mlaq_last_error()
        assert lib.mlaq_uv_run_ex(None, None, None, None, 0, 16, 0, hint, None) == OK


# --------------------------------------------------------------------------
# Dense MLA decode attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("h", [1, 8, 11, 16])
@pytest.mark.parametrize("page,splits", [(1, 1), (64, 16), (4096, 256)])
@pytest.mark.parametrize("pd", [0, 1])
def test_attn_gate_accepts(lib, h, page, splits, pd):
    assert mq.mlaq_attn_plan_supported(h, page, splits, pd) == OK


@pytest.mark.parametrize("args,status,msg", [
    ((0, 64, 4, 0), UNS, "num_heads=0"),
    ((17, 64, 4, 0), UNS, "num_heads=17"),
    ((16, 0, 4, 0), UNS, "page_size=0"),
    ((16, 4097, 4, 0), UNS, "page_size=4097"),
    ((16, 64, 0, 0), UNS, "num_splits=0"),
    ((16, 64, 257, 0), UNS, "num_splits=257"),
    ((16, 64, 4, 2), INV, "partial_dtype"),
])
def test_attn_gate_rejects(lib, args, status, msg):
    assert mq.mlaq_attn_plan_supported(*args) == status
    assert msg in mq.mlaq_last_error()
    assert mq.mlaq_attn_plan_supported(16, 64, 4, 0, arch="gfx942") == UNS
    assert mq.mlaq_attn_plan_supported(16, 64, 4, 0, arch=None) == INV


def test_attn_workspace_size(lib):
    def r256(n):
        return (n + 255) // 256 * 256

    for M, H, S, pd in ((32, 16, 16, 0), (32, 16, 16, 1), (3, 11, 5, 0), (1, 1, 256, 1)):
        esz = 4 if pd else 2
        assert mq.mlaq_attn_workspace_size(M, H, S, pd) == r256(M * S * H * 512 * esz) + r256(M * S * H * 4)
    assert mq.mlaq_attn_workspace_size(32, 16, 1, 0) == 0  # one split writes the output directly
    for bad in ((32, 17, 4, 0), (32, 16, 0, 0), (32, 16, 257, 0), (32, 16, 4, 3), (-1, 16, 4, 0)):
        assert mq.mlaq_attn_workspace_size(*bad) == 0


ATTN_PROBE = r"""
#include <stddef.h>
#include <stdio.h>
#include "mlaq.h"
int main(void) {
  printf("%zu", sizeof(mlaq_attn_args));
#define F(x) printf(" %zu", offsetof(mlaq_attn_args, x));
  F(q) F(q_stride_m) F(q_stride_h) F(kv_cache) F(block_table) F(seq_lens) F(out) F(lse) F(workspace)
  F(workspace_bytes) F(softmax_scale) F(M) F(H) F(page_size) F(num_pages) F(block_table_stride) F(num_splits)
  F(partial_dtype)
  printf("\n");
  return 0;
}
"""


def test_attn_args_layout_matches_header(tmp_path):
    import subprocess

    src = tmp_path / "probe.c"
    src.write_text(ATTN_PROBE)
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", f"-I{HEADER.parent}", "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(mq.AttnArgs)] + [getattr(mq.AttnArgs, name).offset for name, _ in mq.AttnArgs._fields_]
    assert got == want


def attn_run(lib, **kw):
    # q [4,16,576] at A (18 KiB pitch), kv 10 pages of 64 rows at 64A, table at 2A, lens at 3A, out at 4A,
    # workspace at 8A: all disjoint, never dereferenced (every case fails validation first).
    M, H, S = 4, 16, 4
    a = mq.AttnArgs(A, 16 * 576, 576, 64 * A, 2 * A, 3 * A, 4 * A, None, 8 * A,
                    mq.mlaq_attn_workspace_size(M, H, S, 0), 0.07, M, H, 64, 10, 8, S, 0)
    for k, v in kw.items():
        setattr(a, k, v)
    return lib.mlaq_attn_run(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(partial_dtype=5), INV, "partial_dtype"),
    (dict(H=0), UNS, "H=0"),
    (dict(H=17), UNS, "H=17"),
    (dict(page_size=0), UNS, "page_size=0"),
    (dict(num_splits=0), UNS, "num_splits=0"),
    (dict(num_splits=300), UNS, "num_splits=300"),
    (dict(M=70000), UNS, "M=70000"),
    (dict(q=None), INV, "non-NULL"),
    (dict(kv_cache=None), INV, "non-NULL"),
    (dict(block_table=None), INV, "non-NULL"),
    (dict(seq_lens=None), INV, "non-NULL"),
    (dict(out=None), INV, "non-NULL"),
    (dict(num_pages=0), INV, "num_pages"),
    (dict(block_table_stride=0), INV, "block_table_stride"),
    (dict(block_table_stride=1 << 24, page_size=128), UNS, "2^30"),
    (dict(softmax_scale=float("nan")), INV, "finite"),
    (dict(softmax_scale=float("inf")), INV, "finite"),
    (dict(q_stride_h=100), INV, "multiples of 8"),
    (dict(q_stride_m=-8), INV, "multiples of 8"),
    (dict(q_stride_m=1 << 31), INV, "below 2^31"),  # strides travel as 32-bit kernel arguments
    (dict(q=A + 8), INV, "16-byte aligned"),
    (dict(kv_cache=64 * A + 4), INV, "16-byte aligned"),
    (dict(out=4 * A + 2), INV, "16-byte aligned"),
    (dict(block_table=2 * A + 2), INV, "4-byte aligned"),
    (dict(lse=5 * A + 1), INV, "4-byte aligned"),
    (dict(workspace=None), INV, "workspace must hold"),
    (dict(workspace_bytes=1000), INV, "workspace must hold"),
    (dict(workspace=8 * A + 128), INV, "256-byte aligned"),
    (dict(out=64 * A + 4096), INV, "overlaps an input"),
    (dict(workspace=A + 256), INV, "overlaps an input"),
    (dict(lse=4 * A + 1024), INV, "must not overlap"),
])
def test_attn_run_rejects_before_any_device_call(lib, kw, status, msg):
    assert attn_run(lib, **kw) == status
    assert msg in mq.mlaq_last_error()


def test_attn_run_null_args_and_empty_batch(lib):
    assert lib.mlaq_attn_run(None, None) == INV
    assert attn_run(lib, M=0, q=None, kv_cache=None, out=None) == OK
    assert mq.mlaq_last_error() == ""


def test_attn_num_splits_rejects_before_device(lib):
    n = ctypes.c_int(0)
    assert lib.mlaq_attn_num_splits(4, 100, 0, None) == INV
    assert lib.mlaq_attn_num_splits(0, 100, 0, ctypes.byref(n)) == INV
    assert lib.mlaq_attn_num_splits(4, -1, 0, ctypes.byref(n)) == INV
    assert lib.mlaq_attn_num_splits(4, 100, 99, ctypes.byref(n)) == INV  # device ordinal out of range
    assert lib.mlaq_attn_prewarm(7, 0) == INV


def attn_run_noalloc(lib, **kw):
    # The same disjoint, never dereferenced pointers as attn_run, with no workspace.
    M, H, S = 4, 16, 4
    a = mq.AttnArgs(A, 16 * 576, 576, 64 * A, 2 * A, 3 * A, 4 * A, None, None, 0, 0.07, M, H, 64, 10, 8, S, 0)
    for k, v in kw.items():
        setattr(a, k, v)
    return lib.mlaq_attn_run_noalloc(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(workspace=8 * A), INV, "takes no workspace"),
    (dict(workspace_bytes=4096), INV, "takes no workspace"),
    (dict(partial_dtype=5), INV, "partial_dtype"),
    (dict(H=17), UNS, "H=17"),
    (dict(num_splits=300), UNS, "num_splits=300"),
    (dict(q=None), INV, "non-NULL"),
    (dict(q_stride_h=100), INV, "multiples of 8"),
    (dict(out=64 * A + 4096), INV, "overlaps an input"),
    # 4096 sequences x 16 heads x 64 splits of BF16 partials: 1 GiB, above the 32 MiB array.
    (dict(M=4096, num_splits=64), UNS, "bytes of scratch"),
    # FP32 partials of 32 x 16 x 64 splits: 67 MB.
    (dict(M=32, num_splits=64, partial_dtype=1), UNS, "bytes of scratch"),
])
def test_attn_run_noalloc_rejects_before_any_device_call(lib, kw, status, msg):
    assert attn_run_noalloc(lib, **kw) == status
    assert msg in mq.mlaq_last_error()


def test_attn_run_noalloc_null_args_and_empty_batch(lib):
    assert lib.mlaq_attn_run_noalloc(None, None) == INV
    assert attn_run_noalloc(lib, M=0, q=None, kv_cache=None, out=None) == OK
    assert mq.mlaq_last_error() == ""


def test_attn_scratch_limit_matches_header():
    text = HEADER.read_text()
    m = re.search(r"#define MLAQ_ATTN_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mq.MLAQ_ATTN_SCRATCH_BYTES == 32 << 20
    # The decode batch of the benchmark (32 sequences, 16 heads, 16 splits) fits in both partial dtypes.
    assert mq.mlaq_attn_workspace_size(32, 16, 16, 1) <= mq.MLAQ_ATTN_SCRATCH_BYTES
    assert mq.mlaq_attn_workspace_size(32, 16, 16, 0) <= mq.MLAQ_ATTN_SCRATCH_BYTES
