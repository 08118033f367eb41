"""Python binding of libmlaq, the MI355X fused MLA decode query projection.

Argument marshalling only: every step of the operation runs in the HIP
kernels of ``libmlaq.so`` (built in-tree by ``mla_decode_query_amd._build``).
PyTorch supplies device memory and the current stream. There is no fallback:
if the library is missing or a call fails, these functions raise.

The entry points carry the C names (see ``include/mlaq.h``):

* ``mlaq_plan_supported`` -- pure capability gate for an architecture name;
* ``mlaq_can_implement``  -- the gate for a device (sparkinfer PR #75
  "[GG] Add BF16 MLA query projection and assembly", review thread on
  ``api.py``: can_implement with one gate per weight format);
* ``mlaq_prewarm``        -- load the kernels of the graph-visible M regimes
  before capture (vLLM PR #174 "[GG] Fuse MXFP8 and BF16 MLA query
  assembly", "Layout and topology behavior");
* ``mlaq_run``            -- one fused call: ``[M,H,576]`` output with q_pe
  appended in the same launch (sparkinfer page, "What"; vLLM page, "What");
* ``mlaq_run_ex``         -- the same with strided views (a head-major q_nope,
  a pitched output workspace) and nope width 128 or 192;
* ``mlaq_uv_*``           -- the V up-projection that follows attention:
  ``out[m,h,:128] = x[m,h,:512] . W_UV[h]`` (vLLM page, "Layout and topology
  behavior": the UV projection beside the fused query path);
* ``mlaq_attn_*``         -- dense MLA decode attention over a paged latent
  cache, split into ranges whose partials are stored as BF16 or FP32 and
  merged into a BF16 output (b12x PR #441 "Allow FP32 split partials in
  prepared dense MLA", commit text and "Behavior").
"""

from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libmlaq.so"

MLAQ_WEIGHT_BF16, MLAQ_WEIGHT_MXFP8 = 0, 1
MLAQ_OUT_BF16, MLAQ_OUT_E4M3 = 0, 1
MLAQ_CACHE_DEFAULT, MLAQ_CACHE_STREAM = 0, 1
MLAQ_OK, MLAQ_ERR_UNSUPPORTED, MLAQ_ERR_INVALID_ARG, MLAQ_ERR_DEVICE = 0, 1, 2, 3
NOPE_DIM, LATENT_DIM, ROPE_DIM, MAX_M = 128, 512, 64, 32
NOPE_DIM_GLM = 192
V_DIM = 128
ROW = LATENT_DIM + ROPE_DIM
MX_BLOCK = 32
MLAQ_PARTIAL_BF16, MLAQ_PARTIAL_FP32 = 0, 1
MLAQ_ATTN_ROW = ROW
MLAQ_ATTN_MAX_HEADS = 16
MLAQ_ATTN_MAX_SPLITS = 256
MLAQ_ATTN_SPLIT_ALIGN = 64
MLAQ_ATTN_SCRATCH_BYTES = 32 << 20

_STATUS_NAMES = {0: "MLAQ_OK", 1: "MLAQ_ERR_UNSUPPORTED", 2: "MLAQ_ERR_INVALID_ARG", 3: "MLAQ_ERR_DEVICE"}


class RunArgs(ctypes.Structure):
    """Mirror of ``mlaq_run_args`` in include/mlaq.h (same field order and types)."""

    _fields_ = [("q_nope", ctypes.c_void_p), ("q_stride_m", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
                ("q_pe", ctypes.c_void_p), ("pe_stride_m", ctypes.c_int64), ("pe_stride_h", ctypes.c_int64),
                ("w", ctypes.c_void_p), ("w_scales", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("out_stride_m", ctypes.c_int64), ("out_stride_h", ctypes.c_int64),
                ("M", ctypes.c_int), ("H", ctypes.c_int), ("nope_dim", ctypes.c_int),
                ("weight_format", ctypes.c_int), ("out_dtype", ctypes.c_int), ("cache_hint", ctypes.c_int)]


class AttnArgs(ctypes.Structure):
    """Mirror of ``mlaq_attn_args`` in include/mlaq.h (same field order and types)."""

    _fields_ = [("q", ctypes.c_void_p), ("q_stride_m", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
                ("kv_cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("softmax_scale", ctypes.c_float),
                ("M", ctypes.c_int), ("H", ctypes.c_int), ("page_size", ctypes.c_int), ("num_pages", ctypes.c_int),
                ("block_table_stride", ctypes.c_int), ("num_splits", ctypes.c_int), ("partial_dtype", ctypes.c_int)]


class MlaqError(RuntimeError):
    """A non-OK status from libmlaq; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libmlaq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m mla_decode_query_amd._build")
        lib = ctypes.CDLL(str(LIB_PATH))
        I, P = ctypes.c_int, ctypes.c_void_p
        lib.mlaq_plan_supported.argtypes = [I] * 7 + [ctypes.c_char_p]
        lib.mlaq_plan_supported.restype = I
        lib.mlaq_can_implement.argtypes = [I] * 8
        lib.mlaq_can_implement.restype = I
        lib.mlaq_prewarm.argtypes = [I, P, I, I, I, I]
        lib.mlaq_prewarm.restype = I
        lib.mlaq_run.argtypes = [P, P, P, P, P, P, I, I, I, I, P]
        lib.mlaq_run.restype = I
        lib.mlaq_run_ex.argtypes = [ctypes.POINTER(RunArgs), P]
        lib.mlaq_run_ex.restype = I
        lib.mlaq_uv_plan_supported.argtypes = [I] * 5 + [ctypes.c_char_p]
        lib.mlaq_uv_plan_supported.restype = I
        lib.mlaq_uv_can_implement.argtypes = [I] * 6
        lib.mlaq_uv_can_implement.restype = I
        lib.mlaq_uv_prewarm.argtypes = [I, P, I, I, I]
        lib.mlaq_uv_prewarm.restype = I
        lib.mlaq_uv_run.argtypes = [P, P, P, P, I, I, I, P]
        lib.mlaq_uv_run.restype = I
        lib.mlaq_uv_run_ex.argtypes = [P, P, P, P, I, I, I, I, P]
        lib.mlaq_uv_run_ex.restype = I
        lib.mlaq_attn_workspace_size.argtypes = [I, I, I, I]
        lib.mlaq_attn_workspace_size.restype = ctypes.c_size_t
        lib.mlaq_attn_num_splits.argtypes = [I, I, I, ctypes.POINTER(I)]
        lib.mlaq_attn_num_splits.restype = I
        lib.mlaq_attn_plan_supported.argtypes = [I, I, I, I, ctypes.c_char_p]
        lib.mlaq_attn_plan_supported.restype = I
        lib.mlaq_attn_can_implement.argtypes = [I] * 5
        lib.mlaq_attn_can_implement.restype = I
        lib.mlaq_attn_prewarm.argtypes = [I, I]
        lib.mlaq_attn_prewarm.restype = I
        lib.mlaq_attn_run.argtypes = [ctypes.POINTER(AttnArgs), P]
        lib.mlaq_attn_run.restype = I
        lib.mlaq_attn_run_noalloc.argtypes = [ctypes.POINTER(AttnArgs), P]
        lib.mlaq_attn_run_noalloc.restype = I
        lib.mlaq_last_error.argtypes = []
        lib.mlaq_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def mlaq_last_error() -> str:
    return library().mlaq_last_error().decode()


def _check(status: int) -> None:
    if status != MLAQ_OK:
        raise MlaqError(status, mlaq_last_error())


def _device_index(device) -> int:
    if device is None:
        return torch.cuda.current_device()
    if isinstance(device, int):
        return device
    d = torch.device(device)
    return d.index if d.index is not None else torch.cuda.current_device()


def mlaq_plan_supported(num_heads: int, max_m: int, nope_dim: int = NOPE_DIM, latent_dim: int = LATENT_DIM,
                        rope_dim: int = ROPE_DIM, weight_format: int = MLAQ_WEIGHT_MXFP8,
                        out_dtype: int = MLAQ_OUT_BF16, arch: str = "gfx950") -> int:
    """Status of the pure gate for an architecture name (no HIP call)."""
    return library().mlaq_plan_supported(num_heads, max_m, nope_dim, latent_dim, rope_dim, weight_format,
                                         out_dtype, arch.encode() if arch is not None else None)


def mlaq_can_implement(num_heads: int, max_m: int, nope_dim: int = NOPE_DIM, latent_dim: int = LATENT_DIM,
                       rope_dim: int = ROPE_DIM, weight_format: int = MLAQ_WEIGHT_MXFP8,
                       out_dtype: int = MLAQ_OUT_BF16, device=None) -> bool:
    """True when the fused path covers the plan on ``device``."""
    return bool(library().mlaq_can_implement(num_heads, max_m, nope_dim, latent_dim, rope_dim, weight_format,
                                             out_dtype, _device_index(device)))


def mlaq_prewarm(num_heads: int, m_regimes, weight_format: int, out_dtype: int, device=None) -> None:
    """Load the kernels serving ``m_regimes`` (call before graph capture)."""
    regs = list(m_regimes)
    arr = (ctypes.c_int * max(1, len(regs)))(*regs)
    _check(library().mlaq_prewarm(num_heads, arr, len(regs), weight_format, out_dtype, _device_index(device)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def mlaq_run(q_nope: torch.Tensor, q_pe: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor | None,
             q_scale: torch.Tensor | None, out: torch.Tensor, weight_format: int, out_dtype: int,
             stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue one fused call on ``stream`` (default: the current stream).

    q_nope bf16 [M,H,128]; q_pe bf16 [M,H,64]; w bf16 [H,128,512] or
    float8_e4m3fn/uint8 [H,128,512]; w_scales uint8/float8_e8m0fnu [H,128,16]
    (MXFP8) or None; q_scale fp32 [1] (E4M3 output) or None; out bf16 or
    float8_e4m3fn/uint8 [M,H,576]. Shapes and dtypes are checked here; the
    library checks pointers, alignment, scale presence and overlap.
    """
    M, H = int(q_nope.shape[0]), int(q_nope.shape[1]) if q_nope.dim() == 3 else -1
    dev = q_nope.device
    _expect(q_nope, "q_nope", torch.bfloat16, (M, H, NOPE_DIM), dev)
    _expect(q_pe, "q_pe", torch.bfloat16, (M, H, ROPE_DIM), dev)
    if weight_format == MLAQ_WEIGHT_BF16:
        _expect(w, "w", torch.bfloat16, (H, NOPE_DIM, LATENT_DIM), dev)
    else:
        _expect(w, "w", w.dtype if w.dtype in (torch.float8_e4m3fn, torch.uint8) else torch.float8_e4m3fn,
                (H, NOPE_DIM, LATENT_DIM), dev)
    if w_scales is not None:
        _expect(w_scales, "w_scales",
                w_scales.dtype if w_scales.dtype in (torch.uint8, torch.float8_e8m0fnu) else torch.uint8,
                (H, NOPE_DIM, LATENT_DIM // MX_BLOCK), dev)
    if q_scale is not None:
        _expect(q_scale, "q_scale", torch.float32, (1,), dev)
    odt = torch.bfloat16 if out_dtype == MLAQ_OUT_BF16 else (
        out.dtype if out.dtype in (torch.float8_e4m3fn, torch.uint8) else torch.float8_e4m3fn)
    _expect(out, "out", odt, (M, H, ROW), dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _check(library().mlaq_run(_ptr(q_nope), _ptr(q_pe), _ptr(w), _ptr(w_scales), _ptr(q_scale), _ptr(out),
                              M, H, weight_format, out_dtype, ctypes.c_void_p(s.cuda_stream)))


def _expect_view(t, name, dtype, shape, device):
    """A [M,H,width] view whose innermost dimension is contiguous."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be a 3-d view with a contiguous last dimension")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.stride(0), t.stride(1)


def mlaq_run_ex(q_nope: torch.Tensor, q_pe: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor | None,
                q_scale: torch.Tensor | None, out: torch.Tensor, weight_format: int, out_dtype: int,
                stream: torch.cuda.Stream | None = None, cache_hint: int = MLAQ_CACHE_DEFAULT) -> None:
    """Like ``mlaq_run`` but ``q_nope`` ([M,H,K], K = 128 or 192), ``q_pe`` and
    ``out`` may be strided views (e.g. ``q.transpose(0, 1)`` of a head-major
    [H,M,K] tensor, or ``ws[..., :576]`` of a wider workspace). Weights stay
    contiguous [H,K,512] (and [H,K,16] scales). ``cache_hint``:
    ``MLAQ_CACHE_STREAM`` when the weights are read once per decode step (cold
    in HBM), ``MLAQ_CACHE_DEFAULT`` otherwise; results are identical."""
    if q_nope.dim() != 3:
        raise ValueError("q_nope must be [M,H,K]")
    M, H, K = (int(x) for x in q_nope.shape)
    dev = q_nope.device
    q_sm, q_sh = _expect_view(q_nope, "q_nope", torch.bfloat16, (M, H, K), dev)
    pe_sm, pe_sh = _expect_view(q_pe, "q_pe", torch.bfloat16, (M, H, ROPE_DIM), dev)
    wdt = torch.bfloat16 if weight_format == MLAQ_WEIGHT_BF16 else (
        w.dtype if w.dtype in (torch.float8_e4m3fn, torch.uint8) else torch.float8_e4m3fn)
    _expect(w, "w", wdt, (H, K, LATENT_DIM), dev)
    if w_scales is not None:
        _expect(w_scales, "w_scales",
                w_scales.dtype if w_scales.dtype in (torch.uint8, torch.float8_e8m0fnu) else torch.uint8,
                (H, K, LATENT_DIM // MX_BLOCK), dev)
    if q_scale is not None:
        _expect(q_scale, "q_scale", torch.float32, (1,), dev)
    odt = torch.bfloat16 if out_dtype == MLAQ_OUT_BF16 else (
        out.dtype if out.dtype in (torch.float8_e4m3fn, torch.uint8) else torch.float8_e4m3fn)
    o_sm, o_sh = _expect_view(out, "out", odt, (M, H, ROW), dev)
    args = RunArgs(q_nope.data_ptr(), q_sm, q_sh, q_pe.data_ptr(), pe_sm, pe_sh, w.data_ptr(),
                   None if w_scales is None else w_scales.data_ptr(),
                   None if q_scale is None else q_scale.data_ptr(), out.data_ptr(), o_sm, o_sh,
                   M, H, K, weight_format, out_dtype, cache_hint)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _check(library().mlaq_run_ex(ctypes.byref(args), ctypes.c_void_p(s.cuda_stream)))


def fused_query(q_nope, q_pe, w, w_scales=None, q_scale=None, out_dtype: int = MLAQ_OUT_BF16, out=None):
    """Allocate the [M,H,576] output (unless given) and run one fused call."""
    wf = MLAQ_WEIGHT_BF16 if w.dtype == torch.bfloat16 else MLAQ_WEIGHT_MXFP8
    M, H = q_nope.shape[0], q_nope.shape[1]
    if out is None:
        dt = torch.bfloat16 if out_dtype == MLAQ_OUT_BF16 else torch.float8_e4m3fn
        out = torch.empty((M, H, ROW), dtype=dt, device=q_nope.device)
    mlaq_run(q_nope, q_pe, w, w_scales, q_scale, out, wf, out_dtype)
    return out


def mlaq_uv_plan_supported(num_heads: int, max_m: int, latent_dim: int = LATENT_DIM, v_dim: int = V_DIM,
                           weight_format: int = MLAQ_WEIGHT_MXFP8, arch: str = "gfx950") -> int:
    """Status of the pure UV-projection gate for an architecture name."""
    return library().mlaq_uv_plan_supported(num_heads, max_m, latent_dim, v_dim, weight_format,
                                            arch.encode() if arch is not None else None)


def mlaq_uv_can_implement(num_heads: int, max_m: int, latent_dim: int = LATENT_DIM, v_dim: int = V_DIM,
                          weight_format: int = MLAQ_WEIGHT_MXFP8, device=None) -> bool:
    return bool(library().mlaq_uv_can_implement(num_heads, max_m, latent_dim, v_dim, weight_format,
                                                _device_index(device)))


def mlaq_uv_prewarm(num_heads: int, m_regimes, weight_format: int, device=None) -> None:
    regs = list(m_regimes)
    arr = (ctypes.c_int * max(1, len(regs)))(*regs)
    _check(library().mlaq_uv_prewarm(num_heads, arr, len(regs), weight_format, _device_index(device)))


def _uv_views(x, w_uv, w_uv_scales, out, weight_format):
    """Checks of the UV arguments; returns (M, H)."""
    if x.dim() != 3:
        raise ValueError("x must be [M,H,512]")
    M, H = int(x.shape[0]), int(x.shape[1])
    dev = x.device
    _expect(x, "x", torch.bfloat16, (M, H, LATENT_DIM), dev)
    wdt = torch.bfloat16 if weight_format == MLAQ_WEIGHT_BF16 else (
        w_uv.dtype if w_uv.dtype in (torch.float8_e4m3fn, torch.uint8) else torch.float8_e4m3fn)
    _expect(w_uv, "w_uv", wdt, (H, V_DIM, LATENT_DIM), dev)
    if w_uv_scales is not None:
        _expect(w_uv_scales, "w_uv_scales",
                w_uv_scales.dtype if w_uv_scales.dtype in (torch.uint8, torch.float8_e8m0fnu) else torch.uint8,
                (H, V_DIM, LATENT_DIM // MX_BLOCK), dev)
    _expect(out, "out", torch.bfloat16, (M, H, V_DIM), dev)
    return M, H


def mlaq_uv_run(x: torch.Tensor, w_uv: torch.Tensor, w_uv_scales: torch.Tensor | None, out: torch.Tensor,
                weight_format: int, stream: torch.cuda.Stream | None = None) -> None:
    """V up-projection: x bf16 [M,H,512], w_uv bf16 or float8_e4m3fn/uint8
    [H,128,512] (latent contiguous), w_uv_scales uint8/float8_e8m0fnu
    [H,128,16] (MXFP8) or None, out bf16 [M,H,128]."""
    M, H = _uv_views(x, w_uv, w_uv_scales, out, weight_format)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    _check(library().mlaq_uv_run(_ptr(x), _ptr(w_uv), _ptr(w_uv_scales), _ptr(out), M, H, weight_format,
                                 ctypes.c_void_p(s.cuda_stream)))


def mlaq_uv_run_ex(x: torch.Tensor, w_uv: torch.Tensor, w_uv_scales: torch.Tensor | None, out: torch.Tensor,
                   weight_format: int, stream: torch.cuda.Stream | None = None,
                   cache_hint: int = MLAQ_CACHE_DEFAULT) -> None:
    """mlaq_uv_run with a cache hint (MLAQ_CACHE_DEFAULT or MLAQ_CACHE_STREAM),
    accepted so that one policy can be passed to every projection of a layer;
    the UV kernels ignore it (results and timing are those of mlaq_uv_run)."""
    M, H = _uv_views(x, w_uv, w_uv_scales, out, weight_format)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    _check(library().mlaq_uv_run_ex(_ptr(x), _ptr(w_uv), _ptr(w_uv_scales), _ptr(out), M, H, weight_format,
                                    cache_hint, ctypes.c_void_p(s.cuda_stream)))


def mlaq_attn_workspace_size(M: int, H: int, num_splits: int, partial_dtype: int = MLAQ_PARTIAL_BF16) -> int:
    """Workspace bytes of an attention plan (0 for one split or an invalid plan)."""
    return int(library().mlaq_attn_workspace_size(M, H, num_splits, partial_dtype))


def mlaq_attn_num_splits(M: int, max_seq_len: int, device=None) -> int:
    """Split count that fills the device for M sequences of up to max_seq_len tokens."""
    n = ctypes.c_int(0)
    _check(library().mlaq_attn_num_splits(M, max_seq_len, _device_index(device), ctypes.byref(n)))
    return n.value


def mlaq_attn_plan_supported(num_heads: int, page_size: int, num_splits: int,
                             partial_dtype: int = MLAQ_PARTIAL_BF16, arch: str = "gfx950") -> int:
    """Status of the pure attention gate for an architecture name."""
    return library().mlaq_attn_plan_supported(num_heads, page_size, num_splits, partial_dtype,
                                              arch.encode() if arch is not None else None)


def mlaq_attn_can_implement(num_heads: int, page_size: int, num_splits: int,
                            partial_dtype: int = MLAQ_PARTIAL_BF16, device=None) -> bool:
    return bool(library().mlaq_attn_can_implement(num_heads, page_size, num_splits, partial_dtype,
                                                  _device_index(device)))


def mlaq_attn_prewarm(partial_dtype: int = MLAQ_PARTIAL_BF16, device=None) -> None:
    _check(library().mlaq_attn_prewarm(partial_dtype, _device_index(device)))


def _attn_args(q, kv_cache, block_table, seq_lens, out, softmax_scale, num_splits, partial_dtype, workspace,
               lse) -> AttnArgs:
    if q.dim() != 3:
        raise ValueError("q must be [M,H,576]")
    M, H = int(q.shape[0]), int(q.shape[1])
    dev = q.device
    q_sm, q_sh = _expect_view(q, "q", torch.bfloat16, (M, H, ROW), dev)
    if kv_cache.dim() != 3:
        raise ValueError("kv_cache must be [num_pages,page_size,576]")
    num_pages, page_size = int(kv_cache.shape[0]), int(kv_cache.shape[1])
    _expect(kv_cache, "kv_cache", torch.bfloat16, (num_pages, page_size, ROW), dev)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [M,max_blocks]")
    _expect(block_table, "block_table", torch.int32, (M, int(block_table.shape[1])), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (M,), dev)
    _expect(out, "out", torch.bfloat16, (M, H, LATENT_DIM), dev)
    if lse is not None:
        _expect(lse, "lse", torch.float32, (M, H), dev)
    ws_bytes = 0
    if workspace is not None:
        if not workspace.is_contiguous() or workspace.device != dev:
            raise ValueError("workspace must be a contiguous tensor on the query's device")
        ws_bytes = workspace.numel() * workspace.element_size()
    return AttnArgs(q.data_ptr(), q_sm, q_sh, kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
                    out.data_ptr(), None if lse is None else lse.data_ptr(),
                    None if workspace is None else workspace.data_ptr(), ws_bytes, float(softmax_scale),
                    M, H, page_size, num_pages, int(block_table.shape[1]), int(num_splits), int(partial_dtype))


def mlaq_attn_run(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                  out: torch.Tensor, softmax_scale: float, num_splits: int,
                  partial_dtype: int = MLAQ_PARTIAL_BF16, workspace: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> None:
    """Dense MLA decode attention: q bf16 [M,H,576] (a view whose last
    dimension is contiguous), kv_cache bf16 [num_pages,page_size,576],
    block_table int32 [M,max_blocks], seq_lens int32 [M], out bf16 [M,H,512],
    lse fp32 [M,H] or None, workspace a uint8 tensor of at least
    ``mlaq_attn_workspace_size`` bytes (None when that is 0)."""
    args = _attn_args(q, kv_cache, block_table, seq_lens, out, softmax_scale, num_splits, partial_dtype, workspace,
                      lse)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    _check(library().mlaq_attn_run(ctypes.byref(args), ctypes.c_void_p(s.cuda_stream)))


def mlaq_attn_run_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, out: torch.Tensor, softmax_scale: float, num_splits: int,
                          partial_dtype: int = MLAQ_PARTIAL_BF16, lse: torch.Tensor | None = None,
                          stream: torch.cuda.Stream | None = None) -> None:
    """mlaq_attn_run with the partials in the library's device scratch array
    (MLAQ_ATTN_SCRATCH_BYTES per device) instead of a caller workspace; for
    callers that cannot allocate. Calls that overlap in time on one device race."""
    args = _attn_args(q, kv_cache, block_table, seq_lens, out, softmax_scale, num_splits, partial_dtype, None, lse)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    _check(library().mlaq_attn_run_noalloc(ctypes.byref(args), ctypes.c_void_p(s.cuda_stream)))


def dense_mla_decode(q, kv_cache, block_table, seq_lens, softmax_scale: float, num_splits: int | None = None,
                     partial_dtype: int = MLAQ_PARTIAL_BF16, max_seq_len: int | None = None, return_lse=False):
    """Allocate the output (and workspace) and run one attention call. With
    ``num_splits`` None the library's split heuristic picks it from
    ``max_seq_len`` (read from ``seq_lens`` when not given: a device sync)."""
    M, H = int(q.shape[0]), int(q.shape[1])
    if num_splits is None:
        if max_seq_len is None:
            max_seq_len = int(seq_lens.max().item()) if M else 0
        num_splits = mlaq_attn_num_splits(max(M, 1), max_seq_len, q.device)
    out = torch.empty((M, H, LATENT_DIM), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((M, H), dtype=torch.float32, device=q.device) if return_lse else None
    n = mlaq_attn_workspace_size(M, H, num_splits, partial_dtype)
    ws = torch.empty((n,), dtype=torch.uint8, device=q.device) if n else None
    mlaq_attn_run(q, kv_cache, block_table, seq_lens, out, softmax_scale, num_splits, partial_dtype, ws, lse)
    return (out, lse) if return_lse else out
