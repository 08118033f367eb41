// mlaq_api.cpp -- C-ABI front end of libmlaq: argument validation, the
// per-recipe capability gate, prewarm and kernel dispatch. Everything here is
// host code; the only HIP calls are the device query (cached per device),
// function-attribute lookups in prewarm, and the kernel launch itself.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "mlaq.h"
#include "mlaq_internal.h"

namespace {

thread_local char g_err[512];

void clear_error() { g_err[0] = '\0'; }

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

bool known_weight_format(int f) { return f == MLAQ_WEIGHT_BF16 || f == MLAQ_WEIGHT_MXFP8; }
bool known_out_dtype(int d) { return d == MLAQ_OUT_BF16 || d == MLAQ_OUT_E4M3; }
bool supported_heads(int h) { return h == 8 || h == 11 || h == 16; }

bool is_gfx950(const char* arch) {
  // gcnArchName looks like "gfx950:sramecc+:xnack-"; the target id ends at ':'.
  return std::strncmp(arch, "gfx950", 6) == 0 && (arch[6] == '\0' || arch[6] == ':');
}

// Shape and arch checks shared by both recipes.
int common_plan(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim, const char* arch) {
  if (!is_gfx950(arch)) return fail(MLAQ_ERR_UNSUPPORTED, "device architecture '%s' is not gfx950", arch);
  if (!supported_heads(num_heads))
    return fail(MLAQ_ERR_UNSUPPORTED, "num_heads=%d not in {8, 11, 16}", num_heads);
  if (max_m < 1 || max_m > MLAQ_MAX_M) return fail(MLAQ_ERR_UNSUPPORTED, "max_m=%d outside 1..32", max_m);
  if ((nope_dim != MLAQ_NOPE_DIM && nope_dim != MLAQ_NOPE_DIM_GLM) || latent_dim != MLAQ_LATENT_DIM ||
      rope_dim != MLAQ_ROPE_DIM)
    return fail(MLAQ_ERR_UNSUPPORTED, "dims (nope %d, latent %d, rope %d) are not (128 or 192, 512, 64)", nope_dim,
                latent_dim, rope_dim);
  return MLAQ_OK;
}

// Gate of the BF16-weight recipe: its own function, so it never inherits a
// requirement that only the MXFP8 recipe has.
int bf16_recipe_plan(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim, const char* arch) {
  return common_plan(num_heads, max_m, nope_dim, latent_dim, rope_dim, arch);
}

// Gate of the MXFP8-weight recipe (E4M3 payload + E8M0 scales per 32 columns;
// the latent width must hold whole scale groups).
int mxfp8_recipe_plan(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim, const char* arch) {
  if (latent_dim % mlaq::kMxBlock != 0)
    return fail(MLAQ_ERR_UNSUPPORTED, "latent_dim=%d is not a multiple of 32", latent_dim);
  return common_plan(num_heads, max_m, nope_dim, latent_dim, rope_dim, arch);
}

// Per-device architecture cache: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::mutex g_arch_mu;
int g_arch_state[kMaxDevices];
char g_arch_name[kMaxDevices][64];

// Returns MLAQ_OK and the cached arch name of `device`, querying it once.
int device_arch(int device, const char** name) {
  if (device < 0 || device >= kMaxDevices) return fail(MLAQ_ERR_INVALID_ARG, "device ordinal %d out of range", device);
  std::lock_guard<std::mutex> lock(g_arch_mu);
  if (g_arch_state[device] == 0) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
      return fail(MLAQ_ERR_DEVICE, "hipGetDeviceProperties(%d): %s", device, hipGetErrorString(e));
    std::snprintf(g_arch_name[device], sizeof g_arch_name[device], "%s", prop.gcnArchName);
    g_arch_state[device] = is_gfx950(g_arch_name[device]) ? 1 : 2;
  }
  *name = g_arch_name[device];
  return MLAQ_OK;
}

int plan_for(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim, int weight_format,
             int out_dtype, const char* arch) {
  if (!arch) return fail(MLAQ_ERR_INVALID_ARG, "arch is NULL");
  if (!known_weight_format(weight_format)) return fail(MLAQ_ERR_INVALID_ARG, "unknown weight_format %d", weight_format);
  if (!known_out_dtype(out_dtype)) return fail(MLAQ_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  if (weight_format == MLAQ_WEIGHT_BF16)
    return bf16_recipe_plan(num_heads, max_m, nope_dim, latent_dim, rope_dim, arch);
  return mxfp8_recipe_plan(num_heads, max_m, nope_dim, latent_dim, rope_dim, arch);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Bytes spanned by an [M,H,width] view with outer strides (sm, sh) elements.
size_t span_bytes(int M, int H, int64_t sm, int64_t sh, int width, size_t esz) {
  return size_t((int64_t(M) - 1) * sm + (int64_t(H) - 1) * sh + width) * esz;
}

bool stride_ok(int64_t s) { return s >= 0 && s < mlaq::kMaxStride && s % 8 == 0; }

// The M*H output rows [off, off + 576) are pairwise disjoint when one outer
// stride clears a row and the other clears all rows along the first.
bool rows_disjoint(int M, int H, int64_t sm, int64_t sh) {
  const int64_t row = mlaq::kRow;
  if (M == 1) return sh >= row;
  return (sh >= row && sm >= int64_t(H) * sh) || (sm >= row && sh >= int64_t(M) * sm);
}

bool known_partial(int d) { return d == MLAQ_PARTIAL_BF16 || d == MLAQ_PARTIAL_FP32; }

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// Workspace layout: partials [M,S,H,512] (bf16 or fp32) from offset 0, then
// lse_s [M,S,H] fp32 from the next 256-byte boundary.
size_t attn_lse_offset(int M, int H, int S, int partial_dtype) {
  const size_t esz = partial_dtype == MLAQ_PARTIAL_FP32 ? 4 : 2;
  return round256(size_t(M) * S * H * mlaq::kLatent * esz);
}

// Per-device compute-unit count, queried once.
std::mutex g_cu_mu;
int g_cus[kMaxDevices];

int device_cus(int device, int* cus) {
  if (device < 0 || device >= kMaxDevices) return fail(MLAQ_ERR_INVALID_ARG, "device ordinal %d out of range", device);
  std::lock_guard<std::mutex> lock(g_cu_mu);
  if (g_cus[device] == 0) {
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess || n < 1)
      return fail(MLAQ_ERR_DEVICE, "compute-unit count of device %d: %s", device, hipGetErrorString(e));
    g_cus[device] = n;
  }
  *cus = g_cus[device];
  return MLAQ_OK;
}

} // namespace

extern "C" {

int mlaq_plan_supported(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim, int weight_format,
                        int out_dtype, const char* arch) {
  clear_error();
  return plan_for(num_heads, max_m, nope_dim, latent_dim, rope_dim, weight_format, out_dtype, arch);
}

int mlaq_can_implement(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim, int weight_format,
                       int out_dtype, int device) {
  clear_error();
  const char* arch = nullptr;
  if (device_arch(device, &arch) != MLAQ_OK) return 0;
  return plan_for(num_heads, max_m, nope_dim, latent_dim, rope_dim, weight_format, out_dtype, arch) == MLAQ_OK;
}

int mlaq_prewarm(int num_heads, const int* m_regimes, int n_regimes, int weight_format, int out_dtype, int device) {
  clear_error();
  if (n_regimes < 0 || (n_regimes > 0 && !m_regimes))
    return fail(MLAQ_ERR_INVALID_ARG, "m_regimes is NULL or n_regimes < 0");
  const char* arch = nullptr;
  int st = device_arch(device, &arch);
  if (st != MLAQ_OK) return st;
  bool seen[3] = {false, false, false}; // by m_tiles
  for (int i = 0; i < n_regimes; ++i) {
    st = plan_for(num_heads, m_regimes[i], MLAQ_NOPE_DIM, MLAQ_LATENT_DIM, MLAQ_ROPE_DIM, weight_format, out_dtype,
                  arch);
    if (st != MLAQ_OK) return st;
    const int tiles = mlaq::variant_for(weight_format, out_dtype, m_regimes[i], mlaq::kNope, num_heads).m_tiles;
    if (seen[tiles]) continue;
    seen[tiles] = true;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device) e = hipSetDevice(device);
    for (int K : {mlaq::kNope, mlaq::kNopeGlm})
      for (int hint : {MLAQ_CACHE_DEFAULT, MLAQ_CACHE_STREAM}) {
        hipFuncAttributes attr;
        if (e == hipSuccess)
          e = hipFuncGetAttributes(&attr,
                                   mlaq::kernel_for(mlaq::variant_for(weight_format, out_dtype, m_regimes[i], K,
                                                                      num_heads, hint)));
      }
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "loading kernel for M=%d: %s", m_regimes[i], hipGetErrorString(e));
  }
  return MLAQ_OK;
}

int mlaq_run_ex(const mlaq_run_args* args, void* stream) {
  clear_error();
  if (!args) return fail(MLAQ_ERR_INVALID_ARG, "args is NULL");
  const mlaq_run_args& a = *args;
  const int M = a.M, H = a.H, K = a.nope_dim;
  if (!known_weight_format(a.weight_format)) return fail(MLAQ_ERR_INVALID_ARG, "unknown weight_format %d", a.weight_format);
  if (!known_out_dtype(a.out_dtype)) return fail(MLAQ_ERR_INVALID_ARG, "unknown out_dtype %d", a.out_dtype);
  if (a.cache_hint != MLAQ_CACHE_DEFAULT && a.cache_hint != MLAQ_CACHE_STREAM)
    return fail(MLAQ_ERR_INVALID_ARG, "unknown cache_hint %d", a.cache_hint);
  if (!supported_heads(H)) return fail(MLAQ_ERR_UNSUPPORTED, "H=%d not in {8, 11, 16}", H);
  if (M < 0 || M > MLAQ_MAX_M) return fail(MLAQ_ERR_UNSUPPORTED, "M=%d outside 0..32", M);
  if (K != MLAQ_NOPE_DIM && K != MLAQ_NOPE_DIM_GLM) return fail(MLAQ_ERR_UNSUPPORTED, "nope_dim=%d not 128 or 192", K);
  if (M == 0) return MLAQ_OK; // empty batch: nothing to read or write
  if (!a.q_nope || !a.q_pe || !a.w || !a.out)
    return fail(MLAQ_ERR_INVALID_ARG, "q_nope, q_pe, w and out must be non-NULL");
  if (a.weight_format == MLAQ_WEIGHT_MXFP8 && !a.w_scales)
    return fail(MLAQ_ERR_INVALID_ARG, "MXFP8 weights need w_scales");
  if (a.weight_format == MLAQ_WEIGHT_BF16 && a.w_scales)
    return fail(MLAQ_ERR_INVALID_ARG, "BF16 weights take no w_scales (pass NULL)");
  if (a.out_dtype == MLAQ_OUT_E4M3 && !a.q_scale) return fail(MLAQ_ERR_INVALID_ARG, "E4M3 output needs q_scale");
  if (a.out_dtype == MLAQ_OUT_BF16 && a.q_scale)
    return fail(MLAQ_ERR_INVALID_ARG, "BF16 output takes no q_scale (pass NULL)");
  if (!aligned(a.q_nope, 16) || !aligned(a.q_pe, 16) || !aligned(a.w, 16) || !aligned(a.out, 16))
    return fail(MLAQ_ERR_INVALID_ARG, "q_nope, q_pe, w and out must be 16-byte aligned");
  if (a.q_scale && !aligned(a.q_scale, 4)) return fail(MLAQ_ERR_INVALID_ARG, "q_scale must be 4-byte aligned");
  if (!stride_ok(a.q_stride_m) || !stride_ok(a.q_stride_h) || !stride_ok(a.pe_stride_m) ||
      !stride_ok(a.pe_stride_h) || !stride_ok(a.out_stride_m) || !stride_ok(a.out_stride_h))
    return fail(MLAQ_ERR_INVALID_ARG, "strides must be non-negative multiples of 8 elements below 2^24");
  if (a.q_stride_h >= mlaq::kMaxHeadStride || a.pe_stride_h >= mlaq::kMaxHeadStride)
    return fail(MLAQ_ERR_INVALID_ARG, "head strides of q_nope and q_pe must be below 2^16 elements");
  if (!rows_disjoint(M, H, a.out_stride_m, a.out_stride_h))
    return fail(MLAQ_ERR_INVALID_ARG, "out strides (%lld, %lld) make output rows overlap",
                (long long)a.out_stride_m, (long long)a.out_stride_h);

  const size_t esz_w = a.weight_format == MLAQ_WEIGHT_BF16 ? 2 : 1;
  const size_t esz_o = a.out_dtype == MLAQ_OUT_BF16 ? 2 : 1;
  const size_t out_bytes = span_bytes(M, H, a.out_stride_m, a.out_stride_h, mlaq::kRow, esz_o);
  if (overlaps(a.out, out_bytes, a.q_nope, span_bytes(M, H, a.q_stride_m, a.q_stride_h, K, 2)) ||
      overlaps(a.out, out_bytes, a.q_pe, span_bytes(M, H, a.pe_stride_m, a.pe_stride_h, mlaq::kRope, 2)) ||
      overlaps(a.out, out_bytes, a.w, size_t(H) * K * mlaq::kLatent * esz_w) ||
      overlaps(a.out, out_bytes, a.w_scales, size_t(H) * K * (mlaq::kLatent / mlaq::kMxBlock)) ||
      overlaps(a.out, out_bytes, a.q_scale, sizeof(float)))
    return fail(MLAQ_ERR_INVALID_ARG, "out overlaps an input buffer");

  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  const char* arch = nullptr;
  int st = device_arch(device, &arch);
  if (st != MLAQ_OK) return st;
  st = plan_for(H, M, K, MLAQ_LATENT_DIM, MLAQ_ROPE_DIM, a.weight_format, a.out_dtype, arch);
  if (st != MLAQ_OK) return st;

  const mlaq::Variant v = mlaq::variant_for(a.weight_format, a.out_dtype, M, K, H, a.cache_hint);
  const void* fn = mlaq::kernel_for(v);
  if (!fn) return fail(MLAQ_ERR_UNSUPPORTED, "no kernel for this plan");
  dim3 grid, block;
  mlaq::launch_shape(v, H, &grid, &block);
  mlaq::FusedArgs ka{static_cast<const uint16_t*>(a.q_nope), static_cast<const uint16_t*>(a.q_pe), a.w,
                     static_cast<const uint8_t*>(a.w_scales), a.q_scale, a.out,
                     uint32_t(a.q_stride_m), uint32_t(a.q_stride_h), uint32_t(a.pe_stride_m),
                     uint32_t(a.pe_stride_h), uint32_t(a.out_stride_m), uint32_t(a.out_stride_h), M, H};
  // The kernel's argument order (the first 14 dwords are preloaded): head
  // strides and (M, H) travel packed as two 16-bit halves each.
  uint32_t head_strides = ka.q_sh | (ka.pe_sh << 16), m_h = uint32_t(M) | (uint32_t(H) << 16);
  void* kargs[] = {&ka.q_pe, &ka.w, &ka.q_nope, &ka.w_scales, &ka.q_scale, &ka.pe_sm, &ka.q_sm,
                   &head_strides, &m_h, &ka.out, &ka.out_sm, &ka.out_sh};
  e = hipLaunchKernel(fn, grid, block, kargs, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "kernel launch: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

int mlaq_run(const void* q_nope, const void* q_pe, const void* w, const void* w_scales, const float* q_scale,
             void* out, int M, int H, int weight_format, int out_dtype, void* stream) {
  mlaq_run_args a;
  a.q_nope = q_nope;
  a.q_stride_m = int64_t(H) * mlaq::kNope;
  a.q_stride_h = mlaq::kNope;
  a.q_pe = q_pe;
  a.pe_stride_m = int64_t(H) * mlaq::kRope;
  a.pe_stride_h = mlaq::kRope;
  a.w = w;
  a.w_scales = w_scales;
  a.q_scale = q_scale;
  a.out = out;
  a.out_stride_m = int64_t(H) * mlaq::kRow;
  a.out_stride_h = mlaq::kRow;
  a.M = M;
  a.H = H;
  a.nope_dim = mlaq::kNope;
  a.weight_format = weight_format;
  a.out_dtype = out_dtype;
  a.cache_hint = MLAQ_CACHE_DEFAULT;
  return mlaq_run_ex(&a, stream);
}

int mlaq_uv_plan_supported(int num_heads, int max_m, int latent_dim, int v_dim, int weight_format, const char* arch) {
  clear_error();
  if (!arch) return fail(MLAQ_ERR_INVALID_ARG, "arch is NULL");
  if (!known_weight_format(weight_format)) return fail(MLAQ_ERR_INVALID_ARG, "unknown weight_format %d", weight_format);
  if (!is_gfx950(arch)) return fail(MLAQ_ERR_UNSUPPORTED, "device architecture '%s' is not gfx950", arch);
  if (!supported_heads(num_heads)) return fail(MLAQ_ERR_UNSUPPORTED, "num_heads=%d not in {8, 11, 16}", num_heads);
  if (max_m < 1 || max_m > MLAQ_MAX_M) return fail(MLAQ_ERR_UNSUPPORTED, "max_m=%d outside 1..32", max_m);
  if (latent_dim != MLAQ_LATENT_DIM || v_dim != MLAQ_V_DIM)
    return fail(MLAQ_ERR_UNSUPPORTED, "dims (latent %d, v %d) are not (512, 128)", latent_dim, v_dim);
  return MLAQ_OK;
}

int mlaq_uv_can_implement(int num_heads, int max_m, int latent_dim, int v_dim, int weight_format, int device) {
  clear_error();
  const char* arch = nullptr;
  if (device_arch(device, &arch) != MLAQ_OK) return 0;
  return mlaq_uv_plan_supported(num_heads, max_m, latent_dim, v_dim, weight_format, arch) == MLAQ_OK;
}

int mlaq_uv_prewarm(int num_heads, const int* m_regimes, int n_regimes, int weight_format, int device) {
  clear_error();
  if (n_regimes < 0 || (n_regimes > 0 && !m_regimes))
    return fail(MLAQ_ERR_INVALID_ARG, "m_regimes is NULL or n_regimes < 0");
  const char* arch = nullptr;
  int st = device_arch(device, &arch);
  if (st != MLAQ_OK) return st;
  for (int i = 0; i < n_regimes; ++i) {
    st = mlaq_uv_plan_supported(num_heads, m_regimes[i], MLAQ_LATENT_DIM, MLAQ_V_DIM, weight_format, arch);
    if (st != MLAQ_OK) return st;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device) e = hipSetDevice(device);
    const void* fn = mlaq::uv_kernel_for(weight_format, m_regimes[i] <= 16 ? 1 : 2);
    hipFuncAttributes attr;
    if (e == hipSuccess && fn) e = hipFuncGetAttributes(&attr, fn);
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "loading kernel for M=%d: %s", m_regimes[i], hipGetErrorString(e));
  }
  return MLAQ_OK;
}

int mlaq_uv_run(const void* x, const void* w_uv, const void* w_uv_scales, void* out, int M, int H, int weight_format,
                void* stream) {
  return mlaq_uv_run_ex(x, w_uv, w_uv_scales, out, M, H, weight_format, MLAQ_CACHE_DEFAULT, stream);
}

int mlaq_uv_run_ex(const void* x, const void* w_uv, const void* w_uv_scales, void* out, int M, int H,
                   int weight_format, int cache_hint, void* stream) {
  clear_error();
  if (!known_weight_format(weight_format)) return fail(MLAQ_ERR_INVALID_ARG, "unknown weight_format %d", weight_format);
  if (cache_hint != MLAQ_CACHE_DEFAULT && cache_hint != MLAQ_CACHE_STREAM)
    return fail(MLAQ_ERR_INVALID_ARG, "unknown cache_hint %d", cache_hint);
  if (!supported_heads(H)) return fail(MLAQ_ERR_UNSUPPORTED, "H=%d not in {8, 11, 16}", H);
  if (M < 0 || M > MLAQ_MAX_M) return fail(MLAQ_ERR_UNSUPPORTED, "M=%d outside 0..32", M);
  if (M == 0) return MLAQ_OK;
  if (!x || !w_uv || !out) return fail(MLAQ_ERR_INVALID_ARG, "x, w_uv and out must be non-NULL");
  if (weight_format == MLAQ_WEIGHT_MXFP8 && !w_uv_scales) return fail(MLAQ_ERR_INVALID_ARG, "MXFP8 weights need w_uv_scales");
  if (weight_format == MLAQ_WEIGHT_BF16 && w_uv_scales)
    return fail(MLAQ_ERR_INVALID_ARG, "BF16 weights take no w_uv_scales (pass NULL)");
  if (!aligned(x, 16) || !aligned(w_uv, 16) || !aligned(out, 16))
    return fail(MLAQ_ERR_INVALID_ARG, "x, w_uv and out must be 16-byte aligned");
  const size_t mh = size_t(M) * size_t(H);
  const size_t out_bytes = mh * mlaq::kValue * 2;
  const size_t esz_w = weight_format == MLAQ_WEIGHT_BF16 ? 2 : 1;
  if (overlaps(out, out_bytes, x, mh * mlaq::kLatent * 2) ||
      overlaps(out, out_bytes, w_uv, size_t(H) * mlaq::kValue * mlaq::kLatent * esz_w) ||
      overlaps(out, out_bytes, w_uv_scales, size_t(H) * mlaq::kValue * (mlaq::kLatent / mlaq::kMxBlock)))
    return fail(MLAQ_ERR_INVALID_ARG, "out overlaps an input buffer");
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  const char* arch = nullptr;
  int st = device_arch(device, &arch);
  if (st != MLAQ_OK) return st;
  st = mlaq_uv_plan_supported(H, M, MLAQ_LATENT_DIM, MLAQ_V_DIM, weight_format, arch);
  if (st != MLAQ_OK) return st;
  const int m_tiles = M <= 16 ? 1 : 2;
  const void* fn = mlaq::uv_kernel_for(weight_format, m_tiles); // the cache hint is validated above, not used
  if (!fn) return fail(MLAQ_ERR_UNSUPPORTED, "no kernel for this plan");
  dim3 grid, block;
  mlaq::uv_launch_shape(H, m_tiles, &grid, &block);
  mlaq::UvArgs ka{static_cast<const uint16_t*>(x), w_uv, static_cast<const uint8_t*>(w_uv_scales), out, M, H};
  void* kargs[] = {&ka.x, &ka.w, &ka.w_scales, &ka.out, &ka.M, &ka.H};
  e = hipLaunchKernel(fn, grid, block, kargs, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "kernel launch: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

// ---------------------------------------------------------------------------
// Dense MLA decode attention
// ---------------------------------------------------------------------------

size_t mlaq_attn_workspace_size(int M, int H, int num_splits, int partial_dtype) {
  if (M < 0 || M > mlaq::kAttnMaxM || H < 1 || H > mlaq::kAttnMaxHeads || num_splits < 1 ||
      num_splits > mlaq::kAttnMaxSplits || !known_partial(partial_dtype))
    return 0;
  if (num_splits == 1) return 0;
  return attn_lse_offset(M, H, num_splits, partial_dtype) + round256(size_t(M) * num_splits * H * sizeof(float));
}

int mlaq_attn_num_splits(int M, int max_seq_len, int device, int* num_splits) {
  clear_error();
  if (!num_splits) return fail(MLAQ_ERR_INVALID_ARG, "num_splits is NULL");
  if (M < 1 || max_seq_len < 0) return fail(MLAQ_ERR_INVALID_ARG, "M must be >= 1 and max_seq_len >= 0");
  int cus = 0;
  int st = device_cus(device, &cus);
  if (st != MLAQ_OK) return st;
  // Two split workgroups per compute unit (each holds a 66 KiB LDS tile),
  // ranges of at least 256 tokens (four 64-token tiles).
  long long want = 2LL * cus / M;
  const long long by_len = (max_seq_len + 255) / 256;
  if (want > by_len) want = by_len;
  if (want > mlaq::kAttnMaxSplits) want = mlaq::kAttnMaxSplits;
  *num_splits = want < 1 ? 1 : int(want);
  return MLAQ_OK;
}

int mlaq_attn_plan_supported(int num_heads, int page_size, int num_splits, int partial_dtype, const char* arch) {
  clear_error();
  if (!arch) return fail(MLAQ_ERR_INVALID_ARG, "arch is NULL");
  if (!known_partial(partial_dtype)) return fail(MLAQ_ERR_INVALID_ARG, "unknown partial_dtype %d", partial_dtype);
  if (!is_gfx950(arch)) return fail(MLAQ_ERR_UNSUPPORTED, "device architecture '%s' is not gfx950", arch);
  if (num_heads < 1 || num_heads > mlaq::kAttnMaxHeads)
    return fail(MLAQ_ERR_UNSUPPORTED, "num_heads=%d outside 1..16", num_heads);
  if (page_size < 1 || page_size > mlaq::kAttnMaxPage)
    return fail(MLAQ_ERR_UNSUPPORTED, "page_size=%d outside 1..4096", page_size);
  if (num_splits < 1 || num_splits > mlaq::kAttnMaxSplits)
    return fail(MLAQ_ERR_UNSUPPORTED, "num_splits=%d outside 1..256", num_splits);
  return MLAQ_OK;
}

int mlaq_attn_can_implement(int num_heads, int page_size, int num_splits, int partial_dtype, int device) {
  clear_error();
  const char* arch = nullptr;
  if (device_arch(device, &arch) != MLAQ_OK) return 0;
  return mlaq_attn_plan_supported(num_heads, page_size, num_splits, partial_dtype, arch) == MLAQ_OK;
}

int mlaq_attn_prewarm(int partial_dtype, int device) {
  clear_error();
  if (!known_partial(partial_dtype)) return fail(MLAQ_ERR_INVALID_ARG, "unknown partial_dtype %d", partial_dtype);
  const char* arch = nullptr;
  int st = device_arch(device, &arch);
  if (st != MLAQ_OK) return st;
  if (!is_gfx950(arch)) return fail(MLAQ_ERR_UNSUPPORTED, "device architecture '%s' is not gfx950", arch);
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess && cur != device) e = hipSetDevice(device);
  const void* split[] = {mlaq::attn_split_kernel_for(partial_dtype, false),
                         mlaq::attn_split_kernel_for(partial_dtype, true)};
  for (const void* fn : split) {
    hipFuncAttributes attr;
    if (e == hipSuccess) e = hipFuncGetAttributes(&attr, fn);
  }
  for (int parts = 1; parts <= 16; parts *= 2)
    for (int r = 1; r <= 8; r *= 2) {
      hipFuncAttributes attr;
      if (e == hipSuccess) e = hipFuncGetAttributes(&attr, mlaq::attn_merge_kernel_for(partial_dtype, parts, r));
    }
  void* scratch = nullptr; // the allocation-free entry point's array: address looked up once here
  if (e == hipSuccess) e = mlaq::scratch_address(device, &scratch);
  if (cur != device) (void)hipSetDevice(cur);
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "loading attention kernels: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

} // extern "C"

namespace {

// mlaq_attn_run (use_scratch false: the caller's workspace) and
// mlaq_attn_run_noalloc (use_scratch true: the library's device array, no
// caller workspace). Every check that needs no HIP call comes first, so both
// entry points report the same argument errors in the same order.
int attn_run(const mlaq_attn_args* args, bool use_scratch, void* stream) {
  clear_error();
  if (!args) return fail(MLAQ_ERR_INVALID_ARG, "args is NULL");
  const mlaq_attn_args& a = *args;
  if (use_scratch && (a.workspace || a.workspace_bytes))
    return fail(MLAQ_ERR_INVALID_ARG, "mlaq_attn_run_noalloc takes no workspace (pass NULL and 0 bytes)");
  if (!known_partial(a.partial_dtype)) return fail(MLAQ_ERR_INVALID_ARG, "unknown partial_dtype %d", a.partial_dtype);
  if (a.H < 1 || a.H > mlaq::kAttnMaxHeads) return fail(MLAQ_ERR_UNSUPPORTED, "H=%d outside 1..16", a.H);
  if (a.page_size < 1 || a.page_size > mlaq::kAttnMaxPage)
    return fail(MLAQ_ERR_UNSUPPORTED, "page_size=%d outside 1..4096", a.page_size);
  if (a.num_splits < 1 || a.num_splits > mlaq::kAttnMaxSplits)
    return fail(MLAQ_ERR_UNSUPPORTED, "num_splits=%d outside 1..256", a.num_splits);
  if (a.M < 0 || a.M > mlaq::kAttnMaxM) return fail(MLAQ_ERR_UNSUPPORTED, "M=%d outside 0..65536", a.M);
  if (a.M == 0) return MLAQ_OK;
  if (!a.q || !a.kv_cache || !a.block_table || !a.seq_lens || !a.out)
    return fail(MLAQ_ERR_INVALID_ARG, "q, kv_cache, block_table, seq_lens and out must be non-NULL");
  if (a.num_pages < 1 || a.block_table_stride < 1)
    return fail(MLAQ_ERR_INVALID_ARG, "num_pages and block_table_stride must be >= 1");
  if (int64_t(a.block_table_stride) * a.page_size > (int64_t(1) << 30))
    return fail(MLAQ_ERR_UNSUPPORTED, "block_table_stride * page_size exceeds 2^30 tokens");
  if (!(a.softmax_scale == a.softmax_scale) || a.softmax_scale > 3.4e38f || a.softmax_scale < -3.4e38f)
    return fail(MLAQ_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (a.q_stride_m < 0 || a.q_stride_h < 0 || a.q_stride_m % 8 || a.q_stride_h % 8 ||
      a.q_stride_m >= (int64_t(1) << 31) || a.q_stride_h >= (int64_t(1) << 31))
    return fail(MLAQ_ERR_INVALID_ARG, "q strides must be non-negative multiples of 8 elements below 2^31");
  if (!aligned(a.q, 16) || !aligned(a.kv_cache, 16) || !aligned(a.out, 16))
    return fail(MLAQ_ERR_INVALID_ARG, "q, kv_cache and out must be 16-byte aligned");
  if (!aligned(a.block_table, 4) || !aligned(a.seq_lens, 4) || !aligned(a.lse, 4))
    return fail(MLAQ_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");
  const size_t ws = mlaq_attn_workspace_size(a.M, a.H, a.num_splits, a.partial_dtype);
  if (use_scratch) {
    if (ws > mlaq::kAttnScratchBytes)
      return fail(MLAQ_ERR_UNSUPPORTED, "plan needs %zu bytes of scratch; the library's array holds %zu", ws,
                  mlaq::kAttnScratchBytes);
  } else {
    if (ws > 0 && (!a.workspace || a.workspace_bytes < ws))
      return fail(MLAQ_ERR_INVALID_ARG, "workspace must hold %zu bytes", ws);
    if (ws > 0 && !aligned(a.workspace, 256)) return fail(MLAQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  // Address spans: inputs and outputs must not overlap.
  const size_t mh = size_t(a.M) * size_t(a.H);
  const size_t q_bytes = size_t((int64_t(a.M) - 1) * a.q_stride_m + (int64_t(a.H) - 1) * a.q_stride_h + mlaq::kRow) * 2;
  const size_t kv_bytes = size_t(a.num_pages) * size_t(a.page_size) * mlaq::kRow * 2;
  const size_t bt_bytes = size_t(a.M) * size_t(a.block_table_stride) * 4;
  const size_t sl_bytes = size_t(a.M) * 4;
  const size_t out_bytes = mh * mlaq::kLatent * 2, lse_bytes = a.lse ? mh * 4 : 0;
  const void* ins[] = {a.q, a.kv_cache, a.block_table, a.seq_lens};
  const size_t in_bytes[] = {q_bytes, kv_bytes, bt_bytes, sl_bytes};
  const void* outs[] = {a.out, a.lse, ws > 0 && !use_scratch ? a.workspace : nullptr};
  const size_t out_sizes[] = {out_bytes, lse_bytes, ws};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[o], out_sizes[o], ins[i], in_bytes[i]))
        return fail(MLAQ_ERR_INVALID_ARG, "an output or the workspace overlaps an input buffer");
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], out_sizes[o], outs[o2], out_sizes[o2]))
        return fail(MLAQ_ERR_INVALID_ARG, "out, lse and workspace must not overlap");
  }
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  const char* arch = nullptr;
  int st = device_arch(device, &arch);
  if (st != MLAQ_OK) return st;
  st = mlaq_attn_plan_supported(a.H, a.page_size, a.num_splits, a.partial_dtype, arch);
  if (st != MLAQ_OK) return st;
  void* workspace = a.workspace;
  if (use_scratch && ws > 0) {
    e = mlaq::scratch_address(device, &workspace);
    if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "scratch array address on device %d: %s", device,
                                     hipGetErrorString(e));
  }

  mlaq::AttnArgs ka{};
  ka.q = static_cast<const uint16_t*>(a.q);
  ka.kv = static_cast<const uint16_t*>(a.kv_cache);
  ka.bt = a.block_table;
  ka.seq_lens = a.seq_lens;
  ka.part = ws > 0 ? workspace : nullptr;
  ka.part_lse = ws > 0 ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                 attn_lse_offset(a.M, a.H, a.num_splits, a.partial_dtype))
                       : nullptr;
  ka.out = static_cast<uint16_t*>(a.out);
  ka.lse = a.lse;
  ka.q_sm = size_t(a.q_stride_m);
  ka.q_sh = size_t(a.q_stride_h);
  ka.scale_log2 = float(double(a.softmax_scale) * 1.4426950408889634);
  ka.M = a.M;
  ka.H = a.H;
  ka.P = a.page_size;
  ka.num_pages = a.num_pages;
  ka.bt_stride = a.block_table_stride;
  ka.S = a.num_splits;
  dim3 split_grid, merge_grid, block;
  mlaq::attn_launch_shapes(a.M, a.H, a.num_splits, &split_grid, &merge_grid, &block);
  // The kernels' scalar arguments (S, H and M packed into one word).
  uint32_t q_sm32 = uint32_t(ka.q_sm), q_sh32 = uint32_t(ka.q_sh);
  uint32_t shm = uint32_t(ka.S) | (uint32_t(ka.H) << 9) | (uint32_t(ka.M) << 14);
  void* split_args[] = {&ka.seq_lens, &ka.bt, &ka.kv, &ka.q, &q_sm32, &q_sh32, &shm, &ka.P, &ka.bt_stride,
                        &ka.num_pages, &ka.part, &ka.part_lse, &ka.out, &ka.lse, &ka.scale_log2};
  void* merge_args[] = {&ka.part_lse, &ka.part, &ka.out, &ka.lse, &shm};
  const hipStream_t st_ = static_cast<hipStream_t>(stream);
  const bool direct = a.num_splits == 1;
  int parts = 1, per_thread = 1;
  mlaq::attn_merge_shape(a.M, a.H, a.num_splits, &parts, &per_thread);
  // Both kernels are resolved before the first launch, so a plan without a
  // kernel fails with nothing enqueued.
  const void* split_fn = mlaq::attn_split_kernel_for(a.partial_dtype, direct);
  const void* merge_fn = direct ? nullptr : mlaq::attn_merge_kernel_for(a.partial_dtype, parts, per_thread);
  if (!split_fn || (!direct && !merge_fn)) return fail(MLAQ_ERR_UNSUPPORTED, "no attention kernel for this plan");
  e = hipLaunchKernel(split_fn, split_grid, block, split_args, 0, st_);
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "split kernel launch: %s", hipGetErrorString(e));
  if (!direct) {
    // The split kernel of a multi-split call writes only the workspace, so a
    // failed merge launch still leaves out and lse untouched.
    e = hipLaunchKernel(merge_fn, merge_grid, block, merge_args, 0, st_);
    if (e != hipSuccess)
      return fail(MLAQ_ERR_DEVICE, "merge kernel launch (the split kernel, which writes only the workspace, is "
                                   "enqueued): %s", hipGetErrorString(e));
  }
  return MLAQ_OK;
}

} // namespace

extern "C" {

int mlaq_attn_run(const mlaq_attn_args* args, void* stream) { return attn_run(args, false, stream); }

int mlaq_attn_run_noalloc(const mlaq_attn_args* args, void* stream) { return attn_run(args, true, stream); }

const char* mlaq_last_error(void) { return g_err; }

} // extern "C"
