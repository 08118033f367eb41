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
  if (nope_dim != MLAQ_NOPE_DIM || latent_dim != MLAQ_LATENT_DIM || rope_dim != MLAQ_ROPE_DIM)
    return fail(MLAQ_ERR_UNSUPPORTED, "dims (nope %d, latent %d, rope %d) are not (128, 512, 64)", nope_dim,
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
    const mlaq::Variant v = mlaq::variant_for(weight_format, out_dtype, m_regimes[i]);
    if (seen[v.m_tiles]) continue;
    seen[v.m_tiles] = true;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device) e = hipSetDevice(device);
    hipFuncAttributes attr;
    if (e == hipSuccess) e = hipFuncGetAttributes(&attr, mlaq::kernel_for(v));
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "loading kernel for M=%d: %s", m_regimes[i], hipGetErrorString(e));
  }
  return MLAQ_OK;
}

int mlaq_run(const void* q_nope, const void* q_pe, const void* w, const void* w_scales, const float* q_scale,
             void* out, int M, int H, int weight_format, int out_dtype, void* stream) {
  clear_error();
  if (!known_weight_format(weight_format)) return fail(MLAQ_ERR_INVALID_ARG, "unknown weight_format %d", weight_format);
  if (!known_out_dtype(out_dtype)) return fail(MLAQ_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  if (!supported_heads(H)) return fail(MLAQ_ERR_UNSUPPORTED, "H=%d not in {8, 11, 16}", H);
  if (M < 0 || M > MLAQ_MAX_M) return fail(MLAQ_ERR_UNSUPPORTED, "M=%d outside 0..32", M);
  if (M == 0) return MLAQ_OK; // empty batch: nothing to read or write
  if (!q_nope || !q_pe || !w || !out) return fail(MLAQ_ERR_INVALID_ARG, "q_nope, q_pe, w and out must be non-NULL");
  if (weight_format == MLAQ_WEIGHT_MXFP8 && !w_scales)
    return fail(MLAQ_ERR_INVALID_ARG, "MXFP8 weights need w_scales");
  if (weight_format == MLAQ_WEIGHT_BF16 && w_scales)
    return fail(MLAQ_ERR_INVALID_ARG, "BF16 weights take no w_scales (pass NULL)");
  if (out_dtype == MLAQ_OUT_E4M3 && !q_scale) return fail(MLAQ_ERR_INVALID_ARG, "E4M3 output needs q_scale");
  if (out_dtype == MLAQ_OUT_BF16 && q_scale)
    return fail(MLAQ_ERR_INVALID_ARG, "BF16 output takes no q_scale (pass NULL)");
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(w, 16) || !aligned(out, 16))
    return fail(MLAQ_ERR_INVALID_ARG, "q_nope, q_pe, w and out must be 16-byte aligned");
  if (q_scale && !aligned(q_scale, 4)) return fail(MLAQ_ERR_INVALID_ARG, "q_scale must be 4-byte aligned");

  const size_t mh = size_t(M) * size_t(H);
  const size_t esz_w = weight_format == MLAQ_WEIGHT_BF16 ? 2 : 1;
  const size_t esz_o = out_dtype == MLAQ_OUT_BF16 ? 2 : 1;
  const size_t out_bytes = mh * mlaq::kRow * esz_o;
  if (overlaps(out, out_bytes, q_nope, mh * mlaq::kNope * 2) || overlaps(out, out_bytes, q_pe, mh * mlaq::kRope * 2) ||
      overlaps(out, out_bytes, w, size_t(H) * mlaq::kNope * mlaq::kLatent * esz_w) ||
      overlaps(out, out_bytes, w_scales, size_t(H) * mlaq::kNope * (mlaq::kLatent / mlaq::kMxBlock)) ||
      overlaps(out, out_bytes, q_scale, sizeof(float)))
    return fail(MLAQ_ERR_INVALID_ARG, "out overlaps an input buffer");

  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  const char* arch = nullptr;
  int st = device_arch(device, &arch);
  if (st != MLAQ_OK) return st;
  st = plan_for(H, M, MLAQ_NOPE_DIM, MLAQ_LATENT_DIM, MLAQ_ROPE_DIM, weight_format, out_dtype, arch);
  if (st != MLAQ_OK) return st;

  const mlaq::Variant v = mlaq::variant_for(weight_format, out_dtype, M);
  const void* fn = mlaq::kernel_for(v);
  if (!fn) return fail(MLAQ_ERR_UNSUPPORTED, "no kernel for this plan");
  dim3 grid, block;
  mlaq::launch_shape(v, H, &grid, &block);
  mlaq::FusedArgs args{static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe), w,
                       static_cast<const uint8_t*>(w_scales), q_scale, out, M, H};
  void* kargs[] = {&args};
  e = hipLaunchKernel(fn, grid, block, kargs, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLAQ_ERR_DEVICE, "kernel launch: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

const char* mlaq_last_error(void) { return g_err; }

} // extern "C"
