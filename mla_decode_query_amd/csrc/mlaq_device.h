// Device helpers shared by the gfx950 kernels of libmlaq (mlaq_kernels.hip,
// mlaq_uv.hip, mlaq_attn.hip). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mlaq_internal.h"

namespace mlaq {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr int kScalesPerRow = kLatent / kMxBlock;

// An LDS byte pointer as the operand type of the gfx950 transpose read
// (__builtin_amdgcn_ds_read_tr16_b64_v4i16, ds_read_b64_tr_b16).
__device__ __forceinline__ __attribute__((address_space(3))) v4i16_t* lds_v4i16(const uint8_t* p) {
  return (__attribute__((address_space(3))) v4i16_t*)(
      (__attribute__((address_space(3))) uint8_t*)(const_cast<uint8_t*>(p)));
}

// ---------------------------------------------------------------------------
// Conversions. bf16 and E4M3 encodes use the gfx950 convert instructions,
// whose rounding (nearest even) and special values were checked bit for bit
// against an independent definition of OCP E4M3FN and bf16 rounding on every
// bf16 pattern, 2.5 M other fp32 values, all E4M3 midpoints and denormals.
// ---------------------------------------------------------------------------

// Two fp32 -> packed bf16 (low half = lo), round to nearest even, NaN kept
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// The E4M3 conversion saturates: every finite or infinite value past 448 is
// 448 (NaN stays NaN). v_cvt_pk_fp8_f32 rounds to nearest even into OCP
// E4M3FN but turns out-of-range values into NaN, hence the clamp.
__device__ __forceinline__ float clamp448(float v) {
  return __builtin_isnan(v) ? v : __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
}

// Four fp32 -> four OCP E4M3FN codes (byte c holds value c), round to nearest
// even, saturating to +-448.
__device__ __forceinline__ uint32_t e4m3x4_satfinite(float v0, float v1, float v2, float v3) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v0), clamp448(v1), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v2), clamp448(v3), r, true);
  return uint32_t(r);
}

// The E4M3 epilogue's quotient, from rb = RN(1/b) and lim = RN(448 |b|)
// (both once per call), for divisors accepted by quot_e4m3_covers. Returns a
// value whose plain E4M3 conversion (e4m3x4_in_range) is the code of
// e4m3_satfinite(RN(y / b)) for every y:
//  - y is first clamped to [-lim, lim] with IEEE maximum/minimum, which keep
//    NaN (an infinite y becomes +-lim). A clamped quotient lies within a few
//    ulp of +-448 and encodes to +-448, as every quotient past 448 does under
//    saturation, and no quotient left can round past 448, so the convert
//    needs no clamp of its own;
//  - q0 = RN(y * rb) is within one ulp of y / b, the residual y - q0 * b is
//    exact in one FMA, and one FMA correction gives RN(y / b) (Markstein's
//    correction step);
//  - for |y| < 2^-100 the residual may underflow, but the quotient is then
//    at most 2^-10 in magnitude and encodes to a zero; its sign is that of
//    q0, which the final sign copy restores (the correction alone can turn
//    -0 into +0).
__device__ __forceinline__ float quot_e4m3(float y, float b, float rb, float lim) {
  const float yc = __builtin_elementwise_minimum(__builtin_elementwise_maximum(y, -lim), lim);
  const float q0 = yc * rb;
  const float rho = __builtin_fmaf(-q0, b, yc);
  const float q1 = __builtin_fmaf(rho, rb, q0);
  return __builtin_copysignf(q1, q0);
}

// Divisors for which quot_e4m3 holds: 1/b is a normal fp32, 448 |b| is
// finite, and a quotient of |y| < 2^-100 stays at most 2^-10. Others (0,
// subnormal or huge b, inf, NaN) take the IEEE division and the saturating
// encoder.
__device__ __forceinline__ bool quot_e4m3_covers(float b) {
  const float ab = __builtin_fabsf(b);
  return ab >= 0x1p-90f && ab <= 0x1p118f;
}

// Four values in E4M3 range (|v| rounds to at most 448, or NaN) -> four OCP
// E4M3FN codes, round to nearest even.
__device__ __forceinline__ uint32_t e4m3x4_in_range(float v0, float v1, float v2, float v3) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, r, true);
  return uint32_t(r);
}

// E8M0 scale byte s as the scale operand of the scaled convert below: the
// byte in the fp32 exponent field. The instruction reads only that field, so
// this is the same operand as the exact value 2^(s-127) (with s = 0 as the
// subnormal 2^-127 and s = 255 as NaN): an in-bounds probe gave identical
// results for all 256 codes under all 256 scale bytes, one shift instead of
// two compares and two selects per row.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t s) { return __uint_as_float(s << 23); }

// Two E4M3 bytes of `word` (bytes 0-1, or 2-3 with hi) times `scale` as a
// packed bf16 pair (low half = the lower byte), in one gfx950 instruction
// (v_cvt_scalef32_pk_bf16_fp8). With scale = e8m0_scale_operand(s) this is the
// exact bf16 of every code's value times 2^(s-127) for s in 3..254 (checked
// bit for bit against the fp32 conversion and product for all 256 codes and
// all 256 scale bytes); below that the result is a bf16 subnormal, rounded to
// nearest; s = 255 gives NaN.
__device__ __forceinline__ uint32_t e4m3x2_scaled_bf16(uint32_t word, float scale, bool hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(word), scale, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(word), scale, false);
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// Addressing
// ---------------------------------------------------------------------------

// Base pointer + 32-bit byte offset: a uniform base and a zero-extended
// 32-bit offset let the compiler use the SGPR-base form of global memory ops.
template <typename T, typename P>
__device__ __forceinline__ T* at_byte(P* base, uint32_t byte_off) {
  return reinterpret_cast<T*>(reinterpret_cast<typename std::conditional<std::is_const<P>::value, const uint8_t,
                                                                          uint8_t>::type*>(base) + byte_off);
}

// Block -> tile. The dispatcher deals blocks round-robin over the 8 XCDs
// (block b runs on XCD b % 8), and each XCD has its own L2. Tiles are numbered
// head-major (tile = h * NCT + column tile), and XCD x is given the
// contiguous tile range [x * n/8, (x+1) * n/8): every head's tiles then sit
// on one or two XCDs, so its q_nope rows, its q_pe rows and the 128-byte
// weight lines that neighbouring column tiles share are fetched into one L2
// instead of eight. Needs n % 8 == 0 (n = H * NCT with NCT >= 8).
__device__ __forceinline__ int tile_of_block(int b, int nblocks) {
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

} // namespace dev
} // namespace mlaq
