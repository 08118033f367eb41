// Internal interface between the C-ABI front end (mlaq_api.cpp) and the
// kernels (mlaq_kernels.hip). Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mlaq.h"

namespace mlaq {

constexpr int kNope = 128;   // K of the contiguous entry point (mlaq_run)
constexpr int kNopeGlm = 192; // the other supported K (the GLM shape)
constexpr int kLatent = 512; // N: projection width
constexpr int kRope = 64;    // R: appended q_pe width
constexpr int kRow = kLatent + kRope;
constexpr int kMxBlock = 32; // E8M0 scale group along n
constexpr int kValue = 128;  // V: value width of the UV projection
constexpr int kMaxM = 32;
constexpr int64_t kMaxStride = int64_t(1) << 24; // elements; keeps kernel offsets 32-bit
constexpr int64_t kMaxHeadStride = int64_t(1) << 16; // q_nope / q_pe head strides travel as 16-bit halves

// Kernel arguments, passed by value (one kernarg segment). Strides are in
// elements (below 2^24, so offsets stay 32-bit and multiplies 24-bit); the
// innermost dimension of every tensor is contiguous.
struct FusedArgs {
  const uint16_t* q_nope;  // bf16 [M,H,K] at (q_sm, q_sh, 1)
  const uint16_t* q_pe;    // bf16 [M,H,R] at (pe_sm, pe_sh, 1)
  const void* w;           // bf16 or E4M3 [H,K,N], contiguous
  const uint8_t* w_scales; // E8M0 [H,K,N/32], contiguous, or null
  const float* q_scale;    // device fp32 or null
  void* out;               // bf16 or E4M3 [M,H,N+R] at (out_sm, out_sh, 1)
  uint32_t q_sm, q_sh, pe_sm, pe_sh, out_sm, out_sh;
  int M;
  int H;
};

// Identifies one compiled kernel.
struct Variant {
  int weight_format; // MLAQ_WEIGHT_*
  int out_dtype;     // MLAQ_OUT_*
  int m_tiles;       // 16-token tiles: 1 (M <= 16) or 2 (M <= 32)
  int nope;          // K: 128 or 192
  bool stream;       // nontemporal weight loads and output stores (BF16 weights only)
  int cols;          // latent columns per workgroup: 32 or 16
};

// Latent columns per workgroup: 32 (16 workgroups per head), except at
// H = 8 with one 16-token tile, where 16-column tiles (256 workgroups instead
// of 128) measured 1-2% shorter cold launches (K = 128 and 192, bit-identical
// results); at H = 11, H = 16 and M > 16 they were 5% to 25% slower.
inline int tile_cols(int H, int M) { return H == 8 && M <= 16 ? 16 : 32; }

// MLAQ_CACHE_STREAM selects the nontemporal kernels for BF16 weights; MXFP8
// weights always use the ordinary ones (the hint measured slower there).
inline Variant variant_for(int weight_format, int out_dtype, int M, int nope, int H,
                           int cache_hint = MLAQ_CACHE_DEFAULT) {
  return Variant{weight_format, out_dtype, M <= 16 ? 1 : 2, nope,
                 cache_hint == MLAQ_CACHE_STREAM && weight_format == MLAQ_WEIGHT_BF16, tile_cols(H, M)};
}

// V up-projection arguments (all contiguous).
struct UvArgs {
  const uint16_t* x;       // bf16 [M,H,512]
  const void* w;           // bf16 or E4M3 [H,128,512] (latent contiguous)
  const uint8_t* w_scales; // E8M0 [H,128,16] or null
  void* out;               // bf16 [M,H,128]
  int M;
  int H;
};

// V up-projection kernel for a weight format and M tile count, and its grid
// (one kernel per pair: the cache hint does not select a UV kernel).
const void* uv_kernel_for(int weight_format, int m_tiles);
void uv_launch_shape(int H, int m_tiles, dim3* grid, dim3* block);

// Dense MLA decode attention (all tensors contiguous in their inner
// dimension; q rows strided).
constexpr int kAttnTile = 64;       // tokens per kernel iteration = split alignment
constexpr int kAttnMaxHeads = 16;   // heads are the 16 rows of one MFMA tile
constexpr int kAttnMaxSplits = 256;
constexpr int kAttnMaxPage = 4096;  // tokens per cache page
constexpr int kAttnMaxM = 65536;

// Library-owned device scratch of mlaq_attn_run_noalloc (one per device,
// held until the process ends): its size, and the device address of the
// copy on `device` (looked up once per device with that device current).
constexpr size_t kAttnScratchBytes = size_t(MLAQ_ATTN_SCRATCH_BYTES);
hipError_t scratch_address(int device, void** ptr);

struct AttnArgs {
  const uint16_t* q;        // bf16 [M,H,576] at (q_sm, q_sh, 1)
  const uint16_t* kv;       // bf16 [num_pages, P, 576], contiguous
  const int32_t* bt;        // [M, bt_stride]: physical page of each block of P tokens
  const int32_t* seq_lens;  // [M]
  void* part;               // workspace: partials [M,S,H,512] (bf16 or fp32)
  float* part_lse;          // workspace: lse_s [M,S,H] (natural log)
  uint16_t* out;            // bf16 [M,H,512], contiguous
  float* lse;               // optional [M,H]
  size_t q_sm, q_sh;        // elements
  float scale_log2;         // softmax_scale * log2(e)
  int M, H, P, num_pages, bt_stride, S;
};

// Split kernel (per partial dtype, or the direct one-split form) and merge
// kernel, and their launch shapes.
const void* attn_split_kernel_for(int partial_dtype, bool direct);
// The merge kernel for a shape (column parts 1, 2, 4, 8 or 16; ranges per
// thread 1, 2, 4 or 8; null otherwise), and the shape used for M rows of H
// heads and S ranges.
const void* attn_merge_kernel_for(int partial_dtype, int parts, int per_thread);
void attn_merge_shape(int M, int H, int S, int* parts, int* per_thread);
void attn_launch_shapes(int M, int H, int S, dim3* split_grid, dim3* merge_grid, dim3* block);

// Host function pointer of the kernel for a variant (null if none).
const void* kernel_for(const Variant& v);
// Launch geometry of a variant for H heads.
void launch_shape(const Variant& v, int H, dim3* grid, dim3* block);

} // namespace mlaq
