// mlaq_uv.hip -- gfx950 kernel of the V up-projection that follows MLA decode
// attention: for every token m < M and head h < H,
//   out[m,h,v] = bf16_rne( sum_{c<512} x[m,h,c] * W_UV[h,v,c] )    fp32 accumulation
// with x the attention output in the latent space (bf16 [M,H,512]) and W_UV
// stored as the checkpoint holds it, one 512-wide latent row per value column
// (bf16 or E4M3 [H,128,512]; MXFP8 scales along the latent, [H,128,16]).
// (vLLM PR #174 "[GG] Fuse MXFP8 and BF16 MLA query assembly" names this UV
// projection beside the fused query path, in "Layout and topology behavior"
// and "Safety scope and PR 173"; the widths are readings.)
//
// Layout makes the MFMA easy: the reduction axis (latent c) is contiguous in
// memory, so a lane's load of 8 consecutive c of one value column is
// directly its B fragment for v_mfma_f32_16x16x32_bf16, and the A fragment
// is the same 8 c of token j's x row. The MFMA sums element e of lane
// j + 16g of A against element e of lane i + 16g of B over all g and e, so
// any assignment of c to (g, e) that A and B share is valid. A workgroup of
// W waves (W = 1 here; each wave reduces S = 512/W latent values in S/32
// k-blocks, chained in one accumulator) owns one head, CB value columns and
// one 16-token tile. BF16 weights: lane (j, g) of wave w takes
// c = S w + 32kb + 8g + e in k-block kb, so one load instruction covers 64
// contiguous bytes of each of 16 rows. MXFP8 weights: the lane takes
// S/4 consecutive c from S w + (S/4) g (c = S w + (S/4) g + 8kb + e), i.e.
// whole MX scale groups of 32 (four with one wave), in 16-byte loads and one
// scale byte per group, instead of 8-byte loads and a scale byte for each.
// (BF16 rows keep the ungrouped form: grouped, with the nontemporal loads
// they then had, cold BF16 launches ran about 10% longer, each instruction
// touching every 128-byte line of a row segment in 16-byte pieces; BF16 rows
// have no scale loads for grouping to save.) The waves' partial tiles are summed through LDS in a
// fixed order, and the tile goes through LDS anyway so that each thread
// stores 4 consecutive columns. Every workgroup reads its head's x rows for
// its tile from L2, which is the per-CU traffic that grows with M, so the
// shape keeps 256 workgroups at H = 16 either way: for M <= 16, CB = 8 (the
// upper 8 MFMA columns repeat the lower 8 at the same addresses, so no extra
// HBM traffic, and are dropped), 16 workgroups per head; for M <= 32, CB = 16
// and the two token tiles in workgroups of their own (8 column blocks x 2
// tiles per head), the two tiles of a column block on the same XCD so its
// weights come from HBM once.
//
// MXFP8: v_cvt_scalef32_pk_bf16_fp8 gives the exact bf16 of each E4M3 byte
// times 2^(S-127), so the MFMA forms exact products as the oracle's
// dequantization does.
#include "mlaq.h"
#include "mlaq_device.h"
#include "mlaq_internal.h"

namespace mlaq {
namespace {

using namespace dev;

// Waves per workgroup, each reducing kUvSpan latent values in kUvKb
// k-blocks of 32. One wave over all 512 measured shortest in same-box A/B
// runs over cold rotations (against four waves of 128: -2.1% BF16, -2.8%
// MXFP8 at M = 32, -2.9% both at M = 8; two waves of 256 were in between,
// eight waves of 64 were 2-6% slower).
constexpr int kUvWaves = 1;
constexpr int kUvThreads = 64 * kUvWaves;
constexpr int kUvKb = 16 / kUvWaves;    // k-blocks of 32 latent values per wave
constexpr int kUvSpan = 512 / kUvWaves; // latent values per wave
static_assert(kUvWaves == 1 || kUvWaves == 2 || kUvWaves == 4 || kUvWaves == 8, "k-blocks split evenly");
constexpr int kUvScalesPerRow = kLatent / kMxBlock;

// W_UV rows are loaded with the ordinary cache policy whatever the caller's
// cache hint. A nontemporal form for BF16 rows was measured: 3% shorter cold
// BF16 launches only while the other layers' weights stayed in the Infinity
// Cache (which streamed rows do not claim); with every layer of the step cold
// it made the BF16 layers ~3% longer (the 64-layer UV step 2.78 -> 2.82 us per
// layer, three bench runs), and back-to-back calls on one warm weight set
// 7.5% longer. Nontemporal output stores and MXFP8 rows gained nothing.
template <int WF, int NMT, int CB>
__global__ __launch_bounds__(kUvThreads) void uv_projection_kernel(const uint16_t* x, const void* w,
                                                                   const uint8_t* w_scales, void* out, int M_,
                                                                   int H_) {
  // Scalar arguments (all preloaded into SGPRs with the wave, no
  // kernel-argument load before the first weight request).
  const UvArgs a{x, w, w_scales, out, M_, H_};
  constexpr int NVB = kValue / CB; // column blocks per head
  constexpr int MROWS = 16;        // tokens per workgroup
  constexpr int LDW = CB + 4;
  static_assert(CB == 8 || CB == 16, "8 or 16 value columns per workgroup");
  __shared__ __attribute__((aligned(16))) float part[kUvWaves * MROWS * LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  // Tile = (head, column block, token tile), the token tile fastest, so the
  // XCD-contiguous tile ranges keep both token tiles of a block together.
  const int tile = tile_of_block(blockIdx.x, a.H * (NVB * NMT)); // the grid is H x NVB x NMT workgroups
  const int h = tile / (NVB * NMT), hr = tile - h * (NVB * NMT);
  const int vb = hr / NMT, mt = hr - (hr / NMT) * NMT;
  const int v = vb * CB + (j % CB); // this lane's value column
  const int M = a.M, H = a.H;
  // This lane's first latent value, and the step between its k-blocks.
  constexpr bool kGrouped = WF == MLAQ_WEIGHT_MXFP8;
  constexpr int kStep = kGrouped ? 8 : 32;
  const int cbase = kUvSpan * wave + (kGrouped ? 8 * kUvKb : 8) * g;

  // 1. Weight fragments: kUvKb k-blocks of 8 consecutive latent values.
  u32x4_t wb[kUvKb];
  constexpr int kGroups = kUvKb >= 4 ? kUvKb / 4 : 1; // MX scale groups a lane's latent values touch
  uint32_t sc[kGroups];
  if constexpr (WF == MLAQ_WEIGHT_BF16) {
    const uint32_t off = ((uint32_t(h) * kValue + v) * kLatent + cbase) * 2;
#pragma unroll
    for (int kb = 0; kb < kUvKb; ++kb) wb[kb] = *at_byte<const u32x4_t>(a.w, off + 2 * kStep * kb);
  } else {
    const uint32_t off = (uint32_t(h) * kValue + v) * kLatent + cbase;
#pragma unroll
    for (int q = 0; q < kGroups; ++q)
      sc[q] = a.w_scales[(uint32_t(h) * kValue + v) * kUvScalesPerRow + cbase / kMxBlock + q];
#pragma unroll
    for (int q = 0; q < kUvKb / 2; ++q) {
      const u32x4_t wq = *at_byte<const u32x4_t>(a.w, off + 16 * q);
      wb[2 * q] = u32x4_t{wq[0], wq[1], 0u, 0u}; // decoded below
      wb[2 * q + 1] = u32x4_t{wq[2], wq[3], 0u, 0u};
    }
  }

  // 2. A fragments: token 16 mt + j, the same 8 latent values per k-block.
  //    Rows past M read token 0; their MFMA output rows are never stored.
  u32x4_t xa[kUvKb];
  {
    const int m = 16 * mt + j;
    const int mc = m < M ? m : 0;
    const uint32_t off = ((uint32_t(mc) * H + h) * kLatent + cbase) * 2;
#pragma unroll
    for (int kb = 0; kb < kUvKb; ++kb) xa[kb] = *at_byte<const u32x4_t>(a.x, off + 2 * kStep * kb);
  }
  __builtin_amdgcn_sched_barrier(0); // every load is in flight before any wait

  // 3. Contraction over this wave's kUvSpan latent values.
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kUvKb; ++kb) {
    u32x4_t b = wb[kb];
    if constexpr (WF == MLAQ_WEIGHT_MXFP8) {
      // 8 E4M3 values of one column (consecutive latent) -> 4 dwords of bf16
      // pairs, one scaled conversion each.
      const float s = e8m0_scale_operand(sc[kUvKb >= 4 ? kb / 4 : 0]); // a lane's groups start at a group boundary
      u32x4_t d;
#pragma unroll
      for (int p = 0; p < 4; ++p) d[p] = e4m3x2_scaled_bf16(b[p >> 1], s, p & 1);
      b = d;
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[kb]),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }

  // 4. Partial tiles to LDS: lane (j, g) holds tokens 16 mt + 4g + r of column j.
  if (j < CB) {
    float* pw = part + wave * MROWS * LDW;
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[(4 * g + r) * LDW + j] = acc[r];
  }
  __syncthreads();

  // 5. Epilogue: sum the waves' partials in order, round, store 4 columns.
  constexpr int GPR = CB / 4;
  const int m0 = 16 * mt, rows = M - m0 < MROWS ? M - m0 : MROWS; // tokens of this tile below M
  for (int x = tid; x < rows * GPR; x += kUvThreads) {
    const int ml = x / GPR, cg = x - ml * GPR, m = m0 + ml;
    const int off = ml * LDW + 4 * cg;
    f32x4_t sum = *reinterpret_cast<const f32x4_t*>(part + off);
#pragma unroll
    for (int w = 1; w < kUvWaves; ++w) sum += *reinterpret_cast<const f32x4_t*>(part + w * MROWS * LDW + off);
    const uint32_t o = (uint32_t(m) * H + h) * kValue + vb * CB + 4 * cg;
    *at_byte<u32x2_t>(a.out, 2 * o) = u32x2_t{bf16x2_rne(sum[0], sum[1]), bf16x2_rne(sum[2], sum[3])};
  }
}

// Value columns per workgroup: 8 with one token tile, 16 with two (256
// workgroups at H = 16 either way).
constexpr int uv_cols(int m_tiles) { return m_tiles == 1 ? 8 : 16; }

template <int WF, int NMT>
const void* uv_kernel_ptr() {
  return reinterpret_cast<const void*>(&uv_projection_kernel<WF, NMT, uv_cols(NMT)>);
}

} // namespace

const void* uv_kernel_for(int weight_format, int m_tiles) {
  if (weight_format == MLAQ_WEIGHT_BF16)
    return m_tiles == 1 ? uv_kernel_ptr<MLAQ_WEIGHT_BF16, 1>() : uv_kernel_ptr<MLAQ_WEIGHT_BF16, 2>();
  if (weight_format == MLAQ_WEIGHT_MXFP8)
    return m_tiles == 1 ? uv_kernel_ptr<MLAQ_WEIGHT_MXFP8, 1>() : uv_kernel_ptr<MLAQ_WEIGHT_MXFP8, 2>();
  return nullptr;
}

void uv_launch_shape(int H, int m_tiles, dim3* grid, dim3* block) {
  *grid = dim3(unsigned(H * (kValue / uv_cols(m_tiles)) * m_tiles), 1, 1);
  *block = dim3(kUvThreads, 1, 1);
}

} // namespace mlaq
