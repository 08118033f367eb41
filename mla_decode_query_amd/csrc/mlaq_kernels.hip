// mlaq_kernels.hip -- gfx950 kernels of the fused MLA decode query projection
// and assembly (sparkinfer PR #75 "[GG] Add BF16 MLA query projection and
// assembly", sections "What" and "Contract"; vLLM PR #174 "[GG] Fuse MXFP8
// and BF16 MLA query assembly", section "What").
//
// One launch computes, for all M tokens and H heads,
//   out[m,h,0:512]   = cvt(bf16_rne(sum_k q_nope[m,h,k] * W[h,k,n]))
//   out[m,h,512:576] = cvt(q_pe[m,h,:])
// with cvt = identity (BF16 output) or e4m3_satfinite(x / q_scale).
//
// Decomposition. The call moves ~1-3 MiB of weights and little else, so the
// kernel is an HBM stream whose cost is latency: every weight byte is
// requested at kernel entry, spread over as many CUs as the tiling allows.
// A workgroup of K/32 waves (4 for K = 128, 6 for K = 192) owns one head h
// and one slice of WCOLS = 16*VEC latent columns, over all K. Wave w takes k
// rows [32w, 32w+32).
//
// Contraction on MFMA without any transpose. v_mfma_f32_16x16x32_bf16 pairs
// element e of lane (i + 16g) of A with element e of lane (j + 16g) of B, for
// output (i, j). A lane loads VEC consecutive columns of 8 consecutive k rows
// (the weight is n-major, so each row segment is a coalesced load). For each
// of its VEC columns it builds a B fragment from those 8 rows (v_perm packs
// two rows' bf16 into one dword) and issues one MFMA whose output column j is
// relabelled as latent column c0 + VEC*j + i. The A fragment is the q_nope
// row of token i over the same 8 k per lane group, loaded straight from
// global memory. So the 16-wide MFMA column index walks 16 column groups, the
// 4 lane groups walk the 4 k octets, and no LDS round trip is needed for
// either operand. M <= 16 uses one 16-token tile, M <= 32 two.
//
// The waves' fp32 partial tiles are summed through LDS in a fixed order
// (wave 0 + 1 + 2 + ...), so results are deterministic. The epilogue rounds to
// bf16 (and for E4M3 output divides by q_scale and encodes), and the same
// workgroups copy q_pe into columns 512..575 of the row, storing it before
// they wait for their weights.
//
// Cache policy. A decode step reads each layer's weights once, cold in HBM;
// the MLAQ_CACHE_STREAM kernels (template flag NT, BF16 weights only) load
// the weight rows and store the output with the nontemporal hint, which
// shortened the cold BF16-weight launch by 8-10% in same-box A/B runs
// (identical output bits) and lengthened back-to-back calls on one cached
// weight set by 5-14%, hence a caller's hint rather than the only form.
// MXFP8 rows are 32-byte segments whose 128-byte lines four workgroups share;
// there every nontemporal form was slower, so those kernels have no NT form.
//
// MXFP8 weights are decoded in registers: v_cvt_scalef32_pk_bf16_fp8 turns
// two E4M3 bytes and the 2^(S-127) scale into their exact bf16 values in one
// instruction. The bf16 MFMA then forms exact products with q_nope, as the
// pages' exact dequantization requires.
#include "mlaq.h"
#include "mlaq_device.h"
#include "mlaq_internal.h"

namespace mlaq {
namespace {

using namespace dev;

// An output store, nontemporal in the NT kernels.
template <bool NT, typename T>
__device__ __forceinline__ void store_out(T* p, T v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// ---------------------------------------------------------------------------
// The fused kernel
// ---------------------------------------------------------------------------

template <int WF, int OF, int MT, int VEC, int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void fused_query_kernel(FusedArgs a) {
  constexpr int K = 32 * NW;                            // reduction width
  constexpr int THREADS = 64 * NW;
  constexpr int ESZ = (WF == MLAQ_WEIGHT_BF16) ? 2 : 1; // bytes per weight
  constexpr int WCOLS = 16 * VEC;                       // latent columns per workgroup
  constexpr int NCT = kLatent / WCOLS;                  // column tiles per head
  constexpr int RB = VEC * ESZ;                         // bytes per lane per k row
  constexpr int D = (RB + 3) / 4;                       // dwords per lane per k row
  constexpr int MROWS = 16 * MT;
  constexpr int LDW = WCOLS + 4; // padded LDS row, in floats
  static_assert(WF != MLAQ_WEIGHT_BF16 || VEC % 2 == 0, "bf16 columns come in dword pairs");
  static_assert(WF != MLAQ_WEIGHT_MXFP8 || VEC % 2 == 0, "E4M3 columns are decoded in pairs");
  static_assert(!NT || WF == MLAQ_WEIGHT_BF16, "only BF16 weight rows are streamed nontemporally");
  __shared__ __attribute__((aligned(16))) float part[NW * MROWS * LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int tile = tile_of_block(blockIdx.x, gridDim.x);
  const int h = tile / NCT, ct = tile - h * NCT;
  const int c0 = ct * WCOLS;
  const int M = a.M;
  const int k0 = 32 * wave + 8 * g; // first of this lane's 8 k rows
  const int col = c0 + VEC * j;     // first of this lane's VEC columns

  // 1. This thread's q_pe chunk (8 elements), requested first so that its
  //    store can leave while the weights are still in flight. Chunk x of the
  //    head goes to column tile x % NCT, thread x / NCT.
  const int pe_chunk = ct + NCT * tid;
  const bool has_pe = pe_chunk < M * (kRope / 8);
  const int pe_x = has_pe ? pe_chunk : 0; // loads stay unconditional (no branch, no early wait)
  const int pe_m = pe_x >> 3, pe_c = pe_x & 7;
  const uint32_t pe_off = __umul24(pe_m, a.pe_sm) + __umul24(h, a.pe_sh) + 8 * pe_c;
  const u32x4_t pe_v = *at_byte<const u32x4_t>(a.q_pe, 2 * pe_off);
  __builtin_amdgcn_sched_barrier(0); // keep the q_pe load ahead of the weight loads

  // 2. Weight rows (the bulk of the bytes), all requested up front.
  uint32_t wr[8][D];
  {
    const uint32_t off = ((uint32_t(h) * K + k0) * kLatent + col) * ESZ; // < 2^22
    __builtin_assume(off < (1u << 22));
#pragma unroll
    for (int r = 0; r < 8; ++r)
      load_row<RB, NT>(static_cast<const uint8_t*>(a.w) + (off + uint32_t(r) * kLatent * ESZ), wr[r]);
  }
  uint32_t sc[8];
  if constexpr (WF == MLAQ_WEIGHT_MXFP8) {
    const uint32_t off = (uint32_t(h) * K + k0) * kScalesPerRow + col / kMxBlock;
#pragma unroll
    for (int r = 0; r < 8; ++r) sc[r] = a.w_scales[off + uint32_t(r) * kScalesPerRow];
  }

  // 3. q_nope A fragments: token 16t + j, k rows k0..k0+7. Rows past M read
  //    token 0 instead; MFMA output row i depends only on A row i, and rows
  //    past M are never stored, so they need no zeroing.
  u32x4_t qa[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + j;
    const int mc = m < M ? m : 0;
    qa[t] = *at_byte<const u32x4_t>(a.q_nope, 2 * (__umul24(mc, a.q_sm) + __umul24(h, a.q_sh) + k0));
  }
  __builtin_amdgcn_sched_barrier(0); // all loads are in flight before any wait

  // 4. q_pe into columns 512..575 of its row (a bit copy, or the E4M3
  //    conversion with the same per-tensor q_scale).
  float qs = 1.0f, rqs = 1.0f;
  if constexpr (OF == MLAQ_OUT_E4M3) {
    qs = *a.q_scale;
    rqs = 1.0f / qs;
  }
  // Everything from here on, in two copies: x / q_scale by the one-FMA
  // correction (the scales where it is exact), or by IEEE division (0, inf,
  // NaN, subnormal or huge scales). The choice is uniform over the launch, so
  // the usual copy runs as straight-line code.
  auto tail = [&](auto ieee_div) __attribute__((always_inline)) {
    auto quot = [&](float (&x)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = decltype(ieee_div)::value ? x[c] / qs : div_rn(x[c], qs, rqs);
    };
    if (has_pe) {
      const uint32_t o = __umul24(pe_m, a.out_sm) + __umul24(h, a.out_sh) + kLatent + 8 * pe_c;
      if constexpr (OF == MLAQ_OUT_BF16) {
        store_out<NT>(at_byte<u32x4_t>(a.out, 2 * o), pe_v);
      } else {
        float x[2][4];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          x[c >> 2][c & 3] = __uint_as_float(((pe_v[c >> 1] >> (16 * (c & 1))) & 0xffffu) << 16);
        quot(x[0]);
        quot(x[1]);
        u32x2_t v;
        v[0] = e4m3x4_satfinite(x[0][0], x[0][1], x[0][2], x[0][3]);
        v[1] = e4m3x4_satfinite(x[1][0], x[1][1], x[1][2], x[1][3]);
        store_out<NT>(at_byte<u32x2_t>(a.out, o), v);
      }
    }
    __builtin_amdgcn_sched_barrier(0); // the q_pe store leaves before the weight wait

    // 5. Contraction over this wave's 32 k rows.
    f32x4_t acc[MT][VEC];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if constexpr (WF == MLAQ_WEIGHT_BF16) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t b;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          b[p] = __builtin_amdgcn_perm(wr[2 * p + 1][i >> 1], wr[2 * p][i >> 1], sel);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, qa[t]), __builtin_bit_cast(bf16x8_t, b), acc[t][i], 0, 0, 0);
      }
    } else {
      // Exact decode, one scaled conversion per column pair and row: bf16 of
      // E4M3 * 2^(S-127), laid out as the BF16 path's row dwords.
      uint32_t wb[8][VEC / 2];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float s = e8m0_scale_operand(sc[r]);
#pragma unroll
        for (int e = 0; e < VEC; e += 2) wb[r][e >> 1] = e4m3x2_scaled_bf16(wr[r][e >> 2], s, (e >> 1) & 1);
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t b;
#pragma unroll
        for (int p = 0; p < 4; ++p) b[p] = __builtin_amdgcn_perm(wb[2 * p + 1][i >> 1], wb[2 * p][i >> 1], sel);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, qa[t]), __builtin_bit_cast(bf16x8_t, b), acc[t][i], 0, 0, 0);
      }
    }

    // 5b. Partial tiles to LDS: lane (j, g) holds tokens 16t + 4g + r of
    //    columns VEC*j + i.
    {
      float* pw = part + wave * MROWS * LDW;
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = pw + (16 * t + 4 * g + r) * LDW + VEC * j;
#pragma unroll
          for (int i = 0; i < VEC; ++i) dst[i] = acc[t][i][r];
        }
    }
    __syncthreads();

    // 6. Epilogue: sum the k slices in a fixed order, round, convert and
    //    store; each thread finishes 4 consecutive columns of one token.
    constexpr int GPR = WCOLS / 4;
    for (int x = tid; x < M * GPR; x += THREADS) {
      const int m = x / GPR, cg = x - m * GPR;
      const int off = m * LDW + 4 * cg;
      f32x4_t sum = *reinterpret_cast<const f32x4_t*>(part + off);
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += *reinterpret_cast<const f32x4_t*>(part + w * MROWS * LDW + off);
      const uint32_t o = __umul24(m, a.out_sm) + __umul24(h, a.out_sh) + c0 + 4 * cg;
      const uint32_t b01 = bf16x2_rne(sum[0], sum[1]);
      const uint32_t b23 = bf16x2_rne(sum[2], sum[3]);
      if constexpr (OF == MLAQ_OUT_BF16) {
        store_out<NT>(at_byte<u32x2_t>(a.out, 2 * o), u32x2_t{b01, b23});
      } else {
        float y[4] = {__uint_as_float(b01 << 16), __uint_as_float(b01 & 0xffff0000u), __uint_as_float(b23 << 16),
                      __uint_as_float(b23 & 0xffff0000u)};
        quot(y);
        store_out<NT>(at_byte<uint32_t>(a.out, o), e4m3x4_satfinite(y[0], y[1], y[2], y[3]));
      }
    }
  };
  if constexpr (OF == MLAQ_OUT_E4M3) {
    if (__builtin_expect(div_rn_covers(qs), 1))
      tail(Flag<false>{});
    else
      tail(Flag<true>{});
  } else {
    tail(Flag<false>{});
  }
}

// Columns per lane per k row: 2 for both weight formats and every M (32
// columns and 16 workgroups per head; a 4-byte BF16 or 2-byte E4M3 row
// segment per lane). Chosen by cold-cache timing of 2, 4 and 8 columns in
// hipGraph loops; for MXFP8 at M <= 16, 4 columns (8 workgroups per head)
// was ahead once, and is 3-5% behind 2 with the current kernel.
template <int WF, int MT>
constexpr int vec_of() {
  return 2;
}

template <int WF, int OF, int MT, int NW, bool NT = false>
const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&fused_query_kernel<WF, OF, MT, vec_of<WF, MT>(), NW, NT>);
}

} // namespace

const void* kernel_for(const Variant& v) {
#define MLAQ_CASE(WF, OF, MT, K)                                                                 \
  if (v.weight_format == WF && v.out_dtype == OF && v.m_tiles == MT && v.nope == K) {      \
    if constexpr (WF == MLAQ_WEIGHT_BF16)                                                  \
      return v.stream ? kernel_ptr<WF, OF, MT, K / 32, true>() : kernel_ptr<WF, OF, MT, K / 32>(); \
    else                                                                                   \
      return v.stream ? nullptr : kernel_ptr<WF, OF, MT, K / 32>();                        \
  }
#define MLAQ_CASES(K)                                \
  MLAQ_CASE(MLAQ_WEIGHT_BF16, MLAQ_OUT_BF16, 1, K)  \
  MLAQ_CASE(MLAQ_WEIGHT_BF16, MLAQ_OUT_BF16, 2, K)  \
  MLAQ_CASE(MLAQ_WEIGHT_BF16, MLAQ_OUT_E4M3, 1, K)  \
  MLAQ_CASE(MLAQ_WEIGHT_BF16, MLAQ_OUT_E4M3, 2, K)  \
  MLAQ_CASE(MLAQ_WEIGHT_MXFP8, MLAQ_OUT_BF16, 1, K) \
  MLAQ_CASE(MLAQ_WEIGHT_MXFP8, MLAQ_OUT_BF16, 2, K) \
  MLAQ_CASE(MLAQ_WEIGHT_MXFP8, MLAQ_OUT_E4M3, 1, K) \
  MLAQ_CASE(MLAQ_WEIGHT_MXFP8, MLAQ_OUT_E4M3, 2, K)
  MLAQ_CASES(128)
  MLAQ_CASES(192)
#undef MLAQ_CASES
#undef MLAQ_CASE
  return nullptr;
}

void launch_shape(const Variant& v, int H, dim3* grid, dim3* block) {
  // The grid must use the column tile of the very kernel kernel_for() picks.
  const bool bf = v.weight_format == MLAQ_WEIGHT_BF16, one = v.m_tiles == 1;
  const int vec = bf ? (one ? vec_of<MLAQ_WEIGHT_BF16, 1>() : vec_of<MLAQ_WEIGHT_BF16, 2>())
                     : (one ? vec_of<MLAQ_WEIGHT_MXFP8, 1>() : vec_of<MLAQ_WEIGHT_MXFP8, 2>());
  *grid = dim3(unsigned(H * (kLatent / (16 * vec))), 1, 1);
  *block = dim3(unsigned(64 * (v.nope / 32)), 1, 1);
}

} // namespace mlaq
