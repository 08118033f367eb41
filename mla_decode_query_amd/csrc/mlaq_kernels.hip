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
// A workgroup owns one head h and one tile of WC latent columns (WC = 32:
// 16 workgroups per head), over all K, in K/(32 KB) waves: wave w takes the
// KB k-blocks of 32 rows from 32 KB w on. KB = 1 (4 waves at K = 128, 6 at
// K = 192) for two token tiles; with one token tile fewer, longer waves
// measured shorter cold launches: KB = 2 at K = 128 (BF16 out -2.7%, MXFP8
// -0.5..-0.9%, BF16 weights with E4M3 out +0.4%) and KB = 3 at K = 192
// (the pages' shape, H = 8, M = 1: -7%; M = 4: -6%), while KB = 2 at M = 32
// lengthened the launch by 1-5% (the epilogue then has fewer threads).
//
// Loads. Each lane requests pieces of whole weight rows of up to 16 bytes
// (the weight is n-major, so a tile's row segment is contiguous): one load
// instruction covers 16 (BF16) or 32 (E4M3) whole row segments, and an MXFP8
// lane also loads the one E8M0 byte of its row and column group, 5 memory
// requests per wave of one k-block in all with q_pe and the q_nope
// fragments (a k-block more adds its weight piece(s) and fragment). The
// arguments the first requests need are the kernel's first scalar
// arguments, which arrive preloaded in SGPRs (no kernel-argument load on the
// critical path).
//
// Contraction on MFMA. v_mfma_f32_16x16x32_bf16 pairs element e of lane
// (i + 16g) of A with element e of lane (j + 16g) of B, for output (i, j):
// A is q_nope of token i over 8 consecutive k (one 16-byte load straight
// from global memory), B is the weight column j over the same 8 k. A wave
// writes its 32 KB x WC bf16 tile (MXFP8 decoded first) to its own LDS slice
// and reads the B fragments back with the gfx950 transpose read, so no
// workgroup barrier separates the loads from the MFMAs; its KB k-blocks are
// chained in ascending k in one accumulator. M <= 16 uses one 16-token
// tile, M <= 32 two.
//
// The waves' fp32 partial tiles are summed through LDS in a fixed order
// (wave 0 + 1 + 2 + ...), so results are deterministic. The epilogue rounds to
// bf16 (and for E4M3 output divides by q_scale and encodes), and the same
// workgroups copy q_pe into columns 512..575 of the row (a BF16 copy leaves
// before the weights arrive, an E4M3 one right after).
//
// Cache policy. A decode step reads each layer's weights once, cold in HBM;
// the MLAQ_CACHE_STREAM kernels (template flag NT, BF16 weights only) load
// the weight rows and store a BF16 output with the nontemporal hint, which
// shortened the cold BF16-weight launch by 8-10% in same-box A/B runs
// (identical output bits) and lengthened back-to-back calls on one cached
// weight set by 5-14%, hence a caller's hint rather than the only form.
// An E4M3 output (32-byte row pieces per workgroup, four workgroups to a
// 128-byte line) is stored with the default policy: nontemporal, those
// pieces made the cold M = 32 launch 1.5% longer.
// A 128-byte line of MXFP8 rows is shared by four workgroups; there every
// nontemporal form was slower, so those kernels have no NT form.
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
// The fused kernel. One workgroup per head and WC-column tile (WC = 32 or
// 16; wave w owns k rows [32 KB w, 32 KB (w+1))); each lane loads whole
// pieces of weight rows, of up to 16 bytes: a row segment of the wave's tile
// is RBY = WC * (bytes per weight) bytes, every lane takes RBY/2 of them per
// 32 rows (16 or 32 bytes for BF16, 8 or 16 for E4M3) in loads of PB bytes,
// LPR lanes per row segment, so each load instruction covers 64/LPR whole row
// segments. MXFP8 rows come with the one scale byte
// of that row and column group, and are decoded to bf16 in registers. The
// wave then writes its 32 KB x WC bf16 tile to its own LDS slice and reads the
// MFMA B fragments back with the gfx950 transpose read (ds_read_b64_tr_b16):
// within a 16-lane group, output lane i gets element i%4 of the 8 bytes that
// lane 4e + i/4 points at, so lane 4e + q points at columns 4q..4q+3 of k row
// 8g + e (and 8g + 4 + e for the second read), and lane (j, g) receives k rows
// 8g..8g+7 of column j (of each k-block): exactly the B operand pairing with
// the q_nope A fragment of the same k. Each wave reads only rows it wrote itself, so the
// hand-off needs no workgroup barrier. Every output sums the same products in
// the same MFMA positions whatever WC is, so the tile widths give identical
// bits.
// ---------------------------------------------------------------------------

template <int WF, int OF, int MT, int NW, bool NT, int WC, int KB>
__global__ __launch_bounds__(64 * NW) void fused_query_kernel(
    const uint16_t* q_pe, const void* w, const uint16_t* q_nope, const uint8_t* w_scales, const float* q_scale,
    uint32_t pe_sm, uint32_t q_sm, uint32_t head_strides, uint32_t m_h, void* out, uint32_t out_sm, uint32_t out_sh) {
  // Scalar arguments, ordered so that everything the first requests need
  // (the input pointers, q_scale's among them, and the input strides, M and
  // H) lies in the 14 dwords of the kernel-argument segment that are
  // preloaded into SGPRs with the wave: no wave waits for a kernel-argument
  // load before it requests its data, and q_scale is one memory round trip
  // away, not two. head_strides packs the head strides of q_nope (low 16
  // bits) and q_pe (high), m_h packs M (low 16 bits) and H (high).
  const FusedArgs a{q_nope, q_pe, w, w_scales, q_scale, out, q_sm, head_strides & 0xffffu, pe_sm,
                    head_strides >> 16, out_sm, out_sh, int(m_h & 0xffffu), int(m_h >> 16)};
  constexpr int K = 32 * NW * KB;
  constexpr int KR = 32 * KB;                           // k rows per wave
  constexpr int THREADS = 64 * NW;
  constexpr int NCT = kLatent / WC;
  constexpr int MROWS = 16 * MT;
  constexpr int LDW = WC + 4;                           // padded partial-tile row, in floats
  constexpr int TP = 2 * WC + 16;                       // weight-tile row pitch in bytes (bf16 + padding)
  constexpr int ESZ = (WF == MLAQ_WEIGHT_BF16) ? 2 : 1; // bytes per weight in HBM
  constexpr int RBY = WC * ESZ;                         // bytes per row segment
  constexpr int PB = RBY / 2 < 16 ? RBY / 2 : 16;       // bytes per load
  constexpr int NL = KB * ((RBY / 2) / PB);             // loads per lane
  constexpr int LPR = RBY / PB;                         // lanes per row segment
  constexpr int RPL = 64 / LPR;                         // row segments per load
  constexpr int PD = PB / 4;                            // dwords per load
  constexpr int OD = PD * (2 / ESZ);                    // bf16 dwords per load
  static_assert(WC == 16 || WC == 32, "tiles of 16 or 32 columns");
  static_assert(PD == 2 || PD == 4, "8- or 16-byte pieces");
  static_assert(!NT || WF == MLAQ_WEIGHT_BF16, "only BF16 weight rows are streamed nontemporally");
  constexpr bool kNtOut = NT && OF == MLAQ_OUT_BF16; // nontemporal output stores (BF16 rows only)
  __shared__ __attribute__((aligned(16))) float part[NW * MROWS * LDW];
  __shared__ __attribute__((aligned(16))) uint8_t wtile[NW * KR * TP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int tile = tile_of_block(blockIdx.x, a.H * NCT); // the grid is H x NCT workgroups
  const int h = tile / NCT, ct = tile - h * NCT;
  const int c0 = ct * WC;
  const int M = a.M;
  const int k0 = KR * wave + 8 * g;      // first k of this lane's A and B fragments (k-block 0)
  const int r0 = lane / LPR;             // wave-local row of this lane's first piece (+RPL per load)
  const int pcol = (PB / ESZ) * (lane % LPR); // first tile column of each piece

  // 1. This thread's q_pe chunk (8 elements), requested first so that its
  //    store can leave while the weights are still in flight. Token m's 8
  //    chunks go to column tile m % NCT, threads 8 (m / NCT) + c, so one
  //    workgroup writes each token's whole q_pe piece of the row (one line
  //    with BF16 output, half a line with E4M3). When a head's tiles straddle
  //    two XCDs (H = 11), pieces written from two L2s into one line cost
  //    much more: spreading the chunks over the head's tiles (chunk x to tile
  //    x % NCT) made H = 11 launches 5-9% longer (same-box A/B, cold: 2.503 vs
  //    2.365 us at M = 1, 2.944 vs 2.673 us at M = 32), H = 16 equal.
  const int pe_tok = ct + NCT * (tid >> 3);
  const bool has_pe = pe_tok < M;
  const int pe_m = has_pe ? pe_tok : 0, pe_c = tid & 7;
  const uint32_t pe_off = __umul24(pe_m, a.pe_sm) + __umul24(h, a.pe_sh) + 8 * pe_c;
  const u32x4_t pe_v = *at_byte<const u32x4_t>(a.q_pe, 2 * pe_off);
  __builtin_amdgcn_sched_barrier(0);

  // 2. This lane's pieces of its weight rows (and scale byte).
  uint32_t wv[NL][PD];
  uint32_t sb[NL];                       // MXFP8: the scale byte of each piece's row
  {
    const uint32_t off = ((uint32_t(h) * K + KR * wave + r0) * kLatent + c0 + pcol) * ESZ; // < 2^22
    __builtin_assume(off < (1u << 22));
#pragma unroll
    for (int v = 0; v < NL; ++v) {
      const uint8_t* p = static_cast<const uint8_t*>(a.w) + (off + uint32_t(v) * RPL * kLatent * ESZ);
      if constexpr (PD == 4) {
        const u32x4_t x = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p))
                             : *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
        for (int d = 0; d < 4; ++d) wv[v][d] = x[d];
      } else {
        const u32x2_t x = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p))
                             : *reinterpret_cast<const u32x2_t*>(p);
        wv[v][0] = x[0];
        wv[v][1] = x[1];
      }
    }
    if constexpr (WF == MLAQ_WEIGHT_MXFP8)
#pragma unroll
      for (int v = 0; v < NL; ++v)
        sb[v] = a.w_scales[(uint32_t(h) * K + KR * wave + r0 + RPL * v) * kScalesPerRow + (c0 / kMxBlock)];
  }

  // 3. q_nope A fragments: token 16t + j, k rows k0..k0+7. Rows past M read
  //    token 0 instead; MFMA output row i depends only on A row i, and rows
  //    past M are never stored, so they need no zeroing.
  u32x4_t qa[MT][KB];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + j;
    const int mc = m < M ? m : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qa[t][kb] = *at_byte<const u32x4_t>(a.q_nope, 2 * (__umul24(mc, a.q_sm) + __umul24(h, a.q_sh) + k0 + 32 * kb));
  }
  __builtin_amdgcn_sched_barrier(0);

  float qs = 1.0f, rqs = 1.0f, lim = 0.0f;
  if constexpr (OF == MLAQ_OUT_E4M3) {
    qs = *a.q_scale;
    rqs = 1.0f / qs;
    lim = 448.0f * __builtin_fabsf(qs);
  }
  auto tail = [&](auto ieee_div) __attribute__((always_inline)) {
    // Four values -> their E4M3 codes e4m3_satfinite(RN(x / q_scale)).
    auto encode = [&](float x0, float x1, float x2, float x3) __attribute__((always_inline)) {
      if constexpr (decltype(ieee_div)::value)
        return e4m3x4_satfinite(x0 / qs, x1 / qs, x2 / qs, x3 / qs);
      else
        return e4m3x4_in_range(quot_e4m3(x0, qs, rqs, lim), quot_e4m3(x1, qs, rqs, lim),
                               quot_e4m3(x2, qs, rqs, lim), quot_e4m3(x3, qs, rqs, lim));
    };
    // 4. q_pe into columns 512..575. Loads and stores share one counter of
    //    outstanding memory operations, so a store issued before the last
    //    load has arrived must be acknowledged before that load can be
    //    waited for. The BF16 bit copy leaves as soon as q_pe arrives (its
    //    acknowledgement returns while the weights are still in flight); the
    //    E4M3 conversion also needs q_scale, so its store is held back until
    //    the weights have arrived (step 6), which measured 6-8% shorter MXFP8
    //    launches and no change for BF16 weights.
    const uint32_t pe_o = __umul24(pe_m, a.out_sm) + __umul24(h, a.out_sh) + kLatent + 8 * pe_c;
    u32x2_t pe_e4 = {0u, 0u};
    if (has_pe) {
      if constexpr (OF == MLAQ_OUT_BF16) {
        store_out<kNtOut>(at_byte<u32x4_t>(a.out, 2 * pe_o), pe_v);
      } else {
        float x[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = __uint_as_float(((pe_v[c >> 1] >> (16 * (c & 1))) & 0xffffu) << 16);
        pe_e4[0] = encode(x[0], x[1], x[2], x[3]);
        pe_e4[1] = encode(x[4], x[5], x[6], x[7]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 5. The weight pieces as bf16 (exact decode for MXFP8) into this wave's
    //    LDS tile, then the B fragments back through the transpose read.
    uint8_t* wt = wtile + wave * KR * TP;
#pragma unroll
    for (int v = 0; v < NL; ++v) {
      uint32_t b[OD];
      if constexpr (WF == MLAQ_WEIGHT_BF16) {
#pragma unroll
        for (int d = 0; d < PD; ++d) b[d] = wv[v][d];
      } else {
        const float sc = e8m0_scale_operand(sb[v]);
#pragma unroll
        for (int d = 0; d < PD; ++d) {
          b[2 * d] = e4m3x2_scaled_bf16(wv[v][d], sc, false);
          b[2 * d + 1] = e4m3x2_scaled_bf16(wv[v][d], sc, true);
        }
      }
      uint8_t* dst = wt + (r0 + RPL * v) * TP + 2 * pcol;
#pragma unroll
      for (int q = 0; q < OD / 4; ++q)
        *reinterpret_cast<u32x4_t*>(dst + 16 * q) = u32x4_t{b[4 * q], b[4 * q + 1], b[4 * q + 2], b[4 * q + 3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    f32x4_t acc[MT][WC / 16];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < WC / 16; ++i) acc[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint8_t* src = wt + (32 * kb + 8 * g + (j >> 2)) * TP + 8 * (j & 3);
#pragma unroll
      for (int i = 0; i < WC / 16; ++i) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(src + 32 * i));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(src + 32 * i + 4 * TP));
        const u32x4_t bf = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                            __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, qa[t][kb]), __builtin_bit_cast(bf16x8_t, bf), acc[t][i], 0, 0, 0);
      }
    }

    if constexpr (OF == MLAQ_OUT_E4M3) {
      if (has_pe) store_out<kNtOut>(at_byte<u32x2_t>(a.out, pe_o), pe_e4);
    }
    // 6. Partial tiles to LDS: lane (j, g) holds tokens 16t + 4g + r of
    //    column 16i + j.
    {
      float* pw = part + wave * MROWS * LDW;
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < WC / 16; ++i) pw[(16 * t + 4 * g + r) * LDW + 16 * i + j] = acc[t][i][r];
    }
    __syncthreads();

    // 7. Epilogue: sum the k slices in a fixed order, round, convert and
    //    store; each thread finishes 4 consecutive columns of one token.
    constexpr int GPR = WC / 4;
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
        store_out<kNtOut>(at_byte<u32x2_t>(a.out, 2 * o), u32x2_t{b01, b23});
      } else {
        store_out<kNtOut>(at_byte<uint32_t>(a.out, o),
                      encode(__uint_as_float(b01 << 16), __uint_as_float(b01 & 0xffff0000u),
                             __uint_as_float(b23 << 16), __uint_as_float(b23 & 0xffff0000u)));
      }
    }
  };
  if constexpr (OF == MLAQ_OUT_E4M3) {
    if (__builtin_expect(quot_e4m3_covers(qs), 1))
      tail(Flag<false>{});
    else
      tail(Flag<true>{});
  } else {
    tail(Flag<false>{});
  }
}

template <int WF, int OF, int MT, int NW, bool NT, int KB>
const void* kernel_ptr(int wc) {
  if (wc == 16) return reinterpret_cast<const void*>(&fused_query_kernel<WF, OF, MT, NW, NT, 16, KB>);
  return reinterpret_cast<const void*>(&fused_query_kernel<WF, OF, MT, NW, NT, 32, KB>);
}

// k-blocks of 32 rows per wave (the header above gives the measurements).
constexpr int k_blocks_per_wave(int K, int MT) { return MT == 1 ? (K == 192 ? 3 : 2) : 1; }

} // namespace

const void* kernel_for(const Variant& v) {
  if (v.cols != 16 && v.cols != 32) return nullptr;
#define MLAQ_CASE(WF, OF, MT, K)                                                                 \
  if (v.weight_format == WF && v.out_dtype == OF && v.m_tiles == MT && v.nope == K) {      \
    constexpr int KB = k_blocks_per_wave(K, MT), NW = K / (32 * KB);                       \
    if constexpr (WF == MLAQ_WEIGHT_BF16)                                                  \
      return v.stream ? kernel_ptr<WF, OF, MT, NW, true, KB>(v.cols) : kernel_ptr<WF, OF, MT, NW, false, KB>(v.cols); \
    else                                                                                   \
      return v.stream ? nullptr : kernel_ptr<WF, OF, MT, NW, false, KB>(v.cols);           \
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
  // One workgroup per head and column tile of the kernel kernel_for() picks.
  *grid = dim3(unsigned(H * (kLatent / v.cols)), 1, 1);
  *block = dim3(unsigned(64 * (v.nope / (32 * k_blocks_per_wave(v.nope, v.m_tiles)))), 1, 1);
}

} // namespace mlaq
