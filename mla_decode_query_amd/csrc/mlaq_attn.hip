// mlaq_attn.hip -- gfx950 kernels of dense MLA decode attention with split
// partials: the consumer of the 576-wide query row.
//
// For each decode token m (one sequence, T_m = seq_lens[m] cached tokens in a
// paged latent cache) and head h, over the token range of split s:
//
//   s_t   = softmax_scale * q[m,h,0:576] . kv_t[0:576]      (key = whole row)
//   o_s   = sum_t exp(s_t - L_s) kv_t[0:512] / sum_t exp(s_t - L_s)
//   lse_s = L_s + log sum_t exp(s_t - L_s)
//
// stored as FP32 or BF16 partials, then merged into a BF16 output:
//   o = sum_s exp(lse_s - L) o_s / sum_s exp(lse_s - L),  L = max_s lse_s.
// (b12x PR #441 "Allow FP32 split partials in prepared dense MLA": commit
// text, walkthrough and "Behavior" -- partials in FP32 or BF16, BF16 the
// default, merge output BF16. The attention itself is the plain latent-space
// reading: the key is the 512 latent + 64 rotary row, the value its latent
// part, shared by all heads.) Range s covers tokens [s*chunk, (s+1)*chunk)
// of the sequence, chunk = ceil(T/S) rounded up to 64, so every range starts
// on a 64-token tile.
//
// Split kernel, one workgroup (4 waves) per (m, s), two workgroups per
// compute unit (each holds a 66 KiB LDS tile), so one workgroup's compute
// covers the other's waits. Heads are the 16 rows of
// v_mfma_f32_16x16x32_bf16 (H <= 16; missing rows repeat head H-1 and are
// never stored). Tokens go in 64-token tiles:
//  - lane (j, g) of wave w loads token 16w + j of a tile: 16 bytes at byte
//    offset 16(4kb + g) of its 1152-byte row for kb = 0..17, i.e. 64
//    contiguous bytes of each of 16 rows per instruction;
//  - scores: the B fragment of K^T for lane (j, g) is exactly that 16-byte
//    chunk (8 consecutive dims of token j), so S[h, token] is 18 MFMAs
//    straight from the loaded registers, with Q held in registers as A
//    fragments. Right after each k-block's MFMA, its chunk is written to the
//    LDS tile (the value part: the row's first 1024 bytes, row-major) and its
//    registers are refilled with the same chunk of the next tile, so the next
//    tile's requests leave during the score product (1.6% shorter decode
//    batch calls, 2.9% at 64k, than issuing them after it) and every tile has
//    a whole iteration of compute to arrive; its page indices are fetched one
//    tile earlier still;
//  - online softmax in the log2 domain, against a reference maximum that
//    moves only when a score exceeds it by more than 8 (weights up to 2^8,
//    exact in fp32, in range for bf16): a tile then needs no exchange of row
//    maxima before its weights, one workgroup barrier fewer (0.7% shorter
//    decode batch calls, 1.1% at 64k); when a wave sees such a score (always
//    on the first tile), the reference moves to the tile's row maximum, whose
//    wave parts (DPP within rows) are published in LDS beside the flags; the
//    running sums stay per lane until the end;
//  - P (bf16; for FP32 partials also its bf16 remainder, so that P enters
//    the value product with 16 significant bits) goes to LDS; wave w
//    multiplies it by the value columns
//    [128w, 128w+128): 2 k-blocks of 32 tokens x 8 column tiles. The value
//    B fragments come from the row-major tile through the gfx950 LDS
//    transpose read (two 8-byte reads per fragment), with no gathers.
// Tokens past the range end are clamped to its last token (so every loaded
// row is finite data of the sequence) and masked to -inf before the softmax.
// Finally the running sums are reduced (DPP + LDS, fixed order), o_s = acc * (1/l)
// goes through LDS so each lane stores 16 contiguous bytes, and o_s and lse_s
// are written to the workspace, or -- with one split -- the BF16 output and lse
// directly (merging one partial is the identity).
#include <math.h>

#include "mlaq.h"
#include "mlaq_device.h"
#include "mlaq_internal.h"

namespace mlaq {
namespace {

using namespace dev;

constexpr int kAttnThreads = 256;           // 4 waves
constexpr int kKb = kRow / 32;              // 18 k-blocks of the 576-wide score product
constexpr int kVb = kLatent / 32;           // the first 16 of them are the value
// The LDS tile holds the value part of each token row (1024 bytes) at a
// 1056-byte pitch: consecutive rows start 8 banks apart, so the 16 lanes of
// a transpose read (4 rows x 32 bytes) hit 32 different banks. Before the
// first tile it stages the 16 query rows (1152 bytes each) at their own pitch.
constexpr int kVPitch = 2 * kLatent + 32;   // 1056
constexpr int kQPitch = 2 * kRow + 32;      // 1184
constexpr int kTileBytes = kAttnTile * kVPitch;
static_assert(16 * kQPitch <= kTileBytes, "query staging fits the tile");
constexpr int kPPitch = kAttnTile + 8;      // bf16 per head row of the LDS P tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefSlack = 8.f; // log2 of the largest softmax weight allowed against a stale reference

constexpr int kPartialBf16 = MLAQ_PARTIAL_BF16;
constexpr int kPartialFp32 = MLAQ_PARTIAL_FP32;
constexpr int kDirect = 2; // one split: write the final output
constexpr int kMergeMaxR = 8;  // most ranges per merge thread (all requested at once)

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// DPP lane exchange within rows of 16 lanes (float payload).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16
constexpr int kRowRor4 = 0x124;       // lane i <- lane (i+4) mod 16
constexpr int kRowRor8 = 0x128;       // lane i <- lane (i+8) mod 16

// Max / sum over the 16 lanes of a DPP row; every lane gets the result.
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, dpp<kQuadXor1>(v));
  v = __builtin_fmaxf(v, dpp<kQuadXor2>(v));
  v = __builtin_fmaxf(v, dpp<kRowHalfMirror>(v));
  return __builtin_fmaxf(v, dpp<kRowMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  return v + dpp<kRowMirror>(v);
}

// Maxima of four rows over the 16 lanes of a DPP row, transposed: lane j
// returns the maximum of row 2*(j&1) + ((j>>1)&1) of (v0, v1, v2, v3). The
// xor-1 partners swap halves (each keeps two rows), the xor-2 partners swap
// quarters (each keeps one), then two rotations cover all 16 lanes: 5 DPP
// moves instead of 16 for four separate reductions.
__device__ __forceinline__ float rows4_max_transposed(float v0, float v1, float v2, float v3, int j) {
  const bool b0 = j & 1, b1 = (j >> 1) & 1;
  float k0 = b0 ? v2 : v0, k1 = b0 ? v3 : v1;
  const float s0 = b0 ? v0 : v2, s1 = b0 ? v1 : v3;
  k0 = __builtin_fmaxf(k0, dpp<kQuadXor1>(s0));
  k1 = __builtin_fmaxf(k1, dpp<kQuadXor1>(s1));
  float k = b1 ? k1 : k0;
  const float sx = b1 ? k0 : k1;
  k = __builtin_fmaxf(k, dpp<kQuadXor2>(sx));
  k = __builtin_fmaxf(k, dpp<kRowRor4>(k));
  return __builtin_fmaxf(k, dpp<kRowRor8>(k));
}

// Token range [a, b) of split s of a sequence of T tokens.
__device__ __forceinline__ void split_range(int T, int S, int s, int* a, int* b) {
  int chunk = (T + S - 1) / S;
  chunk = (chunk + kAttnTile - 1) / kAttnTile * kAttnTile;
  const long long lo = (long long)s * chunk;
  *a = lo < T ? int(lo) : T;
  *b = lo + chunk < T ? int(lo + chunk) : T;
}

__device__ __forceinline__ int clamp_len(const AttnArgs& a, int m) {
  const int T = a.seq_lens[m];
  const long long cap = (long long)a.bt_stride * a.P;
  return T < 0 ? 0 : (T > cap ? int(cap) : T);
}

// The logical block of this workgroup. Blocks are dealt round-robin over the
// 8 XCDs (block b runs on XCD b % 8), each with its own L2. When the grid is a
// multiple of 8, block b takes the logical index tile_of_block(b), so XCD x
// holds a contiguous eighth of the logical blocks: the split workgroups of a
// sequence share its query rows in one L2 (the split kernel's fetch drops from
// 1.028x to 0.999x the algorithmic bytes at 32 x 4096), and merge workgroups of
// neighbouring column parts, whose 64-byte partial segments share 128-byte
// lines, fetch each line once (the 64k merge's fetch halves). Measured 1.2-1.4%
// shorter calls with bit-identical results.
__device__ __forceinline__ int xcd_local_block(int n) { // n: the grid's block count
  return (n & 7) == 0 ? dev::tile_of_block(blockIdx.x, n) : int(blockIdx.x);
}

// (S, H, M) travel packed in one kernel argument: S in bits 0-8, H in 9-13,
// M in 14-30 (S <= 256, H <= 16, M <= 65536).
__device__ __forceinline__ void unpack_shm(uint32_t shm, int* S, int* H, int* M) {
  *S = int(shm & 0x1ffu);
  *H = int((shm >> 9) & 0x1fu);
  *M = int(shm >> 14);
}

// Scalar arguments: the first 14 dwords (everything the start-up chain of
// length -> block table -> cache row needs, and the query rows) are preloaded
// into SGPRs with the wave, so no wave waits for a kernel-argument load first.
template <int PD>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_split_kernel(
    const int32_t* seq_lens_, const int32_t* bt_, const uint16_t* kv_, const uint16_t* q_, uint32_t q_sm_,
    uint32_t q_sh_, uint32_t shm_, int P_, int bt_stride_, int num_pages_, void* part_, float* part_lse_,
    uint16_t* out_, float* lse_, float scale_log2_) {
  AttnArgs a{};
  a.q = q_;
  a.kv = kv_;
  a.bt = bt_;
  a.seq_lens = seq_lens_;
  a.part = part_;
  a.part_lse = part_lse_;
  a.out = out_;
  a.lse = lse_;
  a.q_sm = q_sm_;
  a.q_sh = q_sh_;
  a.scale_log2 = scale_log2_;
  unpack_shm(shm_, &a.S, &a.H, &a.M);
  a.P = P_;
  a.num_pages = num_pages_;
  a.bt_stride = bt_stride_;
  // FP32 partials keep P to 16 significant bits: P = hi + lo, two bf16
  // tiles and two value products, so the partial is not limited by a bf16
  // rounding of the softmax weights. BF16 partials (and the one-split form,
  // whose output is bf16) use P rounded to bf16 once.
  constexpr bool kSplitP = PD == kPartialFp32;
  __shared__ __attribute__((aligned(16))) uint8_t kvt[kTileBytes]; // the current tile, row = token
  __shared__ __attribute__((aligned(16))) uint16_t pt[(kSplitP ? 2 : 1) * 16 * kPPitch]; // P (hi, lo), row = head
  __shared__ __attribute__((aligned(16))) float red[4][16];            // per-wave row max / sum
  __shared__ __attribute__((aligned(16))) int flags[4];                // per-wave: a score above the reference

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int S = a.S;
  const int bx = xcd_local_block(a.M * a.S);
  const int m = bx / S, s = bx - (bx / S) * S;
  const int H = a.H;
  const int T = clamp_len(a, m);
  int ta, tb;
  split_range(T, S, s, &ta, &tb);

  if (ta >= tb) {
    // Empty range (or empty sequence): lse_s = -inf, and the merge skips it.
    if constexpr (PD == kDirect) {
      for (int x = tid; x < H * kLatent / 8; x += kAttnThreads) {
        const int h = x / (kLatent / 8), c = x - h * (kLatent / 8);
        *reinterpret_cast<u32x4_t*>(a.out + (size_t(m) * H + h) * kLatent + 8 * c) = u32x4_t{0u, 0u, 0u, 0u};
      }
      if (a.lse && tid < H) a.lse[size_t(m) * H + tid] = -INFINITY;
    } else {
      if (tid < H) a.part_lse[(size_t(m) * S + s) * H + tid] = -INFINITY;
    }
    return;
  }

  const int32_t* bt = a.bt + size_t(m) * a.bt_stride;
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(a.kv);
  const int trow = 16 * w + j; // this lane's token within a tile
  // This lane's token in the tile at t0, clamped into the range.
  auto token = [&](int t0) { return t0 + trow < tb ? t0 + trow : tb - 1; };
  // Its block-table entry (raw: clamped into the pool only where it is used,
  // so the load's latency is not waited for until the next tile needs it).
  auto page_of = [&](int t0) { return bt[token(t0) / a.P]; };
  // This lane's chunk of kb = 0 in the tile at t0 (page: its raw block-table
  // entry, clamped into the pool here); chunk kb lies 64 kb bytes further.
  auto tile_row = [&](int t0, int page) {
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    const int tc = token(t0);
    const uint64_t row = uint64_t(uint32_t(page)) * uint32_t(a.P) + uint32_t(tc % a.P);
    return kvb + row * (2 * kRow) + 16 * g;
  };

  // Q rows (16 heads, missing ones repeating head H-1) are read from memory
  // once per workgroup, in 16-byte chunks spread over all threads, before the
  // first tile's loads (so waiting for them never waits for the tile).
  constexpr int kQChunks = 16 * kRow / 8;                          // 1152
  constexpr int kQPerThread = (kQChunks + kAttnThreads - 1) / kAttnThreads; // 5
  u32x4_t qc[kQPerThread];
#pragma unroll
  for (int k = 0; k < kQPerThread; ++k) {
    const int cidx = tid + kAttnThreads * k;
    const int cc = cidx < kQChunks ? cidx : kQChunks - 1;
    const int hh = cc / (kRow / 8), part = cc - hh * (kRow / 8);
    const int hq = hh < H ? hh : H - 1;
    qc[k] = *reinterpret_cast<const u32x4_t*>(a.q + size_t(m) * a.q_sm + size_t(hq) * a.q_sh + 8 * part);
  }
  // Prologue: as at the end of every iteration, the next tile's loads and
  // the page of the one after are in flight (nothing older is, so the loop
  // never waits for them early).
  u32x4_t kr[kKb];
  {
    const uint8_t* rp = tile_row(ta, page_of(ta));
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) kr[kb] = *reinterpret_cast<const u32x4_t*>(rp + 64 * kb);
  }
  int pg_next = ta + kAttnTile < tb ? page_of(ta + kAttnTile) : 0;
  // Q through the (still free) LDS tile into A fragments: lane (i = j, g)
  // holds q[m, head i, 32kb + 8g .. +8].
#pragma unroll
  for (int k = 0; k < kQPerThread; ++k) {
    const int cidx = tid + kAttnThreads * k;
    if (cidx < kQChunks) {
      const int hh = cidx / (kRow / 8), part = cidx - hh * (kRow / 8);
      *reinterpret_cast<u32x4_t*>(kvt + hh * kQPitch + 16 * part) = qc[k];
    }
  }
  __syncthreads();
  u32x4_t qa[kKb];
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb) qa[kb] = *reinterpret_cast<const u32x4_t*>(kvt + j * kQPitch + 16 * (4 * kb + g));
  __syncthreads(); // the first staging overwrites the tile

  float m_run[4], l_run[4];
  f32x4_t acc[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // P column of this lane's token (the k slot of the value product).
  const int pslot = trow;
  const float sl2 = a.scale_log2;

  for (int t0 = ta; t0 < tb; t0 += kAttnTile) {
    const uint8_t* tile = kvt;
    // 1. Scores S[h = 4g + r, token 16w + j] straight from this lane's
    //    registers (its token's row, loaded during the previous iteration):
    //    the B fragment needs no LDS round trip. Each k-block's chunk is
    //    staged for the value product below (visible after the next barrier)
    //    and its registers are refilled with the next tile's chunk right after
    //    its MFMA (in that order: the scheduling barriers keep it).
    f32x4_t sacc;
    {
      // Two independent accumulator chains (even and odd k-blocks), summed
      // at the end, so consecutive MFMAs do not wait on each other.
      f32x4_t s2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      uint8_t* dst = kvt + trow * kVPitch + 16 * g;
      auto scores = [&](auto refill, const uint8_t* rp) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < kKb; ++kb) {
          s2[kb & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[kb]),
                                                               __builtin_bit_cast(bf16x8_t, kr[kb]), s2[kb & 1], 0, 0, 0);
          if (kb < kVb) *reinterpret_cast<u32x4_t*>(dst + 64 * kb) = kr[kb];
          if constexpr (decltype(refill)::value) kr[kb] = *reinterpret_cast<const u32x4_t*>(rp + 64 * kb);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (t0 + kAttnTile < tb) {
        scores(Flag<true>{}, tile_row(t0 + kAttnTile, pg_next));
        pg_next = t0 + 2 * kAttnTile < tb ? page_of(t0 + 2 * kAttnTile) : 0;
      } else {
        scores(Flag<false>{}, nullptr);
      }
      sacc = s2[0] + s2[1];
    }
    // 2. Masked scores in the log2 domain. The softmax weights are taken
    //    against the reference m_run (the running maximum as of the last
    //    tile that raised it) as long as no score exceeds it by more than
    //    kRefSlack, so that a tile needs no exchange of row maxima before its
    //    weights: weights up to 2^kRefSlack are exact in fp32 and in range for
    //    bf16. A wave with a score above that raises its flag; if any wave
    //    did (always on the first tile), the reference moves to the tile's
    //    row maximum, from the wave maxima published beside the flags.
    const bool valid = t0 + trow < tb;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = valid ? sacc[r] * sl2 : -INFINITY;
    {
      const float mx = rows4_max_transposed(sc[0], sc[1], sc[2], sc[3], j);
      if (j < 4) red[w][4 * g + 2 * (j & 1) + ((j >> 1) & 1)] = mx;
    }
    const bool over = __any((sc[0] > m_run[0] + kRefSlack) | (sc[1] > m_run[1] + kRefSlack) |
                            (sc[2] > m_run[2] + kRefSlack) | (sc[3] > m_run[3] + kRefSlack));
    if (lane == 0) flags[w] = over ? 1 : 0;
    // 3. P (bf16, and for FP32 partials its bf16 remainder p - hi, exact in
    //    fp32) into LDS in slot order.
    auto put_p = [&](const float (&pv)[4]) __attribute__((always_inline)) {
      const uint32_t p01 = bf16x2_rne(pv[0], pv[1]), p23 = bf16x2_rne(pv[2], pv[3]);
      pt[(4 * g + 0) * kPPitch + pslot] = uint16_t(p01);
      pt[(4 * g + 1) * kPPitch + pslot] = uint16_t(p01 >> 16);
      pt[(4 * g + 2) * kPPitch + pslot] = uint16_t(p23);
      pt[(4 * g + 3) * kPPitch + pslot] = uint16_t(p23 >> 16);
      if constexpr (kSplitP) {
        const uint32_t l01 = bf16x2_rne(pv[0] - __uint_as_float(p01 << 16), pv[1] - __uint_as_float(p01 & 0xffff0000u));
        const uint32_t l23 = bf16x2_rne(pv[2] - __uint_as_float(p23 << 16), pv[3] - __uint_as_float(p23 & 0xffff0000u));
        uint16_t* plo = pt + 16 * kPPitch;
        plo[(4 * g + 0) * kPPitch + pslot] = uint16_t(l01);
        plo[(4 * g + 1) * kPPitch + pslot] = uint16_t(l01 >> 16);
        plo[(4 * g + 2) * kPPitch + pslot] = uint16_t(l23);
        plo[(4 * g + 3) * kPPitch + pslot] = uint16_t(l23 >> 16);
      }
    };
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(sc[r] - m_run[r]);
    if (!over) put_p(pv);
    __syncthreads(); // publishes the staged tile, the weights, the wave maxima and the flags
    const int4 fl = *reinterpret_cast<const int4*>(flags);
    if ((fl.x | fl.y | fl.z | fl.w) == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) l_run[r] += pv[r];
    } else {
      float alpha[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * g + r;
        const float tmax = __builtin_fmaxf(__builtin_fmaxf(red[0][h], red[1][h]), __builtin_fmaxf(red[2][h], red[3][h]));
        const float mn = __builtin_fmaxf(m_run[r], tmax); // finite: every tile holds a valid token
        alpha[r] = __builtin_amdgcn_exp2f(m_run[r] - mn);
        m_run[r] = mn;
        pv[r] = __builtin_amdgcn_exp2f(sc[r] - mn);
        l_run[r] = l_run[r] * alpha[r] + pv[r];
      }
      put_p(pv);
      // (skipped when no row maximum of this wave's rows moved: alpha is then 1)
      if (__any((alpha[0] != 1.f) | (alpha[1] != 1.f) | (alpha[2] != 1.f) | (alpha[3] != 1.f))) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ct][r] *= alpha[r];
      }
      __syncthreads();
    }
    // 4. O[:, 128w + 16ct + j] += P . V over the tile's two 32-token blocks.
    //    B fragment of lane (j, g): V[token 32kb2 + 8g + e][128w + 16ct + j],
    //    e = 0..7, as two LDS transpose reads (ds_read_b64_tr_b16): within a
    //    16-lane group, output lane i gets element i%4 of the 8 bytes that
    //    lane 4e + i/4 addresses, so lane 4e + q points at columns
    //    16ct + 4q .. +3 of token 8g + e (and of 8g + 4 + e for the second).
    {
      const int e = j >> 2, q = j & 3;
      const uint8_t* vsrc = tile + (8 * g + e) * kVPitch + 2 * (128 * w + 4 * q);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const u32x4_t pa = *reinterpret_cast<const u32x4_t*>(pt + j * kPPitch + 32 * kb2 + 8 * g);
        u32x4_t pl = {0u, 0u, 0u, 0u};
        if constexpr (kSplitP) pl = *reinterpret_cast<const u32x4_t*>(pt + (16 + j) * kPPitch + 32 * kb2 + 8 * g);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const uint8_t* vp = vsrc + 32 * kb2 * kVPitch + 32 * ct;
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vp));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(vp + 4 * kVPitch));
          const u32x4_t vb = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                              __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pa),
                                                            __builtin_bit_cast(bf16x8_t, vb), acc[ct], 0, 0, 0);
          if constexpr (kSplitP)
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pl),
                                                              __builtin_bit_cast(bf16x8_t, vb), acc[ct], 0, 0, 0);
        }
      }
    }
    __syncthreads(); // the tile, P and the row maxima are free again
  }

  // Row sums: 16 lanes (DPP), then the 4 waves in order.
  float lsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lsum[r] = row16_sum(l_run[r]);
  if (j == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][4 * g + r] = lsum[r];
  }
  __syncthreads(); // also: every wave is done with the last tile
  // Normalized rows through LDS (wave w's 16 x 128 block, fp32, row pitch
  // 132), so that the stores are 16 bytes per lane.
  constexpr int kOPitch = 128 + 4;
  static_assert(4 * 16 * kOPitch * 4 <= kTileBytes, "output staging fits the tile");
  float* ob = reinterpret_cast<float*>(kvt) + w * 16 * kOPitch;
  // This lane's four rows 4g..4g+3: the waves' sums in order, then one
  // reciprocal per row (the outputs take a product; l >= 1, since the row
  // maximum's own weight is 1).
  float l[4], inv[4];
  {
    const f32x4_t r0 = *reinterpret_cast<const f32x4_t*>(&red[0][4 * g]);
    const f32x4_t r1 = *reinterpret_cast<const f32x4_t*>(&red[1][4 * g]);
    const f32x4_t r2 = *reinterpret_cast<const f32x4_t*>(&red[2][4 * g]);
    const f32x4_t r3 = *reinterpret_cast<const f32x4_t*>(&red[3][4 * g]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      l[r] = ((r0[r] + r1[r]) + r2[r]) + r3[r];
      inv[r] = __builtin_amdgcn_rcpf(l[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) ob[(4 * g + r) * kOPitch + 16 * ct + j] = acc[ct][r] * inv[r];
  if (w == 0 && j == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      if (h >= H) break;
      const float lse = (m_run[r] + __builtin_amdgcn_logf(l[r])) * kLn2;
      if constexpr (PD == kDirect) {
        if (a.lse) a.lse[size_t(m) * H + h] = lse;
      } else {
        a.part_lse[(size_t(m) * S + s) * H + h] = lse;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // Lane (row = lane / 4, quarter = lane % 4) of each of four passes writes 8
  // consecutive columns (16 bytes of bf16, 32 of fp32) of one row.
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int h = lane >> 2, c8 = 8 * (4 * pass + (lane & 3)); // column within the wave's 128
    if (h >= H) continue;
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(ob + h * kOPitch + c8);
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(ob + h * kOPitch + c8 + 4);
    const int col = 128 * w + c8;
    if constexpr (PD == kPartialFp32) {
      float* dst = static_cast<float*>(a.part) + ((size_t(m) * S + s) * H + h) * kLatent + col;
      *reinterpret_cast<f32x4_t*>(dst) = x0;
      *reinterpret_cast<f32x4_t*>(dst + 4) = x1;
    } else {
      uint16_t* dst = PD == kDirect ? a.out + (size_t(m) * H + h) * kLatent + col
                                    : static_cast<uint16_t*>(a.part) + ((size_t(m) * S + s) * H + h) * kLatent + col;
      *reinterpret_cast<u32x4_t*>(dst) =
          u32x4_t{bf16x2_rne(x0[0], x0[1]), bf16x2_rne(x0[2], x0[3]), bf16x2_rne(x1[0], x1[1]), bf16x2_rne(x1[2], x1[3])};
    }
  }
}

// The value of `v` in lane `src` of the wave (ds_bpermute).
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// Max / sum over the 64 lanes of a wave (DPP within rows, then across rows);
// every lane gets the result, in the same order in every wave.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const int lane = threadIdx.x & 63;
  v = __builtin_fmaxf(v, lane_value(v, lane ^ 16));
  return __builtin_fmaxf(v, lane_value(v, lane ^ 32));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const int lane = threadIdx.x & 63;
  v += lane_value(v, lane ^ 16);
  return v + lane_value(v, lane ^ 32);
}

// Merge: one workgroup per (m, h, column part), QN parts of 512/QN columns.
// Thread t takes 8 columns (t % CG) of the ranges s = t/CG + RG u,
// u = 0..R-1, with RG = 4 QN range groups and R >= S / RG chosen by the host,
// so every partial a thread reads is requested at once, together with the
// lse values, with no branch between the loads. Each wave forms L = max_s lse_s and the weights
// exp(lse_s - L) on its own (no workgroup barrier). The range groups' sums
// are then added in a fixed order: four per thread into QN slices, then the
// QN slices (deterministic, no atomics).
template <int PD, int QN, int R>
__global__ __launch_bounds__(kAttnThreads) void attn_merge_kernel(const float* part_lse_, const void* part_,
                                                                  uint16_t* out_, float* lse_, uint32_t shm_) {
  // Scalar arguments, all preloaded into SGPRs with the wave.
  AttnArgs a{};
  a.part_lse = const_cast<float*>(part_lse_);
  a.part = const_cast<void*>(part_);
  a.out = out_;
  a.lse = lse_;
  unpack_shm(shm_, &a.S, &a.H, &a.M);
  constexpr int kCols = kLatent / QN;         // columns per workgroup
  constexpr int CG = kCols / 8;               // column groups (8 columns each)
  constexpr int RG = kAttnThreads / CG;       // range groups (4 QN)
  constexpr int kPairs = kCols / 2;           // column pairs
  constexpr int KS = kAttnThreads / kPairs;   // slices of the range groups (QN)
  constexpr int RPS = RG / KS;                // range groups per slice (4)
  static_assert(RG == 4 * QN && KS == QN && RPS == 4, "merge shape");
  static_assert(R >= 1 && R <= kMergeMaxR, "ranges per thread");
  constexpr int kLv = (RG * R + 63) / 64; // lse values per lane (S <= RG R)
  static_assert(kAttnMaxSplits <= 4 * 16 * kMergeMaxR, "every split count has a shape");
  __shared__ float wts[4][kAttnMaxSplits];    // each wave's copy of the weights
  __shared__ __attribute__((aligned(16))) float part_sum[RG][kCols];
  __shared__ __attribute__((aligned(8))) float slice_sum[KS][kCols];
  const int H = a.H, S = a.S;
  const int bx = xcd_local_block(a.M * a.H * QN);
  const int mh = bx / QN, part = bx - (bx / QN) * QN;
  const int m = mh / H, h = mh - (mh / H) * H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;
  const int c = kCols * part + 8 * cg;
  const size_t stride = size_t(H) * kLatent; // elements between consecutive ranges
  const size_t base = (size_t(m) * S * H + h) * kLatent + c;

  // 1. lse values (lane l holds s = l + 64i), then this thread's ranges, all
  //    requested before any wait (the loads take no branch: an index past
  //    S re-reads range S-1 and is replaced by -inf once loaded).
  const float* pl = a.part_lse + size_t(m) * S * H + h;
  float lv[kLv];
#pragma unroll
  for (int i = 0; i < kLv; ++i) {
    const int s = lane + 64 * i;
    lv[i] = pl[size_t(s < S ? s : S - 1) * H];
  }
  // Raw partials (8 bf16 in 16 bytes, or 8 fp32 in 32). A slot past this
  // thread's last range re-reads range S-1 (a line other threads read
  // anyway) and is never added.
  typedef u32x4_t raw_t[PD == kPartialFp32 ? 2 : 1];
  raw_t v[R];
  auto load_range = [&](int s, raw_t& dst) {
    const size_t off = base + size_t(s < S ? s : S - 1) * stride;
    if constexpr (PD == kPartialFp32) {
      dst[0] = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(a.part) + off);
      dst[1] = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(a.part) + off + 4);
    } else {
      dst[0] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.part) + off);
    }
  };
  const int nr = rg < S ? (S - rg + RG - 1) / RG : 0; // this thread's ranges
#pragma unroll
  for (int u = 0; u < R; ++u) load_range(rg + RG * u, v[u]);

  // 2. L and the weights, per wave.
#pragma unroll
  for (int i = 0; i < kLv; ++i)
    if (lane + 64 * i >= S) lv[i] = -INFINITY;
  float L = lv[0];
#pragma unroll
  for (int i = 1; i < kLv; ++i) L = __builtin_fmaxf(L, lv[i]);
  L = wave_max(L);
  uint16_t* orow = a.out + (size_t(m) * H + h) * kLatent;
  // (L = -inf: no tokens at all; every weight is 0 and so is the output.)
  float wsum = 0.f;
#pragma unroll
  for (int i = 0; i < kLv; ++i) {
    const int s = lane + 64 * i;
    const float wt = lv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lv[i] - L) * kLog2e);
    if (s < S) wts[w][s] = wt;
    wsum += wt;
  }
  wsum = wave_sum(wsum);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 3. Weighted sum of this thread's ranges, in order of s.
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // A range without tokens (weight 0) holds no partial: its bytes are not
  // used. The products are selected rather than branched over, so the loads
  // above stay ahead of every wait.
  auto add = [&](int u, const raw_t& x) {
    const float wt = u < nr ? wts[w][rg + RG * (u < nr ? u : 0)] : 0.f;
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (PD == kPartialFp32) {
        f[i] = __uint_as_float(x[0][i]);
        f[4 + i] = __uint_as_float(x[1][i]);
      } else {
        f[2 * i] = __uint_as_float(x[0][i] << 16);
        f[2 * i + 1] = __uint_as_float(x[0][i] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] += wt != 0.f ? wt * f[i] : 0.f;
  };
#pragma unroll
  for (int u = 0; u < R; ++u) add(u, v[u]);

  // 4. The range groups' sums: RPS consecutive groups per slice, then the
  //    slices, each in order.
#pragma unroll
  for (int i = 0; i < 8; i += 4)
    *reinterpret_cast<f32x4_t*>(&part_sum[rg][8 * cg + i]) = f32x4_t{o[i], o[i + 1], o[i + 2], o[i + 3]};
  __syncthreads();
  const int pr = tid % kPairs, ks = tid / kPairs;
  float x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int k = 0; k < RPS; ++k) {
    x0 += part_sum[RPS * ks + k][2 * pr];
    x1 += part_sum[RPS * ks + k][2 * pr + 1];
  }
  if constexpr (KS > 1) {
    slice_sum[ks][2 * pr] = x0;
    slice_sum[ks][2 * pr + 1] = x1;
    __syncthreads();
    if (tid >= kPairs) return;
    x0 = 0.f;
    x1 = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      x0 += slice_sum[k][2 * pr];
      x1 += slice_sum[k][2 * pr + 1];
    }
  }
  const bool any = wsum > 0.f;
  *reinterpret_cast<uint32_t*>(orow + kCols * part + 2 * pr) =
      bf16x2_rne(any ? x0 / wsum : 0.f, any ? x1 / wsum : 0.f);
  if (a.lse && part == 0 && tid == 0) a.lse[size_t(m) * H + h] = any ? L + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
}

} // namespace

const void* attn_split_kernel_for(int partial_dtype, bool direct) {
  if (direct) return reinterpret_cast<const void*>(&attn_split_kernel<kDirect>);
  if (partial_dtype == MLAQ_PARTIAL_FP32) return reinterpret_cast<const void*>(&attn_split_kernel<kPartialFp32>);
  if (partial_dtype == MLAQ_PARTIAL_BF16) return reinterpret_cast<const void*>(&attn_split_kernel<kPartialBf16>);
  return nullptr;
}

// Merge shape for M rows of H heads and S ranges: QN column parts (RG =
// 4 QN range groups) and R ranges per thread. QN is the smallest power of two
// with 4 QN kMergeMaxR >= S, doubled while M H QN workgroups would leave
// compute units idle (at most 16); R is the smallest power of two covering
// the ranges of a thread.
void attn_merge_shape(int M, int H, int S, int* parts, int* per_thread) {
  int qn = 1;
  while (qn < 16 && 4 * qn * kMergeMaxR < S) qn *= 2;
  while (qn < 16 && (long long)M * H * qn < 256) qn *= 2;
  int r = 1;
  while (r < kMergeMaxR && 4 * qn * r < S) r *= 2;
  *parts = qn;
  *per_thread = r;
}

template <int PD, int QN>
const void* merge_kernel_r(int r) {
  switch (r) {
  case 1: return reinterpret_cast<const void*>(&attn_merge_kernel<PD, QN, 1>);
  case 2: return reinterpret_cast<const void*>(&attn_merge_kernel<PD, QN, 2>);
  case 4: return reinterpret_cast<const void*>(&attn_merge_kernel<PD, QN, 4>);
  case 8: return reinterpret_cast<const void*>(&attn_merge_kernel<PD, QN, 8>);
  default: return nullptr;
  }
}

template <int PD>
const void* merge_kernel(int parts, int r) {
  switch (parts) {
  case 1: return merge_kernel_r<PD, 1>(r);
  case 2: return merge_kernel_r<PD, 2>(r);
  case 4: return merge_kernel_r<PD, 4>(r);
  case 8: return merge_kernel_r<PD, 8>(r);
  case 16: return merge_kernel_r<PD, 16>(r);
  default: return nullptr;
  }
}

const void* attn_merge_kernel_for(int partial_dtype, int parts, int per_thread) {
  if (partial_dtype == MLAQ_PARTIAL_FP32) return merge_kernel<kPartialFp32>(parts, per_thread);
  if (partial_dtype == MLAQ_PARTIAL_BF16) return merge_kernel<kPartialBf16>(parts, per_thread);
  return nullptr;
}

void attn_launch_shapes(int M, int H, int S, dim3* split_grid, dim3* merge_grid, dim3* block) {
  *split_grid = dim3(unsigned(M) * unsigned(S), 1, 1);
  int parts = 1, r = 1;
  attn_merge_shape(M, H, S, &parts, &r);
  *merge_grid = dim3(unsigned(M) * unsigned(H) * unsigned(parts), 1, 1);
  *block = dim3(kAttnThreads, 1, 1);
}

} // namespace mlaq
