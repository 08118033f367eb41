/*
 * mlaq_oracle.c -- plain, slow, CPU oracle for the fused MLA decode query
 * projection and assembly, and for the two steps around it that the pages
 * name: the V up-projection after attention and dense MLA decode attention
 * with split partials (each in its own section below).
 *
 * TEST INFRASTRUCTURE ONLY. The product library never links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or helper with the HIP
 * path: every codec below is written here from the OCP "8-bit Floating Point
 * Specification (OFP8)" and "Microscaling Formats (MX) v1.0" definitions.
 *
 * What is computed, per decode token m < M and local head h < H:
 *
 *   acc[m,h,n]    = sum over k = 0..K-1 (ascending) of q_nope[m,h,k] * W[h,k,n]
 *                   accumulated in fp32, each product formed exactly
 *   y[m,h,n]      = bf16 round-to-nearest-even of acc
 *   out[m,h,n]    = y                               BF16 output
 *                 = e4m3_satfinite(fp32(y) / q_scale)  E4M3 output
 *   out[m,h,N+r]  = q_pe[m,h,r]                     BF16 output (bit copy)
 *                 = e4m3_satfinite(fp32(q_pe) / q_scale)  E4M3 output
 *
 * Sources (page title, then section):
 *  - sparkinfer PR #75 "[GG] Add BF16 MLA query projection and assembly",
 *    section "What": the per-head product q_nope x W_UK_T into a [M,H,576]
 *    buffer with the 64-wide RoPE part appended in the same launch.
 *  - same page, section "Contract": fp32 accumulation, rounding of the
 *    512-wide projection to BF16 before any E4M3 conversion; E4M3 output takes
 *    a q_scale, BF16 output takes none; K order may differ between
 *    implementations, so the BF16 projection is not a bitwise contract.
 *  - same page, review thread on api.py: the MXFP8 weight is N-major with its
 *    scale factors along n (b_major "n", sf_axis "n"), batched over heads.
 *  - vLLM PR #174 "[GG] Fuse MXFP8 and BF16 MLA query assembly", section
 *    "What": native MXFP8 and materialized BF16 W_UK_T; the epilogue writes
 *    [M,H,576] directly and appends q_pe; E4M3 output passes the query scale.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - the MXFP8 scale is one E8M0 byte per 32 contiguous n of each k row,
 *    stored row-major as [H,K,N/32];
 *  - "q / q_scale" is an IEEE fp32 division, correctly rounded;
 *  - E4M3 is OCP E4M3FN (max 448, no infinities), conversion rounds to
 *    nearest-even and saturates every finite or infinite overflow to +-448;
 *    NaN maps to 0x7F with the sign kept;
 *  - q_pe is quantized with the same per-tensor q_scale in E4M3 output.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fPIC -shared
 * -pthread (no FMA contraction, so every fp32 add rounds once).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_WEIGHT_BF16 0
#define ORACLE_WEIGHT_MXFP8 1
#define ORACLE_OUT_BF16 0
#define ORACLE_OUT_E4M3 1
#define ORACLE_MX_BLOCK 32 /* MX block size along n (OCP MX v1.0) */

/* ------------------------------------------------------------------------ */
/* Codecs                                                                   */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t bits_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* bf16 is the upper 16 bits of an IEEE binary32 pattern. */
static float bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* fp32 -> bf16, round to nearest, ties to even, written as the definition:
 * take the two bf16 values that bracket x, return the nearer one, and on a
 * tie the one whose last significand bit is 0. Past the largest finite bf16
 * the upper neighbour is 2^128 (infinity), as in IEEE overflow rounding.
 * NaN stays NaN (quiet, sign kept). */
static uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = bits_from_f32(x);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
  uint16_t lo = (uint16_t)(u >> 16); /* neighbour toward zero */
  if ((u & 0xFFFFu) == 0) return lo; /* x is exactly a bf16 */
  uint16_t hi = (uint16_t)(lo + 1);  /* neighbour away from zero */
  double ax = fabs((double)x);
  double alo = fabs((double)bf16_to_f32(lo));
  double ahi = ((hi & 0x7FFFu) == 0x7F80u) ? ldexp(1.0, 128) : fabs((double)bf16_to_f32(hi));
  double dlo = ax - alo, dhi = ahi - ax;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1u) ? hi : lo;
}

/* OCP E4M3FN decode: 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is
 * no infinity. */
static double e4m3_to_f64(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9); /* (m/8) * 2^(1-7) */
  else
    mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -mag : mag;
}

/* OCP MX E8M0 scale: 2^(b-127); 0xFF is NaN. */
static double e8m0_to_f64(uint8_t b) { return b == 0xFF ? NAN : ldexp(1.0, (int)b - 127); }

/* Magnitudes of the 127 non-negative finite E4M3 codes 0x00..0x7E, filled
 * from e4m3_to_f64 once. */
static double g_e4m3_mag[0x7F];
static pthread_once_t g_e4m3_once = PTHREAD_ONCE_INIT;
static void e4m3_table_init(void) {
  for (int c = 0; c < 0x7F; ++c) g_e4m3_mag[c] = e4m3_to_f64((uint8_t)c);
}

/* fp32 -> E4M3FN, round to nearest, ties to the even code, saturating:
 * the result is the finite E4M3 value nearest to x (so everything past 448,
 * infinity included, lands on 448). Written as a search over all finite
 * codes. NaN -> 0x7F with the sign bit of x. */
static uint8_t f32_to_e4m3_satfinite(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(0x7F | sign);
  if (isinf(x)) return (uint8_t)(0x7E | sign);
  pthread_once(&g_e4m3_once, e4m3_table_init);
  double a = fabs((double)x);
  int best = 0;
  double bestd = a; /* distance to code 0 (+0.0) */
  for (int c = 1; c < 0x7F; ++c) {
    double d = fabs(a - g_e4m3_mag[c]);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)(best | sign);
}

/* ------------------------------------------------------------------------ */
/* The projection                                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  const uint16_t* q_nope; /* bf16 [M,H,K] */
  const uint16_t* q_pe;   /* bf16 [M,H,R] */
  const void* w;          /* bf16 [H,K,N] or e4m3 [H,K,N] */
  const uint8_t* w_scales; /* e8m0 [H,K,N/32] (MXFP8 only) */
  float q_scale;
  void* out; /* bf16 or e4m3 [M,H,N+R] */
  int M, H, K, N, R, weight_format, out_dtype;
  float* acc_out;    /* optional fp32 [M,H,N] */
  double* sabs_out;  /* optional fp64 [M,H,N]: sum |q*w| */
  double* ref64_out; /* optional fp64 [M,H,N]: sum q*w in double */
  int next_head;     /* work counter (heads), under the lock */
  pthread_mutex_t lock;
  int status;
} oracle_job;

/* Dequantized weight of head h, element (k,n), as an exact double. */
static double weight_at(const oracle_job* j, int h, int k, int n) {
  size_t idx = ((size_t)h * j->K + k) * j->N + n;
  if (j->weight_format == ORACLE_WEIGHT_BF16)
    return (double)bf16_to_f32(((const uint16_t*)j->w)[idx]);
  {
    uint8_t p = ((const uint8_t*)j->w)[idx];
    uint8_t s = j->w_scales[((size_t)h * j->K + k) * (j->N / ORACLE_MX_BLOCK) + n / ORACLE_MX_BLOCK];
    return e4m3_to_f64(p) * e8m0_to_f64(s);
  }
}

/* Output conversion of one fp32 value (already bf16-valued for the
 * projection) for E4M3 output. */
static uint8_t to_e4m3_out(float v, float q_scale) { return f32_to_e4m3_satfinite(v / q_scale); }

static void run_head(oracle_job* j, int h, double* wdq) {
  const int K = j->K, N = j->N, R = j->R, H = j->H, OW = N + R;
  /* Step 1: dequantize this head's weight slab W[h] (exact in double). */
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n) wdq[(size_t)k * N + n] = weight_at(j, h, k, n);

  for (int m = 0; m < j->M; ++m) {
    const uint16_t* q = j->q_nope + ((size_t)m * H + h) * K;
    const uint16_t* pe = j->q_pe + ((size_t)m * H + h) * R;
    size_t orow = ((size_t)m * H + h) * OW;
    size_t arow = ((size_t)m * H + h) * N;
    /* Step 2: contract over k in ascending order, fp32 accumulator. */
    for (int n = 0; n < N; ++n) {
      float acc = 0.0f;
      double sabs = 0.0, ref = 0.0;
      for (int k = 0; k < K; ++k) {
        double p = (double)bf16_to_f32(q[k]) * wdq[(size_t)k * N + n]; /* exact */
        acc = acc + (float)p;
        sabs += fabs(p);
        ref += p;
      }
      if (j->acc_out) j->acc_out[arow + n] = acc;
      if (j->sabs_out) j->sabs_out[arow + n] = sabs;
      if (j->ref64_out) j->ref64_out[arow + n] = ref;
      /* Step 3: round the projection to bf16. */
      uint16_t y = f32_to_bf16_rne(acc);
      /* Step 4: write it, converting for E4M3 output. */
      if (j->out_dtype == ORACLE_OUT_BF16)
        ((uint16_t*)j->out)[orow + n] = y;
      else
        ((uint8_t*)j->out)[orow + n] = to_e4m3_out(bf16_to_f32(y), j->q_scale);
    }
    /* Step 5: append q_pe after the projection in the same row. */
    for (int r = 0; r < R; ++r) {
      if (j->out_dtype == ORACLE_OUT_BF16)
        ((uint16_t*)j->out)[orow + N + r] = pe[r];
      else
        ((uint8_t*)j->out)[orow + N + r] = to_e4m3_out(bf16_to_f32(pe[r]), j->q_scale);
    }
  }
}

static void* worker(void* arg) {
  oracle_job* j = (oracle_job*)arg;
  double* wdq = (double*)malloc(sizeof(double) * (size_t)j->K * j->N);
  if (!wdq) {
    pthread_mutex_lock(&j->lock);
    j->status = 3;
    pthread_mutex_unlock(&j->lock);
    return NULL;
  }
  for (;;) {
    pthread_mutex_lock(&j->lock);
    int h = j->next_head++;
    pthread_mutex_unlock(&j->lock);
    if (h >= j->H) break;
    run_head(j, h, wdq);
  }
  free(wdq);
  return NULL;
}

/*
 * Full fused call. Returns 0 on success, 1 on bad sizes or formats, 2 on
 * missing buffers, 3 on host allocation failure. Heads are independent, so
 * the work is split over `nthreads` threads by head; results do not depend
 * on the thread count.
 */
int mlaq_oracle_run(const uint16_t* q_nope, const uint16_t* q_pe, const void* w,
                    const uint8_t* w_scales, float q_scale, void* out, int M, int H, int K,
                    int N, int R, int weight_format, int out_dtype, float* acc_out,
                    double* sabs_out, double* ref64_out, int nthreads) {
  oracle_job j;
  if (M < 0 || H < 0 || K < 1 || N < ORACLE_MX_BLOCK || N % ORACLE_MX_BLOCK || R < 0) return 1;
  if (weight_format != ORACLE_WEIGHT_BF16 && weight_format != ORACLE_WEIGHT_MXFP8) return 1;
  if (out_dtype != ORACLE_OUT_BF16 && out_dtype != ORACLE_OUT_E4M3) return 1;
  if (M == 0 || H == 0) return 0;
  if (!q_nope || !w || !out || (R > 0 && !q_pe)) return 2;
  if (weight_format == ORACLE_WEIGHT_MXFP8 && !w_scales) return 2;
  memset(&j, 0, sizeof j);
  j.q_nope = q_nope;
  j.q_pe = q_pe;
  j.w = w;
  j.w_scales = w_scales;
  j.q_scale = q_scale;
  j.out = out;
  j.M = M;
  j.H = H;
  j.K = K;
  j.N = N;
  j.R = R;
  j.weight_format = weight_format;
  j.out_dtype = out_dtype;
  j.acc_out = acc_out;
  j.sabs_out = sabs_out;
  j.ref64_out = ref64_out;
  pthread_mutex_init(&j.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > H) nthreads = H;
  if (nthreads == 1) {
    worker(&j);
  } else {
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    if (!tids) {
      pthread_mutex_destroy(&j.lock);
      return 3;
    }
    for (int t = 0; t < nthreads; ++t)
      if (pthread_create(&tids[t], NULL, worker, &j) == 0) ++started;
    if (started == 0) worker(&j);
    for (int t = 0; t < started; ++t) pthread_join(tids[t], NULL);
    free(tids);
  }
  pthread_mutex_destroy(&j.lock);
  return j.status;
}

/*
 * Per-tensor query scale for E4M3 output: amax / 448 over the layer's fp32
 * result (the projection accumulators before bf16 rounding, and q_pe read as
 * fp32); 1 when amax is 0. 448 is the largest finite E4M3FN value.
 */
float mlaq_oracle_qscale(const float* acc, size_t n_acc, const uint16_t* q_pe, size_t n_pe) {
  float amax = 0.0f;
  for (size_t i = 0; i < n_acc; ++i) {
    float a = fabsf(acc[i]);
    if (a > amax) amax = a;
  }
  for (size_t i = 0; i < n_pe; ++i) {
    float a = fabsf(bf16_to_f32(q_pe[i]));
    if (a > amax) amax = a;
  }
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

/* Element-wise codec entry points, for pinning the codecs in tests. */
void mlaq_oracle_bf16_round(const float* in, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
void mlaq_oracle_e4m3_encode(const float* in, uint8_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = f32_to_e4m3_satfinite(in[i]);
}
void mlaq_oracle_e4m3_decode(const uint8_t* in, double* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = e4m3_to_f64(in[i]);
}
void mlaq_oracle_e8m0_decode(const uint8_t* in, double* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = e8m0_to_f64(in[i]);
}

/* ------------------------------------------------------------------------ */
/* V up-projection (the step after MLA decode attention)                    */
/* ------------------------------------------------------------------------ */

/*
 * For every token m < M, head h < H and value column v < V:
 *
 *   acc[m,h,v] = sum over c = 0..C-1 (ascending) of x[m,h,c] * W_UV[h,v,c]
 *                accumulated in fp32, each product formed exactly
 *   out[m,h,v] = bf16 round-to-nearest-even of acc
 *
 * x is the attention output in the latent space, bf16 [M,H,C]; W_UV is stored
 * as the checkpoint holds it, one row of C latent values per value column,
 * bf16 or E4M3 [H,V,C], with MXFP8 scales along the latent (reduction) axis,
 * one E8M0 byte per 32 contiguous c of each row: [H,V,C/32]. (The pages name
 * this projection -- vLLM PR #174 "[GG] Fuse MXFP8 and BF16 MLA query
 * assembly", "Layout and topology behavior" and "Safety scope and PR 173" --
 * without its shapes; C = 512 latent and V = 128 value dims are the readings.)
 * Same codecs and accumulation as the query projection above. Returns 0, or 1
 * on bad sizes/formats, 2 on missing buffers, 3 on host allocation failure.
 */
int mlaq_oracle_uv_run(const uint16_t* x, const void* w, const uint8_t* w_scales, uint16_t* out, int M, int H,
                       int C, int V, int weight_format, float* acc_out, double* sabs_out) {
  if (M < 0 || H < 0 || C < ORACLE_MX_BLOCK || C % ORACLE_MX_BLOCK || V < 1) return 1;
  if (weight_format != ORACLE_WEIGHT_BF16 && weight_format != ORACLE_WEIGHT_MXFP8) return 1;
  if (M == 0 || H == 0) return 0;
  if (!x || !w || !out || (weight_format == ORACLE_WEIGHT_MXFP8 && !w_scales)) return 2;
  double* wdq = (double*)malloc(sizeof(double) * (size_t)V * C);
  if (!wdq) return 3;
  for (int h = 0; h < H; ++h) {
    /* Step 1: dequantize this head's W_UV[h] (exact in double). */
    for (int v = 0; v < V; ++v)
      for (int c = 0; c < C; ++c) {
        size_t idx = ((size_t)h * V + v) * C + c;
        if (weight_format == ORACLE_WEIGHT_BF16) {
          wdq[(size_t)v * C + c] = (double)bf16_to_f32(((const uint16_t*)w)[idx]);
        } else {
          uint8_t p = ((const uint8_t*)w)[idx];
          uint8_t s = w_scales[((size_t)h * V + v) * (C / ORACLE_MX_BLOCK) + c / ORACLE_MX_BLOCK];
          wdq[(size_t)v * C + c] = e4m3_to_f64(p) * e8m0_to_f64(s);
        }
      }
    /* Step 2: contract over c in ascending order (fp32), step 3: round. */
    for (int m = 0; m < M; ++m) {
      const uint16_t* xr = x + ((size_t)m * H + h) * C;
      for (int v = 0; v < V; ++v) {
        float acc = 0.0f;
        double sabs = 0.0;
        for (int c = 0; c < C; ++c) {
          double p = (double)bf16_to_f32(xr[c]) * wdq[(size_t)v * C + c];
          acc = acc + (float)p;
          sabs += fabs(p);
        }
        size_t o = ((size_t)m * H + h) * V + v;
        if (acc_out) acc_out[o] = acc;
        if (sabs_out) sabs_out[o] = sabs;
        out[o] = f32_to_bf16_rne(acc);
      }
    }
  }
  free(wdq);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dense MLA decode attention with split partials (the query's consumer)    */
/* ------------------------------------------------------------------------ */

/*
 * Each of the M decode tokens m belongs to its own sequence, whose T_m =
 * seq_lens[m] cached tokens live in a paged latent cache: token t of sequence
 * m is row (t mod P) of physical page block_table[m][t / P], and a row holds
 * the D = 576 values "512 latent, then 64 rotary" -- the same split as the
 * query row. Attention runs in the latent space (keys are the whole row,
 * values its first DV = 512 entries), per head h:
 *
 *   s_t  = softmax_scale * sum_{d<D} q[m,h,d] * kv_t[d]
 *   o    = sum_{t<T} exp(s_t - L) kv_t[0:DV] / sum_{t<T} exp(s_t - L)
 *   lse  = L + log sum_{t<T} exp(s_t - L),      L = max_t s_t
 *
 * Split procedure (b12x PR #441 "Allow FP32 split partials in prepared dense
 * MLA": commit text, walkthrough and "Behavior"): the T tokens are cut into S
 * contiguous ranges; range s yields its own normalized output o_s and lse_s;
 * o_s is stored as FP32 or as BF16 (the default) and lse_s as fp32; a merge
 * then forms
 *
 *   L' = max_s lse_s,  w_s = exp(lse_s - L'),
 *   o  = sum_s w_s o_s / sum_s w_s,  lse = L' + log sum_s w_s,
 *
 * and the output is BF16 in every case. Readings where the page is silent
 * (each is listed in the design notes):
 *  - range boundaries: chunk = ceil(T / S) rounded up to a multiple of 64
 *    tokens, range s = [s*chunk, min(T, (s+1)*chunk)); an empty range has
 *    lse_s = -inf and takes no part in the merge;
 *  - T = 0 gives o = 0 and lse = -inf;
 *  - "stored as BF16/FP32" is round-to-nearest-even of the range's exact
 *    normalized output; lse_s is stored as fp32 in both cases.
 * Everything else is evaluated in double (bf16 inputs make each product
 * exact; exp and log are the C library's).
 */

#define ORACLE_PARTIAL_BF16 0
#define ORACLE_PARTIAL_FP32 1
#define ORACLE_PARTIAL_EXACT 2 /* keep partials and lse_s in double (for checks) */
#define ORACLE_SPLIT_ALIGN 64

/* double -> bf16, round to nearest, ties to even, from the definition: bf16
 * keeps 8 significant bits, so in the binade [2^(e-1), 2^e) its values are
 * the multiples of 2^(e-8) (never finer than 2^-133, the subnormal spacing);
 * take the two multiples that bracket |x|, keep the nearer, on a tie the even
 * multiple. Results past the largest finite bf16 become infinity. */
static uint16_t f64_to_bf16_rne(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
  double a = fabs(x);
  double r;
  if (a == 0.0 || isinf(a)) {
    r = a;
  } else {
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    int se = e - 8;
    if (se < -133) se = -133;
    double step = ldexp(1.0, se);
    double lo = floor(a / step); /* exact: a / step only shifts the exponent */
    double dlo = a - lo * step, dhi = (lo + 1.0) * step - a;
    if (dlo < dhi)
      r = lo * step;
    else if (dhi < dlo)
      r = (lo + 1.0) * step;
    else
      r = fmod(lo, 2.0) == 0.0 ? lo * step : (lo + 1.0) * step;
    if (r > 3.3895313892515355e38) r = INFINITY; /* past (2 - 2^-7) * 2^127 */
  }
  uint16_t b = (uint16_t)(bits_from_f32((float)r) >> 16); /* r is a bf16 value: exact */
  return signbit(x) ? (uint16_t)(b | 0x8000u) : b;
}

typedef struct {
  const uint16_t* q;           /* bf16 [M,H,D] */
  const uint16_t* kv;          /* bf16 [num_pages,P,D] */
  const int32_t* block_table;  /* [M, max_blocks] */
  const int32_t* seq_lens;     /* [M] */
  int M, H, D, DV, P, num_pages, max_blocks, num_splits, partial_dtype;
  double softmax_scale;
  uint16_t* out;      /* bf16 [M,H,DV] */
  double* o_out;      /* optional [M,H,DV]: merged o before the bf16 rounding */
  double* lse_out;    /* optional [M,H] */
  double* vabs_out;   /* optional [M,H,DV]: sum_t p_t |kv_t[d]| with exact p */
  double* smag_out;   /* optional [M,H]: max_t softmax_scale * sum_d |q_d kv_t[d]| */
  double* part_out;   /* optional [M,S,H,DV]: stored partials (after rounding) */
  double* plse_out;   /* optional [M,S,H]: stored lse_s (fp32 values) */
  double* pvabs_out;  /* optional [M,S,H,DV]: sum_t p_t |kv_t[d]| within each range */
  int next_item;      /* work counter over (m, h) pairs, under the lock */
  pthread_mutex_t lock;
} attn_job;

/* Pointer to the cached row of token t of sequence m. */
static const uint16_t* attn_row(const attn_job* j, int m, int t) {
  int page = j->block_table[(size_t)m * j->max_blocks + t / j->P];
  return j->kv + ((size_t)page * j->P + (size_t)(t % j->P)) * j->D;
}

/* Softmax over tokens [a, b) of one (m, h): normalized output into o[DV]
 * (and, if vabs is given, the same weights applied to |kv_t[d]|), returns
 * lse. Scores s[] are the precomputed s_t of the whole sequence. */
static double attn_range(const attn_job* j, int m, const double* s, int a, int b, double* o, double* vabs) {
  double L = -INFINITY, sum = 0.0;
  for (int t = a; t < b; ++t)
    if (s[t] > L) L = s[t];
  for (int d = 0; d < j->DV; ++d) o[d] = 0.0;
  if (vabs)
    for (int d = 0; d < j->DV; ++d) vabs[d] = 0.0;
  for (int t = a; t < b; ++t) {
    double e = exp(s[t] - L);
    const uint16_t* row = attn_row(j, m, t);
    sum += e;
    for (int d = 0; d < j->DV; ++d) o[d] += e * (double)bf16_to_f32(row[d]);
    if (vabs)
      for (int d = 0; d < j->DV; ++d) vabs[d] += e * fabs((double)bf16_to_f32(row[d]));
  }
  for (int d = 0; d < j->DV; ++d) o[d] /= sum;
  if (vabs)
    for (int d = 0; d < j->DV; ++d) vabs[d] /= sum;
  return L + log(sum);
}

static void attn_head(attn_job* j, int m, int h, double* s, double* o, double* ps) {
  const int H = j->H, D = j->D, DV = j->DV, T = j->seq_lens[m];
  const int S = j->num_splits;
  {
    const uint16_t* qr = j->q + ((size_t)m * H + h) * D;
    const size_t orow = ((size_t)m * H + h) * DV;
    double smag = 0.0;
    /* Step 1: scores s_t = scale * q . kv_t over all D dims. */
    for (int t = 0; t < T; ++t) {
      const uint16_t* row = attn_row(j, m, t);
      double acc = 0.0, mag = 0.0;
      for (int d = 0; d < D; ++d) {
        double p = (double)bf16_to_f32(qr[d]) * (double)bf16_to_f32(row[d]); /* exact */
        acc += p;
        mag += fabs(p);
      }
      s[t] = j->softmax_scale * acc;
      if (j->softmax_scale * mag > smag) smag = j->softmax_scale * mag;
    }
    if (j->smag_out) j->smag_out[(size_t)m * H + h] = smag;
    /* Bound helper: sum_t p_t |v_t| with the exact (unsplit) weights. */
    if (j->vabs_out) {
      double L = -INFINITY, sum = 0.0;
      for (int t = 0; t < T; ++t)
        if (s[t] > L) L = s[t];
      for (int d = 0; d < DV; ++d) j->vabs_out[orow + d] = 0.0;
      for (int t = 0; t < T; ++t) {
        double e = exp(s[t] - L);
        const uint16_t* row = attn_row(j, m, t);
        sum += e;
        for (int d = 0; d < DV; ++d) j->vabs_out[orow + d] += e * fabs((double)bf16_to_f32(row[d]));
      }
      for (int d = 0; d < DV; ++d) j->vabs_out[orow + d] = T > 0 ? j->vabs_out[orow + d] / sum : 0.0;
    }
    double lse;
    if (T == 0) {
      /* Step 2 for an empty sequence: nothing to attend to. */
      for (int d = 0; d < DV; ++d) o[d] = 0.0;
      lse = -INFINITY;
      for (int sp = 0; sp < S; ++sp) {
        if (j->plse_out) j->plse_out[((size_t)m * S + sp) * H + h] = -INFINITY;
        if (j->part_out)
          for (int d = 0; d < DV; ++d) j->part_out[(((size_t)m * S + sp) * H + h) * DV + d] = 0.0;
      }
    } else if (S == 0) {
      /* Step 2 without splitting: the definition itself. */
      lse = attn_range(j, m, s, 0, T, o, NULL);
    } else {
      /* Step 2: one normalized partial per range, stored in its dtype. */
      int chunk = (T + S - 1) / S;
      chunk = (chunk + ORACLE_SPLIT_ALIGN - 1) / ORACLE_SPLIT_ALIGN * ORACLE_SPLIT_ALIGN;
      double Lp = -INFINITY;
      double* plse = ps + (size_t)S * DV; /* S lse values after the S partial rows */
      for (int sp = 0; sp < S; ++sp) {
        double* po = ps + (size_t)sp * DV;
        long a = (long)sp * chunk, b = a + chunk < T ? a + chunk : T;
        if (a >= b) {
          plse[sp] = -INFINITY;
          for (int d = 0; d < DV; ++d) po[d] = 0.0;
        } else {
          double* pv = j->pvabs_out ? j->pvabs_out + (((size_t)m * S + sp) * H + h) * DV : NULL;
          plse[sp] = attn_range(j, m, s, (int)a, (int)b, po, pv);
          if (j->partial_dtype != ORACLE_PARTIAL_EXACT) plse[sp] = (double)(float)plse[sp];
          for (int d = 0; d < DV; ++d) {
            if (j->partial_dtype == ORACLE_PARTIAL_BF16)
              po[d] = (double)bf16_to_f32(f64_to_bf16_rne(po[d]));
            else if (j->partial_dtype == ORACLE_PARTIAL_FP32)
              po[d] = (double)(float)po[d];
          }
        }
        if (plse[sp] > Lp) Lp = plse[sp];
        if (j->plse_out) j->plse_out[((size_t)m * S + sp) * H + h] = plse[sp];
        if (j->part_out)
          for (int d = 0; d < DV; ++d) j->part_out[(((size_t)m * S + sp) * H + h) * DV + d] = po[d];
      }
      /* Step 3: merge the ranges that hold tokens. */
      double wsum = 0.0;
      for (int d = 0; d < DV; ++d) o[d] = 0.0;
      for (int sp = 0; sp < S; ++sp) {
        if (plse[sp] == -INFINITY) continue;
        double w = exp(plse[sp] - Lp);
        wsum += w;
        for (int d = 0; d < DV; ++d) o[d] += w * ps[(size_t)sp * DV + d];
      }
      for (int d = 0; d < DV; ++d) o[d] /= wsum;
      lse = Lp + log(wsum);
    }
    /* Step 4: BF16 output. */
    for (int d = 0; d < DV; ++d) {
      j->out[orow + d] = f64_to_bf16_rne(o[d]);
      if (j->o_out) j->o_out[orow + d] = o[d];
    }
    if (j->lse_out) j->lse_out[(size_t)m * H + h] = lse;
  }
}

static void* attn_worker(void* arg) {
  attn_job* j = (attn_job*)arg;
  int tmax = 0;
  for (int m = 0; m < j->M; ++m)
    if (j->seq_lens[m] > tmax) tmax = j->seq_lens[m];
  double* s = (double*)malloc(sizeof(double) * (size_t)(tmax > 0 ? tmax : 1));
  double* o = (double*)malloc(sizeof(double) * (size_t)j->DV);
  double* ps = (double*)malloc(sizeof(double) * ((size_t)j->num_splits * (j->DV + 1) + 1));
  if (s && o && ps)
    for (;;) {
      pthread_mutex_lock(&j->lock);
      int item = j->next_item++;
      pthread_mutex_unlock(&j->lock);
      if (item >= j->M * j->H) break;
      attn_head(j, item / j->H, item % j->H, s, o, ps);
    }
  int failed = !(s && o && ps);
  free(s);
  free(o);
  free(ps);
  return failed ? (void*)1 : NULL;
}

/*
 * Dense MLA decode attention over a paged latent cache. num_splits = 0
 * evaluates the definition directly; num_splits >= 1 runs the split procedure
 * with partials stored per partial_dtype (0 BF16, 1 FP32, 2 kept in double).
 * Returns 0, or 1 on bad sizes or modes, 2 on missing buffers, 3 on host
 * allocation failure, 4 on a block-table entry or sequence length outside the
 * cache. (Sequence, head) pairs are independent and split over `nthreads`
 * threads; results do not depend on the thread count.
 */
int mlaq_oracle_attn_run(const uint16_t* q, const uint16_t* kv, const int32_t* block_table,
                         const int32_t* seq_lens, int M, int H, int D, int DV, int P, int num_pages,
                         int max_blocks, double softmax_scale, int num_splits, int partial_dtype,
                         uint16_t* out, double* o_out, double* lse_out, double* vabs_out, double* smag_out,
                         double* part_out, double* plse_out, double* pvabs_out, int nthreads) {
  attn_job j;
  if (M < 0 || H < 0 || D < 1 || DV < 1 || DV > D || P < 1 || num_pages < 0 || max_blocks < 0) return 1;
  if (num_splits < 0 || partial_dtype < ORACLE_PARTIAL_BF16 || partial_dtype > ORACLE_PARTIAL_EXACT) return 1;
  if (M == 0 || H == 0) return 0;
  if (!q || !seq_lens || !out) return 2;
  for (int m = 0; m < M; ++m) {
    long T = seq_lens[m];
    if (T < 0 || T > (long)max_blocks * P) return 4;
    if (T > 0 && (!kv || !block_table)) return 2;
    for (long b = 0; b < (T + P - 1) / P; ++b) {
      int page = block_table[(size_t)m * max_blocks + b];
      if (page < 0 || page >= num_pages) return 4;
    }
  }
  memset(&j, 0, sizeof j);
  j.q = q;
  j.kv = kv;
  j.block_table = block_table;
  j.seq_lens = seq_lens;
  j.M = M;
  j.H = H;
  j.D = D;
  j.DV = DV;
  j.P = P;
  j.num_pages = num_pages;
  j.max_blocks = max_blocks;
  j.num_splits = num_splits;
  j.partial_dtype = partial_dtype;
  j.softmax_scale = softmax_scale;
  j.out = out;
  j.o_out = o_out;
  j.lse_out = lse_out;
  j.vabs_out = vabs_out;
  j.smag_out = smag_out;
  j.part_out = num_splits > 0 ? part_out : NULL;
  j.plse_out = num_splits > 0 ? plse_out : NULL;
  j.pvabs_out = num_splits > 0 ? pvabs_out : NULL;
  pthread_mutex_init(&j.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > M * H) nthreads = M * H;
  int status = 0;
  if (nthreads == 1) {
    if (attn_worker(&j)) status = 3;
  } else {
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    if (!tids) {
      pthread_mutex_destroy(&j.lock);
      return 3;
    }
    for (int t = 0; t < nthreads; ++t)
      if (pthread_create(&tids[t], NULL, attn_worker, &j) == 0) ++started;
    if (started == 0 && attn_worker(&j)) status = 3;
    for (int t = 0; t < started; ++t) {
      void* r = NULL;
      pthread_join(tids[t], &r);
      if (r) status = 3;
    }
    free(tids);
  }
  pthread_mutex_destroy(&j.lock);
  return status;
}

/* Element-wise entry point of the double -> bf16 rounding, for pinning it. */
void mlaq_oracle_bf16_round_f64(const double* in, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = f64_to_bf16_rne(in[i]);
}
