/*
 * kvq_oracle.c -- plain, slow CPU oracle for Jensen-bias-corrected low-bit
 * KV-cache attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library and must never be used as a
 * fallback for it.
 *
 * Sources (web pages on the method; cited by title and section):
 *  [S1] "量化鍵值偷走注意力：針對 KV-Cache 的 Jensen 偏差校正還原影片擴散品質"
 *       (agents-report.net summary of "Quantized Keys Steal Attention"),
 *       sections 問題 (problem), 方法 (method), 為何校正有效 (why it works),
 *       限制與邊界情況 (limitations).
 *  [S2] "Quantized Keys Steal Attention: Bias Correction for KV-Cache
 *       Compression in Video Diffusion" (fugumt.com abstract page), Abstract.
 *  [S3] "QuantWM：保住时间一致性的两比特键值缓存量化" (pchao.org review),
 *       section 研究缺口 (research gap), Eq. (5): logits are QK^T / sqrt(d).
 *  [S4] gist.science explainer of the TurboQuant-inspired KV/KQV study,
 *       section Metodologia / Estrutura Teórica: keys enter through the
 *       exponential, values enter linearly.
 *
 * What is computed (plain definitions, no blocking or fusion):
 *  - Q: group-wise asymmetric uniform quantizer, fp32, bit-exact contract.
 *  - b: the per-score Jensen bias of a cached key, Taylor or exact form.
 *  - attention: one softmax over [cached keys ; current keys] with b
 *    subtracted from cached logits only, in fp64, brute force.
 *  - an online (tiled, split, LSE-merged) evaluation of the same softmax,
 *    used only to check the online formulation against brute force;
 *  - attention-balance statistics of a row: the softmax over unquantised
 *    cached keys against the quantised one (log-sum-exps, current-chunk
 *    mass, KL divergence, top-5 keys).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *  - step  D = fl32(fl32(mx - mn) / (2^bits - 1)), zero-point z = mn (fp32);
 *    with 16-bit metadata (IEEE binary16 or bfloat16), D and z are rounded
 *    to that format (nearest, ties to even) and the codes below use the
 *    rounded D and z;
 *  - code  c = clamp(rne(fl32(fl32(x - mn) / D)), 0, 2^bits - 1), 0 if D == 0;
 *  - mn and mx are canonicalised with "+ 0.0f" so a zero extreme is +0;
 *  - packing is LSB-first: element k of a row sits in byte floor(k*bits/8)
 *    at bit (k*bits) mod 8; rows are contiguous along the head dimension and
 *    groups are consecutive runs of `group` elements of a row;
 *  - groups along the tokens instead (per channel, the grouping the pages
 *    name beside per-group steps): channel c of `group` consecutive tokens
 *    of one head shares D and z; the last group of a quantised run may be
 *    shorter; codes are packed per token row as above, and D, z are stored
 *    [token group][channel]; the bias then uses D_{g(t),c} per channel;
 *  - dequantised value  x^ = z + D * c  (fp64 here);
 *  - tau = 1/sqrt(d) unless a scale is given; the Taylor bias is
 *    (tau^2/24) * sum_g D_g^2 * sum_{c in g} q_c^2, which equals the page's
 *    (1/(24 d)) sum_c q_c^2 D_{i,c}^2 when tau = 1/sqrt(d);
 *  - the exact bias is sum_c log(sinh x_c / x_c), x_c = tau q_c D_{g(c)} / 2,
 *    the log-MGF of independent U(-D/2, D/2) key noise;
 *  - GQA: query head h reads KV head h / (Hq / Hkv);
 *  - by default no mask: every query sees every cached and current key
 *    (chunk-wise video generation); optionally a causal mask within the
 *    current chunk aligned to its end (query row j sees current keys
 *    i <= j + Ncur - Nq and the whole cache), for chunked prefill.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 * (no -ffast-math: the quantizer relies on IEEE fp32 division and rint).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Every float expression must round to fp32 at each step. */
#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the quantizer contract needs FLT_EVAL_METHOD == 0 (SSE fp32 arithmetic)"
#endif

#define KVO_OK 0
#define KVO_ERR_ARG 1
#define KVO_ERR_MEM 2

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_bits_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int kvo_bf16_to_f32(const uint16_t *in, int64_t n, float *out) {
  if (!in || !out || n < 0) return KVO_ERR_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_f32(in[i]);
  return KVO_OK;
}

/* ------------------------------------------------------------------ */
/* Q: group-wise asymmetric uniform quantizer                          */
/* [S1] 問題: keys/values are rounded to INT4/INT2 with near-zero-mean  */
/* rounding error; [S1] 方法: one step size per group (or channel).     */
/* ------------------------------------------------------------------ */

static int qparams_ok(int32_t d, int32_t group, int32_t bits) {
  if (bits != 2 && bits != 4) return 0;
  if (group <= 0 || d <= 0 || d % group != 0) return 0;
  if ((d * bits) % 8 != 0) return 0;
  return 1;
}

/* The binary16 value nearest to a finite fp32 x (round half to even),
 * returned as fp32 (exactly).  binary16: 10 fraction bits, normals from
 * 2^-14, subnormals spaced 2^-24, largest finite 65504; larger magnitudes
 * round to infinity (outside the quantizer's contract).  The spacing of
 * binary16 numbers in x's binade is a power of two u, so x/u is exact and
 * rint(x/u)*u is the rounded value. */
static float round_fp16(float x) {
  if (x == 0.0f || !isfinite(x)) return x;
  const float a = fabsf(x);
  int e;
  frexpf(a, &e);              /* a in [2^(e-1), 2^e) */
  int ue = (e - 1) - 10;      /* spacing in that binade */
  if (ue < -24) ue = -24;     /* subnormal spacing */
  const float u = ldexpf(1.0f, ue);
  const float r = rintf(a / u) * u;
  if (r > 65504.0f) return copysignf(INFINITY, x);
  return copysignf(r, x);
}

float kvo_round_fp16(float x) { return round_fp16(x); }

/* The bfloat16 value nearest to a finite fp32 x (round half to even),
 * returned as fp32 (exactly).  bfloat16 keeps fp32's exponent range with 7
 * fraction bits: normals from 2^-126 spaced 2^(e-8) in [2^(e-1), 2^e),
 * subnormals spaced 2^-133, largest finite (2 - 2^-7) 2^127; magnitudes
 * that round past it become infinity.  As for binary16, x/u is exact for
 * the spacing u of x's binade and rint(x/u) u is the rounded value (the
 * product overflows to infinity exactly when the rounded value does). */
static float round_bf16(float x) {
  if (x == 0.0f || !isfinite(x)) return x;
  const float a = fabsf(x);
  int e;
  frexpf(a, &e);              /* a in [2^(e-1), 2^e) */
  int ue = (e - 1) - 7;       /* spacing in that binade */
  if (ue < -133) ue = -133;   /* subnormal spacing */
  const float r = rintf(ldexpf(a, -ue));
  return copysignf(ldexpf(r, ue), x);
}

float kvo_round_bf16(float x) { return round_bf16(x); }

/* The stored value of a step or zero point: meta 0 fp32 (unchanged),
 * 1 binary16, 2 bfloat16. */
static float round_meta(float x, int32_t meta) {
  return meta == 1 ? round_fp16(x) : meta == 2 ? round_bf16(x) : x;
}

/* Quantize one group of `group` fp32 values.  codes_out gets one code per
 * element (unpacked).  The order of fp32 operations is the contract.
 * meta: the storage of the step and zero point (0 fp32, 1 binary16,
 * 2 bfloat16); with 16 bits they are rounded first and the codes are taken
 * against the rounded grid, so that the dequantised value z + D c uses
 * exactly what is stored. */
static void quantize_group(const float *x, int32_t group, int32_t bits, int32_t meta,
                           uint8_t *codes_out, float *step_out, float *zero_out) {
  const int32_t top = (1 << bits) - 1;
  float mn = x[0], mx = x[0];
  for (int32_t k = 1; k < group; ++k) {
    if (x[k] < mn) mn = x[k];
    if (x[k] > mx) mx = x[k];
  }
  mn = mn + 0.0f; /* canonical zero sign */
  mx = mx + 0.0f;
  float range = mx - mn;             /* fl32 subtraction */
  float step = range / (float)top;   /* fl32 IEEE division */
  float zero = mn;
  step = round_meta(step, meta);
  zero = round_meta(mn, meta);
  *step_out = step;
  *zero_out = zero;
  for (int32_t k = 0; k < group; ++k) {
    int32_t c = 0;
    if (step > 0.0f) {
      float num = x[k] - zero;         /* fl32 subtraction */
      float t = num / step;            /* fl32 IEEE division */
      float r = rintf(t);                      /* round half to even */
      if (r < 0.0f) r = 0.0f;
      if (r > (float)top) r = (float)top;
      c = (int32_t)r;
    }
    codes_out[k] = (uint8_t)c;
  }
}

/* Pack one row of d codes LSB-first into d*bits/8 bytes. */
static void pack_row(const uint8_t *c, int32_t d, int32_t bits, uint8_t *out) {
  memset(out, 0, (size_t)(d * bits / 8));
  for (int32_t k = 0; k < d; ++k) {
    int64_t bit = (int64_t)k * bits;
    out[bit / 8] |= (uint8_t)(c[k] << (bit % 8));
  }
}

/* Quantize `rows` rows of d fp32 values.  codes: rows x (d*bits/8) bytes;
 * step, zero: rows x (d/group) fp32 (holding the 16-bit values when meta is 1 or 2). */
int kvo_quantize_f32_meta(const float *x, int64_t rows, int32_t d, int32_t group,
                          int32_t bits, int32_t meta, uint8_t *codes, float *step, float *zero) {
  if (!x || !codes || !step || !zero || rows < 0 || (meta < 0 || meta > 2)) return KVO_ERR_ARG;
  if (!qparams_ok(d, group, bits)) return KVO_ERR_ARG;
  const int32_t ng = d / group;
  const int64_t row_bytes = d * bits / 8;
  int err = KVO_OK;
#pragma omp parallel
  {
    uint8_t *c = (uint8_t *)malloc((size_t)d);
    if (!c) {
#pragma omp atomic write
      err = KVO_ERR_MEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t r = 0; r < rows; ++r) {
        for (int32_t g = 0; g < ng; ++g)
          quantize_group(x + r * d + (int64_t)g * group, group, bits, meta, c + g * group,
                         step + r * ng + g, zero + r * ng + g);
        pack_row(c, d, bits, codes + r * row_bytes);
      }
      free(c);
    }
  }
  return err;
}

int kvo_quantize_f32(const float *x, int64_t rows, int32_t d, int32_t group,
                     int32_t bits, uint8_t *codes, float *step, float *zero) {
  return kvo_quantize_f32_meta(x, rows, d, group, bits, 0, codes, step, zero);
}

/* Same, for bf16 input (widened exactly to fp32 first). */
int kvo_quantize_bf16_meta(const uint16_t *x, int64_t rows, int32_t d, int32_t group,
                           int32_t bits, int32_t meta, uint8_t *codes, float *step, float *zero) {
  if (!x || rows < 0 || d <= 0) return KVO_ERR_ARG;
  float *f = (float *)malloc((size_t)(rows * d) * sizeof(float) + 1);
  if (!f) return KVO_ERR_MEM;
  kvo_bf16_to_f32(x, rows * d, f);
  int rc = kvo_quantize_f32_meta(f, rows, d, group, bits, meta, codes, step, zero);
  free(f);
  return rc;
}

/* Groups along the tokens: x is `outer` runs of n tokens of d fp32 values
 * ([outer][n][d], one run per (b, h)); within a run, channel c of tokens
 * [j*group, min(n, (j+1)*group)) is one group, quantised exactly like a
 * group of the head-dimension layout.  codes: [outer][n][d*bits/8] (token
 * rows, packed as above); step, zero: [outer][ceil(n/group)][d].  Any
 * group >= 1 is accepted here. */
int kvo_quantize_tokens_f32_meta(const float *x, int64_t outer, int64_t n, int32_t d, int32_t group,
                                 int32_t bits, int32_t meta, uint8_t *codes, float *step, float *zero) {
  if (!x || !codes || !step || !zero || outer < 0 || n < 0 || d <= 0 || group < 1) return KVO_ERR_ARG;
  if ((bits != 2 && bits != 4) || (d * bits) % 8 != 0 || (meta < 0 || meta > 2)) return KVO_ERR_ARG;
  const int64_t ngr = (n + group - 1) / group;
  const int64_t row_bytes = d * bits / 8;
  int err = KVO_OK;
#pragma omp parallel
  {
    float *vals = (float *)malloc(sizeof(float) * (size_t)group);
    uint8_t *gc = (uint8_t *)malloc((size_t)group);
    uint8_t *u = (uint8_t *)malloc((size_t)(n * d) + 1); /* unpacked codes of one run */
    if (!vals || !gc || !u) {
#pragma omp atomic write
      err = KVO_ERR_MEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t o = 0; o < outer; ++o) {
        const float *xo = x + o * n * d;
        for (int64_t j = 0; j < ngr; ++j) {
          const int64_t t0 = j * group;
          const int32_t cnt = (int32_t)(n - t0 < group ? n - t0 : group);
          for (int32_t c = 0; c < d; ++c) {
            for (int32_t i = 0; i < cnt; ++i) vals[i] = xo[(t0 + i) * d + c];
            quantize_group(vals, cnt, bits, meta, gc, step + (o * ngr + j) * d + c,
                           zero + (o * ngr + j) * d + c);
            for (int32_t i = 0; i < cnt; ++i) u[(t0 + i) * d + c] = gc[i];
          }
        }
        for (int64_t t = 0; t < n; ++t) pack_row(u + t * d, d, bits, codes + (o * n + t) * row_bytes);
      }
    }
    free(vals);
    free(gc);
    free(u);
  }
  return err;
}

int kvo_quantize_tokens_bf16_meta(const uint16_t *x, int64_t outer, int64_t n, int32_t d, int32_t group,
                                  int32_t bits, int32_t meta, uint8_t *codes, float *step, float *zero) {
  if (!x || outer < 0 || n < 0 || d <= 0) return KVO_ERR_ARG;
  float *f = (float *)malloc((size_t)(outer * n * d) * sizeof(float) + 1);
  if (!f) return KVO_ERR_MEM;
  kvo_bf16_to_f32(x, outer * n * d, f);
  int rc = kvo_quantize_tokens_f32_meta(f, outer, n, d, group, bits, meta, codes, step, zero);
  free(f);
  return rc;
}

int kvo_quantize_bf16(const uint16_t *x, int64_t rows, int32_t d, int32_t group,
                      int32_t bits, uint8_t *codes, float *step, float *zero) {
  return kvo_quantize_bf16_meta(x, rows, d, group, bits, 0, codes, step, zero);
}

/* Read code k of a packed row (LSB-first). */
static int32_t code_at(const uint8_t *row, int32_t k, int32_t bits) {
  int64_t bit = (int64_t)k * bits;
  return (row[bit / 8] >> (bit % 8)) & ((1 << bits) - 1);
}

int kvo_unpack(const uint8_t *codes, int64_t rows, int32_t d, int32_t bits, uint8_t *out) {
  if (!codes || !out || rows < 0 || (bits != 2 && bits != 4) || (d * bits) % 8) return KVO_ERR_ARG;
  const int64_t row_bytes = d * bits / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t k = 0; k < d; ++k) out[r * d + k] = (uint8_t)code_at(codes + r * row_bytes, k, bits);
  return KVO_OK;
}

int kvo_pack(const uint8_t *c, int64_t rows, int32_t d, int32_t bits, uint8_t *codes) {
  if (!codes || !c || rows < 0 || (bits != 2 && bits != 4) || (d * bits) % 8) return KVO_ERR_ARG;
  for (int64_t r = 0; r < rows; ++r) pack_row(c + r * d, d, bits, codes + r * (d * bits / 8));
  return KVO_OK;
}

/* x^ = z + D * c, in fp64. */
int kvo_dequant(const uint8_t *codes, const float *step, const float *zero, int64_t rows,
                int32_t d, int32_t group, int32_t bits, double *out) {
  if (!codes || !step || !zero || !out || rows < 0) return KVO_ERR_ARG;
  if (!qparams_ok(d, group, bits)) return KVO_ERR_ARG;
  const int32_t ng = d / group;
  const int64_t row_bytes = d * bits / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t k = 0; k < d; ++k) {
      int32_t g = k / group;
      out[r * d + k] = (double)zero[r * ng + g] +
                       (double)step[r * ng + g] * (double)code_at(codes + r * row_bytes, k, bits);
    }
  return KVO_OK;
}

/* ------------------------------------------------------------------ */
/* b: the Jensen bias of one (query, cached key) score                 */
/* [S1] 方法: b_i = log E[exp(delta_i)], delta_i the score error from   */
/* the query times the key quantisation noise; for uniform noise an     */
/* exact form exists; the second-order Taylor form is                   */
/* (1/(24 d)) sum_c q_c^2 D_{i,c}^2.  [S2] Abstract: computed on the    */
/* fly from the cached keys' step sizes and the query norm.             */
/* ------------------------------------------------------------------ */

/* L(x) = log(sinh(x) / x), even, L(0) = 0.  Log of the moment generating
 * function of a U(-1/2, 1/2) variable at 2x.  Series below 0.1 (terms
 * 2^{2n} B_{2n} x^{2n} / (2n (2n)!), n = 1..4); the identity
 * log(sinh a / a) = a - log(2a) + log1p(-exp(-2a)) above. */
double kvo_logsinhc(double x) {
  double a = fabs(x);
  if (a < 0.1) {
    double y = a * a;
    return y * (1.0 / 6.0 + y * (-1.0 / 180.0 + y * (1.0 / 2835.0 + y * (-1.0 / 37800.0))));
  }
  return a - log(2.0 * a) + log1p(-exp(-2.0 * a));
}

static double default_tau(int32_t d, double scale) {
  return scale > 0.0 ? scale : 1.0 / sqrt((double)d);
}

/* Taylor form: (tau^2 / 24) * sum_g D_g^2 * ||q_g||^2.  `step` holds the
 * d/group step sizes of one cached key. */
double kvo_bias_taylor(const double *q, const float *step, int32_t d, int32_t group, double tau) {
  double b = 0.0;
  for (int32_t g = 0; g < d / group; ++g) {
    double qn = 0.0;
    for (int32_t c = g * group; c < (g + 1) * group; ++c) qn += q[c] * q[c];
    double s = (double)step[g];
    b += s * s * qn;
  }
  return tau * tau / 24.0 * b;
}

/* Exact form: sum_c L(tau * q_c * D_{g(c)} / 2). */
double kvo_bias_exact(const double *q, const float *step, int32_t d, int32_t group, double tau) {
  double b = 0.0;
  for (int32_t c = 0; c < d; ++c) b += kvo_logsinhc(tau * q[c] * (double)step[c / group] / 2.0);
  return b;
}

/* ------------------------------------------------------------------ */
/* attention over [cached ; current]                                   */
/* ------------------------------------------------------------------ */

typedef struct {
  int64_t B, Hq, Hkv, Nq, Ncur, Nc;
  int32_t d;
  int32_t group;
  const uint16_t *q;     /* bf16 bits [B][Hq][Nq][d] */
  const uint16_t *k_cur; /* bf16 bits [B][Hkv][Ncur][d] */
  const uint16_t *v_cur; /* bf16 bits [B][Hkv][Ncur][d] */
  const uint8_t *kc_codes; /* [B][Hkv][cap][d*kbits/8] */
  const float *kc_step;    /* [B][Hkv][cap][d/group], or [B][Hkv][ceil(cap/group)][d] (kaxis 1) */
  const float *kc_zero;
  const uint8_t *vc_codes;
  const float *vc_step;
  const float *vc_zero;
  int32_t kbits, vbits;
  int64_t cap;
  double scale; /* softmax scale tau; <= 0 means 1/sqrt(d) */
  int32_t corr; /* 0 off, 1 Taylor, 2 exact */
  int32_t causal; /* 0 no mask; 1 end-aligned causal mask on the current chunk */
  int32_t kaxis;  /* 0: K groups along the head dimension; 1: along the tokens (per channel) */
  int32_t vaxis;  /* the same for V */
} kvo_attn;

static int attn_ok(const kvo_attn *a) {
  if (!a || a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Hq % a->Hkv) return 0;
  if (a->Nq < 1 || a->Ncur < 0 || a->Nc < 0 || a->Nc + a->Ncur < 1) return 0;
  if (a->corr < 0 || a->corr > 2 || !a->q) return 0;
  if (a->causal != 0 && a->causal != 1) return 0;
  if (a->causal && a->Nc == 0 && a->Nq > a->Ncur) return 0; /* a row would see no key */
  if (a->Ncur > 0 && (!a->k_cur || !a->v_cur)) return 0;
  if (a->Nc > 0) {
    if (!a->kc_codes || !a->kc_step || !a->kc_zero || !a->vc_codes || !a->vc_step || !a->vc_zero) return 0;
    if (a->kaxis < 0 || a->kaxis > 1 || a->vaxis < 0 || a->vaxis > 1) return 0;
    if (a->kaxis == 0 ? !qparams_ok(a->d, a->group, a->kbits)
                      : (a->group < 1 || (a->kbits != 2 && a->kbits != 4) || (a->d * a->kbits) % 8))
      return 0;
    if (a->vaxis == 0 ? !qparams_ok(a->d, a->group, a->vbits)
                      : (a->group < 1 || (a->vbits != 2 && a->vbits != 4) || (a->d * a->vbits) % 8))
      return 0;
    if (a->cap < a->Nc) return 0;
  }
  return a->d > 0;
}

/* Per-row view of the inputs. */
typedef struct {
  const kvo_attn *a;
  int64_t b, h, hk;
  double tau;
  double *q; /* d */
} rowctx;

static void row_setup(const kvo_attn *a, int64_t row, rowctx *rc, double *qbuf) {
  rc->a = a;
  rc->b = row / (a->Hq * a->Nq);
  rc->h = (row / a->Nq) % a->Hq;
  rc->hk = rc->h / (a->Hq / a->Hkv);
  rc->tau = default_tau(a->d, a->scale);
  rc->q = qbuf;
  const uint16_t *qp = a->q + row * a->d;
  for (int32_t c = 0; c < a->d; ++c) rc->q[c] = (double)bf16_bits_to_f32(qp[c]);
}

/* Whether key t is visible to flat query row `row` (query j = row mod Nq):
 * every cached key; current key i = t - Nc unless the causal mask hides it
 * (i > j + Ncur - Nq). */
static int visible(const kvo_attn *a, int64_t row, int64_t t) {
  if (t < a->Nc || !a->causal) return 1;
  const int64_t j = row % a->Nq;
  return t - a->Nc <= j + a->Ncur - a->Nq;
}

/* Index of the step and zero point of channel c of cached token t of
 * (b, hk) = bkv: groups along the head dimension (axis 0: [cap][d/group])
 * or along the tokens (axis 1: [ceil(cap/group)][d]). */
static int64_t meta_index(const kvo_attn *a, int32_t axis, int64_t bkv, int64_t t, int32_t c) {
  if (axis == 0) return (bkv * a->cap + t) * (a->d / a->group) + c / a->group;
  const int64_t capg = (a->cap + a->group - 1) / a->group;
  return (bkv * capg + t / a->group) * a->d + c;
}

/* Key index t in [0, Nc + Ncur): t < Nc is cached key t, else current key
 * t - Nc. Writes the (fp64) key and value vectors. */
static void key_value(const rowctx *rc, int64_t t, double *k, double *v) {
  const kvo_attn *a = rc->a;
  const int32_t d = a->d;
  if (t < a->Nc) {
    const int64_t bkv = rc->b * a->Hkv + rc->hk;
    const int64_t base = bkv * a->cap + t;
    const uint8_t *kr = a->kc_codes + base * (d * a->kbits / 8);
    const uint8_t *vr = a->vc_codes + base * (d * a->vbits / 8);
    /* channel c's step is at meta_index(.., 0) plus its group c / group, or
     * plus c along the tokens */
    const int64_t mk0 = meta_index(a, a->kaxis, bkv, t, 0), mv0 = meta_index(a, a->vaxis, bkv, t, 0);
    for (int32_t c = 0; c < d; ++c) {
      const int32_t g = c / a->group;
      const int64_t mk = mk0 + (a->kaxis == 0 ? g : c), mv = mv0 + (a->vaxis == 0 ? g : c);
      k[c] = (double)a->kc_zero[mk] + (double)a->kc_step[mk] * code_at(kr, c, a->kbits);
      v[c] = (double)a->vc_zero[mv] + (double)a->vc_step[mv] * code_at(vr, c, a->vbits);
    }
  } else {
    const int64_t base = ((rc->b * a->Hkv + rc->hk) * a->Ncur + (t - a->Nc)) * d;
    for (int32_t c = 0; c < d; ++c) {
      k[c] = (double)bf16_bits_to_f32(a->k_cur[base + c]);
      v[c] = (double)bf16_bits_to_f32(a->v_cur[base + c]);
    }
  }
}

/* The corrected logit of key t:
 *   cached  (t < Nc): tau * q.k^ - b     ([S1] 為何校正有效: b is subtracted
 *                                          from quantised keys' scores before
 *                                          softmax)
 *   current (t >= Nc): tau * q.k          (current-chunk logits untouched)
 * Logit scale tau = 1/sqrt(d): [S3] 研究缺口, Eq. (5). */
static double logit_of(const rowctx *rc, int64_t t, const double *k) {
  const kvo_attn *a = rc->a;
  double s = 0.0;
  for (int32_t c = 0; c < a->d; ++c) s += rc->q[c] * k[c];
  s *= rc->tau;
  if (t < a->Nc && a->corr != 0) {
    /* the key's steps: d/group of them, or one per channel (groups along
     * the tokens: a group of one channel each) */
    const int64_t bkv = rc->b * a->Hkv + rc->hk;
    const float *step = a->kc_step + meta_index(a, a->kaxis, bkv, t, 0);
    const int32_t gsz = a->kaxis == 0 ? a->group : 1;
    s -= (a->corr == 1) ? kvo_bias_taylor(rc->q, step, a->d, gsz, rc->tau)
                        : kvo_bias_exact(rc->q, step, a->d, gsz, rc->tau);
  }
  return s;
}

/* All Nc + Ncur logits of one flat query row (row = (b*Hq + h)*Nq + j). */
int kvo_logits(const kvo_attn *a, int64_t row, double *logits) {
  if (!attn_ok(a) || !logits || row < 0 || row >= a->B * a->Hq * a->Nq) return KVO_ERR_ARG;
  const int32_t d = a->d;
  double *buf = (double *)malloc(sizeof(double) * 3 * (size_t)d);
  if (!buf) return KVO_ERR_MEM;
  rowctx rc;
  row_setup(a, row, &rc, buf);
  for (int64_t t = 0; t < a->Nc + a->Ncur; ++t) {
    key_value(&rc, t, buf + d, buf + 2 * d);
    logits[t] = visible(a, row, t) ? logit_of(&rc, t, buf + d) : -INFINITY;
  }
  free(buf);
  return KVO_OK;
}

/* Brute force: the full softmax over the concatenation, then the weighted
 * sum of values ([S4] Estrutura Teórica: values enter linearly and get no
 * correction).  out: nrows x d. */
static int attention_row(const kvo_attn *a, int64_t row, double *out, double *work) {
  const int32_t d = a->d;
  const int64_t n = a->Nc + a->Ncur;
  double *q = work, *k = work + d, *v = work + 2 * d, *s = work + 3 * d;
  rowctx rc;
  row_setup(a, row, &rc, q);
  double m = -INFINITY;
  for (int64_t t = 0; t < n; ++t) {
    key_value(&rc, t, k, v);
    s[t] = visible(a, row, t) ? logit_of(&rc, t, k) : -INFINITY;
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    if (s[t] == -INFINITY) continue; /* masked */
    double p = exp(s[t] - m);
    l += p;
    key_value(&rc, t, k, v);
    for (int32_t c = 0; c < d; ++c) out[c] += p * v[c];
  }
  for (int32_t c = 0; c < d; ++c) out[c] /= l;
  return KVO_OK;
}

/* rows: nrows flat query-row indices (NULL = all rows in order).
 * threads <= 0 uses the OpenMP default. */
int kvo_attention(const kvo_attn *a, const int64_t *rows, int64_t nrows, double *out, int32_t threads) {
  if (!attn_ok(a) || !out) return KVO_ERR_ARG;
  const int64_t total = a->B * a->Hq * a->Nq;
  if (!rows) nrows = total;
  for (int64_t i = 0; rows && i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= total) return KVO_ERR_ARG;
  const size_t wsz = (size_t)(3 * a->d + a->Nc + a->Ncur);
  int err = KVO_OK;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#else
  (void)threads;
#endif
#pragma omp parallel num_threads(threads)
  {
    double *work = (double *)malloc(wsz * sizeof(double));
    if (!work) {
#pragma omp atomic write
      err = KVO_ERR_MEM;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows ? rows[i] : i;
        attention_row(a, row, out + i * a->d, work);
      }
      free(work);
    }
  }
  return err;
}

/* ------------------------------------------------------------------ */
/* Online mirror: the same softmax evaluated tile by tile with a       */
/* running (max, sum, accumulator), over arbitrary contiguous parts of */
/* the key sequence, merged by log-sum-exp.  Not a different method:   */
/* it must reproduce the brute-force result up to rounding.            */
/* ------------------------------------------------------------------ */

/* Key order position p -> key index t.  cur_first puts the current chunk
 * before the cache. */
static int64_t order_key(const kvo_attn *a, int64_t p, int32_t cur_first) {
  if (!cur_first) return p;
  return p < a->Ncur ? a->Nc + p : p - a->Ncur;
}

/* bounds: nparts+1 increasing positions from 0 to Nc+Ncur (a partition of
 * the key order into contiguous parts); tile >= 1 keys per online step. */
int kvo_attention_online(const kvo_attn *a, int64_t row, int64_t tile, const int64_t *bounds,
                         int64_t nparts, int32_t cur_first, double *out) {
  if (!attn_ok(a) || !out || !bounds || nparts < 1 || tile < 1) return KVO_ERR_ARG;
  const int64_t n = a->Nc + a->Ncur;
  if (bounds[0] != 0 || bounds[nparts] != n) return KVO_ERR_ARG;
  for (int64_t i = 0; i < nparts; ++i)
    if (bounds[i + 1] < bounds[i]) return KVO_ERR_ARG;
  if (row < 0 || row >= a->B * a->Hq * a->Nq) return KVO_ERR_ARG;
  const int32_t d = a->d;
  double *buf = (double *)malloc(sizeof(double) * ((size_t)(3 * d + tile) + (size_t)nparts * (d + 2)));
  if (!buf) return KVO_ERR_MEM;
  double *q = buf, *k = buf + d, *v = buf + 2 * d, *s = buf + 3 * d;
  double *part = buf + 3 * d + tile; /* per part: m, l, o[d] */
  rowctx rc;
  row_setup(a, row, &rc, q);
  for (int64_t pi = 0; pi < nparts; ++pi) {
    double *pm = part + pi * (d + 2), *pl = pm + 1, *po = pm + 2;
    double m = -INFINITY, l = 0.0;
    for (int32_t c = 0; c < d; ++c) po[c] = 0.0;
    for (int64_t p0 = bounds[pi]; p0 < bounds[pi + 1]; p0 += tile) {
      int64_t p1 = p0 + tile < bounds[pi + 1] ? p0 + tile : bounds[pi + 1];
      double mt = -INFINITY;
      for (int64_t p = p0; p < p1; ++p) {
        int64_t t = order_key(a, p, cur_first);
        key_value(&rc, t, k, v);
        s[p - p0] = visible(a, row, t) ? logit_of(&rc, t, k) : -INFINITY;
        if (s[p - p0] > mt) mt = s[p - p0];
      }
      double mnew = mt > m ? mt : m;
      double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
      l *= alpha;
      for (int32_t c = 0; c < d; ++c) po[c] *= alpha;
      for (int64_t p = p0; p < p1; ++p) {
        int64_t t = order_key(a, p, cur_first);
        if (s[p - p0] == -INFINITY) continue; /* masked */
        key_value(&rc, t, k, v);
        double w = exp(s[p - p0] - mnew);
        l += w;
        for (int32_t c = 0; c < d; ++c) po[c] += w * v[c];
      }
      m = mnew;
    }
    *pm = m;
    *pl = l;
  }
  /* log-sum-exp merge of the parts */
  double M = -INFINITY;
  for (int64_t pi = 0; pi < nparts; ++pi)
    if (part[pi * (d + 2)] > M) M = part[pi * (d + 2)];
  double L = 0.0;
  for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
  for (int64_t pi = 0; pi < nparts; ++pi) {
    double *pm = part + pi * (d + 2);
    if (pm[0] == -INFINITY) continue; /* empty part */
    double w = exp(pm[0] - M);
    L += w * pm[1];
    for (int32_t c = 0; c < d; ++c) out[c] += w * pm[2 + c];
  }
  for (int32_t c = 0; c < d; ++c) out[c] /= L;
  free(buf);
  return KVO_OK;
}

/* ------------------------------------------------------------------ */
/* Attention-balance diagnostics ([S1] 問題: quantisation noise on the */
/* keys raises the cached logits' share of the softmax through the     */
/* exponential's convexity, so attention moves from the current chunk  */
/* to the cache; [S1] 為何校正有效: subtracting b restores the balance). */
/* For one row, the softmax over the unquantised cached keys (given as */
/* bf16 k_ref) is compared with the one over the quantised cache under */
/* the problem's correction mode; current keys are the same in both.   */
/* ------------------------------------------------------------------ */

#define KVO_TOPK 5

/* The k largest of s[0..n) in (value descending, index ascending) order,
 * skipping -inf (masked) entries; unused slots are -1.  Repeated scans:
 * slot r takes the best entry that is ordered after slot r-1's. */
static void top_k(const double *s, int64_t n, int64_t *idx) {
  int64_t prev = -1;
  for (int32_t r = 0; r < KVO_TOPK; ++r) {
    int64_t best = -1;
    for (int64_t t = 0; t < n; ++t) {
      if (s[t] == -INFINITY) continue;
      if (prev >= 0 && (s[t] > s[prev] || (s[t] == s[prev] && t <= prev))) continue; /* already taken */
      if (best < 0 || s[t] > s[best]) best = t; /* first index wins ties (t increases) */
    }
    idx[r] = best;
    if (best < 0) {
      for (int32_t q = r + 1; q < KVO_TOPK; ++q) idx[q] = -1;
      return;
    }
    prev = best;
  }
}

/* log sum exp of the visible entries. */
static double lse_of(const double *s, int64_t n) {
  double m = -INFINITY;
  for (int64_t t = 0; t < n; ++t)
    if (s[t] > m) m = s[t];
  double l = 0.0;
  for (int64_t t = 0; t < n; ++t)
    if (s[t] != -INFINITY) l += exp(s[t] - m);
  return m + log(l);
}

/* k_ref: bf16 bits [B][Hkv][Nc][d], the cached keys before quantisation.
 * Per row (flat index, NULL rows = all rows in order):
 *   stats[5]: lse_ref, lse_q   log sum_t exp(logit_t) over visible keys,
 *             mass_ref, mass_q the softmax mass on current-chunk keys,
 *             kl               KL(p_ref || p_q) = sum_t p_ref,t log(p_ref,t / p_q,t);
 *   top[10]:  the 5 largest logits' key indices (descending, ties by lower
 *             index; -1 past the visible count) of ref, then of q.
 * ref logits: tau q.k_ref for cached keys, tau q.k for current keys;
 * q logits: as kvo_logits (tau q.k^ - b for cached keys). */
int kvo_diagnostics(const kvo_attn *a, const uint16_t *k_ref, const int64_t *rows, int64_t nrows,
                    double *stats, int64_t *top, int32_t threads) {
  if (!attn_ok(a) || !stats || !top || (a->Nc > 0 && !k_ref)) return KVO_ERR_ARG;
  const int64_t total = a->B * a->Hq * a->Nq;
  if (!rows) nrows = total;
  for (int64_t i = 0; rows && i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= total) return KVO_ERR_ARG;
  const int32_t d = a->d;
  const int64_t n = a->Nc + a->Ncur;
  int err = KVO_OK;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#else
  (void)threads;
#endif
#pragma omp parallel num_threads(threads)
  {
    double *work = (double *)malloc(sizeof(double) * (size_t)(3 * d + 2 * n));
    if (!work) {
#pragma omp atomic write
      err = KVO_ERR_MEM;
    } else {
      double *q = work, *k = work + d, *v = work + 2 * d, *sr = work + 3 * d, *sq = sr + n;
#pragma omp for schedule(dynamic, 4)
      for (int64_t i = 0; i < nrows; ++i) {
        const int64_t row = rows ? rows[i] : i;
        rowctx rc;
        row_setup(a, row, &rc, q);
        for (int64_t t = 0; t < n; ++t) {
          if (!visible(a, row, t)) {
            sr[t] = sq[t] = -INFINITY;
            continue;
          }
          key_value(&rc, t, k, v);
          sq[t] = logit_of(&rc, t, k);
          if (t < a->Nc) {
            const uint16_t *kr = k_ref + ((rc.b * a->Hkv + rc.hk) * a->Nc + t) * d;
            double s = 0.0;
            for (int32_t c = 0; c < d; ++c) s += q[c] * (double)bf16_bits_to_f32(kr[c]);
            sr[t] = s * rc.tau;
          } else {
            sr[t] = sq[t]; /* current keys: the same logit in both */
          }
        }
        const double lr = lse_of(sr, n), lq = lse_of(sq, n);
        double mr = 0.0, mq = 0.0, kl = 0.0;
        for (int64_t t = 0; t < n; ++t) {
          if (sr[t] == -INFINITY) continue;
          const double pr = exp(sr[t] - lr);
          kl += pr * ((sr[t] - lr) - (sq[t] - lq));
          if (t >= a->Nc) {
            mr += pr;
            mq += exp(sq[t] - lq);
          }
        }
        double *st = stats + i * 5;
        st[0] = lr;
        st[1] = lq;
        st[2] = mr;
        st[3] = mq;
        st[4] = kl;
        top_k(sr, n, top + i * 2 * KVO_TOPK);
        top_k(sq, n, top + i * 2 * KVO_TOPK + KVO_TOPK);
      }
      free(work);
    }
  }
  return err;
}

int kvo_version(void) { return 4; }
