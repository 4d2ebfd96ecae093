/* Sanitizer driver for the oracle (test infrastructure, built only by
 * tests/test_sanitizers.py with AddressSanitizer and UndefinedBehaviorSanitizer):
 * runs every entry point of oracle/kvq_oracle.c on small seeded inputs with
 * ragged sizes (groups along the head dimension and along the tokens,
 * binary16 metadata, no cache, no current chunk, the causal mask) and checks
 * the return codes and a few identities that hold exactly, so that an
 * out-of-bounds access or undefined operation in any of them aborts the run. */
#include "../../oracle/kvq_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) { /* splitmix64 -> [0, 1) */
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return (double)((z ^ (z >> 31)) >> 11) * 0x1p-53;
}
static uint16_t bf16_of(double x) { /* truncation is enough for inputs */
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static uint16_t *bf16_array(int64_t n, double scale) {
  uint16_t *p = (uint16_t *)malloc((size_t)n * 2 + 2);
  for (int64_t i = 0; i < n; ++i) p[i] = bf16_of((uniform() * 2.0 - 1.0) * scale);
  return p;
}

#define CHECK(c)                                                           \
  do {                                                                     \
    if (!(c)) {                                                            \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);     \
      return 1;                                                            \
    }                                                                      \
  } while (0)

/* One attention problem through kvo_attention, kvo_attention_online,
 * kvo_logits and kvo_diagnostics. */
static int run_case(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Ncur, int64_t Nc, int32_t d,
                    int32_t group, int32_t kbits, int32_t vbits, int32_t corr, int32_t causal, int32_t kaxis,
                    int32_t vaxis, int32_t meta16) {
  const int64_t cap = Nc + 3;
  const int64_t mrows_k = kaxis ? (cap + group - 1) / group : cap, mrows_v = vaxis ? (cap + group - 1) / group : cap;
  const int64_t mper_k = kaxis ? d : d / group, mper_v = vaxis ? d : d / group;
  uint16_t *q = bf16_array(B * Hq * Nq * d, 2.0);
  uint16_t *kc = bf16_array(B * Hkv * Ncur * d + 1, 1.5), *vc = bf16_array(B * Hkv * Ncur * d + 1, 1.0);
  uint16_t *kref = bf16_array(B * Hkv * cap * d, 1.5), *vref = bf16_array(B * Hkv * cap * d, 1.0);
  uint8_t *kcodes = (uint8_t *)calloc((size_t)(B * Hkv * cap * d * kbits / 8) + 1, 1);
  uint8_t *vcodes = (uint8_t *)calloc((size_t)(B * Hkv * cap * d * vbits / 8) + 1, 1);
  float *ks = (float *)calloc((size_t)(B * Hkv * mrows_k * mper_k) + 1, 4);
  float *kz = (float *)calloc((size_t)(B * Hkv * mrows_k * mper_k) + 1, 4);
  float *vs = (float *)calloc((size_t)(B * Hkv * mrows_v * mper_v) + 1, 4);
  float *vz = (float *)calloc((size_t)(B * Hkv * mrows_v * mper_v) + 1, 4);
  if (kaxis)
    CHECK(kvo_quantize_tokens_bf16_meta(kref, B * Hkv, cap, d, group, kbits, meta16, kcodes, ks, kz) == KVO_OK);
  else
    CHECK(kvo_quantize_bf16_meta(kref, B * Hkv * cap, d, group, kbits, meta16, kcodes, ks, kz) == KVO_OK);
  if (vaxis)
    CHECK(kvo_quantize_tokens_bf16_meta(vref, B * Hkv, cap, d, group, vbits, meta16, vcodes, vs, vz) == KVO_OK);
  else
    CHECK(kvo_quantize_bf16_meta(vref, B * Hkv * cap, d, group, vbits, meta16, vcodes, vs, vz) == KVO_OK);
  kvo_attn a;
  memset(&a, 0, sizeof a);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Ncur = Ncur; a.Nc = Nc; a.d = d; a.group = group;
  a.q = q; a.k_cur = kc; a.v_cur = vc;
  a.kc_codes = kcodes; a.kc_step = ks; a.kc_zero = kz; a.vc_codes = vcodes; a.vc_step = vs; a.vc_zero = vz;
  a.kbits = kbits; a.vbits = vbits; a.cap = cap; a.scale = 0.0; a.corr = corr; a.causal = causal;
  a.kaxis = kaxis; a.vaxis = vaxis;
  const int64_t rows = B * Hq * Nq, n = Nc + Ncur;
  double *out = (double *)malloc(sizeof(double) * (size_t)(rows * d));
  double *on = (double *)malloc(sizeof(double) * (size_t)d);
  double *lg = (double *)malloc(sizeof(double) * (size_t)(n + 1));
  CHECK(kvo_attention(&a, NULL, 0, out, 1) == KVO_OK);
  const int64_t bounds[3] = {0, n / 2, n};
  for (int64_t r = 0; r < rows; r += 3) {
    CHECK(kvo_attention_online(&a, r, 5, bounds, 2, r & 1, on) == KVO_OK);
    for (int32_t c = 0; c < d; ++c) CHECK(fabs(on[c] - out[r * d + c]) <= 1e-9 * (1.0 + fabs(out[r * d + c])));
    CHECK(kvo_logits(&a, r, lg) == KVO_OK);
  }
  double *stats = (double *)malloc(sizeof(double) * (size_t)(rows * 5));
  int64_t *top = (int64_t *)malloc(sizeof(int64_t) * (size_t)(rows * 10));
  if (kaxis == 0 || Nc == 0) {
    uint16_t *kr = bf16_array(B * Hkv * (Nc > 0 ? Nc : 1) * d, 1.5);
    CHECK(kvo_diagnostics(&a, kr, NULL, 0, stats, top, 1) == KVO_OK);
    for (int64_t r = 0; r < rows; ++r) CHECK(stats[r * 5 + 4] >= -1e-9);  /* KL >= 0 */
    free(kr);
  }
  /* invalid arguments are refused without touching memory */
  kvo_attn bad = a;
  bad.corr = 3;
  CHECK(kvo_attention(&bad, NULL, 0, out, 1) == KVO_ERR_ARG);
  const int64_t oob = rows;
  CHECK(kvo_attention(&a, &oob, 1, out, 1) == KVO_ERR_ARG);
  free(q); free(kc); free(vc); free(kref); free(vref); free(kcodes); free(vcodes);
  free(ks); free(kz); free(vs); free(vz); free(out); free(on); free(lg); free(stats); free(top);
  return 0;
}

int main(void) {
  /* quantiser, pack/unpack, dequantisation: ragged rows, every group */
  const int32_t ds[2] = {64, 128}, groups[3] = {32, 64, 128}, bitss[2] = {2, 4};
  for (int di = 0; di < 2; ++di)
    for (int gi = 0; gi < 3; ++gi)
      for (int bi = 0; bi < 2; ++bi)
        for (int32_t m16 = 0; m16 < 2; ++m16) {
          const int32_t d = ds[di], g = groups[gi], bits = bitss[bi];
          if (g > d) continue;
          const int64_t rows = 7;
          float *x = (float *)malloc(sizeof(float) * (size_t)(rows * d));
          for (int64_t i = 0; i < rows * d; ++i) x[i] = (float)((uniform() * 2 - 1) * 3);
          uint8_t *codes = (uint8_t *)malloc((size_t)(rows * d * bits / 8));
          uint8_t *c = (uint8_t *)malloc((size_t)(rows * d)), *codes2 = (uint8_t *)malloc((size_t)(rows * d * bits / 8));
          float *st = (float *)malloc(sizeof(float) * (size_t)(rows * d / g));
          float *zp = (float *)malloc(sizeof(float) * (size_t)(rows * d / g));
          double *dq = (double *)malloc(sizeof(double) * (size_t)(rows * d));
          CHECK(kvo_quantize_f32_meta(x, rows, d, g, bits, m16, codes, st, zp) == KVO_OK);
          CHECK(kvo_unpack(codes, rows, d, bits, c) == KVO_OK);
          CHECK(kvo_pack(c, rows, d, bits, codes2) == KVO_OK);
          CHECK(memcmp(codes, codes2, (size_t)(rows * d * bits / 8)) == 0);
          CHECK(kvo_dequant(codes, st, zp, rows, d, g, bits, dq) == KVO_OK);
          if (!m16)
            for (int64_t i = 0; i < rows * d; ++i) /* |x - x^| <= D/2 inside the grid */
              CHECK(fabs((double)x[i] - dq[i]) <= 0.5 * st[i / g] * (1 + 1e-6) + 1e-30);
          double qv[128];
          for (int32_t k = 0; k < d; ++k) qv[k] = uniform() - 0.5;
          const double bt = kvo_bias_taylor(qv, st, d, g, 0.0), be = kvo_bias_exact(qv, st, d, g, 0.0);
          CHECK(bt >= 0 && be >= 0 && be <= bt * (1 + 1e-12));
          CHECK(kvo_quantize_f32_meta(x, rows, d, g + 1, bits, m16, codes, st, zp) == KVO_ERR_ARG);
          free(x); free(codes); free(c); free(codes2); free(st); free(zp); free(dq);
        }
  /* attention: head-dim and token groups, with and without cache or chunk */
  CHECK(run_case(2, 4, 2, 3, 5, 37, 128, 64, 2, 4, 1, 0, 0, 0, 0) == 0);
  CHECK(run_case(1, 2, 1, 4, 6, 19, 64, 32, 4, 2, 2, 1, 0, 0, 1) == 0);
  CHECK(run_case(1, 3, 3, 2, 0, 23, 128, 128, 2, 2, 1, 0, 0, 0, 0) == 0);
  CHECK(run_case(2, 2, 2, 5, 5, 0, 64, 64, 2, 2, 1, 1, 0, 0, 0) == 0);
  CHECK(run_case(1, 4, 2, 3, 4, 41, 128, 32, 4, 4, 1, 0, 1, 1, 0) == 0);
  CHECK(run_case(1, 2, 2, 2, 3, 70, 64, 64, 2, 4, 0, 1, 1, 0, 1) == 0);
  printf("oracle sanitizer run: ok\n");
  return 0;
}
