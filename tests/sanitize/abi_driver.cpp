// Sanitizer driver for the library's host code (test infrastructure, built
// only by tests/test_sanitizers.py: every library source compiled for the
// host only, with AddressSanitizer and UndefinedBehaviorSanitizer).  It calls
// the C ABI with invalid arguments (each must be refused with its status) and
// asks the planner for workspace sizes of valid calls; device addresses are
// fake and never dereferenced, and no call here reaches a kernel launch.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvq.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }
constexpr uintptr_t A = 0x100000000;  // q, k_cur, v_cur, out 4 GiB apart

static kv_qtensor qt(uintptr_t base, int32_t bits = 2, int32_t group = 64, int64_t cap = 100) {
  kv_qtensor t;
  memset(&t, 0, sizeof t);
  t.codes = static_cast<uint8_t *>(P(base));
  t.scale = P(base + 0x100000);
  t.zero = P(base + 0x200000);
  t.bits = bits;
  t.group = group;
  t.cap = cap;
  t.meta = KV_META_F32;
  t.axis = KV_AXIS_DIM;
  return t;
}

struct Call {
  kv_attn_args a;
  kv_qtensor k, v;
  Call() {
    memset(&a, 0, sizeof a);
    a.B = 1; a.Hq = 4; a.Hkv = 2; a.Nq = 8; a.Ncur = 8; a.Nc = 50; a.d = 128;
    a.q = P(A); a.k_cur = P(2 * A); a.v_cur = P(3 * A); a.out = P(4 * A);
    k = qt(0x10000000);
    v = qt(0x20000000);
    a.k_cache = &k;
    a.v_cache = &v;
    a.corr = KV_CORR_TAYLOR;
  }
};

int main() {
  for (int s = 0; s <= 9; ++s) CHECK(kv_status_string(static_cast<kv_status>(s)) != nullptr);
  CHECK(kv_version() > 0);

  // ---- kv_quantize: refused arguments, then N = 0 (validated, nothing launched)
  {
    kv_qtensor t = qt(0x30000000, 4, 64, 64);
    CHECK(kv_quantize(nullptr, KV_BF16, 1, 2, 8, 128, &t, 0, nullptr) == KV_ERR_NULL);
    CHECK(kv_quantize(P(A), static_cast<kv_dtype>(9), 1, 2, 8, 128, &t, 0, nullptr) == KV_ERR_UNSUPPORTED);
    CHECK(kv_quantize(P(A), KV_BF16, 1, 2, 8, 96, &t, 0, nullptr) == KV_ERR_UNSUPPORTED);
    CHECK(kv_quantize(P(A), KV_BF16, 1, 2, 60, 128, &t, 10, nullptr) == KV_ERR_SHAPE);
    CHECK(kv_quantize(P(A + 2), KV_BF16, 1, 2, 8, 128, &t, 0, nullptr) == KV_ERR_ALIGN);
    CHECK(kv_quantize(P(0x30000000 + 64), KV_BF16, 1, 2, 8, 128, &t, 0, nullptr) == KV_ERR_ALIAS);
    CHECK(kv_quantize(P(A), KV_BF16, INT64_MAX / 2, 2, 8, 128, &t, 0, nullptr) != KV_OK);
    CHECK(kv_quantize(P(A), KV_BF16, 1, 2, 0, 128, &t, 0, nullptr) == KV_OK);
    kv_qtensor tk = t;
    tk.axis = KV_AXIS_TOKENS;
    CHECK(kv_quantize(P(A), KV_BF16, 1, 2, 8, 128, &tk, 3, nullptr) == KV_ERR_SHAPE);
    kv_qtensor pg = t;
    pg.page_table = static_cast<const int32_t *>(P(0x7000000));
    pg.page_size = 48;
    pg.num_pages = 4;
    CHECK(kv_quantize(P(A), KV_BF16, 1, 2, 0, 128, &pg, 0, nullptr) == KV_ERR_SHAPE);
  }

  // ---- kv_attention_corrected / workspace size: refused arguments
  {
    struct Bad {
      void (*edit)(Call &);
      kv_status want;
    } bad[] = {
        {[](Call &c) { c.a.q = nullptr; }, KV_ERR_NULL},
        {[](Call &c) { c.a.k_cache = nullptr; }, KV_ERR_NULL},
        {[](Call &c) { c.a.B = 0; }, KV_ERR_SHAPE},
        {[](Call &c) { c.a.Hq = 3; }, KV_ERR_SHAPE},
        {[](Call &c) { c.a.Nc = 0; c.a.Ncur = 0; }, KV_ERR_SHAPE},
        {[](Call &c) { c.a.Nc = -1; }, KV_ERR_SHAPE},
        {[](Call &c) { c.a.Nq = INT64_MAX / 4; }, KV_ERR_SHAPE},
        {[](Call &c) { c.a.d = 96; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.corr = 3; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.path = 7; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.splits = 1025; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.softmax_scale = -1.0f; }, KV_ERR_SHAPE},
        {[](Call &c) { c.a.q = P(A + 2); }, KV_ERR_ALIGN},
        {[](Call &c) { c.a.out = P(A + 64); }, KV_ERR_ALIAS},
        {[](Call &c) { c.a.causal = 2; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.causal = 1; c.a.Nc = 0; c.a.Nq = 9; }, KV_ERR_SHAPE},
        {[](Call &c) { c.k.bits = 3; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.k.bound = static_cast<float *>(P(0x50000002)); }, KV_ERR_ALIGN},
        {[](Call &c) {  // appending writes the running bound: it may not lie inside q
           c.a.append = 1;
           c.v.bound = static_cast<float *>(P(A));
         },
         KV_ERR_ALIAS},
        {[](Call &c) { c.k.cap = 10; }, KV_ERR_SHAPE},
        {[](Call &c) { c.v.group = 32; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.append = 2; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.reserved = 1; }, KV_ERR_UNSUPPORTED},
        {[](Call &c) { c.a.append = 1; c.a.Nc = 93; }, KV_ERR_SHAPE},
        {[](Call &c) { c.a.append = 1; c.a.k_cur = P(0x10000000 + 4096); }, KV_ERR_ALIAS},
        {[](Call &c) { c.a.append = 1; c.v = qt(0x10000000 + 256); }, KV_ERR_ALIAS},
        {[](Call &c) {
           c.a.append = 1;
           c.k.axis = c.v.axis = KV_AXIS_TOKENS;
           c.k.cap = c.v.cap = 128;
         },
         KV_ERR_UNSUPPORTED},
    };
    int i = 0;
    for (const Bad &b : bad) {
      Call c;
      b.edit(c);
      const kv_status got = kv_attention_corrected(&c.a, nullptr);
      if (got != b.want) fprintf(stderr, "case %d: status %d, want %d\n", i, got, b.want);
      ++i;
      CHECK(got == b.want);
      CHECK(kv_attention_corrected_static(&c.a, nullptr) == b.want);
      CHECK(kv_attention_workspace_size(&c.a) == 0);
    }
    Call c;  // valid but no workspace: refused before any launch
    c.a.path = KV_PATH_SHORT;
    CHECK(kv_attention_corrected(&c.a, nullptr) == KV_ERR_WORKSPACE);
  }

  // ---- planner: workspace sizes of valid calls on every path (no launch)
  {
    struct Plan {
      void (*edit)(Call &);
    } plans[] = {
        {[](Call &) {}},
        {[](Call &c) { c.a.path = KV_PATH_SHORT; }},
        {[](Call &c) { c.a.Nq = 4096; c.a.Ncur = 4096; c.k.cap = c.v.cap = 1 << 20; c.a.Nc = 1 << 19; }},
        {[](Call &c) { c.a.d = 64; c.k.group = c.v.group = 32; }},
        {[](Call &c) { c.a.corr = KV_CORR_EXACT; c.a.path = KV_PATH_SHORT; }},
        {[](Call &c) { c.k.axis = c.v.axis = KV_AXIS_TOKENS; c.k.cap = c.v.cap = 128; }},
        {[](Call &c) { c.a.splits = 1024; c.a.path = KV_PATH_SHORT; }},
        {[](Call &c) { c.a.append = 1; c.a.Nc = 0; }},
        {[](Call &c) {
          c.k.page_table = c.v.page_table = static_cast<const int32_t *>(P(0x7000000));
          c.k.page_size = c.v.page_size = 64;
          c.k.num_pages = c.v.num_pages = 8;
          c.k.cap = c.v.cap = 128;
        }},
    };
    int i = 0;
    for (const Plan &p : plans) {
      Call c;
      p.edit(c);
      const size_t ws = kv_attention_workspace_size(&c.a);
      if (ws == 0) fprintf(stderr, "plan %d: no workspace (status %d)\n", i, kv_attention_corrected(&c.a, nullptr));
      ++i;
      CHECK(ws > 0);
    }
    Call big;  // the static entry's scratch limit, checked before any device call
    big.a.path = KV_PATH_SHORT;
    big.a.splits = 1024;
    big.a.B = 64; big.a.Hq = 64; big.a.Hkv = 64; big.a.Nq = 16; big.a.Ncur = 16;
    CHECK(kv_attention_corrected_static(&big.a, nullptr) == KV_ERR_SCRATCH);
  }

  // ---- diagnostics: refused arguments
  {
    kv_diag_args d;
    memset(&d, 0, sizeof d);
    kv_qtensor k = qt(0x10000000);
    d.B = 1; d.Hq = 4; d.Hkv = 2; d.Nq = 8; d.Ncur = 8; d.Nc = 50; d.d = 128; d.corr = KV_CORR_TAYLOR;
    d.q = P(A); d.k_cur = P(2 * A); d.k_ref = P(3 * A); d.k_cache = &k;
    d.out = static_cast<kv_diag_row *>(P(4 * A));
    kv_diag_args x = d;
    x.out = nullptr;
    CHECK(kv_attention_diagnostics(&x, nullptr) == KV_ERR_NULL);
    x = d;
    x.out = static_cast<kv_diag_row *>(P(A + 16));
    CHECK(kv_attention_diagnostics(&x, nullptr) == KV_ERR_ALIAS);
    x = d;
    k.cap = 49;
    CHECK(kv_attention_diagnostics(&x, nullptr) == KV_ERR_SHAPE);
  }
  printf("host sanitizer run: ok\n");
  return 0;
}
