// Host side of libkvq.so: argument validation (before any HIP call, so every
// error path can be exercised on a machine without a GPU), path selection
// and kernel launch.  No allocation, no state kept between calls.
#include <math.h>
#include <stdlib.h>
#include <stdio.h>

#include <mutex>

#include "kvq_internal.h"

namespace {

using kvq::AttnLaunch;

constexpr int32_t kAbiVersion = 10;
constexpr int32_t kMaxSplits = 1024;  // grid z extent of the split path
constexpr int64_t kMaxTokensPerHead = int64_t(1) << 23;  // 8M tokens: 32-bit in-head offsets

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Page sizes of the paged layout: powers of two from 16 tokens (shifts and
// masks in the kernels).  The throughput kernel needs pages of at least 64
// tokens (whole tiles) and the short-query kernel of at least 32 (whole
// blocks); smaller pages run on the general kernel, which looks every row up.
bool page_size_ok(int32_t ps) { return ps >= 16 && ps <= (1 << 23) && (ps & (ps - 1)) == 0; }

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

static_assert(KV_META_F32 == kvq::kMetaF32 && KV_META_F16 == kvq::kMetaF16 && KV_META_BF16 == kvq::kMetaBF16,
              "the kernels take kv_meta values as their metadata kinds");
bool meta_ok(int32_t m) { return m == KV_META_F32 || m == KV_META_F16 || m == KV_META_BF16; }

bool group_ok(int32_t group, int32_t d) {
  return (group == 32 || group == 64 || group == 128) && group <= d && d % group == 0;
}

// Group size of a cache tensor: along the head dimension it must divide d;
// along the tokens any of 32, 64, 128.
bool tensor_group_ok(const kv_qtensor *t, int32_t d) {
  if (t->axis == KV_AXIS_TOKENS) return t->group == 32 || t->group == 64 || t->group == 128;
  return group_ok(t->group, d);
}

// Byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checked a*b for non-negative int64 (false on overflow).
bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

kv_status check_qtensor(const kv_qtensor *t, int32_t d, int64_t need_rows, int64_t B) {
  if (!t) return KV_ERR_NULL;
  if (!t->codes || !t->scale || !t->zero) return KV_ERR_NULL;
  if (t->bits != 2 && t->bits != 4) return KV_ERR_UNSUPPORTED;
  if (t->axis != KV_AXIS_DIM && t->axis != KV_AXIS_TOKENS) return KV_ERR_UNSUPPORTED;
  if (!tensor_group_ok(t, d)) return KV_ERR_UNSUPPORTED;
  if (t->cap < need_rows || t->cap < 0) return KV_ERR_SHAPE;
  if (t->axis == KV_AXIS_TOKENS && (t->cap % t->group != 0 || (t->page_table && t->page_size % t->group != 0)))
    return KV_ERR_SHAPE;
  if (t->cap > kMaxTokensPerHead) return KV_ERR_UNSUPPORTED;
  if (!aligned16(t->codes) || !aligned16(t->scale) || !aligned16(t->zero)) return KV_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(t->bound) & 3u) != 0) return KV_ERR_ALIGN;
  if (!meta_ok(t->meta)) return KV_ERR_UNSUPPORTED;
  if (t->page_table) {
    if (!page_size_ok(t->page_size) || t->cap % t->page_size != 0) return KV_ERR_SHAPE;
    if (t->num_pages < 1) return KV_ERR_SHAPE;
    if (B * (t->cap / t->page_size) > INT32_MAX) return KV_ERR_SHAPE;  // page-table indices are 32-bit
    if ((reinterpret_cast<uintptr_t>(t->page_table) & 3u) != 0) return KV_ERR_ALIGN;
  } else if (t->page_size != 0 || t->num_pages != 0) {
    return KV_ERR_SHAPE;
  }
  return KV_OK;
}

kvq::CacheLayout layout_of(const kv_qtensor *t) {
  if (!t->page_table) return kvq::CacheLayout{nullptr, 0, 0};
  return kvq::CacheLayout{t->page_table, __builtin_ctz(static_cast<unsigned>(t->page_size)),
                          static_cast<int32_t>(t->cap / t->page_size)};
}

// Token rows a cache tensor of B x H heads spans in memory (its pool when paged).
int64_t tensor_rows(const kv_qtensor *t, int64_t B, int64_t H) {
  return t->page_table ? static_cast<int64_t>(t->num_pages) * H * t->page_size : B * H * t->cap;
}

bool same_layout(const kv_qtensor *a, const kv_qtensor *b) {
  return a->page_table == b->page_table && a->page_size == b->page_size && a->meta == b->meta;
}

// Bytes of one step or zero-point element.
size_t meta_bytes(const kv_qtensor *t) { return t->meta == KV_META_F32 ? 4 : 2; }

// Bytes of a cache tensor's step (or zero-point) array over `rows` token rows.
size_t meta_array_bytes(const kv_qtensor *t, size_t rows, int32_t d) {
  const size_t elems = t->axis == KV_AXIS_TOKENS ? rows / static_cast<size_t>(t->group) * static_cast<size_t>(d)
                                                 : rows * static_cast<size_t>(d / t->group);
  return elems * meta_bytes(t);
}

// Page size of a call's caches (0: contiguous or no cache).
int32_t cache_page_size(const kv_attn_args *a) {
  return a->Nc > 0 && a->k_cache->page_table ? a->k_cache->page_size : 0;
}

// The K / V cache of a call (when it reads one) groups along the tokens.
bool k_tokens(const kv_attn_args *a) { return a->Nc > 0 && a->k_cache->axis == KV_AXIS_TOKENS; }
bool v_tokens(const kv_attn_args *a) { return a->Nc > 0 && a->v_cache->axis == KV_AXIS_TOKENS; }

// Either cache of a call groups along the tokens (the general kernel, or on
// the short path with K alone along the tokens the 16-row kernel).
bool tokens_axis(const kv_attn_args *a) { return k_tokens(a) || v_tokens(a); }

bool debug_log() {
  const char *e = getenv("KVQ_LOG");
  return e && e[0] == '1';
}

struct Plan {
  int path;  // KV_PATH_LONG or KV_PATH_SHORT
  int splits;
  size_t workspace;
  int64_t full_units;  // throughput kernel: units run unsplit
};

// Rows per KV head at or below which the split-over-cache path is used.
constexpr int64_t kShortRows = 64;

int device_cu_count() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  return cus;
}

// The call reads its caches (Nc > 0) or writes the chunk into them (append).
bool uses_caches(const kv_attn_args *a) { return a->Nc > 0 || (a->append == 1 && a->Ncur > 0); }

// [p, p + n) overlaps the codes, steps or zero points of cache tensor c.
bool overlaps_cache(const kv_attn_args *a, const kv_qtensor *c, const void *p, size_t n) {
  const size_t rows = static_cast<size_t>(tensor_rows(c, a->B, a->Hkv));
  return overlaps(p, n, c->codes, rows * static_cast<size_t>(a->d * c->bits / 8)) ||
         overlaps(p, n, c->scale, meta_array_bytes(c, rows, a->d)) ||
         overlaps(p, n, c->zero, meta_array_bytes(c, rows, a->d)) ||
         overlaps(p, n, c->bound, static_cast<size_t>(a->B * a->Hkv) * sizeof(float));
}

kv_status validate_attention(const kv_attn_args *a) {
  if (!a) return KV_ERR_NULL;
  if (!a->q || !a->out) return KV_ERR_NULL;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Nq < 1 || a->Ncur < 0 || a->Nc < 0) return KV_ERR_SHAPE;
  if (a->Hq % a->Hkv != 0) return KV_ERR_SHAPE;
  if (a->Nc + a->Ncur < 1) return KV_ERR_SHAPE;
  if (!head_dim_ok(a->d)) return KV_ERR_UNSUPPORTED;
  if (a->corr < KV_CORR_OFF || a->corr > KV_CORR_EXACT) return KV_ERR_UNSUPPORTED;
  if (a->path < KV_PATH_AUTO || a->path > KV_PATH_SHORT) return KV_ERR_UNSUPPORTED;
  if (a->splits < 0) return KV_ERR_SHAPE;
  if (a->splits > kMaxSplits) return KV_ERR_UNSUPPORTED;
  if (a->causal != 0 && a->causal != 1) return KV_ERR_UNSUPPORTED;
  if (a->causal && a->Nc == 0 && a->Nq > a->Ncur) return KV_ERR_SHAPE;  // a row would see no key
  if (!(a->softmax_scale >= 0.0f) || !isfinite(a->softmax_scale)) return KV_ERR_SHAPE;
  // sizes: every element count must fit comfortably in int64 and the grid
  int64_t nq_el = 0, ncur_el = 0, t = 0;
  if (!mul_ok(a->B, a->Hq, &t) || !mul_ok(t, a->Nq, &t) || !mul_ok(t, a->d, &nq_el)) return KV_ERR_SHAPE;
  if (!mul_ok(a->B, a->Hkv, &t) || !mul_ok(t, a->Ncur, &t) || !mul_ok(t, a->d, &ncur_el)) return KV_ERR_SHAPE;
  if (a->B * a->Hkv > 65535) return KV_ERR_UNSUPPORTED;
  // per-head token counts: kernels index rows within a head in 32 bits
  if (a->Ncur > kMaxTokensPerHead || a->Nc > kMaxTokensPerHead) return KV_ERR_UNSUPPORTED;
  if ((a->Nq * (a->Hq / a->Hkv)) > (int64_t(1) << 40)) return KV_ERR_SHAPE;
  if (!aligned16(a->q) || !aligned16(a->out)) return KV_ERR_ALIGN;
  if (a->Ncur > 0) {
    if (!a->k_cur || !a->v_cur) return KV_ERR_NULL;
    if (!aligned16(a->k_cur) || !aligned16(a->v_cur)) return KV_ERR_ALIGN;
  }
  if (a->append != 0 && a->append != 1) return KV_ERR_UNSUPPORTED;
  if (a->reserved != 0) return KV_ERR_UNSUPPORTED;
  if (uses_caches(a)) {
    // appending needs room for the chunk after the cached rows
    const int64_t need = a->Nc + (a->append ? a->Ncur : 0);
    kv_status s = check_qtensor(a->k_cache, a->d, need, a->B);
    if (s != KV_OK) return s;
    s = check_qtensor(a->v_cache, a->d, need, a->B);
    if (s != KV_OK) return s;
    if (a->k_cache->group != a->v_cache->group) return KV_ERR_UNSUPPORTED;
    if (a->k_cache->cap != a->v_cache->cap) return KV_ERR_SHAPE;
    if (!same_layout(a->k_cache, a->v_cache)) return KV_ERR_UNSUPPORTED;
    if (a->append && (a->k_cache->axis != KV_AXIS_DIM || a->v_cache->axis != KV_AXIS_DIM))
      return KV_ERR_UNSUPPORTED;
  }
  // the output must not overlap any input
  const size_t out_b = static_cast<size_t>(nq_el) * 2;
  if (overlaps(a->out, out_b, a->q, out_b)) return KV_ERR_ALIAS;
  if (a->Ncur > 0 && (overlaps(a->out, out_b, a->k_cur, static_cast<size_t>(ncur_el) * 2) ||
                      overlaps(a->out, out_b, a->v_cur, static_cast<size_t>(ncur_el) * 2)))
    return KV_ERR_ALIAS;
  if (uses_caches(a)) {
    const kv_qtensor *ts[2] = {a->k_cache, a->v_cache};
    for (const kv_qtensor *c : ts)
      if (overlaps_cache(a, c, a->out, out_b)) return KV_ERR_ALIAS;
  }
  if (a->append && a->Ncur > 0) {  // the caches are written: nothing else the call touches may share their bytes
    const size_t cur_b = static_cast<size_t>(ncur_el) * 2;
    const kv_qtensor *ts[2] = {a->k_cache, a->v_cache};
    for (const kv_qtensor *c : ts)
      if (overlaps_cache(a, c, a->q, out_b) || overlaps_cache(a, c, a->k_cur, cur_b) ||
          overlaps_cache(a, c, a->v_cur, cur_b))
        return KV_ERR_ALIAS;
    const kv_qtensor *k = a->k_cache, *v = a->v_cache;
    const size_t rows = static_cast<size_t>(tensor_rows(k, a->B, a->Hkv));
    const size_t kc = rows * static_cast<size_t>(a->d * k->bits / 8), km = meta_array_bytes(k, rows, a->d);
    if (overlaps_cache(a, v, k->codes, kc) || overlaps_cache(a, v, k->scale, km) || overlaps_cache(a, v, k->zero, km) ||
        overlaps(k->codes, kc, k->scale, km) || overlaps(k->codes, kc, k->zero, km) ||
        overlaps(k->scale, km, k->zero, km))
      return KV_ERR_ALIAS;
    const size_t vrows = static_cast<size_t>(tensor_rows(v, a->B, a->Hkv));
    const size_t vcb = vrows * static_cast<size_t>(a->d * v->bits / 8), vm = meta_array_bytes(v, vrows, a->d);
    if (overlaps(v->codes, vcb, v->scale, vm) || overlaps(v->codes, vcb, v->zero, vm) ||
        overlaps(v->scale, vm, v->zero, vm))
      return KV_ERR_ALIAS;
  }
  return KV_OK;
}

// The byte range [p, p + n) overlaps the output or an input of the call
// (used for the workspace).
bool overlaps_call(const kv_attn_args *a, const void *p, size_t n) {
  const size_t q_b = static_cast<size_t>(a->B * a->Hq * a->Nq * a->d) * 2;
  const size_t cur_b = static_cast<size_t>(a->B * a->Hkv * a->Ncur * a->d) * 2;
  if (overlaps(p, n, a->out, q_b) || overlaps(p, n, a->q, q_b)) return true;
  if (a->Ncur > 0 && (overlaps(p, n, a->k_cur, cur_b) || overlaps(p, n, a->v_cur, cur_b))) return true;
  if (uses_caches(a)) {
    const kv_qtensor *ts[2] = {a->k_cache, a->v_cache};
    for (const kv_qtensor *c : ts) {
      if (overlaps_cache(a, c, p, n)) return true;
      if (c->page_table &&
          overlaps(p, n, c->page_table, static_cast<size_t>(a->B * (c->cap / c->page_size)) * sizeof(int32_t)))
        return true;
    }
  }
  return false;
}

kv_status validate_diagnostics(const kv_diag_args *a) {
  if (!a) return KV_ERR_NULL;
  if (!a->q || !a->out) return KV_ERR_NULL;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Nq < 1 || a->Ncur < 0 || a->Nc < 0) return KV_ERR_SHAPE;
  if (a->Hq % a->Hkv != 0 || a->Nc + a->Ncur < 1) return KV_ERR_SHAPE;
  if (!head_dim_ok(a->d)) return KV_ERR_UNSUPPORTED;
  if (a->corr < KV_CORR_OFF || a->corr > KV_CORR_EXACT) return KV_ERR_UNSUPPORTED;
  if (a->causal != 0 && a->causal != 1) return KV_ERR_UNSUPPORTED;
  if (a->causal && a->Nc == 0 && a->Nq > a->Ncur) return KV_ERR_SHAPE;  // a row would see no key
  if (!(a->softmax_scale >= 0.0f) || !isfinite(a->softmax_scale)) return KV_ERR_SHAPE;
  int64_t nq_el = 0, ncur_el = 0, nc_el = 0, t = 0;
  if (!mul_ok(a->B, a->Hq, &t) || !mul_ok(t, a->Nq, &t) || !mul_ok(t, a->d, &nq_el)) return KV_ERR_SHAPE;
  if (!mul_ok(a->B, a->Hkv, &t) || !mul_ok(t, a->Ncur, &t) || !mul_ok(t, a->d, &ncur_el)) return KV_ERR_SHAPE;
  if (!mul_ok(a->B, a->Hkv, &t) || !mul_ok(t, a->Nc, &t) || !mul_ok(t, a->d, &nc_el)) return KV_ERR_SHAPE;
  if (a->B * a->Hkv > 65535) return KV_ERR_UNSUPPORTED;
  if (a->Ncur > kMaxTokensPerHead || a->Nc > kMaxTokensPerHead) return KV_ERR_UNSUPPORTED;
  if ((a->Nq * (a->Hq / a->Hkv)) > (int64_t(1) << 36)) return KV_ERR_SHAPE;
  if (!aligned16(a->q) || !aligned16(a->out)) return KV_ERR_ALIGN;
  if (a->Ncur > 0) {
    if (!a->k_cur) return KV_ERR_NULL;
    if (!aligned16(a->k_cur)) return KV_ERR_ALIGN;
  }
  if (a->Nc > 0) {
    if (!a->k_ref) return KV_ERR_NULL;
    const kv_status s = check_qtensor(a->k_cache, a->d, a->Nc, a->B);
    if (s != KV_OK) return s;
    if (!aligned16(a->k_ref)) return KV_ERR_ALIGN;
  }
  // the records must not overlap any input
  const size_t out_b = static_cast<size_t>(nq_el / a->d) * sizeof(kv_diag_row);
  if (overlaps(a->out, out_b, a->q, static_cast<size_t>(nq_el) * 2)) return KV_ERR_ALIAS;
  if (a->Ncur > 0 && overlaps(a->out, out_b, a->k_cur, static_cast<size_t>(ncur_el) * 2)) return KV_ERR_ALIAS;
  if (a->Nc > 0) {
    const kv_qtensor *c = a->k_cache;
    const size_t rows = static_cast<size_t>(tensor_rows(c, a->B, a->Hkv));
    if (overlaps(a->out, out_b, a->k_ref, static_cast<size_t>(nc_el) * 2) ||
        overlaps(a->out, out_b, c->codes, rows * static_cast<size_t>(a->d * c->bits / 8)) ||
        overlaps(a->out, out_b, c->scale, meta_array_bytes(c, rows, a->d)) ||
        overlaps(a->out, out_b, c->zero, meta_array_bytes(c, rows, a->d)))
      return KV_ERR_ALIAS;
  }
  return KV_OK;
}

// Scratch of kv_attention_corrected_static: one copy per device, addressed
// only through the pointer hipGetSymbolAddress returns for that device.
constexpr size_t kScratchBytes = KV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

// Device address of the current device's scratch array (nullptr on failure),
// looked up on the first call per device and kept.
void *scratch_ptr() {
  static std::mutex mu;
  static void *ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// `limit`: most workspace bytes the caller can give; an automatic split
// count is lowered to fit it where possible (a forced one is kept).
Plan plan_attention(const kv_attn_args *a, bool query_device, size_t limit = SIZE_MAX) {
  Plan pl{KV_PATH_LONG, 0, 0, 0};
  const int64_t rows = a->Nq * (a->Hq / a->Hkv);
  int path = a->path;
  if (path == KV_PATH_AUTO) {
    // caches grouped along the tokens take the short-query kernels at any row
    // count where they can (the throughput kernel takes head-dimension groups
    // only, and the general kernel is 2-2.5x slower than row groups of 32 on
    // the short-query tiles)
    const int meta = a->Nc > 0 ? static_cast<int>(a->k_cache->meta) : 0;
    const bool tok_short = tokens_axis(a) &&
                           (kvq::short16_tok_supported(a->d, a->corr, k_tokens(a), v_tokens(a), cache_page_size(a),
                                                       meta, rows) ||
                            kvq::short_tok_supported(a->d, a->corr, k_tokens(a), v_tokens(a), cache_page_size(a), meta));
    path = ((rows <= kShortRows || tok_short) && a->Nc > 0) ? KV_PATH_SHORT : KV_PATH_LONG;
  }
  pl.path = path;
  if (path == KV_PATH_SHORT) {
    const int cus = query_device ? device_cu_count() : 256;
    const bool fast = kvq::short_fast_supported(a->d, a->corr, tokens_axis(a), cache_page_size(a)) ||
                      kvq::short16_tok_supported(a->d, a->corr, k_tokens(a), v_tokens(a), cache_page_size(a),
                                                 a->Nc > 0 ? static_cast<int>(a->k_cache->meta) : 0, rows) ||
                      kvq::short_tok_supported(a->d, a->corr, k_tokens(a), v_tokens(a), cache_page_size(a),
                                               a->Nc > 0 ? static_cast<int>(a->k_cache->meta) : 0);
    auto bytes = [&](int s) {
      return fast ? kvq::short_path_workspace_bytes(a->B, a->Hq, a->Nq, a->d, s)
                  : kvq::general_path_workspace_bytes(a->B, a->Hq, a->Hkv, a->Nq, a->d, s, true);
    };
    pl.splits = a->splits > 0 ? a->splits
                : fast        ? kvq::short_fast_splits(a->B, a->Hkv, rows, a->Nc, a->Ncur, cus)
                              : kvq::short_path_splits(a->B, a->Hkv, rows, a->Nc, cus);
    pl.workspace = bytes(pl.splits);
    if (pl.workspace > limit && a->splits == 0) {  // the partials grow linearly with the split count
      const size_t fixed = bytes(1) - kvq::short_path_workspace_bytes(a->B, a->Hq, a->Nq, a->d, 1);
      const size_t per = kvq::short_path_workspace_bytes(a->B, a->Hq, a->Nq, a->d, 1);
      const size_t fit = limit > fixed && per > 0 ? (limit - fixed) / per : 0;
      pl.splits = static_cast<int>(fit < 1 ? 1 : fit < static_cast<size_t>(pl.splits) ? fit : pl.splits);
      while (pl.splits > 1 && bytes(pl.splits) > limit) --pl.splits;  // rounding of the general layout
      pl.workspace = bytes(pl.splits);
    }
  } else if (kvq::fast_kernel_ok(a->d, a->corr, tokens_axis(a), cache_page_size(a))) {  // split-K when it balances
    const int cus = query_device ? device_cu_count() : 256;
    kvq::FastPlan fp = kvq::fast_path_plan(a->B, a->Hq, a->Hkv, a->Nq, a->Nc, a->Ncur, cus, a->splits);
    if (a->splits == 0 && fp.splits > 1 &&
        kvq::fast_path_workspace_bytes(a->B, a->Hq, a->Hkv, a->Nq, fp.splits) > limit) {
      const int64_t units = (a->Nq * (a->Hq / a->Hkv) + 255) / 256 * a->B * a->Hkv;
      fp = kvq::FastPlan{1, units};  // no key-range split: no partials
    }
    pl.splits = fp.splits;
    pl.full_units = fp.full_units;
    pl.workspace = kvq::fast_path_workspace_bytes(a->B, a->Hq, a->Hkv, a->Nq, pl.splits);
  } else {
    pl.workspace = kvq::general_path_workspace_bytes(a->B, a->Hq, a->Hkv, a->Nq, a->d, 1, false);
  }
  return pl;
}

}  // namespace

extern "C" {

const char *kv_status_string(kv_status s) {
  switch (s) {
    case KV_OK: return "ok";
    case KV_ERR_NULL: return "a required pointer is NULL";
    case KV_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case KV_ERR_UNSUPPORTED: return "unsupported bits, group, head dimension, correction or path";
    case KV_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KV_ERR_ALIAS: return "an output or the workspace overlaps an input";
    case KV_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case KV_ERR_SCRATCH: return "the call needs more scratch than the library's static array holds";
  }
  return "unknown status";
}

int32_t kv_version(void) { return kAbiVersion; }

kv_status kv_quantize(const void *x, kv_dtype xdt, int64_t B, int64_t H, int64_t N, int32_t d,
                      const kv_qtensor *dst, int64_t tok_offset, void *stream) {
  if (!x || !dst) return KV_ERR_NULL;
  if (!dst->codes || !dst->scale || !dst->zero) return KV_ERR_NULL;
  if (xdt != KV_BF16 && xdt != KV_F32) return KV_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 0 || tok_offset < 0) return KV_ERR_SHAPE;
  if (B > 65535 || H > 65535) return KV_ERR_UNSUPPORTED;  // grid y and z extents
  if (!head_dim_ok(d)) return KV_ERR_UNSUPPORTED;
  if (dst->bits != 2 && dst->bits != 4) return KV_ERR_UNSUPPORTED;
  if (dst->axis != KV_AXIS_DIM && dst->axis != KV_AXIS_TOKENS) return KV_ERR_UNSUPPORTED;
  if (!tensor_group_ok(dst, d)) return KV_ERR_UNSUPPORTED;
  if (dst->cap < 0 || tok_offset > dst->cap || N > dst->cap - tok_offset) return KV_ERR_SHAPE;
  if (dst->cap > kMaxTokensPerHead) return KV_ERR_UNSUPPORTED;  // the attention would refuse the cache
  if (dst->axis == KV_AXIS_TOKENS &&
      (tok_offset % dst->group != 0 || dst->cap % dst->group != 0 ||
       (dst->page_table && dst->page_size % dst->group != 0)))
    return KV_ERR_SHAPE;
  if (dst->page_table) {
    if (!page_size_ok(dst->page_size) || dst->cap % dst->page_size != 0) return KV_ERR_SHAPE;
    if (dst->num_pages < 1) return KV_ERR_SHAPE;
    if (B * (dst->cap / dst->page_size) > INT32_MAX) return KV_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(dst->page_table) & 3u) != 0) return KV_ERR_ALIGN;
  } else if (dst->page_size != 0 || dst->num_pages != 0) {
    return KV_ERR_SHAPE;
  }
  int64_t t = 0;
  if (!mul_ok(B, H, &t) || !mul_ok(t, N, &t) || !mul_ok(t, d, &t) || t > (int64_t(1) << 40)) return KV_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(dst->codes) || !aligned16(dst->scale) || !aligned16(dst->zero))
    return KV_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(dst->bound) & 3u) != 0) return KV_ERR_ALIGN;
  if (!meta_ok(dst->meta)) return KV_ERR_UNSUPPORTED;
  {  // the input must not overlap the cache it is written into
    const size_t xb = static_cast<size_t>(t) * (xdt == KV_BF16 ? 2 : 4);
    const size_t rows = static_cast<size_t>(tensor_rows(dst, B, H));
    if (overlaps(x, xb, dst->codes, rows * static_cast<size_t>(d * dst->bits / 8)) ||
        overlaps(x, xb, dst->scale, meta_array_bytes(dst, rows, d)) ||
        overlaps(x, xb, dst->zero, meta_array_bytes(dst, rows, d)) ||
        overlaps(x, xb, dst->bound, static_cast<size_t>(B * H) * sizeof(float)))
      return KV_ERR_ALIAS;
  }
  if (N == 0) return KV_OK;
  kvq::QuantizeLaunch p{x, static_cast<int>(xdt), B, H, N, d, dst->codes, static_cast<float *>(dst->scale),
                        static_cast<float *>(dst->zero), dst->bits, dst->group, dst->cap, tok_offset,
                        layout_of(dst), static_cast<int>(dst->meta), dst->axis == KV_AXIS_TOKENS, dst->bound};
  return kvq::launch_quantize(p, static_cast<hipStream_t>(stream)) == hipSuccess ? KV_OK : KV_ERR_HIP;
}

size_t kv_attention_workspace_size(const kv_attn_args *a) {
  if (validate_attention(a) != KV_OK) return 0;
  return plan_attention(a, true).workspace;
}

}  // extern "C"

namespace {

// Launches a validated call with its plan and workspace.
kv_status launch_attention(const kv_attn_args *a, const Plan &pl, void *workspace, void *stream) {
  AttnLaunch p{};
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.Nq = a->Nq; p.Ncur = a->Ncur; p.Nc = a->Nc; p.d = a->d;
  p.q = static_cast<const uint16_t *>(a->q);
  p.k_cur = static_cast<const uint16_t *>(a->k_cur);
  p.v_cur = static_cast<const uint16_t *>(a->v_cur);
  p.out = static_cast<uint16_t *>(a->out);
  if (a->Nc > 0) {
    p.kc_codes = a->k_cache->codes;
    p.kc_scale = static_cast<const float *>(a->k_cache->scale);
    p.kc_zero = static_cast<const float *>(a->k_cache->zero);
    p.vc_codes = a->v_cache->codes;
    p.vc_scale = static_cast<const float *>(a->v_cache->scale);
    p.vc_zero = static_cast<const float *>(a->v_cache->zero);
    p.meta = static_cast<int>(a->k_cache->meta);
    p.ktok = a->k_cache->axis == KV_AXIS_TOKENS;
    p.vtok = a->v_cache->axis == KV_AXIS_TOKENS;
    p.kbits = a->k_cache->bits; p.vbits = a->v_cache->bits; p.group = a->k_cache->group; p.cap = a->k_cache->cap;
    p.layout = layout_of(a->k_cache);
    p.kc_bound = a->k_cache->bound;
    p.vc_bound = a->v_cache->bound;
  } else {
    p.kbits = 2; p.vbits = 2; p.group = a->d; p.cap = 0;
  }
  p.tau = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / sqrtf(static_cast<float>(a->d));
  p.corr = a->corr;
  p.causal = a->causal;
  p.splits = pl.splits;
  p.fast_full_units = pl.full_units;
  p.workspace = workspace;
  if (a->append && a->Ncur > 0) {
    const kv_qtensor *k = a->k_cache, *v = a->v_cache;
    p.app.on = true;
    p.app.codes[0] = k->codes;
    p.app.codes[1] = v->codes;
    p.app.scale[0] = static_cast<float *>(k->scale);
    p.app.scale[1] = static_cast<float *>(v->scale);
    p.app.zero[0] = static_cast<float *>(k->zero);
    p.app.zero[1] = static_cast<float *>(v->zero);
    p.app.bits[0] = k->bits;
    p.app.bits[1] = v->bits;
    p.app.group = k->group;
    p.app.meta = static_cast<int>(k->meta);
    p.app.cap = k->cap;
    p.app.layout = layout_of(k);
    p.app.bound[0] = k->bound;
    p.app.bound[1] = v->bound;
  }
  if (debug_log())
    fprintf(stderr,
            "kvq: attention path=%s rows/kvhead=%lld splits=%d full_units=%lld workspace=%zu corr=%d append=%d\n",
            pl.path == KV_PATH_SHORT ? "short" : "long", static_cast<long long>(a->Nq * (a->Hq / a->Hkv)),
            pl.splits, static_cast<long long>(pl.full_units), pl.workspace, a->corr, p.app.on ? 1 : 0);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = pl.path == KV_PATH_SHORT ? kvq::launch_attention_short(p, s) : kvq::launch_attention_long(p, s);
  return e == hipSuccess ? KV_OK : KV_ERR_HIP;
}

}  // namespace

extern "C" {

kv_status kv_attention_corrected(const kv_attn_args *a, void *stream) {
  const kv_status v = validate_attention(a);
  if (v != KV_OK) return v;
  const Plan pl = plan_attention(a, true);
  if (pl.workspace > 0 && (!a->workspace || a->workspace_bytes < pl.workspace)) return KV_ERR_WORKSPACE;
  if (pl.workspace > 0 && !aligned16(a->workspace)) return KV_ERR_ALIGN;
  if (pl.workspace > 0 && overlaps_call(a, a->workspace, pl.workspace)) return KV_ERR_ALIAS;
  return launch_attention(a, pl, a->workspace, stream);
}

kv_status kv_attention_corrected_static(const kv_attn_args *a, void *stream) {
  const kv_status v = validate_attention(a);
  if (v != KV_OK) return v;
  const Plan pl = plan_attention(a, true, kScratchBytes);
  if (pl.workspace > kScratchBytes) return KV_ERR_SCRATCH;
  void *ws = nullptr;
  if (pl.workspace > 0 && !(ws = scratch_ptr())) return KV_ERR_HIP;
  return launch_attention(a, pl, ws, stream);
}

kv_status kv_attention_diagnostics(const kv_diag_args *a, void *stream) {
  const kv_status v = validate_diagnostics(a);
  if (v != KV_OK) return v;
  kvq::DiagLaunch p{};
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.Nq = a->Nq; p.Ncur = a->Ncur; p.Nc = a->Nc; p.d = a->d;
  p.q = static_cast<const uint16_t *>(a->q);
  p.k_cur = static_cast<const uint16_t *>(a->k_cur);
  p.k_ref = static_cast<const uint16_t *>(a->k_ref);
  if (a->Nc > 0) {
    p.kc_codes = a->k_cache->codes;
    p.kc_scale = static_cast<const float *>(a->k_cache->scale);
    p.kc_zero = static_cast<const float *>(a->k_cache->zero);
    p.meta = static_cast<int>(a->k_cache->meta);
    p.ktok = a->k_cache->axis == KV_AXIS_TOKENS;
    p.kbits = a->k_cache->bits; p.group = a->k_cache->group; p.cap = a->k_cache->cap;
    p.layout = layout_of(a->k_cache);
  } else {
    p.kbits = 2; p.group = a->d; p.cap = 0;
  }
  p.tau = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / sqrtf(static_cast<float>(a->d));
  p.corr = a->corr;
  p.causal = a->causal;
  p.out = a->out;
  return kvq::launch_diagnostics(p, static_cast<hipStream_t>(stream)) == hipSuccess ? KV_OK : KV_ERR_HIP;
}

}  // extern "C"
