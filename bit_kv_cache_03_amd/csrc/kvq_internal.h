// Internal declarations shared by the host entry points (kvq_api.cpp) and the
// gfx950 kernels.  Not part of the ABI; include/kvq.h is.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// Cache layout shared by a launch's cache tensors: contiguous, or paged
// (see kv_qtensor; the page size is a power of two).  Physical row of token
// t of head h of sequence b in a tensor of H heads:
//   contiguous: (b*H + h)*cap + t
//   paged:      (table[b*(cap/P) + t/P]*H + h)*P + t%P
// A tile of 64 tokens starting at a multiple of 64 lies in one page.
struct CacheLayout {
  const int32_t *page_table;  // nullptr: contiguous
  int32_t page_shift;         // log2(page size)
  int32_t pages_per_seq;      // cap / page size
  __host__ __device__ int64_t row(int64_t cap, int64_t H, int64_t b, int64_t h, int64_t t) const {
    if (!page_table) return (b * H + h) * cap + t;
    const int64_t page = page_table[b * pages_per_seq + (t >> page_shift)];
    return ((page * H + h) << page_shift) + (t & ((int64_t(1) << page_shift) - 1));
  }
};

// Storage of a cache tensor's step and zero-point elements (the values of
// kv_meta): fp32, IEEE binary16 or bfloat16.  With 16 bits the float
// pointers of the arrays address 16-bit elements.
constexpr int kMetaF32 = 0, kMetaF16 = 1, kMetaBF16 = 2;

// A 16-bit step or zero-point element of kind mk as fp32 (exact: a bfloat16
// pattern is the upper half of the fp32 one).
__host__ __device__ inline float meta16_value(uint16_t h, int mk) {
  if (mk == kMetaBF16) return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// The 16-bit pattern of kind mk nearest to x (ties to even), as stored.
// bfloat16: adding 0x7fff plus the kept half's lowest bit to the fp32 bits
// carries into the kept half exactly when the dropped half exceeds one half
// of its unit, or equals it with an odd kept half (NaN stays a quiet NaN).
__host__ __device__ inline uint16_t meta16_bits(float x, int mk) {
  if (mk == kMetaBF16) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// The stored value of an fp32 step or zero point.
__host__ __device__ inline float meta_round(float x, int mk) {
  return mk == kMetaF32 ? x : meta16_value(meta16_bits(x, mk), mk);
}

// Metadata element i of a step or zero-point array of kind mk.
__host__ __device__ inline float meta_at(const float *p, int64_t i, int mk) {
  return mk == kMetaF32 ? p[i] : meta16_value(reinterpret_cast<const uint16_t *>(p)[i], mk);
}

// Everything a quantize launch needs, already validated by the host.
struct QuantizeLaunch {
  const void *x;
  int xdt;  // kv_dtype
  int64_t B, H, N;
  int32_t d;
  uint8_t *codes;
  float *scale;
  float *zero;
  int32_t bits, group;
  int64_t cap, off;
  CacheLayout layout;
  int meta;     // kind of the scale and zero arrays (kMetaF32 / kMetaF16 / kMetaBF16)
  bool tokens;  // groups along the tokens: scale/zero [row / group][d], row the cache row
  float *bound;  // [B][H] running bound of |z|, |z + top D| (atomic max), or nullptr
};

// The chunk append an attention call may carry: K_cur and V_cur quantised
// into rows [Nc, Nc + Ncur) of the caches (index 0: K, 1: V), groups along
// the head dimension, in the workgroups of a pre-pass or in extra
// workgroups of the attention launch (ids wg0 .. wg0 + wgs - 1).
struct AppendLaunch {
  bool on;
  uint8_t *codes[2];
  float *scale[2], *zero[2];  // 16-bit arrays unless meta is kMetaF32
  int32_t bits[2];
  int32_t group;
  int meta;  // kind of the caches' scale and zero arrays
  int64_t cap;
  CacheLayout layout;
  float *bound[2];  // the caches' running bounds [B][Hkv], or nullptr
  int64_t wg0;  // set by the launcher that adds append workgroups
  int32_t wgs;
};

// Everything an attention launch needs, already validated by the host.
struct AttnLaunch {
  int64_t B, Hq, Hkv, Nq, Ncur, Nc;
  int32_t d;
  const uint16_t *q, *k_cur, *v_cur;
  uint16_t *out;
  const uint8_t *kc_codes, *vc_codes;
  const float *kc_scale, *kc_zero, *vc_scale, *vc_zero;
  const float *kc_bound, *vc_bound;  // running bounds [B][Hkv] of the caches, or nullptr (scan the metadata)
  int32_t kbits, vbits, group;
  int64_t cap;
  CacheLayout layout;  // of both caches
  int meta;            // kind of both caches' scale and zero arrays (kMetaF32 / kMetaF16 / kMetaBF16)
  bool ktok, vtok;     // K / V groups along the tokens (per channel): scale/zero [row >> log2 group][d]
  float tau;   // resolved softmax scale
  int corr;    // kv_corr
  int causal;  // 1: current key i visible to query row j only if i <= j + Ncur - Nq
  int splits;  // resolved key-range split count
  int64_t fast_full_units;  // throughput kernel: work units run unsplit before the split ones
  void *workspace;
  AppendLaunch app;
};

// Split path partials: per (split, query row) the unnormalised O[d] then the
// running max (exp2 domain) and sum, padded to keep rows 16-byte aligned.
constexpr __host__ __device__ int64_t kPartialStride(int32_t d) { return d + 4; }

hipError_t launch_quantize(const QuantizeLaunch &p, hipStream_t stream);
hipError_t launch_attention_long(const AttnLaunch &p, hipStream_t stream);
// The general kernel over caches grouped along the tokens (split: the
// short-query path's key-range split), built in attention_tokens.hip.
hipError_t launch_attention_tokens(const AttnLaunch &p, hipStream_t stream, bool split);
hipError_t launch_attention_short(const AttnLaunch &p, hipStream_t stream);
// Throughput kernel (attention_fast.hip): head dim 128, correction off or
// Taylor.  Its workspace holds the split partials (when splits > 1, laid out
// as on the short path), then 32 fp32 partial key bounds and 32 partial
// query bounds per (b, KV head).
bool fast_path_supported(const AttnLaunch &p);
// The throughput kernel: d = 128, correction off or Taylor, groups along the
// head dimension, and (paged) pages that hold whole 64-key tiles.  The
// host's plan and the device dispatch both decide with this.
inline bool fast_kernel_ok(int32_t d, int corr, bool tokens_axis, int32_t page_size) {
  return d == 128 && corr != KV_CORR_EXACT && !tokens_axis && (page_size == 0 || page_size >= 64);
}
// Page size of a launch's layout (0: contiguous).
inline int32_t layout_page_size(const CacheLayout &l) { return l.page_table ? (1 << l.page_shift) : 0; }
size_t fast_path_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int splits);
int fast_path_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nc, int64_t Ncur, int cu_count);
struct FastPlan {
  int splits;          // key ranges of each split work unit
  int64_t full_units;  // leading (b, KV head, 256-row block) units that run unsplit
};
FastPlan fast_path_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nc, int64_t Ncur, int cu_count,
                        int forced);
hipError_t launch_attention_fast(const AttnLaunch &p, hipStream_t stream);
// The same with the causal mask (built in attention_fast_causal.hip), over
// a paged cache (attention_fast_paged.hip), and both
// (attention_fast_paged_causal.hip).
hipError_t launch_attention_fast_causal(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_paged_causal(const AttnLaunch &p, hipStream_t stream);
// Binary16 steps and zero points: the same four variants
// (attention_fast_m16*.hip); bfloat16 ones: attention_fast_mb16*.hip.
hipError_t launch_attention_fast_m16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_m16_causal(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_m16_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_m16_paged_causal(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_mb16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_mb16_causal(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_mb16_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_fast_mb16_paged_causal(const AttnLaunch &p, hipStream_t stream);
// Pre-pass of the throughput kernel: per (b, KV head), 32 partial bounds of
// |key| (dequantised cache and current chunk) and of |query|, from which the
// kernel takes the exponent that balances its fp16 key and query operands.
void launch_key_scale(const AttnLaunch &p, hipStream_t stream, float *part);

// Short path: cached-token split count chosen for a problem and the
// workspace it needs (partials of every split for every query row).
int short_path_splits(int64_t B, int64_t Hkv, int64_t rows_per_kvhead, int64_t Nc, int cu_count);
size_t short_path_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int32_t d, int splits);
// General kernel (attention.hip; head dim 64, the exact form, groups along
// the tokens, small pages): its workspace holds the split partials (split:
// the short path's key-range split), then, from a 256-byte boundary, 32
// fp32 partial bounds of |value| per (b, KV head) written by its pre-pass.
size_t general_bound_offset(int64_t B, int64_t Hq, int64_t Nq, int32_t d, int splits, bool split);
size_t general_path_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int32_t d, int splits,
                                    bool split);
// Log-sum-exp merge of split partials into the bf16 output.
hipError_t launch_combine(const float *ws, uint16_t *out, int64_t nrows, int splits, int32_t d, hipStream_t stream);
// Short-query kernel (attention_short.hip): head dim 128, correction off or
// Taylor; workspace = the split partials.
bool short_fast_supported(int32_t d, int corr, bool tokens_axis, int32_t page_size);
int short_fast_splits(int64_t B, int64_t Hkv, int64_t rows_per_kvhead, int64_t Nc, int64_t Ncur, int cu_count);
hipError_t launch_attention_short_fast(const AttnLaunch &p, hipStream_t stream);
// The same over a paged cache, with binary16 metadata, and both (built in
// attention_short_paged.hip, attention_short_m16.hip,
// attention_short_m16_paged.hip); with bfloat16 metadata
// (attention_short_mb16.hip, attention_short_mb16_paged.hip).
hipError_t launch_attention_short_fast_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short_fast_m16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short_fast_m16_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short_fast_mb16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short_fast_mb16_paged(const AttnLaunch &p, hipStream_t stream);
// The short-query kernel on 16-row query tiles (attention_short16.hip), for
// at most 16 query rows per KV head; its paged, binary16 and paged binary16
// instances in attention_short16_paged.hip, attention_short16_m16.hip,
// attention_short16_m16_paged.hip, the bfloat16 ones in
// attention_short16_mb16*.hip.  Same workspace and split count.
hipError_t launch_attention_short16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_m16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_m16_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_mb16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_mb16_paged(const AttnLaunch &p, hipStream_t stream);
// The 16-row kernel over caches grouped along the tokens (K, V or both):
// whether it serves a call, its dispatch over the layout and metadata kind,
// and the instances (attention_short16_ktok*.hip: K along the tokens, V
// along the head dimension; attention_short16_vtok*.hip: V along the tokens,
// fp32 metadata).  Same workspace and split count as the short-query kernels.
bool short16_tok_supported(int32_t d, int corr, bool ktok, bool vtok, int32_t page_size, int meta,
                           int64_t rows_per_kvhead);
hipError_t launch_attention_short16_tok(const AttnLaunch &p, hipStream_t stream);
// The 32-row kernel over caches grouped along the tokens (fp32 metadata;
// attention_short_tok*.hip), for calls the 16-row kernel does not take.
bool short_tok_supported(int32_t d, int corr, bool ktok, bool vtok, int32_t page_size, int meta);
hipError_t launch_attention_short_tok(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short_tok_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_vtok(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_vtok_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_ktok(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_ktok_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_ktok_m16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_ktok_m16_paged(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_ktok_mb16(const AttnLaunch &p, hipStream_t stream);
hipError_t launch_attention_short16_ktok_mb16_paged(const AttnLaunch &p, hipStream_t stream);

// Everything a diagnostics launch needs, already validated by the host.
struct DiagLaunch {
  int64_t B, Hq, Hkv, Nq, Ncur, Nc;
  int32_t d;
  const uint16_t *q, *k_cur, *k_ref;
  const uint8_t *kc_codes;
  const float *kc_scale, *kc_zero;
  int32_t kbits, group;
  int64_t cap;
  CacheLayout layout;
  int meta;   // kind of the K cache's scale and zero arrays
  bool ktok;  // the K cache groups along the tokens (per channel)
  float tau;   // resolved softmax scale
  int corr;    // kv_corr
  int causal;
  kv_diag_row *out;
};
// Attention-balance statistics (diagnostics.hip).
hipError_t launch_diagnostics(const DiagLaunch &p, hipStream_t stream);

}  // namespace kvq
