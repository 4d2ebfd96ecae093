/*
 * kvq.h -- C ABI of libkvq.so: Jensen-bias-corrected attention over a
 * group-wise INT2/INT4 KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *  - "量化鍵值偷走注意力：針對 KV-Cache 的 Jensen 偏差校正還原影片擴散品質"
 *    (agents-report.net), sections 問題 and 方法: keys and values of earlier
 *    chunks are cached at INT4/INT2; the exponential in softmax turns the
 *    zero-mean rounding noise of cached keys into an upward bias of their
 *    weight; each cached-key score gets b_i = log E[exp(delta_i)] subtracted,
 *    in practice its second-order form (1/(24 d)) sum_c q_c^2 D_{i,c}^2,
 *    built from per-group query squared norms and the keys' step sizes.
 *    Section 為何校正有效: b is subtracted from the quantised keys' scores
 *    before the softmax; current-chunk scores are left alone.
 *  - "Quantized Keys Steal Attention: Bias Correction for KV-Cache
 *    Compression in Video Diffusion" (fugumt.com), Abstract: the correction is
 *    computed on the fly from the cached keys' step sizes and the query norm,
 *    with no memory beyond the cache.
 *  - "QuantWM：保住时间一致性的两比特键值缓存量化" (pchao.org), section
 *    方法概览: each cache block is quantised once after it is built;
 *    section 研究缺口, Eq. (5): logits are Q K^T / sqrt(d).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library never allocates, frees or retains them and keeps no state
 *    between calls; concurrent calls on different streams are safe.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is only enqueued there; calls return before it completes.
 *  - Arguments are validated on the host before any HIP call; an invalid call
 *    returns an error and touches no memory.  Launch failures return
 *    KV_ERR_HIP.  A device fault surfaces at the caller's next
 *    synchronisation.
 *  - Tensors are dense and row-major in the shapes given; every pointer must
 *    be 16-byte aligned.
 *  - NaN or Inf inputs, and groups whose range max-min overflows fp32, are
 *    outside the contract.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are 32-bit integers.  C++ sees them with that fixed
 * underlying type, so any int32 value a caller passes (including the
 * values that the entry points refuse) is a valid value of the type. */
#ifdef __cplusplus
#define KV_ENUM_TYPE : int32_t
#else
#define KV_ENUM_TYPE
#endif

typedef enum KV_ENUM_TYPE {
  KV_OK = 0,
  KV_ERR_NULL = 1,        /* a required pointer is NULL */
  KV_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  KV_ERR_UNSUPPORTED = 3, /* valid but not implemented (bits, group, d, path) */
  KV_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  KV_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
  KV_ERR_ALIAS = 6,       /* an output or the workspace overlaps an input (or each other) */
  KV_ERR_HIP = 7,         /* a HIP runtime call or launch failed */
  KV_ERR_SCRATCH = 8      /* kv_attention_corrected_static: the call needs more scratch
                             than KV_STATIC_SCRATCH_BYTES */
} kv_status;

typedef enum KV_ENUM_TYPE { KV_BF16 = 0, KV_F32 = 1 } kv_dtype;

/* Correction applied to cached-key logits. */
typedef enum KV_ENUM_TYPE {
  KV_CORR_OFF = 0,    /* plain softmax over [dequantised cache ; current chunk] */
  KV_CORR_TAYLOR = 1, /* b = (tau^2/24) sum_g D_g^2 ||q_g||^2  (page 方法 formula) */
  KV_CORR_EXACT = 2   /* b = sum_c log(sinh x_c / x_c), x_c = tau q_c D_{g(c)} / 2:
                         the uniform-noise closed form; slow path, no perf target */
} kv_corr;

/* Storage type of a cache tensor's step D and zero point z. */
typedef enum KV_ENUM_TYPE {
  KV_META_F32 = 0, /* fp32 (default) */
  KV_META_F16 = 1, /* IEEE binary16: D and z rounded (nearest, ties to even) before
                      the codes are taken, so that z + D c uses what is stored; 2x less
                      metadata (INT2/INT2 at group 64 and d = 128: 80 instead of 96 bytes
                      per token per head); |values| must stay below 65504 */
  KV_META_BF16 = 2 /* bfloat16: the same rounding rule and size as binary16 with fp32's
                      range and 8 significant bits (D and z are each within 2^-9 of
                      their fp32 values, relatively; the codes follow the rounded grid) */
} kv_meta;

/* Axis along which a cache tensor's groups run (agents-report.net page,
 * §方法: the correction uses one step per group or per channel, D_{i,c}). */
typedef enum KV_ENUM_TYPE {
  KV_AXIS_DIM = 0,    /* along the head dimension (default): one D, z per token and
                         group of `group` channels; scale/zero [..][cap][d/group] */
  KV_AXIS_TOKENS = 1  /* along the tokens, per channel: one D, z per channel and group
                         of `group` consecutive tokens (the first at a multiple of
                         `group`); scale/zero [B][H][cap/group][d], paged
                         [num_pages][H][page_size/group][d].  The bias of key i then
                         uses D_{i/group, c} channel by channel.  Attention over such
                         a cache runs on the general kernel */
} kv_axis;

/* Kernel path.  AUTO picks by rows per KV head; tests may force either. */
typedef enum KV_ENUM_TYPE {
  KV_PATH_AUTO = 0,  /* SHORT for at most 64 query rows per KV head, and for caches grouped
                        along the tokens that the short-query kernels take; else LONG */
  KV_PATH_LONG = 1,  /* MFMA tile kernel, query rows tiled, one pass over keys */
  KV_PATH_SHORT = 2  /* split over cached tokens + log-sum-exp combine */
} kv_path;

/*
 * One quantised cache tensor (K or V) of B x H heads and `cap` token slots.
 * Group-wise asymmetric uniform quantisation along the head dimension:
 * token row of d values, groups of `group` consecutive values, per group
 *   step  D = fl32(fl32(max - min) / (2^bits - 1)),   zero z = min
 *   code  c = clamp(round_half_even(fl32(fl32(x - min) / D)), 0, 2^bits - 1)
 *         (c = 0 when D == 0; a zero min or max is taken as +0)
 *   value x^ = z + D * c.
 * Codes are packed LSB-first: element k of a row lives in byte
 * floor(k*bits/8) at bit (k*bits) mod 8.
 */
typedef struct {
  uint8_t *codes; /* [B][H][cap][d*bits/8] bytes (paged: the pool, see below) */
  void *scale;    /* [B][H][cap][d/group]  step D (fp32 or binary16, see `meta`) */
  void *zero;     /* [B][H][cap][d/group]  zero-point z (the group minimum, rounded like D) */
  int32_t bits;   /* 2 or 4 */
  int32_t group;  /* 32, 64 or 128; divides d */
  int64_t cap;    /* token capacity per head, at most 2^23 */
  /* Paged layout (page_table != NULL): tokens live in pages of page_size
   * tokens of all H heads of one sequence.  codes, scale and zero then point
   * to pools of num_pages pages, [num_pages][H][page_size][row], and token t
   * of (b, h) is pool row (page_table[b*(cap/page_size) + t/page_size]*H + h)
   * *page_size + t % page_size.  page_table is a DEVICE int32 array
   * [B][cap/page_size] whose entries must lie in [0, num_pages) (not
   * checked: device data); pages of different blocks may not coincide where
   * a call writes.  page_size is a power of two, at least 16, and divides
   * cap.  Attention over pages of fewer than 64 tokens (32 on the short-query
   * path) runs on the general kernel, which looks up every row.  NULL, with page_size and num_pages 0: the contiguous layout above. */
  const int32_t *page_table;
  int32_t page_size;
  int32_t num_pages;
  int32_t meta;   /* kv_meta of scale and zero; K and V caches of one call share it */
  int32_t axis;   /* kv_axis; KV_AXIS_TOKENS needs cap (and page_size) to be multiples
                     of group; K and V may differ */
  /* Optional running bound, NULL or a DEVICE fp32 array [B][H] (4-byte
   * aligned): for every (b, h), at least max(|z|, |z + (2^bits - 1) D|) over
   * the groups of every row written so far, i.e. a bound on |x^|.
   * kv_quantize and the fused append raise it (atomic max, never lower it);
   * the attention calls read it to pick their fp16 scales instead of
   * scanning every step and zero point of rows [0, Nc).  It must start at 0
   * (or any value at least the bound of the rows already present), and be
   * reset to 0 when the cache is refilled from scratch; a value below the
   * true bound is outside the contract (fp16 overflow of the scaled keys or
   * values).  With NULL the attention scans the metadata. */
  float *bound;
} kv_qtensor;

/*
 * kv_quantize -- quantise N new tokens of every (b, h) and store them in
 * cache rows [tok_offset, tok_offset + N): how a finished chunk is appended
 * (QuantWM page, 方法概览: each block is quantised once after it is built).
 *
 *   x    : [B][H][N][d], bf16 (xdt = KV_BF16) or fp32 (KV_F32), device.
 *   dst  : host pointer to the descriptor of the destination cache.
 * d must be 64 or 128; B and H at most 65535.  N = 0 is a no-op.  Output is bit-exact with the
 * definition above (IEEE fp32 division, round half to even).
 * KV_AXIS_TOKENS: tok_offset must be a multiple of group; the tokens of the
 * call form groups [tok_offset + j*group, +group), the last one shorter when
 * group does not divide N (quantised over the tokens it has; it cannot be
 * extended later: the next call starts at the next multiple of group).
 * Errors: KV_ERR_NULL, KV_ERR_SHAPE (tok_offset + N > cap, tok_offset not a
 * multiple of a token group, ...), KV_ERR_UNSUPPORTED (bits, group, d, axis,
 * cap above 2^23 tokens: no attention call would accept the cache),
 * KV_ERR_ALIGN, KV_ERR_ALIAS (x overlaps the cache's codes, steps or zero
 * points), KV_ERR_HIP.
 */
kv_status kv_quantize(const void *x, kv_dtype xdt, int64_t B, int64_t H, int64_t N, int32_t d,
                      const kv_qtensor *dst, int64_t tok_offset, void *stream);

/*
 * Arguments of one corrected-attention call.  For query head h (KV head
 * hk = h / (Hq/Hkv)) and query row j, with tau = softmax_scale (0 -> 1/sqrt(d)):
 *   cached  logits  s_i = tau q.x^_i - b_i   for i <  Nc  (b per `corr`)
 *   current logits  s_i = tau q.k_i          for i <  Ncur (never corrected)
 *   out = softmax over both segments together, applied to [v^ ; v_cur]
 * Values get no correction (they enter the output linearly).  By default
 * there is no mask (chunk-wise video generation: every query sees every
 * key).  With `causal` = 1 the current chunk is masked causally, aligned to
 * its end: query row j sees current keys i <= j + Ncur - Nq (and the whole
 * cache), as in chunked prefill where the chunk's queries are its last Nq
 * tokens.
 */
typedef struct {
  int64_t B, Hq, Hkv; /* Hq % Hkv == 0 */
  int64_t Nq;         /* query rows per head, >= 1 */
  int64_t Ncur;       /* current-chunk tokens, 0 .. 2^23 */
  int64_t Nc;         /* cached tokens in use (rows [0, Nc) of the caches), 0 .. 2^23 */
  int32_t d;          /* head dimension: 64 or 128 */
  const void *q;      /* bf16 [B][Hq][Nq][d] */
  const void *k_cur;  /* bf16 [B][Hkv][Ncur][d] (may be NULL if Ncur == 0) */
  const void *v_cur;  /* bf16 [B][Hkv][Ncur][d] (may be NULL if Ncur == 0) */
  const kv_qtensor *k_cache; /* host pointers to descriptors; may be NULL if Nc == 0 */
  const kv_qtensor *v_cache; /* both with the same group, cap and layout (the same page
                                table and page size when paged) */
  void *out;          /* bf16 [B][Hq][Nq][d], overwritten; must not overlap inputs */
  float softmax_scale; /* tau; 0 -> 1/sqrt(d); the correction uses tau^2/24 */
  int32_t corr;       /* kv_corr */
  int32_t path;       /* kv_path */
  int32_t splits;     /* key-range splits, 0 = automatic, at most 1024: the short path,
                         and the long path for d = 128 with correction off or Taylor
                         (clamped to the number of 64-key tiles) */
  int32_t causal;     /* 0: no mask; 1: causal within the current chunk, end-aligned
                         (every query row must then see a key: Nc > 0 or Ncur >= Nq) */
  void *workspace;    /* device scratch of kv_attention_workspace_size() bytes */
  size_t workspace_bytes;
  int32_t append;     /* 0: the caches are only read.  1: the call also quantises the
                         chunk into rows [Nc, Nc + Ncur) of the caches, exactly as
                         kv_quantize(k_cur, KV_BF16, B, Hkv, Ncur, d, k_cache, Nc) and
                         the same for v_cur and v_cache write them (each block is
                         quantised once, after it is built: "QuantWM：…" (pchao.org),
                         section 方法概览).  Needs both caches (also when Nc = 0),
                         grouped along the head dimension, with cap >= Nc + Ncur.  The
                         attention itself reads rows [0, Nc) only, so its result is
                         the same with or without the append; on a paged cache no
                         page that rows [0, Nc) use may also hold rows being written. */
  int32_t reserved;   /* must be 0 */
} kv_attn_args;

/* Bytes of device workspace the call needs: on the short path the
 * per-split partial results (splits x B*Hq*Nq rows of d+4 floats); on the
 * long path with d = 128 and correction off or Taylor, the same partials
 * when it splits the key range (more than one split), then 96 fp32 partial
 * key, value and query bounds per (b, KV head) rounded up to 256 bytes;
 * on the general kernel (d = 64, the exact form, groups along the tokens,
 * pages smaller than a tile) 32 fp32 partial value bounds per (b, KV head),
 * after the short path's partials rounded up to 256 bytes.  The
 * contents need no initialisation and are meaningless after the call.
 * Returns 0 for invalid arguments as well; kv_attention_corrected reports
 * those. */
size_t kv_attention_workspace_size(const kv_attn_args *a);

/*
 * kv_attention_corrected -- the hot path: one call computes `out` for all
 * B x Hq x Nq query rows in a single fused pass over the packed cache and the
 * bf16 current chunk (dequantisation, scores, correction, softmax and the
 * value product all inside the kernel).
 * Errors: KV_ERR_NULL, KV_ERR_SHAPE (also: causal with Nc = 0 and
 * Nq > Ncur; with append, cap < Nc + Ncur), KV_ERR_UNSUPPORTED (also: causal
 * or append not 0 or 1, reserved not 0, append to a cache grouped along the
 * tokens), KV_ERR_WORKSPACE, KV_ERR_ALIGN, KV_ERR_ALIAS (out overlaps an
 * input, or the bytes of the workspace the call uses overlap out, an input
 * or a page table; with append, q, k_cur, v_cur, out or the workspace
 * overlaps a cache array, or the K and V caches' arrays overlap), KV_ERR_HIP.
 */
kv_status kv_attention_corrected(const kv_attn_args *a, void *stream);

/* Bytes of the static device scratch array of kv_attention_corrected_static
 * (one copy per GPU the library runs on, held until the process ends). */
#define KV_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * kv_attention_corrected_static -- kv_attention_corrected for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same computation and kernels;
 * a->workspace and a->workspace_bytes are ignored and the scratch is a
 * file-scope device array of KV_STATIC_SCRATCH_BYTES in the library.  The
 * call allocates and frees nothing (its device address is looked up once
 * per GPU, on the first call with that GPU current).
 *  - Splits chosen automatically (a->splits = 0) are lowered where the
 *    partials of the usual choice would not fit the array; a forced split
 *    count, or a call whose scratch does not fit even unsplit, returns
 *    KV_ERR_SCRATCH (kv_attention_workspace_size() reports what
 *    kv_attention_corrected would use).
 *  - Every call on one GPU uses that GPU's one array, and the scratch needs
 *    no initialisation: calls on one stream are safe, calls that may overlap
 *    in time on one GPU (other streams, other host threads) race.
 * Errors: those of kv_attention_corrected except KV_ERR_WORKSPACE, and
 * KV_ERR_SCRATCH; KV_ERR_HIP also when the array's address cannot be found.
 */
kv_status kv_attention_corrected_static(const kv_attn_args *a, void *stream);

/*
 * Attention-balance diagnostics ("量化鍵值偷走注意力…" (agents-report.net),
 * section 問題: rounding noise on cached keys raises their share of the
 * softmax through the exponential's convexity, so attention moves from the
 * current chunk to the cache; section 為何校正有效: subtracting b restores
 * the balance).  For every query row the softmax over the cached keys
 * before quantisation (k_ref, bf16) is compared with the softmax the
 * corrected attention uses (the quantised cache with `corr`); the current
 * chunk's keys are the same in both.  With logits l (natural log units,
 * tau as in kv_attn_args, the same mask):
 *   lse   = log sum_i exp(l_i) over the visible keys,
 *   mass  = sum over visible current keys of exp(l_i - lse),
 *   kl    = KL(p_ref || p_q) = sum_i p_ref,i log(p_ref,i / p_q,i),
 *   top   = the 5 largest logits' key indices, descending, ties to the lower
 *           index; index i < Nc is cached key i, Nc + j is current key j;
 *           -1 past the number of visible keys.
 * One record per query row, rows in [B][Hq][Nq] order; 64 bytes.
 */
typedef struct {
  float lse_ref, lse_q;
  float mass_ref, mass_q;
  float kl;
  int32_t top_ref[5];
  int32_t top_q[5];
  int32_t reserved; /* written as 0 */
} kv_diag_row;

typedef struct {
  int64_t B, Hq, Hkv, Nq, Ncur, Nc; /* as in kv_attn_args (Nc >= 1 or Ncur >= 1) */
  int32_t d;          /* 64 or 128 */
  int32_t corr;       /* kv_corr applied to the quantised cached logits */
  const void *q;      /* bf16 [B][Hq][Nq][d] */
  const void *k_cur;  /* bf16 [B][Hkv][Ncur][d] (may be NULL if Ncur == 0) */
  const void *k_ref;  /* bf16 [B][Hkv][Nc][d]: the cached keys before quantisation
                         (may be NULL if Nc == 0) */
  const kv_qtensor *k_cache; /* host pointer to the quantised keys' descriptor */
  float softmax_scale; /* tau; 0 -> 1/sqrt(d) */
  int32_t causal;     /* as in kv_attn_args */
  kv_diag_row *out;   /* [B*Hq*Nq] records, overwritten; must not overlap inputs */
} kv_diag_args;

/*
 * kv_attention_diagnostics -- the statistics above for every query row, one
 * pass over both key sets (scores only, no value product).  A measurement
 * tool beside the hot path, not part of it.
 * Errors: KV_ERR_NULL, KV_ERR_SHAPE, KV_ERR_UNSUPPORTED (d, bits, group,
 * corr, causal), KV_ERR_ALIGN, KV_ERR_ALIAS, KV_ERR_HIP.
 */
kv_status kv_attention_diagnostics(const kv_diag_args *a, void *stream);

/* Static English description of a status code. */
const char *kv_status_string(kv_status s);

/* ABI version (bumped on any change to these declarations). */
int32_t kv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
