// Throughput kernel of the corrected attention for gfx950 (head dim 128,
// correction off or Taylor): the computation of attn_tile_kernel in
// attention.hip, reorganised for MI355X.
//
// Work split: one workgroup = 8 waves = 256 query rows of one KV head (GQA
// rows of all its query heads packed together), 32 rows per wave; two waves
// per SIMD, so the vector ALU of a SIMD is fed by two instruction streams.
// When the row blocks alone would leave the last round of workgroups
// partly empty, the key range is also split (split-K): each split takes a
// contiguous share of the 64-key tiles of [cache ; current chunk] and writes
// unnormalised partials that attn_combine_kernel merges.  Workgroup ids
// are remapped so that all row blocks of one KV head and split run on one
// XCD and share its L2.
//
// Keys enter the Q K^T product as fp16 with the softmax scale folded in:
// cached keys are dequantised in fp32 as (z + D c) tau log2(e) 2^-ek and
// rounded once to fp16 (11-bit significand, ~8x finer than a bf16 rounding,
// which moved the scores of large-step groups too much); queries enter as
// q 2^ek, exact for bf16 input.  The scores then come out of the MFMA in the
// exp2 domain.  A pre-pass (key_scale_kernel) bounds |k| and |q| per KV head,
// and ek balances the two so both operands stay in fp16 range (keys below
// 2^15 always; queries are clamped there, which only a product
// |q| |k| tau log2(e) beyond ~2^29 can reach).  Values and probabilities
// are fp16 as well: the pre-pass also bounds |v| per KV head, values enter
// as v 2^-ev with |v| 2^-ev below 2^15, and the epilogue multiplies O by
// 2^ev (bf16 values moved the outputs of short INT2 caches with large steps
// past the mean tolerance).
//
// Per 64-key tile, software-pipelined across tiles inside each wave:
//   1. S_t = K_t Q^T - m (fp16 MFMA, then one bf16 step)  with
//      exponentials of tile t-1 (VALU)
//   2. O += V_{t-1}^T P_{t-1}^T   with  dequantisation of tile t+1 into LDS,
//                                       the HBM fetch of t+2
// The running max m of each row enters the score MFMAs through the extra
// bf16 step (below), so an exponential is exp2 of the accumulator itself.
// m starts at 0 and moves only when a row's sum would leave [2^-10, 2^40]
// or a probability overflows fp16 (see fix_growth): fp16 probabilities stay
// out of the subnormals and fp32 O and l keep their relative precision over
// that range, so no per-tile max is needed.
// K tiles are double-buffered and V tiles triple-buffered in LDS; one
// barrier per tile.  Keys past the end of a segment are fetched as copies
// of its last key: their scores equal that key's, so the tile max is
// unchanged, and only their probabilities are zeroed.
//
// Jensen-bias correction ("量化鍵值偷走注意力…" (agents-report.net), §方法:
// b = (1/(24 d)) sum_c q_c^2 D_{i,c}^2; §為何校正有效: subtracted from the
// quantised keys' scores before softmax): one extra K=16 bf16 MFMA step per
// 32x32 score block, accumulated into the same fp32 scores, with operands
// [tau^2/24 log2(e) ||q_g||^2] per query and [-D_g^2] per cached key, each
// split into bf16 hi and lo parts, in slots 4g+{0,1,2}.  Slots 3 and 7 carry
// the running max: 1.0 on every key, -m (hi, lo) on the query side.  The
// step runs with the correction off too (then only the max slots are set).
//
// MFMA lane layouts (32x32x16, wave64): A operand lane l holds row l%32 and
// k-slots 8*(l/32)..+7, B operand column l%32 and the same k-slots, the
// fp32 result column l%32 and rows 8*(i/4) + 4*(l/32) + i%4.  With S^T
// (keys as rows) each lane owns one query: row max and sum are local plus
// one exchange with lane l^32, and the P operand is the score accumulator
// itself; V^T is stored in LDS in the matching permuted key order.
//
// The causal-mask instances are built from this file in a translation unit
// of their own (attention_fast_causal.hip defines KVQ_FAST_CAUSAL to 1):
// compiled next to the unmasked ones, they changed how those were
// optimised (query operands spilled inside the tile loop).  The paged-cache
// instances likewise (attention_fast_paged.hip and
// attention_fast_paged_causal.hip: KVQ_FAST_PAGED), and those reading
// binary16 steps and zero points (attention_fast_m16*.hip: KVQ_FAST_META16):
// one variant per file.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "quant_device.h"

#ifndef KVQ_FAST_CAUSAL
#define KVQ_FAST_CAUSAL 0
#endif
#ifndef KVQ_FAST_PAGED
#define KVQ_FAST_PAGED 0
#endif
#ifndef KVQ_FAST_META16
#define KVQ_FAST_META16 0
#endif

namespace kvq {
namespace {

using namespace dev;

constexpr int D = 128;
constexpr int BM = 256;        // query rows per workgroup
constexpr int BN = 64;         // keys per tile
constexpr int THREADS = 512;   // 8 waves, 32 rows each
constexpr int KS = D + 16 + 8; // K row in LDS: fp16 values[128], bf16 corr[16], pad[8]
constexpr int KEXT = D;
constexpr int VS = BN + 8;     // V^T row in LDS (bf16)
constexpr int KBUF = BN * KS;  // 16-bit elements per K buffer
constexpr int VBUF = D * VS;   // 16-bit elements per V buffer
constexpr int NVBUF = 3;

// Step / zero-point arrays: fp32, or the 16-bit kind KVQ_FAST_META16 names in
// its units (1 binary16, 2 bfloat16; the float pointers then address 16-bit
// elements).
constexpr int kMeta = KVQ_FAST_META16;
template <int MT, typename I>
__device__ inline float meta_ld(const float *p, I i) {
  if (MT != kMetaF32) return meta16_value(reinterpret_cast<const uint16_t *>(p)[i], MT);
  return p[i];
}
template <int MT>
__device__ inline const float *meta_adv(const float *p, int64_t n) {
  return reinterpret_cast<const float *>(reinterpret_cast<const char *>(p) + n * (MT ? 2 : 4));
}

// V^T element (row = head-dim index, col = permuted key slot 0..63).  The
// 16-byte chunks of a row are XOR-swizzled by (row / 16) % 8, which spreads
// the transposed 4-byte stores of unpack_v over the banks; operand reads
// stay 16-byte aligned.
__device__ inline int vt_index(int row, int col) {
  return row * VS + ((((col >> 3) ^ (row >> 4)) & 7) << 3) + (col & 7);
}

// ---- pre-pass: fp16 scales of the keys and queries of each KV head --------
// Dequantised cached keys lie between z and z + (2^bits - 1) D of their
// group (the two ends of the code range), so their bound needs only the
// step and zero arrays; current keys and the queries (the gq query heads of
// the KV head) are scanned directly, and values the same way as keys.  Each
// KV head's rows are split over KCHUNKS workgroups, each writing the
// largest |key|, |query| and |value| of its share
// (part[(3 bkv + 0|1|2) KCHUNKS + chunk]); the attention kernel reduces the
// partial bounds.
constexpr int KCHUNKS = 32;

template <int NT>
__device__ inline float bf16_bound(const uint16_t *x, int64_t lo, int64_t hi, int tid) {  // 8-value chunks
  float b = 0.f;
  for (int64_t i = lo + tid; i < hi; i += NT) {
    const uint4 w = reinterpret_cast<const uint4 *>(x)[i];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) b = fmaxf(b, fmaxf(fabsf(lo_f(u[j])), fabsf(hi_f(u[j]))));
  }
  return b;
}
template <int NT>
__device__ inline float block_max(float b, float *red, int tid) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) b = fmaxf(b, __shfl_xor(b, o, 64));
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = b;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Largest |z|, |z + top D| over this chunk's share of a cache tensor's groups.
template <int MT, int NT>
__device__ inline float cache_bound(const AttnLaunch &p, const float *scale, const float *zero, float top,
                                    int32_t ng, int64_t bkv, int64_t ch, int tid) {
  float bd = 0.f;
  const int64_t n = p.Nc * ng, lo = n * ch / KCHUNKS, hi = n * (ch + 1) / KCHUNKS;
  if (p.layout.page_table) {  // element i = (token i / ng, group i % ng) through the page table
    const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
    for (int64_t i = lo + tid; i < hi; i += NT) {
      const int64_t e = p.layout.row(p.cap, p.Hkv, b, hk, i / ng) * ng + i % ng;
      const float zi = meta_ld<MT>(zero, e);
      bd = fmaxf(bd, fmaxf(fabsf(zi), fabsf(fmaf(meta_ld<MT>(scale, e), top, zi))));
    }
  } else {
    const float *s = meta_adv<MT>(scale, bkv * p.cap * ng);
    const float *z = meta_adv<MT>(zero, bkv * p.cap * ng);
    for (int64_t i = lo + tid; i < hi; i += NT) {
      const float zi = meta_ld<MT>(z, i);
      bd = fmaxf(bd, fmaxf(fabsf(zi), fabsf(fmaf(meta_ld<MT>(s, i), top, zi))));
    }
  }
  return bd;
}

// Pre-pass: workgroup (b * Hkv + hk) * KCHUNKS + chunk bounds |key|, |query|
// and |value| over its share of the head's cache groups (or takes the
// caches' running bounds, chunk 0), current chunk and query rows.  APPEND: the call's chunk append rides along -- the workgroup
// also quantises its share of the chunk's K and V rows into the caches, from
// the values it loads for the bounds.
template <int KBITS, int MT, bool APPEND>
__global__ __launch_bounds__(256) void key_scale_kernel(AttnLaunch p, int32_t ng, float *part) {
  constexpr int NT = 256;
  __shared__ float red[NT / 64];
  const int64_t bkv = blockIdx.x / KCHUNKS;
  const int64_t ch = blockIdx.x % KCHUNKS;
  const int tid = threadIdx.x;
  float kb = 0.f, vb = 0.f;
  if (p.Nc > 0) {  // the caches' running bounds when they keep them, else a scan of the metadata
    kb = p.kc_bound ? (ch == 0 ? p.kc_bound[bkv] : 0.f)
                    : cache_bound<MT, NT>(p, p.kc_scale, p.kc_zero, static_cast<float>((1 << KBITS) - 1), ng, bkv,
                                           ch, tid);
    vb = p.vc_bound ? (ch == 0 ? p.vc_bound[bkv] : 0.f)
                    : cache_bound<MT, NT>(p, p.vc_scale, p.vc_zero, static_cast<float>((1 << p.vbits) - 1), ng, bkv,
                                           ch, tid);
  }
  if (APPEND && p.Ncur > 0) {  // the chunk's rows in this share: their bounds, and their codes
    const int64_t r0 = bkv * p.Ncur + p.Ncur * ch / KCHUNKS, r1 = bkv * p.Ncur + p.Ncur * (ch + 1) / KCHUNKS;
    qdev::RowBounds rb;
    qdev::append_rows<MT>(p, r0, r1, true, tid, NT, kb, vb, rb);
    // the rows are all of (b, KV head) bkv: one atomic per cache for the workgroup
    const float rk = block_max<NT>(rb.k, red, tid), rv = block_max<NT>(rb.v, red, tid);
    if (tid == 0) {
      if (p.app.bound[0]) qdev::bound_max(p.app.bound[0], bkv, rk);
      if (p.app.bound[1]) qdev::bound_max(p.app.bound[1], bkv, rv);
    }
  } else if (p.Ncur > 0) {
    const int64_t n = p.Ncur * D / 8, lo = n * ch / KCHUNKS, hi = n * (ch + 1) / KCHUNKS;
    kb = fmaxf(kb, bf16_bound<NT>(p.k_cur + bkv * p.Ncur * D, lo, hi, tid));
    vb = fmaxf(vb, bf16_bound<NT>(p.v_cur + bkv * p.Ncur * D, lo, hi, tid));
  }
  float qb;
  {
    const int64_t gq = p.Hq / p.Hkv, b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
    const int64_t n = gq * p.Nq * D / 8, lo = n * ch / KCHUNKS, hi = n * (ch + 1) / KCHUNKS;
    qb = bf16_bound<NT>(p.q + (b * p.Hq + hk * gq) * p.Nq * D, lo, hi, tid);
  }
  kb = block_max<NT>(kb, red, tid);
  qb = block_max<NT>(qb, red, tid);
  vb = block_max<NT>(vb, red, tid);
  if (tid == 0) {
    part[3 * bkv * KCHUNKS + ch] = kb;
    part[(3 * bkv + 1) * KCHUNKS + ch] = qb;
    part[(3 * bkv + 2) * KCHUNKS + ch] = vb;
  }
}

// ---- per-wave state ---------------------------------------------------------

// Query-side operands of one lane (its half of each k-step).
struct QState {
  f16x8 q[D / 16];
  bf16x8 qext;
};

// The lane's fp16 query operands (lane half h holds dimensions 16 s + 8 h ..
// +7 of k-step s): q times `scale`, clamped to the fp16 range.  Cached keys
// carry tau log2(e) 2^-ek, so their queries take scale = 2^ek (exact for bf16
// q); current keys are stored as k 2^-ek, so theirs take tau log2(e) 2^ek.
__device__ inline void query_operands(const uint16_t *qptr, int h, float scale, QState &qs) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint4 qw = *reinterpret_cast<const uint4 *>(qptr + 16 * s + 8 * h);
    const uint32_t u[4] = {qw.x, qw.y, qw.z, qw.w};
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack2h(fminf(fmaxf(lo_f(u[i]) * scale, -65504.0f), 65504.0f),
                    fminf(fmaxf(hi_f(u[i]) * scale, -65504.0f), 65504.0f));
    qs.q[s] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// The lane's query operands for the cached keys (query_operands with 2^ek)
// and the extra step's query slots, matching the key slots of unpack_k_item:
// N_g = tau^2/24 log2(e) ||q_g||^2 split into bf16 (N_hi, N_hi, N_lo) against
// (-D_hi, -D_lo, -D_hi), zero without the correction; -m split (hi, lo) in
// slots 3 and 7 (lane half 0; m = 0 at the start); S_g = tau log2(e)
// sum_{c in g} q_c split (S_hi, S_lo) against the centre c_g twice.  Lane
// half h holds slots 8h .. 8h+7: with two groups group h, (N, N, N, max,
// S, S, 0, max); with four groups 2h and 2h+1, (N, N, N, max, N, N, N, max);
// with one group (half 0) (N, N, N, max, S, S, 0, max).
template <bool TAYLOR>
__device__ inline void load_query_folded(const uint16_t *qptr, int h, int group_shift, float tau, int ek,
                                         QState &qs) {
  const int ng = 128 >> group_shift;
  query_operands(qptr, h, ldexpf(1.0f, ek), qs);
  float nsum[4] = {0.f, 0.f, 0.f, 0.f}, qsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint4 qw = *reinterpret_cast<const uint4 *>(qptr + 16 * s + 8 * h);
    const uint32_t u[4] = {qw.x, qw.y, qw.z, qw.w};
    float acc = 0.f, sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += lo_f(u[i]) * lo_f(u[i]) + hi_f(u[i]) * hi_f(u[i]);
      sum += lo_f(u[i]) + hi_f(u[i]);
    }
    const int gs = (16 * s + 8 * h) >> group_shift;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      nsum[g] += g == gs ? acc : 0.f;
      qsum[g] += g == gs ? sum : 0.f;
    }
  }
  float nh[4], nl[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float n = TAYLOR && g < ng ? (nsum[g] + __shfl_xor(nsum[g], 32, 64)) * (tau * tau / 24.0f * kLog2e) : 0.f;
    nh[g] = lo_f(pack2(n, 0.f));
    nl[g] = n - nh[g];
  }
  float sh[2], sl[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float t = (qsum[g] + __shfl_xor(qsum[g], 32, 64)) * (tau * kLog2e);
    sh[g] = g < ng ? lo_f(pack2(t, 0.f)) : 0.f;
    sl[g] = g < ng ? t - sh[g] : 0.f;
  }
  if (ng == 4) {
    const float n0h = h ? nh[2] : nh[0], n0l = h ? nl[2] : nl[0];
    const float n1h = h ? nh[3] : nh[1], n1l = h ? nl[3] : nl[1];
    qs.qext = __builtin_bit_cast(bf16x8, make_uint4(pack2(n0h, n0h), pack2(n0l, 0.f), pack2(n1h, n1h), pack2(n1l, 0.f)));
  } else {  // group h (one group: half 1 empty)
    const bool on = h < ng;
    const float gh = on ? (h ? nh[1] : nh[0]) : 0.f, gl = on ? (h ? nl[1] : nl[0]) : 0.f;
    const float th = on ? (h ? sh[1] : sh[0]) : 0.f, tl = on ? (h ? sl[1] : sl[0]) : 0.f;
    qs.qext = __builtin_bit_cast(bf16x8, make_uint4(pack2(gh, gh), pack2(gl, 0.f), pack2(th, tl), 0u));
  }
}

// Packed data of one tile held in registers between the fetch and the unpack.
struct Fetch {
  uint32_t kw[8];   // K: codes of 16 values (cached) or 16 bf16 values (current)
  uint32_t vw[8];   // V: codes of 2 keys x 8 values (cached) or 2 x 8 bf16 (current)
  float kstep, kzero;
  float vstep[2], vzero[2];
};

// Pointers already offset to this (b, hk) head (uniform per workgroup), so
// every per-lane offset below is a 32-bit row index within the head (the
// host bounds the token counts per head).
struct Ctx {
  const uint8_t *kc_codes, *vc_codes;
  const float *kc_scale, *kc_zero, *vc_scale, *vc_zero;
  const uint16_t *k_cur, *v_cur;
  int ng, group_shift;
  int beg, end;     // key range of the segment
  int climit;       // causal mask: current keys below climit are visible to the lane's row
  float kscale;     // cached keys: tau log2(e) 2^-ek
  float cscale;     // current keys: 2^-ek (exact for bf16 keys; tau log2(e) goes to the query)
  bool centre;      // cached keys centred per group (at most 2 groups per row)
  float vscale;     // 2^-ev: values enter the PV product as fp16 v 2^-ev
  uint32_t kmask;   // code mask of magic8, in a vector register
  CacheLayout layout;         // paged caches: pointers at the pools, rows of (b, hk)
  int64_t cap, H, b, hk;
};

// Paged caches: the pool row of the first row of the tile that holds rows
// [k0, k0 + 64) after clamping to the segment's last row (a tile that starts
// at or past the end holds only clamped rows: the tile of the last row).
// Such a tile lies in one page.
__device__ inline int tile_start(const Ctx &c, int k0) { return min(k0, (c.end - 1) & ~(BN - 1)); }
__device__ inline size_t tile_pool_row(const Ctx &c, int ts) {
  // wave-uniform page index (the host bounds B * pages per sequence to int32): one scalar load
  const int idx = __builtin_amdgcn_readfirstlane(static_cast<int>(c.b) * c.layout.pages_per_seq +
                                                 (ts >> c.layout.page_shift));
  const int64_t page = c.layout.page_table[idx];
  return static_cast<size_t>(((page * c.H + c.hk) << c.layout.page_shift) +
                             (ts & ((1 << c.layout.page_shift) - 1)));
}

// Per-lane softmax state of the lane's query row; m is the value the score
// MFMAs subtract (bf16 hi + lo, exactly as carried in the query operand).
struct Soft {
  f32x16 o[D / 32];
  float m, l;
};

// Thread roles in fetch / unpack:
//  K: key tid / 8, values 16 * (tid % 8) .. +16
//  V: keys 2*kq, 2*kq+1 with kq = tid / 16, values 8 * (tid % 16) .. +8
//     (a wave reads 4 keys' rows whole: 16 lanes per row)
// Rows past the end of the segment clamp to its last row (always in bounds).
template <bool CACHED, int KBITS, bool PAGED = false>
__device__ inline void fetch_k(const Ctx &c, int k0, int tid, Fetch &f, size_t pr = 0) {
  const int last = c.end - 1;
  const int kk = tid >> 3, d0 = (tid & 7) * 16;
  uint32_t krow = static_cast<uint32_t>(k0 + kk <= last ? k0 + kk : last);
  if (CACHED) {
    const uint8_t *kc_codes = c.kc_codes;
    const float *kc_scale = c.kc_scale, *kc_zero = c.kc_zero;
    if (PAGED) {  // pool row pr of the tile (looked up a step earlier), then rows within it
      const int ts = tile_start(c, k0);
      kc_codes += pr * (D * KBITS / 8);
      kc_scale = meta_adv<kMeta>(kc_scale, pr * c.ng);
      kc_zero = meta_adv<kMeta>(kc_zero, pr * c.ng);
      krow -= static_cast<uint32_t>(ts);
    }
    const uint8_t *ks = kc_codes + (krow * (D * KBITS / 8) + static_cast<uint32_t>(d0 * KBITS / 8));
    if (KBITS == 4) {
      const uint2 w = *reinterpret_cast<const uint2 *>(ks);
      f.kw[0] = w.x; f.kw[1] = w.y;
    } else {
      f.kw[0] = *reinterpret_cast<const uint32_t *>(ks);
    }
    const uint32_t km = krow * static_cast<uint32_t>(c.ng);
    f.kstep = meta_ld<kMeta>(kc_scale, km + static_cast<uint32_t>(d0 >> c.group_shift));
    f.kzero = meta_ld<kMeta>(kc_zero, km + static_cast<uint32_t>(d0 >> c.group_shift));
  } else {
    const uint4 *ks = reinterpret_cast<const uint4 *>(c.k_cur + (krow * D + static_cast<uint32_t>(d0)));
    const uint4 a = ks[0], b = ks[1];
    f.kw[0] = a.x; f.kw[1] = a.y; f.kw[2] = a.z; f.kw[3] = a.w;
    f.kw[4] = b.x; f.kw[5] = b.y; f.kw[6] = b.z; f.kw[7] = b.w;
  }
}

template <bool CACHED, int VBITS, bool PAGED = false>
__device__ inline void fetch_v(const Ctx &c, int k0, int tid, int j, Fetch &f, size_t pr = 0) {
  const int last = c.end - 1;
  const int dq = tid & 15, kq = tid >> 4;
  uint32_t vrow = static_cast<uint32_t>(k0 + 2 * kq + j <= last ? k0 + 2 * kq + j : last);
  if (CACHED) {
    const uint8_t *vc_codes = c.vc_codes;
    const float *vc_scale = c.vc_scale, *vc_zero = c.vc_zero;
    if (PAGED) {
      const int ts = tile_start(c, k0);
      vc_codes += pr * (D * VBITS / 8);
      vc_scale = meta_adv<kMeta>(vc_scale, pr * c.ng);
      vc_zero = meta_adv<kMeta>(vc_zero, pr * c.ng);
      vrow -= static_cast<uint32_t>(ts);
    }
    const uint8_t *vs = vc_codes + (vrow * (D * VBITS / 8) + static_cast<uint32_t>(dq * VBITS));
    f.vw[j] = VBITS == 4 ? *reinterpret_cast<const uint32_t *>(vs)
                         : static_cast<uint32_t>(*reinterpret_cast<const uint16_t *>(vs));
    const uint32_t vm = vrow * static_cast<uint32_t>(c.ng) + static_cast<uint32_t>((8 * dq) >> c.group_shift);
    f.vstep[j] = meta_ld<kMeta>(vc_scale, vm);
    f.vzero[j] = meta_ld<kMeta>(vc_zero, vm);
  } else {
    const uint4 v = *reinterpret_cast<const uint4 *>(c.v_cur + (vrow * D + static_cast<uint32_t>(8 * dq)));
    f.vw[4 * j] = v.x; f.vw[4 * j + 1] = v.y; f.vw[4 * j + 2] = v.z; f.vw[4 * j + 3] = v.w;
  }
}

// ---- work items --------------------------------------------------------------
// The VALU work of a tile is cut into items of a few instructions each; every
// item is issued right after one MFMA (see tile_step), so the matrix core and
// the vector ALU stay busy together; each item's results are pinned (see
// pin) so that it stays between its fences.

// K tile row: fp16 values, then the 16 slots of the extra bf16 step, laid
// out so that each thread writes slots of its own group (that of its 16
// values) and loads no other step or zero point.  With g the thread's group:
//   -D_g^2 split (hi, lo, hi) for the Taylor correction (zero without it):
//     two groups: slots 8g + {0, 1, 2}; four groups: 4g + {0, 1, 2}; one: 0..2;
//   1.0 in slots 3 and 7 (the running max carried by the query side);
//   the centre c_g of a cached key's group (see group_centre) in slots
//     8g + 4, 8g + 5 (one or two groups; none with four);
//   zero elsewhere.  Cached values are stored centred, (z - c_g + D code)
// tau log2(e) 2^-ek, and the step adds c_g times the query's group sums
// back; current keys are stored as k 2^-ek, exact.  Item 0 computes the
// scaled step, centred zero point and centre (kept in KWork), items 0 and 1
// write values 8p .. 8p+7 of the thread's 16, item 2 its two slots 2j, 2j+1
// (j = tid % 8).  A 304-byte row stride keeps the 16-byte writes (16 lanes =
// 2 keys x 8 chunks) on disjoint bank quads.
constexpr int kItemsK = 3;

struct KWork {
  float s, z, centre;
};

template <bool CACHED, bool TAYLOR, int KBITS>
__device__ inline void unpack_k_item(int p, const Ctx &c, int tid, const Fetch &f, uint16_t *Kb, KWork &u) {
  const int kk = tid >> 3, j = tid & 7, d0 = j * 16;
  if (CACHED && p == 0) {
    u.centre = c.centre ? group_centre<KBITS>(f.kzero, f.kstep) : 0.f;
    u.s = f.kstep * c.kscale;
    u.z = fmaf(-1024.0f, f.kstep, f.kzero - u.centre) * c.kscale;
  }
  if (p < 2) {
    uint32_t w[4];
    if (CACHED) {
      uint32_t m[4];
      magic8<KBITS>(KBITS == 4 ? f.kw[p] : (f.kw[0] >> (16 * p)), c.kmask, m);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pair_h(dequant_h(magic_code(m, 2 * e), u.s, u.z), dequant_h(magic_code(m, 2 * e + 1), u.s, u.z));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = f.kw[4 * p + e];
        w[e] = pack2h(lo_f(x) * c.cscale, hi_f(x) * c.cscale);
      }
    }
    *reinterpret_cast<uint4 *>(Kb + kk * KS + d0 + 8 * p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {  // slots 2j, 2j+1 (layout above); j's slot pair within its group: r
    const int r = c.ng == 4 ? (j & 1) : c.ng == 2 ? (j & 3) : j;
    const float one = j == 1 || j == 3 ? 1.0f : 0.f;
    float a = 0.f, b = one;
    if (CACHED) {
      const float sq = TAYLOR ? f.kstep * f.kstep : 0.f;
      const float hsq = lo_f(pack2(sq, 0.f));
      if (r == 0) {
        a = -hsq;
        b = -(sq - hsq);
      } else if (r == 1) {
        a = -hsq;
      } else if (r == 2) {  // (one or two groups) the centre, twice
        a = b = u.centre;
      }
    }
    *reinterpret_cast<uint32_t *>(Kb + kk * KS + KEXT + 2 * j) = pack2(a, b);
  }
}

// V^T tile: the thread's 2 keys 2kq, 2kq+1 sit in adjacent permuted slots
// (key r of a 16-key step sits at slot (r&3) + 4*(r>>3) + 8*((r>>2)&1)), so
// each of its 8 head-dim rows gets one 4-byte store.  Item 0 splits the
// codes of both keys into bytes and scales their steps and zero points
// (cached); items 1..4 dequantise and store rows 2(p-1), 2(p-1)+1.  Values
// are stored as fp16 v 2^-ev (ev: the KV head's value exponent, so that
// |v| 2^-ev < 2^15), rounded once from an fp32 fma.
constexpr int kItemsV = 5;

struct VWork {
  uint32_t c[2][2];  // per key: bytes holding codes (INT4: even / odd codes; INT2: codes j, j+4 pairs)
  float s[2], z[2];  // per key: step and zero point times 2^-ev
};

// Code e (0..7) of a key from its VWork bytes.
template <int VBITS>
__device__ inline float vcode(const uint32_t (&c)[2], int e) {
  if (VBITS == 4) {  // byte k of c[0] / c[1] holds code 2k / 2k+1
    return static_cast<float>((c[e & 1] >> (8 * (e >> 1))) & 0xffu);  // one v_cvt_f32_ubyteN
  } else {  // c[0] byte 0/1 = codes 0/4 of (w & 0x0303), etc.: code e = byte (e >> 2) of word e & 3
    const uint32_t w = (e & 3) < 2 ? c[0] : c[1];
    const int sh = 16 * ((e & 3) & 1) + 8 * (e >> 2);
    return static_cast<float>((w >> sh) & 0xffu);
  }
}

template <bool CACHED, int VBITS>
__device__ inline void unpack_v_item(int p, int tid, const Fetch &f, uint16_t *Vb, VWork &u, float vscale) {
  const int dq = tid & 15, kq = tid >> 4;
  if (p == 0) {
    if (CACHED) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        u.s[k] = f.vstep[k] * vscale;
        u.z[k] = f.vzero[k] * vscale;
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t w = f.vw[k];
        if (VBITS == 4) {
          u.c[k][0] = w & 0x0f0f0f0fu;
          u.c[k][1] = (w >> 4) & 0x0f0f0f0fu;
        } else {  // codes j and j+4 of (w >> 2j) & 0x0303 in bytes 0 and 1; j = 0,1 in c[0], j = 2,3 in c[1]
          u.c[k][0] = (w & 0x0303u) | (((w >> 2) & 0x0303u) << 16);
          u.c[k][1] = ((w >> 4) & 0x0303u) | (((w >> 6) & 0x0303u) << 16);
        }
      }
    }
  } else {
    const int r = (2 * kq) & 15;
    const int slot = 16 * (kq >> 3) + ((r & 3) | ((r >> 3) << 2) | (((r >> 2) & 1) << 3));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = 2 * (p - 1) + i;
      uint32_t w;
      if (CACHED) {
        w = pack2h(fmaf(u.s[0], vcode<VBITS>(u.c[0], e), u.z[0]), fmaf(u.s[1], vcode<VBITS>(u.c[1], e), u.z[1]));
      } else {
        // bf16 element e of key 0 (words 0..3) and key 1 (words 4..7), scaled (exact) and rounded to fp16
        const uint32_t w0 = f.vw[e >> 1], w1 = f.vw[4 + (e >> 1)];
        w = (e & 1) ? pack2h(hi_f(w0) * vscale, hi_f(w1) * vscale) : pack2h(lo_f(w0) * vscale, lo_f(w1) * vscale);
      }
      *reinterpret_cast<uint32_t *>(Vb + vt_index(8 * dq + e, slot)) = w;
    }
  }
}

// p = exp2(s) for scores 2k, 2k+1 of the block (k = 0..15): the running max
// is already subtracted by the score MFMAs (SHIFT subtracts a further
// `shift`, in the rare redo of fix_growth); every fourth item packs 8 of
// them into an fp16 P operand and adds the rounded p to the row sum (a p
// above the fp16 range becomes inf, and fix_growth redoes the tile).  MASK
// zeroes keys at or past `count`.
template <bool MASK, bool SHIFT = false>
__device__ inline void exp_item(int k, const f32x16 (&acc)[2], Soft &st, int count, int h, float (&e)[8],
                                f16x8 (&pk)[4], float shift = 0.f) {
  const int kb = k >> 3;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = 2 * (k & 7) + u;
    float x = __builtin_amdgcn_exp2f(SHIFT ? acc[kb][i] - shift : acc[kb][i]);
    if (MASK && kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3) >= count) x = 0.f;
    e[(2 * k + u) & 7] = x;
  }
  pin(e[(2 * k) & 7]);
  pin(e[(2 * k + 1) & 7]);
  if ((k & 3) == 3) {
    pk[k >> 2] = __builtin_bit_cast(f16x8, make_uint4(pack2h(e[0], e[1]), pack2h(e[2], e[3]), pack2h(e[4], e[5]),
                                                      pack2h(e[6], e[7])));
    st.l = sum8h(pk[k >> 2], st.l);
    pin(pk[k >> 2]);
    pin(st.l);
  }
}

// The running max carried by the query operand: -m split into bf16 (hi, lo)
// in slots 3 and 7 (lanes of half 0); returns the m those two carry.
__device__ inline float set_max_slots(QState &qs, float m, int h) {
  const float mh = lo_f(pack2(m, 0.f));
  const float ml = lo_f(pack2(m - mh, 0.f));
  if (h == 0) {
    uint4 w = __builtin_bit_cast(uint4, qs.qext);
    w.y = (w.y & 0xffffu) | (pack2(0.f, -mh) & 0xffff0000u);
    w.w = (w.w & 0xffffu) | (pack2(0.f, -ml) & 0xffff0000u);
    qs.qext = __builtin_bit_cast(bf16x8, w);
  }
  return mh + ml;
}

// Guard of the running max after the exponentials of a tile (sum l0 before
// it): if some row's sum left [kShrink, kGrowth] (or is not finite), move
// that row's m by the tile max (up or down), rescale O and l0, redo the
// tile's probabilities, and shift the already computed next scores sn by the
// same amount.  Rare: it takes a score about 16 binary orders above m (a p
// above 65504 rounds to inf in fp16, which fails the growth test), or all
// of a row's scores so far about 10 below it (the first tile after m = 0
// can be one); the shrink bound keeps a row's largest p away from the fp16
// subnormals.  A row with an empty sum and no visible key in the tile
// (causal mask) is left alone.
constexpr float kGrowth = 1099511627776.0f;  // 2^40
constexpr float kShrink = 0.0009765625f;     // 2^-10

template <bool MASK, bool QK>
__device__ inline void fix_growth(const f32x16 (&s)[2], f32x16 (&sn)[2], QState &qs, Soft &st, float l0, int count,
                                  int h, f16x8 (&pk)[4]) {
  const float lt = xor32_sum(st.l);
  const bool need = !(lt < kGrowth && (lt > kShrink || (MASK && lt == 0.f && count <= 0)));
  if (!__any(need)) return;
  float mt = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!MASK || kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3) < count) mt = fmaxf(mt, s[kb][i]);
  mt = xor32_max(mt);
  const float m_new = set_max_slots(qs, need && mt > -INFINITY ? st.m + mt : st.m, h);
  const float shift = m_new - st.m;
  // A shrink (shift < 0) only happens to a row whose sum was still empty, so
  // O and l are zero; a shift below -128 would make exp2(-shift) infinite
  // and 0 * inf a NaN, hence the clamp to the largest finite float (growth
  // gives sc <= 1).
  const float sc = fminf(exp2f(-shift), 3.4e38f);
  st.l = l0 * sc;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] *= sc;
  st.m = m_new;
  float e[8];
#pragma unroll
  for (int k = 0; k < 16; ++k) exp_item<MASK, true>(k, s, st, count, h, e, pk, shift);
  if (QK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[kb][i] -= shift;
  }
}

// ---- MFMA sequences ------------------------------------------------------------
// S^T of the wave's block: MFMA j < 16 uses the K fragment of k-step j / 2 of
// key block j % 2; j = 16, 17 are the correction steps of the two blocks.
constexpr int kNqk = 18;

__device__ constexpr int qk_off(int j) { return (j & 1) * 32 * KS + (j < 16 ? 16 * (j >> 1) : KEXT); }

// O^T += V^T P^T: MFMA j = (k-step j / 4, head-dim block j % 4); the
// fragment of (row 32 db + qc, slot 16 ks + 8 h) sits at the lane's base
// (qc * VS + 8 h) plus a constant.
__device__ constexpr int pv_off(int j) { return 32 * (j & 3) * VS + 16 * ((j >> 2) ^ (j & 3)); }

__device__ inline uint4 lds16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

#define KVQ_FENCE() __builtin_amdgcn_sched_barrier(0)

// One step of the cross-tile pipeline of a segment:
//   QK:   S_t - m of tile t (LDS K buffer Kl);
//   PREV: P_{t-1} from the saved scores S_{t-1} and O += V_{t-1} P_{t-1}
//         (LDS V buffer Vp), MASK for a ragged last tile of count keys;
//   NEXT: dequantise tile t+1 from f into K buffer Kn / V buffer Vn, and
//         fetch tile t+2 (rows clamp into the segment).
template <bool CACHED, bool TAYLOR, int KBITS, int VBITS, bool QK, bool PREV, bool NEXT, bool MASK, bool PAGED>
__device__ inline void tile_step(const Ctx &c, QState &qs, Soft &st, Fetch &f, const f32x16 (&s)[2],
                                 f32x16 (&sn)[2], const uint16_t *Kl, uint16_t *Kn, const uint16_t *Vp, uint16_t *Vn,
                                 int k0_next2, int count, int tid, size_t &prn) {
  const int lane = tid & 63, qc = lane & 31, h = lane >> 5;
  const uint16_t *Kb = Kl + qc * KS + 8 * h;
  const uint16_t *Vb = Vp + qc * VS + 8 * (h ^ (qc >> 4));
  constexpr int NQK = kNqk;
  constexpr int NK = kItemsK;
  uint4 buf[4];
  float ev[8];
  f16x8 pk[4];

  // 1. S_t - m (fp16 keys, bf16 correction and max step), with the
  //    exponentials of t-1
  const float l0 = st.l;
  if (QK) {
    sn[0] = f32x16{};
    sn[1] = f32x16{};
#pragma unroll
    for (int j = 0; j < 4; ++j) buf[j] = lds16(Kb + qk_off(j));
  }
#pragma unroll
  for (int j = 0; j < (QK ? NQK : 16); ++j) {
    if (QK) {
      if (j < 16)
        sn[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, buf[j & 3]), qs.q[j >> 1],
                                                           sn[j & 1], 0, 0, 0);
      else
        sn[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, buf[j & 3]), qs.qext,
                                                            sn[j & 1], 0, 0, 0);
      if (j + 4 < NQK) buf[j & 3] = lds16(Kb + qk_off(j + 4));
    }
    if (PREV && j < 16) exp_item<MASK>(j, s, st, count, h, ev, pk);
    KVQ_FENCE();
  }
  if (PREV) fix_growth<MASK, QK>(s, sn, qs, st, l0, count, h, pk);

  // 2. O += V_{t-1}^T P_{t-1}^T, with tile t+1 into LDS and the fetch of
  //    tile t+2
  {
    VWork u;
    KWork ku;
    if (PREV) {
#pragma unroll
      for (int j = 0; j < 4; ++j) buf[j] = lds16(Vb + pv_off(j));
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (PREV) {
        st.o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, buf[j & 3]), pk[j >> 2],
                                                             st.o[j & 3], 0, 0, 0);
        if (j + 4 < 16) buf[j & 3] = lds16(Vb + pv_off(j + 4));
      }
      if (NEXT) {
        if (j < NK) unpack_k_item<CACHED, TAYLOR, KBITS>(j, c, tid, f, Kn, ku);
        else if (j >= 4 && j - 4 < kItemsV) unpack_v_item<CACHED, VBITS>(j - 4, tid, f, Vn, u, c.vscale);
        else if (j == 9) fetch_k<CACHED, KBITS, PAGED>(c, k0_next2, tid, f, prn);
        else if (j == 10 || j == 11) fetch_v<CACHED, VBITS, PAGED>(c, k0_next2, tid, j - 10, f, prn);
      }
      KVQ_FENCE();
    }
  }
  // paged: the pool row of the tile the next step fetches, looked up now so
  // that the scalar load has long completed when that fetch needs it
  if (CACHED && PAGED && NEXT) prn = tile_pool_row(c, tile_start(c, k0_next2 + BN));
}

#undef KVQ_FENCE

// One segment (cached or current keys) of the key range; ends with a barrier
// so the next segment may reuse every LDS buffer.  CAUSAL (current keys
// only) masks every tile with the lane's own count of visible keys.
template <bool CACHED, bool TAYLOR, int KBITS, int VBITS, bool CAUSAL = false, bool PAGED = false>
__device__ inline void segment(const Ctx &c, QState &qs, Soft &st, uint16_t *Kl, uint16_t *Vl, int tid) {
  const int nt = c.end > c.beg ? (c.end - c.beg + BN - 1) / BN : 0;
  if (nt == 0) return;
  const int tail = c.end - c.beg - (nt - 1) * BN;  // keys in the last tile
  // keys of tile t that the lane's row sees (n in the tile)
  auto cnt = [&](int t, int n) { return CAUSAL ? min(n, c.climit - (c.beg + t * BN)) : n; };
  Fetch f;
  {
    VWork u;
    KWork ku;
    const size_t pr0 = CACHED && PAGED ? tile_pool_row(c, tile_start(c, c.beg)) : 0;
    fetch_k<CACHED, KBITS, PAGED>(c, c.beg, tid, f, pr0);
    fetch_v<CACHED, VBITS, PAGED>(c, c.beg, tid, 0, f, pr0);
    fetch_v<CACHED, VBITS, PAGED>(c, c.beg, tid, 1, f, pr0);
#pragma unroll
    for (int p = 0; p < kItemsK; ++p) unpack_k_item<CACHED, TAYLOR, KBITS>(p, c, tid, f, Kl, ku);
#pragma unroll
    for (int p = 0; p < kItemsV; ++p) unpack_v_item<CACHED, VBITS>(p, tid, f, Vl, u, c.vscale);
    const size_t pr1 = CACHED && PAGED ? tile_pool_row(c, tile_start(c, c.beg + BN)) : 0;
    fetch_k<CACHED, KBITS, PAGED>(c, c.beg + BN, tid, f, pr1);
    fetch_v<CACHED, VBITS, PAGED>(c, c.beg + BN, tid, 0, f, pr1);
    fetch_v<CACHED, VBITS, PAGED>(c, c.beg + BN, tid, 1, f, pr1);
  }
  __syncthreads();
  // paged: pool row of the tile the next fetch loads (tile 2)
  size_t prn = CACHED && PAGED ? tile_pool_row(c, tile_start(c, c.beg + 2 * BN)) : 0;
  // Scores alternate between sa and sb: step t reads S_{t-1} from one and
  // writes S_t to the other.
  f32x16 sa[2], sb[2];
  // t = 0: S_0 only (and tile 1 into LDS when there is one)
  if (nt > 1)
    tile_step<CACHED, TAYLOR, KBITS, VBITS, true, false, true, false, PAGED>(c, qs, st, f, sb, sa, Kl, Kl + KBUF, Vl,
                                                                      Vl + VBUF, c.beg + 2 * BN, BN, tid, prn);
  else
    tile_step<CACHED, TAYLOR, KBITS, VBITS, true, false, false, false, PAGED>(c, qs, st, f, sb, sa, Kl, Kl + KBUF, Vl,
                                                                       Vl + VBUF, 0, BN, tid, prn);
  __syncthreads();
  // steady state: S_t, P_{t-1} V_{t-1}, tile t+1 into LDS; two steps per trip
  int vb = 0;  // V buffer of tile t-1
  int t = 1;
  for (; t + 1 < nt - 1; t += 2) {
    const int v1 = vb + 1 < NVBUF ? vb + 1 : 0, v2 = v1 + 1 < NVBUF ? v1 + 1 : 0, v3 = vb;
    tile_step<CACHED, TAYLOR, KBITS, VBITS, true, true, true, CAUSAL, PAGED>(c, qs, st, f, sa, sb, Kl + KBUF, Kl,
                                                                      Vl + vb * VBUF, Vl + v2 * VBUF,
                                                                      c.beg + (t + 2) * BN, cnt(t - 1, BN), tid, prn);
    __syncthreads();
    tile_step<CACHED, TAYLOR, KBITS, VBITS, true, true, true, CAUSAL, PAGED>(c, qs, st, f, sb, sa, Kl, Kl + KBUF,
                                                                      Vl + v1 * VBUF, Vl + v3 * VBUF,
                                                                      c.beg + (t + 3) * BN, cnt(t, BN), tid, prn);
    __syncthreads();
    vb = v2;
  }
  if (t < nt - 1) {  // one more steady step (t odd: K buffer 1, S_t into sb)
    const int vn = vb + 2 < NVBUF ? vb + 2 : vb + 2 - NVBUF;
    tile_step<CACHED, TAYLOR, KBITS, VBITS, true, true, true, CAUSAL, PAGED>(c, qs, st, f, sa, sb, Kl + KBUF, Kl,
                                                                      Vl + vb * VBUF, Vl + vn * VBUF,
                                                                      c.beg + (t + 2) * BN, cnt(t - 1, BN), tid, prn);
    __syncthreads();
    vb = vb + 1 < NVBUF ? vb + 1 : 0;
    ++t;
    sa[0] = sb[0];
    sa[1] = sb[1];
  }
  // here t = nt - 1 (nt > 1) with S_{t-1} in sa, or nt == 1 with S_0 in sa
  if (nt > 1) {  // S_{nt-1}, P_{nt-2} V_{nt-2}
    tile_step<CACHED, TAYLOR, KBITS, VBITS, true, true, false, CAUSAL, PAGED>(c, qs, st, f, sa, sb,
                                                                       Kl + ((nt - 1) & 1) * KBUF, Kl, Vl + vb * VBUF,
                                                                       Vl, 0, cnt(nt - 2, BN), tid, prn);
    vb = vb + 1 < NVBUF ? vb + 1 : 0;
    sa[0] = sb[0];
    sa[1] = sb[1];
  }
  // drain: P_{nt-1} V_{nt-1}
  if (tail == BN && !CAUSAL)
    tile_step<CACHED, TAYLOR, KBITS, VBITS, false, true, false, false, PAGED>(c, qs, st, f, sa, sb, Kl, Kl,
                                                                       Vl + vb * VBUF, Vl, 0, BN, tid, prn);
  else
    tile_step<CACHED, TAYLOR, KBITS, VBITS, false, true, false, true, PAGED>(c, qs, st, f, sa, sb, Kl, Kl, Vl + vb * VBUF,
                                                                      Vl, 0, cnt(nt - 1, tail), tid, prn);
  __syncthreads();
}

// (MT names the metadata type in the kernel's symbol; it equals kMeta.)
template <int KBITS, int VBITS, bool TAYLOR, bool CAUSAL, bool PAGED, int MT>
__global__ __launch_bounds__(THREADS, 1) void attn_fast_kernel(AttnLaunch p, int32_t group_shift,
                                                                int64_t rows_per_kvhead, int32_t row_blocks,
                                                                const float *kpart, int32_t nsplit,
                                                                float *partials, int64_t nfull) {
  __shared__ __attribute__((aligned(16))) uint16_t Kl[2 * KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t Vl[NVBUF * VBUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qc = lane & 31, h = lane >> 5;
  const int ng = D >> group_shift;

  // Workgroups are dealt to the 8 XCDs round-robin by id; renumber so that
  // consecutive ids (the row blocks of one KV head) share an XCD.  The first
  // nfull ids (the unsplit units, dispatched first; a multiple of the CU
  // count) and the rest are renumbered separately, so that the unsplit units
  // all start in the first rounds.
  const uint32_t nwg = gridDim.x, wg = blockIdx.x;
  const bool tail = nsplit > 1 && wg >= static_cast<uint32_t>(nfull);
  const uint32_t base = tail ? static_cast<uint32_t>(nfull) : 0u;
  const uint32_t cnt = nsplit > 1 ? (tail ? nwg - base : static_cast<uint32_t>(nfull)) : nwg;
  const uint32_t k = wg - base;
  const uint32_t per = cnt >> 3, extra = cnt & 7, xcd = k & 7, slot = k >> 3;
  const uint32_t lin = base + (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + slot;
  // work units = (b, KV head, row block); the first nfull run over all keys,
  // each of the others is split into nsplit key ranges (split-major, so that
  // adjacent workgroups read the same keys)
  const int64_t units = static_cast<int64_t>(row_blocks) * p.B * p.Hkv;
  int64_t unit, split = 0, ns = 1;
  if (static_cast<int64_t>(lin) < nfull) {
    unit = lin;
  } else {
    const int64_t t = lin - nfull, ntail = units - nfull;
    split = t / ntail;
    unit = nfull + (t - split * ntail);
    ns = nsplit;
  }
  const int64_t bkv = unit / row_blocks;
  const int64_t rb = unit - bkv * row_blocks;
  const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
  const int64_t gq = p.Hq / p.Hkv;
  // exponent ek of the KV head from the pre-pass's partial bounds: key
  // operands (cached: centred, |k - c| <= 2 max|k|, times tau log2(e) 2^-ek;
  // current: k 2^-ek) and query operands (q 2^ek, q tau log2(e) 2^ek) near
  // the same magnitude, keys always below 2^15
  float kb = lane < KCHUNKS ? kpart[3 * bkv * KCHUNKS + lane] : 0.f;
  float qb = lane < KCHUNKS ? kpart[(3 * bkv + 1) * KCHUNKS + lane] : 0.f;
  float vb = lane < KCHUNKS ? kpart[(3 * bkv + 2) * KCHUNKS + lane] : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kb = fmaxf(kb, __shfl_xor(kb, o, 64));
    qb = fmaxf(qb, __shfl_xor(qb, o, 64));
    vb = fmaxf(vb, __shfl_xor(vb, o, 64));
  }
  // values enter the PV product as fp16 v 2^-ev, |v| 2^-ev below 2^15
  const int ev = vb > 0.f ? ilogbf(vb) - 14 : 0;
  const float kt = kb * fmaxf(2.0f * p.tau * kLog2e, 1.0f), qt = qb * fmaxf(p.tau * kLog2e, 1.0f);
  int ek = 0;
  if (kt > 0.f) {
    const int lk = ilogbf(kt);
    if (qt > 0.f) ek = (lk - ilogbf(qt)) >> 1;
    if (lk - ek > kFp16Exp) ek = lk - kFp16Exp;
  }

  // ---- the lane's query row: fp16 operands, scale, correction operands ----
  QState qs;
  const int64_t r = rb * BM + wave * 32 + qc;
  const bool row_ok = r < rows_per_kvhead;
  const int64_t rr = row_ok ? r : rows_per_kvhead - 1;
  const int64_t qrow = (b * p.Hq + hk * gq + rr / p.Nq) * p.Nq + rr % p.Nq;
  Soft st;
  load_query_folded<TAYLOR>(p.q + qrow * D, h, group_shift, p.tau, ek, qs);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16{};
  st.m = 0.f;
  st.l = 0.f;

  Ctx c{};
  c.ng = ng;
  c.group_shift = group_shift;
  c.kscale = ldexpf(p.tau * kLog2e, -ek);
  c.cscale = ldexpf(1.0f, -ek);
  c.centre = ng <= 2;
  c.vscale = ldexpf(1.0f, -ev);
  c.kmask = opaque_u32(kCodeMask<KBITS>);
  c.layout = p.layout;
  c.cap = p.cap;
  c.H = p.Hkv;
  c.b = b;
  c.hk = hk;
  if (p.Nc > 0) {
    const int64_t hrow = PAGED ? 0 : bkv * p.cap;  // first cache row of this head (paged: the pool)
    c.kc_codes = p.kc_codes + hrow * (D * KBITS / 8);
    c.vc_codes = p.vc_codes + hrow * (D * VBITS / 8);
    c.kc_scale = meta_adv<MT>(p.kc_scale, hrow * ng);
    c.kc_zero = meta_adv<MT>(p.kc_zero, hrow * ng);
    c.vc_scale = meta_adv<MT>(p.vc_scale, hrow * ng);
    c.vc_zero = meta_adv<MT>(p.vc_zero, hrow * ng);
  }
  // this split's tiles [t0, t1) of the cached tiles followed by the current ones
  const int tc = static_cast<int>((p.Nc + BN - 1) / BN), tu = static_cast<int>((p.Ncur + BN - 1) / BN);
  const int t0 = static_cast<int>(split * (tc + tu) / ns), t1 = static_cast<int>((split + 1) * (tc + tu) / ns);
  c.beg = min(t0, tc) * BN;
  c.end = min(min(t1, tc) * BN, static_cast<int>(p.Nc));
  segment<true, TAYLOR, KBITS, VBITS, false, PAGED>(c, qs, st, Kl, Vl, tid);
  if (p.Ncur > 0) {
    c.k_cur = p.k_cur + bkv * p.Ncur * D;
    c.v_cur = p.v_cur + bkv * p.Ncur * D;
  }
  c.beg = max(t0 - tc, 0) * BN;
  c.end = min(max(t1 - tc, 0) * BN, static_cast<int>(p.Ncur));
  // current keys are exact fp16 k 2^-ek: the softmax scale moves to the query
  if (c.end > c.beg) query_operands(p.q + qrow * D, h, ldexpf(p.tau * kLog2e, ek), qs);
  if (CAUSAL) {
    // current keys below climit are visible to the lane's row (query j of
    // Nq, aligned to the chunk's end); the workgroup stops at the largest
    // limit of its rows
    c.climit = static_cast<int>(rr % p.Nq + p.Ncur - p.Nq + 1);
    const int64_t r0 = rb * BM, r1 = min(r0 + BM, rows_per_kvhead) - 1;
    const int64_t jmax = r0 / p.Nq == r1 / p.Nq ? r1 % p.Nq : p.Nq - 1;
    c.end = static_cast<int>(min(static_cast<int64_t>(c.end), jmax + p.Ncur - p.Nq + 1));
  }
  segment<false, TAYLOR, KBITS, VBITS, CAUSAL, PAGED>(c, qs, st, Kl, Vl, tid);

  const float l_tot = st.l + __shfl_xor(st.l, 32, 64);
  if (!row_ok) return;
  const float vs = ldexpf(1.0f, ev);  // O accumulated values v 2^-ev
  if (ns > 1) {  // partial: O (unnormalised), then (m, l); [split][qrow][kPartialStride(D)]
    float *w = partials + (split * (p.B * p.Hq * p.Nq) + qrow) * kPartialStride(D);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4 *>(w + 32 * db + 8 * g4 + 4 * h) =
            make_float4(st.o[db][4 * g4] * vs, st.o[db][4 * g4 + 1] * vs, st.o[db][4 * g4 + 2] * vs,
                        st.o[db][4 * g4 + 3] * vs);
    if (h == 0) {
      w[D] = l_tot > 0.f ? st.m : -INFINITY;  // -inf: no key of this split is visible to the row
      w[D + 1] = l_tot;
    }
    return;
  }
  const float inv = vs / l_tot;
  uint16_t *optr = p.out + qrow * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<uint2 *>(optr + 32 * db + 8 * g4 + 4 * h) =
          make_uint2(pack2(st.o[db][4 * g4] * inv, st.o[db][4 * g4 + 1] * inv),
                     pack2(st.o[db][4 * g4 + 2] * inv, st.o[db][4 * g4 + 3] * inv));
}

// Log-sum-exp merge of the split partials of the tail units only (the
// others wrote their output directly): one wave per query row of a tail
// unit, 2 values per lane.
__global__ __launch_bounds__(256) void tail_combine_kernel(const float *__restrict__ ws, uint16_t *__restrict__ out,
                                                           AttnLaunch p, int64_t rows_per_kvhead, int32_t row_blocks,
                                                           int64_t nfull, int32_t nsplit) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // row of the tail units
  const int lane = threadIdx.x & 63;
  const int64_t unit = nfull + idx / BM;
  const int64_t bkv = unit / row_blocks, rb = unit - bkv * row_blocks;
  const int64_t rr = rb * BM + idx % BM;
  if (bkv >= p.B * p.Hkv || rr >= rows_per_kvhead) return;
  const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv, gq = p.Hq / p.Hkv;
  const int64_t qrow = (b * p.Hq + hk * gq + rr / p.Nq) * p.Nq + rr % p.Nq;
  const int64_t nrows = p.B * p.Hq * p.Nq;
  constexpr int64_t W = kPartialStride(D);
  // one pass, running max: a split's loads do not wait for the others' math
  float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll 4
  for (int s = 0; s < nsplit; ++s) {
    const float *w = ws + (s * nrows + qrow) * W;
    const float ms = w[D], ls = w[D + 1];
    const float2 o = *reinterpret_cast<const float2 *>(w + 2 * lane);
    if (ms == -INFINITY) continue;  // no key of this split is visible to the row
    const float mn = fmaxf(m, ms);
    const float c = exp2f(m - mn), f = exp2f(ms - mn);  // c = 0 for the first visible split
    l = fmaf(l, c, f * ls);
    a0 = fmaf(a0, c, f * o.x);
    a1 = fmaf(a1, c, f * o.y);
    m = mn;
  }
  const float inv = 1.0f / l;
  *reinterpret_cast<uint32_t *>(out + qrow * D + 2 * lane) = pack2(a0 * inv, a1 * inv);
}

template <int KB, int VB>
hipError_t launch_bits(const AttnLaunch &p, hipStream_t stream) {
  const int64_t rows = p.Nq * (p.Hq / p.Hkv);
  const int32_t row_blocks = static_cast<int32_t>((rows + BM - 1) / BM);
  const int32_t gshift = __builtin_ctz(static_cast<unsigned>(p.group));
  const int nsplit = p.splits > 1 ? p.splits : 1;
  float *partials = static_cast<float *>(p.workspace);
  float *kpart = reinterpret_cast<float *>(static_cast<char *>(p.workspace) +
                                           (nsplit > 1 ? short_path_workspace_bytes(p.B, p.Hq, p.Nq, p.d, nsplit) : 0));
  launch_key_scale(p, stream, kpart);
  const int64_t units = static_cast<int64_t>(row_blocks) * p.B * p.Hkv;
  const int64_t nfull = nsplit > 1 ? p.fast_full_units : units;
  const dim3 grid(static_cast<uint32_t>(nfull + (units - nfull) * nsplit));
  constexpr bool CAUSAL = KVQ_FAST_CAUSAL != 0, PAGED = KVQ_FAST_PAGED != 0;
  auto kernel = p.corr == KV_CORR_TAYLOR ? attn_fast_kernel<KB, VB, true, CAUSAL, PAGED, kMeta>
                                         : attn_fast_kernel<KB, VB, false, CAUSAL, PAGED, kMeta>;
  kernel<<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows, row_blocks, kpart, nsplit, partials, nfull);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  if (nfull == 0) return launch_combine(partials, p.out, p.B * p.Hq * p.Nq, nsplit, p.d, stream);
  const int64_t tail_rows = (units - nfull) * BM;
  tail_combine_kernel<<<dim3(static_cast<uint32_t>((tail_rows + 3) / 4)), dim3(256), 0, stream>>>(
      partials, p.out, p, rows, row_blocks, nfull, nsplit);
  return hipGetLastError();
}

}  // namespace

#if KVQ_FAST_PAGED || KVQ_FAST_CAUSAL || KVQ_FAST_META16
#if KVQ_FAST_META16 == 2 && KVQ_FAST_PAGED && KVQ_FAST_CAUSAL
hipError_t launch_attention_fast_mb16_paged_causal(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_META16 == 2 && KVQ_FAST_PAGED
hipError_t launch_attention_fast_mb16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_META16 == 2 && KVQ_FAST_CAUSAL
hipError_t launch_attention_fast_mb16_causal(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_META16 == 2
hipError_t launch_attention_fast_mb16(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_META16 && KVQ_FAST_PAGED && KVQ_FAST_CAUSAL
hipError_t launch_attention_fast_m16_paged_causal(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_META16 && KVQ_FAST_PAGED
hipError_t launch_attention_fast_m16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_META16 && KVQ_FAST_CAUSAL
hipError_t launch_attention_fast_m16_causal(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_META16
hipError_t launch_attention_fast_m16(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_PAGED && KVQ_FAST_CAUSAL
hipError_t launch_attention_fast_paged_causal(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_FAST_PAGED
hipError_t launch_attention_fast_paged(const AttnLaunch &p, hipStream_t stream) {
#else
hipError_t launch_attention_fast_causal(const AttnLaunch &p, hipStream_t stream) {
#endif
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<2, 2>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2>(p, stream);
  return launch_bits<4, 4>(p, stream);
}
#else
bool fast_path_supported(const AttnLaunch &p) {
  return fast_kernel_ok(p.d, p.corr, p.ktok || p.vtok, layout_page_size(p.layout));
}

template <int MT>
void key_scale_launch(const AttnLaunch &p, hipStream_t stream, float *part, dim3 grid, int32_t ng, bool k4) {
  // the instances with the chunk append hold its registers; those without stay lean
  auto kernel = p.app.on ? (k4 ? key_scale_kernel<4, MT, true> : key_scale_kernel<2, MT, true>)
                         : (k4 ? key_scale_kernel<4, MT, false> : key_scale_kernel<2, MT, false>);
  kernel<<<grid, dim3(256), 0, stream>>>(p, ng, part);
}

void launch_key_scale(const AttnLaunch &p, hipStream_t stream, float *part) {
  const int32_t ng = D / p.group;
  const dim3 grid(static_cast<uint32_t>(p.B * p.Hkv * KCHUNKS));
  const bool k4 = p.Nc > 0 && p.kbits == 4;
  if (p.meta == kMetaBF16)
    return key_scale_launch<kMetaBF16>(p, stream, part, grid, ng, k4);
  if (p.meta == kMetaF16) return key_scale_launch<kMetaF16>(p, stream, part, grid, ng, k4);
  key_scale_launch<kMetaF32>(p, stream, part, grid, ng, k4);
}

size_t fast_path_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int splits) {
  const size_t part = splits > 1 ? short_path_workspace_bytes(B, Hq, Nq, D, splits) : 0;
  return part + (static_cast<size_t>(B * Hkv) * 3 * KCHUNKS * sizeof(float) + 255) / 256 * 256;
}

// Key-range split of the throughput kernel.  With at least one full round
// of one-per-CU work units (R = units / CUs >= 1), the units of the last,
// partly empty round (r = units mod CUs) are split floor(CUs / r) ways so
// that they fill it, and the others run unsplit: R + 1/s rounds instead of
// R + 1, with partials and their merge for the r tail units only.  With
// fewer units than CUs, all of them split (fast_path_splits).  A forced
// count splits every unit.
FastPlan fast_path_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nc, int64_t Ncur, int cu_count,
                        int forced) {
  const int64_t rows = Nq * (Hq / Hkv);
  const int64_t units = (rows + BM - 1) / BM * B * Hkv;
  const int64_t tiles = (Nc + BN - 1) / BN + (Ncur + BN - 1) / BN;
  if (forced > 0) return FastPlan{static_cast<int>(forced < tiles ? forced : tiles), 0};
  const int64_t R = units / cu_count, r = units - R * cu_count;
  if (R == 0) return FastPlan{fast_path_splits(B, Hq, Hkv, Nq, Nc, Ncur, cu_count), 0};
  int64_t s = r > 0 ? cu_count / r : 1;
  if (s > 64) s = 64;
  if (s * 2 > tiles) s = tiles / 2;
  if (s < 2) return FastPlan{1, units};
  return FastPlan{static_cast<int>(s), units - r};
}

// Split count of the throughput kernel when every work unit splits: rounds
// of one-per-CU workgroups times the tiles each one runs, plus the HBM
// traffic of the partials.
int fast_path_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nc, int64_t Ncur, int cu_count) {
  const int64_t rows = Nq * (Hq / Hkv);
  const int64_t wgs = (rows + BM - 1) / BM * B * Hkv;
  const int64_t tiles = (Nc + BN - 1) / BN + (Ncur + BN - 1) / BN;
  const double t_tile = 2.0e-6;     // one workgroup, one 64-key tile (measured order)
  const double bytes_per_s = 4.0e12;  // partial write + combine read
  const double part_bytes = static_cast<double>(B * Hq * Nq) * kPartialStride(D) * sizeof(float) * 2.0;
  int best = 1;
  double best_t = 0.0;
  for (int64_t s = 1; s <= 64 && s * 2 <= tiles; ++s) {
    const int64_t rounds = (wgs * s + cu_count - 1) / cu_count;
    const double t = static_cast<double>(rounds) * static_cast<double>((tiles + s - 1) / s) * t_tile +
                     (s > 1 ? s * part_bytes / bytes_per_s + 5.0e-6 : 0.0);
    if (s == 1 || t < best_t * 0.98) {
      best = static_cast<int>(s);
      best_t = t;
    }
  }
  return best;
}

hipError_t launch_attention_fast(const AttnLaunch &p, hipStream_t stream) {
  if (p.meta == kMetaBF16) {
    if (p.layout.page_table)
      return p.causal ? launch_attention_fast_mb16_paged_causal(p, stream) : launch_attention_fast_mb16_paged(p, stream);
    return p.causal ? launch_attention_fast_mb16_causal(p, stream) : launch_attention_fast_mb16(p, stream);
  }
  if (p.meta == kMetaF16) {
    if (p.layout.page_table)
      return p.causal ? launch_attention_fast_m16_paged_causal(p, stream) : launch_attention_fast_m16_paged(p, stream);
    return p.causal ? launch_attention_fast_m16_causal(p, stream) : launch_attention_fast_m16(p, stream);
  }
  if (p.layout.page_table)
    return p.causal ? launch_attention_fast_paged_causal(p, stream) : launch_attention_fast_paged(p, stream);
  if (p.causal) return launch_attention_fast_causal(p, stream);
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<2, 2>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2>(p, stream);
  return launch_bits<4, 4>(p, stream);
}
#endif

}  // namespace kvq
