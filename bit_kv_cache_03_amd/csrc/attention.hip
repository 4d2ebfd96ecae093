// Corrected attention over [packed cache ; bf16 current chunk] for gfx950
// (MI355X): the long-query-chunk path, and the split-over-keys variant used
// by the short-query path (partials + log-sum-exp combine).
//
// One workgroup = 4 waves = BM (128) query rows that share one KV head
// (GQA rows of all query heads of that KV head are packed into one row
// space).  It walks the cached tokens, then the current chunk, in tiles of
// BN (64) keys.  Per tile:
//   1. all 256 threads stream the packed INT2/INT4 codes and fp32 step/zero
//      of the tile from HBM, dequantise x^ = z + D*c in fp32 and write bf16
//      K (row-major) and fp16 V (transposed, scaled by 2^-ev) tiles to LDS
//      -- the dequantisation is
//      fused into the attention kernel and no dequantised cache is ever
//      written to memory ("量化后画面闪烁？…" (hotelren.com), §4.3: the unfused
//      version cost +12% end to end, the fused one -3% vs FP16);
//   2. each wave computes S^T = K Q^T for its 32 rows on bf16 MFMA
//      (v_mfma_f32_32x32x16_bf16, fp32 accumulate), cached keys as a hi + lo
//      bf16 pair (two accumulation chains, ~16-bit keys);
//   3. the Jensen-bias correction ("量化鍵值偷走注意力…" (agents-report.net),
//      §方法: b = (1/(24 d)) sum_c q_c^2 D_{i,c}^2, §為何校正有效: subtracted
//      from cached-key scores before softmax) is rank (d/group) per score:
//      b_ij = tau/24 * sum_g ||q_{j,g}||^2 * D_{i,g}^2 in units of q.k.  It is
//      folded into the same MFMA accumulation as one extra K=16 step whose
//      operands are [||q_g||^2 * tau/24] per query and [-D_g^2] per key, each
//      split into bf16 hi + lo parts (hi*hi + hi*lo + lo*hi keeps ~16 bits),
//      so the epilogue costs no per-score VALU work;
//      the exact form sum_c log(sinh x_c/x_c) (§方法: exact for uniform noise)
//      is a per-score epilogue instead (slow path);
//   4. one online softmax (running max and sum per query row, exp2 with
//      log2(e) folded into the scale) spans both segments: cached logits are
//      corrected, current logits are not;
//   5. O^T += V^T P^T on fp16 MFMA (p <= 1 and v 2^-e in fp16: 11-bit
//      significands; bf16 values move the outputs of short, large-step INT2
//      caches by about the mean tolerance).
// Finally O 2^ev / l is rounded to bf16 and stored.
//
// The value exponent ev is fixed per (b, KV head): a pre-pass
// (value_bound_kernel) bounds |v| over the head's cached values (per group
// max(|z|, |z + top D|): the dequantised values lie between the two) and
// its current-chunk values, and ev = ilogb(bound) - 14 keeps |v| 2^-ev
// below 2^15, inside the fp16 range.  Values far below the bound become
// fp16 subnormals; their absolute error stays below 2^-24 of 2^ev, ~2^-39
// of the largest value.
//
// Caches whose groups run along the tokens (per channel: D_{t/G, c}) are
// dequantised channel by channel; their bias is then the same for every key
// of a token group, so with G >= 32 and tiles starting at multiples of 64
// each 32-key half of a tile has one bias per query row:
// tau^2/24 sum_c q_c^2 D_c^2 (or the exact sum_c log(sinh x_c / x_c)),
// computed per row from the half's per-channel steps staged in LDS.
//
// MFMA lane layouts (32x32x16 bf16, wave64): A operand lane l holds row l%32,
// k-slots 8*(l/32)..+7; B operand lane l holds column l%32, the same k-slots;
// the 32x32 fp32 result gives lane l column l%32 and rows
// 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.  With S^T (keys as rows, queries
// as columns) every lane owns one query, so row max and row sum are a local
// reduction plus one exchange with lane l^32, and the P operand of the next
// product is the score accumulator itself (no shuffle): for k-step ks the
// lane's 8 keys are 16*(ks%2) + {4h..4h+3, 8+4h..8+4h+3}.  The V tile is
// written to LDS transposed in that same key order, so both operands of
// O^T = V^T P^T are single 16-byte LDS reads.
//
// The instances for caches grouped along the tokens are built from this file
// in a translation unit of their own (attention_tokens.hip defines
// KVQ_TILE_TOKENS to 1): the head-dimension instances compile exactly as
// without them.  Every instance is built for two workgroups per CU: at
// d = 128 the token instances then spill ~30 registers and still run faster
// than at one; the exact-form instances at d = 128 need 88 KB of LDS, so
// one workgroup per CU is all that fits there anyway.
#include <math.h>

#include "kvq_internal.h"
#include "quant_device.h"

#ifndef KVQ_TILE_TOKENS
#define KVQ_TILE_TOKENS 0
#endif

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 256;  // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMinVExp = -100;  // smallest value exponent (2^100 fits fp32)
constexpr int kVChunks = 32;    // value pre-pass: workgroups and partial bounds per (b, KV head)

// A cached key is dequantised in fp32 and kept as a pair of bf16 values
// (hi = bf16(x^), lo = bf16(x^ - hi)) so that q.x^ carries ~16 significant
// bits: a single bf16 rounding of x^ moves the scores of large-step groups by
// more than the output tolerance allows.  Q K^T is then two MFMA chains.
template <int D>
struct Tile {
  static constexpr int kLo = D;               // offset of the lo half in a K row
  static constexpr int kExt = 2 * D;          // offset of the 16 correction slots
  static constexpr int kStride = 2 * D + 16 + 8;  // K row: hi, lo, correction slots, pad
  static constexpr int vStride = kBN + 8;     // V^T row: 64 keys, pad
};

__device__ inline uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

__device__ inline float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) | (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

// Two floats -> two fp16 (round to nearest even) in one instruction.
__device__ inline uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// log(sinh x / x) in fp32: series to x^10 below 0.5, else the identity
// log(sinh a / a) = a - log(2a) + log1p(-exp(-2a)).
__device__ inline float logsinhc(float x) {
  const float a = fabsf(x);
  if (a < 0.5f) {
    const float y = a * a;
    return y * (1.0f / 6.0f +
                y * (-1.0f / 180.0f + y * (1.0f / 2835.0f + y * (-1.0f / 37800.0f + y * (1.0f / 467775.0f)))));
  }
  return a - logf(2.0f * a) + log1pf(-expf(-2.0f * a));
}

// Metadata elements i .. i+3 (i a multiple of 4) of kind mk: fp32, or 16-bit
// (binary16 or bfloat16); one 16-byte or 8-byte load.
__device__ inline float4 meta4(const float *p, int64_t i, int mk) {
  if (mk == kMetaBF16) {  // bfloat16 patterns are the upper halves of fp32 ones
    const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
  }
  if (mk == kMetaF16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
    const auto h = [](uint32_t x) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x))); };
    return make_float4(h(w.x), h(w.x >> 16), h(w.y), h(w.y >> 16));
  }
  return *reinterpret_cast<const float4 *>(p + i);
}

// code j of a packed word: BITS-wide fields, LSB first.
template <int BITS>
__device__ inline float code_f(uint32_t w, int j) {
  return static_cast<float>((w >> (j * BITS)) & ((1u << BITS) - 1u));
}

// SPLIT: blockIdx.z selects a contiguous range of the key sequence
// [cache ; current]; the workgroup writes unnormalised partials (running max
// in the log2 domain, running sum, O) to the workspace instead of `out`.
// TOK: the caches may group along the tokens (p.ktok / p.vtok); false
// compiles those paths out.
template <int D, int KBITS, int VBITS, bool EXACT, bool SPLIT, bool TOK>
__global__ __launch_bounds__(kThreads, 2) void attn_tile_kernel(AttnLaunch p, int32_t group_shift,
                                                                 int64_t rows_per_kvhead, int64_t split_keys,
                                                                 const float *__restrict__ vbound) {
  constexpr int KS = Tile<D>::kStride;
  constexpr int VS = Tile<D>::vStride;
  constexpr int NS = D / 16;  // k-steps over the head dimension
  constexpr int NDB = D / 32; // 32-row blocks of the head dimension in O^T
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];
  // exact form only: per-key steps and the workgroup's query rows (bf16)
  __shared__ float Dk[EXACT ? kBN * 4 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[EXACT ? kBM * (D + 8) : 1];
  // groups along the tokens: per-channel steps of the token group of each
  // 32-key half of the tile
  __shared__ __attribute__((aligned(16))) float Dt[TOK ? 2 * D : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool ktok = TOK && p.ktok, vtok = TOK && p.vtok;
  const int qc = lane & 31;  // query column owned by this lane
  const int h = lane >> 5;   // lane half
  const int group = 1 << group_shift;
  const int ng = D >> group_shift;  // groups per row (1..4)

  const int64_t bkv = blockIdx.y;  // b * Hkv + hk
  const int64_t b = bkv / p.Hkv;
  const int64_t hk = bkv - b * p.Hkv;
  const int64_t gq = p.Hq / p.Hkv;

  // ---- this lane's query row ----
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kBM + wave * 32 + qc;
  const bool row_ok = r < rows_per_kvhead;
  const int64_t rr = row_ok ? r : rows_per_kvhead - 1;
  const int64_t qh = hk * gq + rr / p.Nq;
  const int64_t qj = rr - (rr / p.Nq) * p.Nq;
  const int64_t qrow = (b * p.Hq + qh) * p.Nq + qj;
  const uint16_t *qptr = p.q + qrow * D;

  bf16x8 qreg[NS];
  float nsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint4 w = *reinterpret_cast<const uint4 *>(qptr + 16 * s + 8 * h);
    qreg[s] = __builtin_bit_cast(bf16x8, w);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(u[i] << 16), hi = __uint_as_float(u[i] & 0xffff0000u);
      acc += lo * lo + hi * hi;
    }
    const int gs = (16 * s + 8 * h) >> group_shift;  // group of these 8 values
#pragma unroll
    for (int g = 0; g < 4; ++g) nsum[g] += g == gs ? acc : 0.f;
  }
  // correction operand of the queries: slots 3g+{0,1,2} = N_hi, N_hi, N_lo with
  // N_g = tau/24 * ||q_g||^2; lane half h holds slots 8h..8h+7
  bf16x8 qext;
  {
    float nh[4], nl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float tot = nsum[g] + __shfl_xor(nsum[g], 32, 64);
      const float n = tot * (p.tau / 24.0f);
      nh[g] = bf16_bits_to_f32(f32_to_bf16_bits(n));
      nl[g] = n - nh[g];
    }
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slot = 8 * h + j, g = slot / 3, part = slot % 3;
      e[j] = 0.f;
      if (g < ng && p.corr == KV_CORR_TAYLOR && !ktok) e[j] = part == 2 ? nl[g] : nh[g];
    }
    qext = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                                 pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])));
  }
  if (EXACT) {
    // stage the workgroup's query rows for the per-channel epilogue
    __syncthreads();
    for (int s = 0; s < NS; ++s)
      *reinterpret_cast<uint4 *>(&Qs[(wave * 32 + qc) * (D + 8) + 16 * s + 8 * h]) =
          __builtin_bit_cast(uint4, qreg[s]);
  }

  // ---- running softmax state ----
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // value exponent of the head from the pre-pass's partial bounds: O holds
  // sum p v 2^-ev
  float vb = lane < kVChunks ? vbound[bkv * kVChunks + lane] : 0.f;
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) vb = fmaxf(vb, __shfl_xor(vb, o2, 64));
  const int ev = vb > 0.f ? max(min(ilogbf(vb), 127) - 14, kMinVExp) : kMinVExp;
  const float vsc = ldexpf(1.0f, -ev);
  const float alpha = p.tau * kLog2e;

  // key range of this workgroup in the concatenated sequence [cache ; current]
  int64_t kbeg = 0, kend = p.Nc + p.Ncur;
  if (SPLIT) {
    kbeg = static_cast<int64_t>(blockIdx.z) * split_keys;
    kend = kbeg + split_keys < kend ? kbeg + split_keys : kend;
  }
  const int64_t c_beg = kbeg < p.Nc ? kbeg : p.Nc, c_end = kend < p.Nc ? kend : p.Nc;
  const int64_t u_beg = (kbeg > p.Nc ? kbeg : p.Nc) - p.Nc;
  int64_t u_end = (kend > p.Nc ? kend : p.Nc) - p.Nc;
  // causal mask: current keys below climit are visible to this lane's row;
  // the workgroup stops at the largest limit of its rows
  const int64_t climit = p.causal ? qj + p.Ncur - p.Nq + 1 : p.Ncur;
  if (p.causal) {
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kBM;
    const int64_t r1 = (r0 + kBM < rows_per_kvhead ? r0 + kBM : rows_per_kvhead) - 1;
    const int64_t jmax = r0 / p.Nq == r1 / p.Nq ? r1 % p.Nq : p.Nq - 1;
    const int64_t wlim = jmax + p.Ncur - p.Nq + 1;
    if (u_end > wlim) u_end = wlim;
  }
  const int64_t nt_c = c_end > c_beg ? (c_end - c_beg + kBN - 1) / kBN : 0;
  const int64_t nt_u = u_end > u_beg ? (u_end - u_beg + kBN - 1) / kBN : 0;
  const int64_t kvbase_u = bkv * p.Ncur;            // first current row of this (b, hk)
  constexpr int KROW = D * KBITS / 8;               // packed bytes per key row
  constexpr int VROW = D * VBITS / 8;

  for (int64_t t = 0; t < nt_c + nt_u; ++t) {
    const bool cached = t < nt_c;
    const int64_t k0 = cached ? c_beg + t * kBN : u_beg + (t - nt_c) * kBN;
    const int64_t kn = cached ? c_end : u_end;
    const int count = static_cast<int>(kn - k0 < kBN ? kn - k0 : kBN);
    // keys of this lane's row in the tile (fewer under the causal mask)
    const int64_t vis = cached ? count : climit - k0;
    const int rcount = vis < count ? static_cast<int>(vis) : count;

    __syncthreads();  // previous tile fully consumed
    // ---------------- K tile -> LDS (row-major, bf16) ----------------
    {
      constexpr int DPT = D / 4;  // head-dim values per thread
      const int key = tid >> 2;
      const int d0 = (tid & 3) * DPT;
      const bool ok = key < count;
      uint32_t outw[DPT / 2];
      if (cached) {
        const int64_t row = p.layout.row(p.cap, p.Hkv, b, hk, k0 + (ok ? key : 0));  // cache row of the key
        constexpr int WORDS = DPT * KBITS / 32;
        uint32_t w[WORDS];
        const uint8_t *src = p.kc_codes + row * KROW + d0 * KBITS / 8;
#pragma unroll
        for (int i = 0; i < WORDS; ++i) w[i] = ok ? reinterpret_cast<const uint32_t *>(src)[i] : 0u;
        constexpr int PER = 32 / KBITS;
        uint32_t low[DPT / 2];
        // values e, e + 1 as a bf16 hi pair and the lo pair of the remainders
        auto put = [&](int e, float a, float c) {
          const uint32_t hi = ok ? pack_bf16x2(a, c) : 0u;
          outw[e / 2] = hi;
          low[e / 2] = ok ? pack_bf16x2(a - __uint_as_float(hi << 16), c - __uint_as_float(hi & 0xffff0000u)) : 0u;
        };
        if (!ktok) {  // one step / zero point for the thread's values (one group of the row)
          const int g = d0 >> group_shift;
          const float stp = ok ? meta_at(p.kc_scale, row * ng + g, p.meta) : 0.f;
          const float zp = ok ? meta_at(p.kc_zero, row * ng + g, p.meta) : 0.f;
#pragma unroll
          for (int e = 0; e < DPT; e += 2)
            put(e, fmaf(stp, code_f<KBITS>(w[e / PER], e % PER), zp),
                fmaf(stp, code_f<KBITS>(w[(e + 1) / PER], (e + 1) % PER), zp));
        } else {  // groups along the tokens: one per channel of the key's token group
          // (row is a valid cache row also for keys past the tile's end;
          // put() zeroes their values)
          const int64_t m0 = (row >> group_shift) * D + d0;
#pragma unroll
          for (int e = 0; e < DPT; e += 4) {
            const float4 s4 = meta4(p.kc_scale, m0 + e, p.meta), z4 = meta4(p.kc_zero, m0 + e, p.meta);
            put(e, fmaf(s4.x, code_f<KBITS>(w[e / PER], e % PER), z4.x),
                fmaf(s4.y, code_f<KBITS>(w[(e + 1) / PER], (e + 1) % PER), z4.y));
            put(e + 2, fmaf(s4.z, code_f<KBITS>(w[(e + 2) / PER], (e + 2) % PER), z4.z),
                fmaf(s4.w, code_f<KBITS>(w[(e + 3) / PER], (e + 3) % PER), z4.w));
          }
        }
        uint4 *dlo = reinterpret_cast<uint4 *>(&Ks[key * KS + Tile<D>::kLo + d0]);
#pragma unroll
        for (int i = 0; i < DPT / 8; ++i)
          dlo[i] = make_uint4(low[4 * i], low[4 * i + 1], low[4 * i + 2], low[4 * i + 3]);
        if ((tid & 3) == 0 && !ktok) {
          // correction slots: 3g+{0,1,2} = -Dsq_hi, -Dsq_lo, -Dsq_hi
          float e16[16];
          float dsh[4] = {0.f, 0.f, 0.f, 0.f}, dsl[4] = {0.f, 0.f, 0.f, 0.f};
          for (int gg = 0; gg < ng; ++gg) {
            const float s = ok ? meta_at(p.kc_scale, row * ng + gg, p.meta) : 0.f;
            const float sq = s * s;
            dsh[gg] = bf16_bits_to_f32(f32_to_bf16_bits(sq));
            dsl[gg] = sq - dsh[gg];
            if (EXACT) Dk[key * 4 + gg] = s;
          }
#pragma unroll
          for (int slot = 0; slot < 16; ++slot) {
            const int gg = slot / 3, part = slot % 3;
            e16[slot] = gg < ng ? -(part == 1 ? dsl[gg] : dsh[gg]) : 0.f;
          }
          uint4 *dst = reinterpret_cast<uint4 *>(&Ks[key * KS + Tile<D>::kExt]);
          dst[0] = make_uint4(pack_bf16x2(e16[0], e16[1]), pack_bf16x2(e16[2], e16[3]),
                              pack_bf16x2(e16[4], e16[5]), pack_bf16x2(e16[6], e16[7]));
          dst[1] = make_uint4(pack_bf16x2(e16[8], e16[9]), pack_bf16x2(e16[10], e16[11]),
                              pack_bf16x2(e16[12], e16[13]), pack_bf16x2(e16[14], e16[15]));
        }
      } else {
        const int64_t row = kvbase_u + k0 + (ok ? key : 0);
        const uint4 *src = reinterpret_cast<const uint4 *>(p.k_cur + row * D + d0);
#pragma unroll
        for (int i = 0; i < DPT / 8; ++i) {
          const uint4 v = ok ? src[i] : make_uint4(0, 0, 0, 0);
          outw[4 * i] = v.x; outw[4 * i + 1] = v.y; outw[4 * i + 2] = v.z; outw[4 * i + 3] = v.w;
        }
      }
      uint4 *dst = reinterpret_cast<uint4 *>(&Ks[key * KS + d0]);
#pragma unroll
      for (int i = 0; i < DPT / 8; ++i)
        dst[i] = make_uint4(outw[4 * i], outw[4 * i + 1], outw[4 * i + 2], outw[4 * i + 3]);
      if (cached && ktok && p.corr != KV_CORR_OFF && tid < 2 * D) {
        const int hk0 = 32 * (tid / D);  // first key of the half
        const bool okh = hk0 < count;
        const int64_t hrow = p.layout.row(p.cap, p.Hkv, b, hk, k0 + (okh ? hk0 : 0));
        Dt[tid] = okh ? meta_at(p.kc_scale, (hrow >> group_shift) * D + tid % D, p.meta) : 0.f;
      }
    }
    // ---------------- V tile -> LDS (transposed, permuted key order) ----------------
    {
      // unit = 4 consecutive keys x 8 consecutive head-dim values
      constexpr int UNITS = (kBN / 4) * (D / 8);
      const int kq = tid & 15;  // key quad
      const int dq = tid >> 4;  // head-dim octet
      // dequantise v 2^-ev (exact scaling), round to fp16, store transposed
      if (tid < UNITS) {
        const int ks = kq >> 2, a = kq & 3;
        const int slot = 16 * ks + ((a >> 1) << 2) + ((a & 1) << 3);
        float v[4][8];
        if (cached) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = 4 * kq + j;
            const bool ok = key < count;
            const int64_t row = p.layout.row(p.cap, p.Hkv, b, hk, k0 + (ok ? key : 0));
            const uint8_t *src = p.vc_codes + row * VROW + dq * VBITS;  // 8 codes = VBITS bytes
            uint32_t w = 0;
            if (ok) w = VBITS == 2 ? *reinterpret_cast<const uint16_t *>(src) : *reinterpret_cast<const uint32_t *>(src);
            if (!vtok) {  // one step per group of the row
              const int64_t m = row * ng + ((8 * dq) >> group_shift);
              const float stp = ok ? meta_at(p.vc_scale, m, p.meta) * vsc : 0.f;
              const float zp = ok ? meta_at(p.vc_zero, m, p.meta) * vsc : 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) v[j][e] = fmaf(stp, code_f<VBITS>(w, e), zp);
            } else {  // groups along the tokens: one per channel
              const int64_t m0 = (row >> group_shift) * D + 8 * dq;
#pragma unroll
              for (int e4 = 0; e4 < 8; e4 += 4) {
                const float4 s4 = meta4(p.vc_scale, m0 + e4, p.meta), z4 = meta4(p.vc_zero, m0 + e4, p.meta);
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w}, zv[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  v[j][e4 + e] = ok ? fmaf(sv[e] * vsc, code_f<VBITS>(w, e4 + e), zv[e] * vsc) : 0.f;
              }
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = 4 * kq + j;
            const bool ok = key < count;
            const int64_t row = kvbase_u + k0 + (ok ? key : 0);
            const uint4 w = ok ? *reinterpret_cast<const uint4 *>(p.v_cur + row * D + 8 * dq) : make_uint4(0, 0, 0, 0);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[j][2 * e] = __uint_as_float(u[e] << 16) * vsc;
              v[j][2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u) * vsc;
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint2 w2 = make_uint2(pack_f16x2(v[0][e], v[1][e]), pack_f16x2(v[2][e], v[3][e]));
          *reinterpret_cast<uint2 *>(&Vt[(8 * dq + e) * VS + slot]) = w2;
        }
      }
    }
    __syncthreads();

    // groups along the tokens: one bias per query row and 32-key half (one
    // token group each), in logit units; the lane sums its half of the
    // channels, then the two lane halves combine
    float tokb[2] = {0.f, 0.f};
    if (cached && ktok && p.corr != KV_CORR_OFF) {
      constexpr bool taylor = !EXACT;  // this instance runs Taylor (EXACT: the exact form)
      const float half_tau = 0.5f * p.tau;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint4 w = __builtin_bit_cast(uint4, qreg[s]);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const float4 *dv = reinterpret_cast<const float4 *>(&Dt[kb * D + 16 * s + 8 * h]);
          const float4 d0v = dv[0], d1v = dv[1];
          const float st[8] = {d0v.x, d0v.y, d0v.z, d0v.w, d1v.x, d1v.y, d1v.z, d1v.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float qv = (i & 1) ? __uint_as_float(u[i >> 1] & 0xffff0000u) : __uint_as_float(u[i >> 1] << 16);
            tokb[kb] += taylor ? qv * qv * (st[i] * st[i]) : logsinhc(half_tau * qv * st[i]);
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float tot = tokb[kb] + __shfl_xor(tokb[kb], 32, 64);
        tokb[kb] = taylor ? tot * (p.tau * p.tau / 24.0f) : tot;  // tau^2/24 sum q^2 D^2, or sum L(x_c)
      }
    }

    // ---------------- S^T = K Q^T (+ correction step) ----------------
    f32x16 acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      acc[kb] = f32x16{};
      const uint16_t *krow = &Ks[(kb * 32 + qc) * KS + 8 * h];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(krow + 16 * s);
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], acc[kb], 0, 0, 0);
      }
      if (cached) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(krow + Tile<D>::kLo + 16 * s);
          acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], acc[kb], 0, 0, 0);
        }
      }
      if (!EXACT && cached && p.corr == KV_CORR_TAYLOR && !ktok) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(krow + Tile<D>::kExt);
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qext, acc[kb], 0, 0, 0);
      }
    }

    // ---------------- logits (log2 domain) ----------------
    float z[2][16];
    if (cached && ktok && p.corr != KV_CORR_OFF) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[kb][i] = (acc[kb][i] * p.tau - tokb[kb]) * kLog2e;
    } else if (EXACT && cached && p.corr == KV_CORR_EXACT) {
      float be[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) be[kb][i] = 0.f;
      const uint16_t *qs = &Qs[(wave * 32 + qc) * (D + 8)];
      const float half_tau = 0.5f * p.tau;
      for (int g = 0; g < ng; ++g) {
        float st[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) st[kb][i] = Dk[(kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3)) * 4 + g];
        for (int c = g * group; c < (g + 1) * group; ++c) {
          const float ac = half_tau * bf16_bits_to_f32(qs[c]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) be[kb][i] += logsinhc(ac * st[kb][i]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[kb][i] = (acc[kb][i] * p.tau - be[kb][i]) * kLog2e;
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[kb][i] = acc[kb][i] * alpha;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= rcount) z[kb][i] = -INFINITY;
        mt = fmaxf(mt, z[kb][i]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    // a row with no visible key yet keeps m = -inf; its terms are all zero
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float sc = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= sc;
    if (__any(sc != 1.0f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= sc;
    }
    f16x8 pk[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float e[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        e[i] = exp2f(z[kb][i] - m_use);
        l_run += e[i];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float *f = &e[8 * half];
        pk[2 * kb + half] = __builtin_bit_cast(
            f16x8, make_uint4(pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]), pack_f16x2(f[4], f[5]),
                              pack_f16x2(f[6], f[7])));
      }
    }

    // ---------------- O^T += V^T P^T ----------------
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t *vrow = &Vt[(32 * db + qc) * VS + 8 * h];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 va = *reinterpret_cast<const f16x8 *>(vrow + 16 * ks);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pk[ks], o[db], 0, 0, 0);
      }
    }
  }

  // ---------------- finalize ----------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float vs = ldexpf(1.0f, ev);
  if (SPLIT) {
    // partial: O (unnormalised) then (m, l), fp32, [split][qrow][kPartialStride(D)]
    if (row_ok) {
      float *w = static_cast<float *>(p.workspace) +
                 (static_cast<int64_t>(blockIdx.z) * (p.B * p.Hq * p.Nq) + qrow) * kPartialStride(D);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int e = 0; e < 4; ++e) w[32 * db + 8 * g4 + 4 * h + e] = o[db][4 * g4 + e] * vs;
      if (h == 0) {
        w[D] = m_run;
        w[D + 1] = l_tot;
      }
    }
    return;
  }
  const float inv = vs / l_tot;
  if (row_ok) {
    uint16_t *optr = p.out + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = 32 * db + 8 * g4 + 4 * h;
        uint2 w = make_uint2(pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                             pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv));
        *reinterpret_cast<uint2 *>(optr + dd) = w;
      }
  }
}

// Value pre-pass: workgroup (chunk, b * Hkv + hk) bounds |v| over its
// share of the head's cached value groups (max(|z|, |z + top D|) per group;
// chunk 0 takes the cache's running bound instead when it keeps one) and of
// its current-chunk values, and writes the bound to
// part[(b * Hkv + hk) * kVChunks + chunk].  APPEND: the call's chunk append
// rides along -- the workgroup also quantises its share of the chunk's K and
// V rows into the caches, from the values it loads for the bound.
template <bool APPEND>
__global__ __launch_bounds__(256) void value_bound_kernel(AttnLaunch p, int32_t group_shift, float *part) {
  const int tid = threadIdx.x;
  const int64_t ch = blockIdx.x, bkv = blockIdx.y;
  const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
  float vm = 0.f;
  if (p.Nc > 0 && p.vc_bound) {  // the value cache's running bound
    vm = ch == 0 ? p.vc_bound[bkv] : 0.f;
  } else if (p.Nc > 0) {
    const float top = static_cast<float>((1 << p.vbits) - 1);
    const bool tok = p.vtok;
    // groups along the head dim: Nc rows of d/G groups; along the tokens:
    // ceil(Nc/G) token groups of d channels
    const int64_t per = tok ? p.d : (p.d >> group_shift);
    const int64_t nrow = tok ? (p.Nc + (int64_t{1} << group_shift) - 1) >> group_shift : p.Nc;
    const int64_t n = nrow * per, lo = n * ch / kVChunks, hi = n * (ch + 1) / kVChunks;
    for (int64_t i = lo + tid; i < hi; i += 256) {
      const int64_t r = i / per, c = i - r * per;
      const int64_t e = tok ? (p.layout.row(p.cap, p.Hkv, b, hk, r << group_shift) >> group_shift) * per + c
                            : p.layout.row(p.cap, p.Hkv, b, hk, r) * per + c;
      const float stp = meta_at(p.vc_scale, e, p.meta), zp = meta_at(p.vc_zero, e, p.meta);
      vm = fmaxf(vm, fmaxf(fabsf(zp), fabsf(fmaf(stp, top, zp))));
    }
  }
  if (APPEND) {  // the chunk's rows in this share: the value bound, and the codes of both tensors
    const int64_t r0 = bkv * p.Ncur + p.Ncur * ch / kVChunks, r1 = bkv * p.Ncur + p.Ncur * (ch + 1) / kVChunks;
    float kb = 0.f;
    qdev::RowBounds rb;
    qdev::append_rows_any(p, r0, r1, true, tid, 256, kb, vm, rb);
    qdev::raise_bound(p.app.bound[0], bkv, rb.k);  // the rows are all of (b, KV head) bkv
    qdev::raise_bound(p.app.bound[1], bkv, rb.v);
  } else {  // current chunk: bf16 pairs
    const uint32_t *w = reinterpret_cast<const uint32_t *>(p.v_cur + bkv * p.Ncur * p.d);
    const int64_t n = p.Ncur * p.d / 2, lo = n * ch / kVChunks, hi = n * (ch + 1) / kVChunks;
    for (int64_t i = lo + tid; i < hi; i += 256) {
      const uint32_t u = w[i] & 0x7fff7fffu;  // |v| of both halves
      vm = fmaxf(vm, fmaxf(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) vm = fmaxf(vm, __shfl_xor(vm, o, 64));
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = vm;
  __syncthreads();
  if (tid == 0) part[bkv * kVChunks + ch] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Log-sum-exp merge of the split partials: one wave per query row.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float *__restrict__ ws, uint16_t *__restrict__ out,
                                                           int64_t nrows, int splits) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= nrows) return;
  constexpr int PER = D / 64;  // values per lane
  constexpr int64_t W = kPartialStride(D);
  // one pass, running max: a split's loads do not wait for the others' math
  float m = -INFINITY, l = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float *w = ws + (s * nrows + row) * W;
    const float ms = w[D], ls = w[D + 1];
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = w[lane * PER + e];
    if (ms == -INFINITY) continue;  // empty split
    const float mn = fmaxf(m, ms);
    const float c = exp2f(m - mn), f = exp2f(ms - mn);  // c = 0 for the first non-empty split
    l = fmaf(l, c, f * ls);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(acc[e], c, f * o[e]);
    m = mn;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[row * D + lane * PER + e] = f32_to_bf16_bits(acc[e] * inv);
}

constexpr bool kTok = KVQ_TILE_TOKENS != 0;

template <int D, int KB, int VB, bool SPLIT>
hipError_t launch_bits(const AttnLaunch &p, hipStream_t stream, bool exact) {
  const int64_t rows = p.Nq * (p.Hq / p.Hkv);
  const int splits = SPLIT ? p.splits : 1;
  const int64_t nkeys = p.Nc + p.Ncur;
  int64_t split_keys = (nkeys + splits - 1) / splits;
  split_keys = (split_keys + kBN - 1) / kBN * kBN;
  const dim3 grid(static_cast<uint32_t>((rows + kBM - 1) / kBM), static_cast<uint32_t>(p.B * p.Hkv),
                  static_cast<uint32_t>(splits));
  const int32_t gshift = __builtin_ctz(static_cast<unsigned>(p.group));
  // value bounds after the split partials
  float *vpart = reinterpret_cast<float *>(static_cast<char *>(p.workspace) +
                                           general_bound_offset(p.B, p.Hq, p.Nq, D, splits, SPLIT));
  const dim3 vgrid(kVChunks, static_cast<uint32_t>(p.B * p.Hkv));
  if (p.app.on)  // the instance with the chunk append holds its registers
    value_bound_kernel<true><<<vgrid, dim3(256), 0, stream>>>(p, gshift, vpart);
  else
    value_bound_kernel<false><<<vgrid, dim3(256), 0, stream>>>(p, gshift, vpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (exact)
    attn_tile_kernel<D, KB, VB, true, SPLIT, kTok>
        <<<grid, dim3(kThreads), 0, stream>>>(p, gshift, rows, split_keys, vpart);
  else
    attn_tile_kernel<D, KB, VB, false, SPLIT, kTok>
        <<<grid, dim3(kThreads), 0, stream>>>(p, gshift, rows, split_keys, vpart);
  e = hipGetLastError();
  if (e != hipSuccess || !SPLIT) return e;
  const int64_t nrows = p.B * p.Hq * p.Nq;
  attn_combine_kernel<D><<<dim3(static_cast<uint32_t>((nrows + 3) / 4)), dim3(256), 0, stream>>>(
      static_cast<const float *>(p.workspace), p.out, nrows, splits);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_d(const AttnLaunch &p, hipStream_t stream) {
  const bool exact = p.corr == KV_CORR_EXACT;
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<D, 2, 2, SPLIT>(p, stream, exact);
  if (kb == 2 && vb == 4) return launch_bits<D, 2, 4, SPLIT>(p, stream, exact);
  if (kb == 4 && vb == 2) return launch_bits<D, 4, 2, SPLIT>(p, stream, exact);
  return launch_bits<D, 4, 4, SPLIT>(p, stream, exact);
}

}  // namespace

#if KVQ_TILE_TOKENS
hipError_t launch_attention_tokens(const AttnLaunch &p, hipStream_t stream, bool split) {
  if (split) return p.d == 64 ? launch_d<64, true>(p, stream) : launch_d<128, true>(p, stream);
  return p.d == 64 ? launch_d<64, false>(p, stream) : launch_d<128, false>(p, stream);
}
#else
hipError_t launch_attention_long(const AttnLaunch &p, hipStream_t stream) {
  if (p.ktok || p.vtok) return launch_attention_tokens(p, stream, false);
  if (fast_path_supported(p)) return launch_attention_fast(p, stream);
  return p.d == 64 ? launch_d<64, false>(p, stream) : launch_d<128, false>(p, stream);
}

hipError_t launch_attention_short(const AttnLaunch &p, hipStream_t stream) {
  if (p.ktok || p.vtok) {
    if (short16_tok_supported(p.d, p.corr, p.ktok, p.vtok, layout_page_size(p.layout), p.meta, p.Nq * (p.Hq / p.Hkv)))
      return launch_attention_short16_tok(p, stream);
    if (short_tok_supported(p.d, p.corr, p.ktok, p.vtok, layout_page_size(p.layout), p.meta))
      return p.layout.page_table ? launch_attention_short_tok_paged(p, stream) : launch_attention_short_tok(p, stream);
    return launch_attention_tokens(p, stream, true);
  }
  if (short_fast_supported(p.d, p.corr, false, layout_page_size(p.layout))) return launch_attention_short_fast(p, stream);
  return p.d == 64 ? launch_d<64, true>(p, stream) : launch_d<128, true>(p, stream);
}

hipError_t launch_combine(const float *ws, uint16_t *out, int64_t nrows, int splits, int32_t d, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((nrows + 3) / 4));
  if (d == 64)
    attn_combine_kernel<64><<<grid, dim3(256), 0, stream>>>(ws, out, nrows, splits);
  else
    attn_combine_kernel<128><<<grid, dim3(256), 0, stream>>>(ws, out, nrows, splits);
  return hipGetLastError();
}

int short_path_splits(int64_t B, int64_t Hkv, int64_t rows_per_kvhead, int64_t Nc, int cu_count) {
  const int64_t tiles = B * Hkv * ((rows_per_kvhead + kBM - 1) / kBM);
  // at most two workgroups per CU (one round where two fit), rounded down:
  // rounding up sent a few workgroups into a further round (24 KV heads on
  // a 61k cache, groups along the tokens: 22 splits 856 us, 21 splits 562)
  int64_t s = 2 * static_cast<int64_t>(cu_count) / tiles;
  const int64_t max_s = (Nc + 4 * kBN - 1) / (4 * kBN);  // at least 4 tiles of keys per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 1024) s = 1024;
  return static_cast<int>(s);
}

size_t short_path_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int32_t d, int splits) {
  return static_cast<size_t>(splits) * static_cast<size_t>(B * Hq * Nq) * static_cast<size_t>(kPartialStride(d)) *
         sizeof(float);
}

size_t general_bound_offset(int64_t B, int64_t Hq, int64_t Nq, int32_t d, int splits, bool split) {
  return split ? (short_path_workspace_bytes(B, Hq, Nq, d, splits) + 255) / 256 * 256 : 0;
}

size_t general_path_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int32_t d, int splits,
                                    bool split) {
  return general_bound_offset(B, Hq, Nq, d, splits, split) +
         (static_cast<size_t>(B * Hkv) * kVChunks * sizeof(float) + 255) / 256 * 256;
}
#endif

}  // namespace kvq
