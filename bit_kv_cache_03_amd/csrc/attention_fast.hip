// Throughput kernel of the corrected attention for gfx950 (head dim 128,
// correction off or Taylor): the computation of attn_tile_kernel in
// attention.hip, reorganised for MI355X.
//
//  - 8 waves = 256 query rows per workgroup (one workgroup per CU), so each
//    dequantised K/V tile in LDS feeds 256 rows: the per-element unpack work
//    is amortised over twice as many scores as with 128 rows.
//  - The next packed tile is fetched from HBM into registers one tile ahead
//    and dequantised into the other half of a double-buffered LDS, its K
//    part interleaved with the current tile's Q K^T MFMAs and its V part
//    with P V, so the VALU work fills the matrix-core shadow.
//  - Ping-pong schedule (see segment()): two barrier-separated phases per
//    64-key tile, waves 4-7 one phase behind waves 0-3, so each SIMD pairs
//    an MFMA-heavy phase of one wave with the softmax of the other.
//  - Every wave dequantises 1/8 of the K tile (hi/lo bf16 pairs and the
//    correction slots) and 1/8 of the V tile (transposed, bank-conflict-free
//    in both directions).
//  - The cached and the current segment run in separate loops (no
//    per-tile branch on the segment kind); keys past the end of a segment
//    are fetched as duplicates of a valid row and masked out of the softmax,
//    so the dequantisation itself never needs predication.
//  - Lazy running max: O is rescaled only when a tile's max exceeds the
//    running max by more than 2^8 (in the exp2 domain).
// The Jensen-bias correction ("量化鍵值偷走注意力…" (agents-report.net),
// §方法 and §為何校正有效) enters as one extra K=16 MFMA step per 32x32
// score block: operands [tau/24 * ||q_g||^2] per query and [-D_g^2] per
// cached key, each split into bf16 hi and lo parts.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int BM = 256;        // query rows per workgroup
constexpr int BN = 64;         // keys per tile
constexpr int THREADS = 512;   // 8 waves
constexpr int KS = 2 * D + 16 + 8;  // K row in LDS: hi[128] lo[128] corr[16] pad[8] (bf16)
constexpr int KLO = D;
constexpr int KEXT = 2 * D;
constexpr int VS = BN + 8;     // V^T row in LDS (bf16)
constexpr int KBUF = BN * KS;  // bf16 elements per K buffer
constexpr int VBUF = D * VS;   // bf16 elements per V buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // rescale threshold (exp2 domain)

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // round to nearest even
}
// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
// (x, y) -> the bf16 pair h = (bf16(x), bf16(y)) and the pair of residuals
// (bf16(x - h.x), bf16(y - h.y)).  Each residual is one v_dot2_f32_bf16:
// h.x * -1 + h.y * 0 + x = x - h.x, exact in fp32.
// The weight pair (-1, -0.0) is written so that it is emitted as the 32-bit
// literal 0x8000bf80: the pair (-1, 0) gets encoded as the inline constant
// -1.0, which the hardware reads as the fp32 bit pattern 0xbf800000, i.e.
// the bf16 pair (0, -1).
__device__ inline void split2(float x, float y, uint32_t &hi, uint32_t &lo) {
  hi = pack2(x, y);
  const bf16x2 h = __builtin_bit_cast(bf16x2, hi);
  const bf16x2 e0 = {static_cast<__bf16>(-1.0f), static_cast<__bf16>(-0.0f)};
  const bf16x2 e1 = {static_cast<__bf16>(0.0f), static_cast<__bf16>(-1.0f)};
  lo = pack2(__builtin_amdgcn_fdot2_f32_bf16(h, e0, x, false), __builtin_amdgcn_fdot2_f32_bf16(h, e1, y, false));
}

// Sum of the 8 bf16 values of v, added to acc (two per v_dot2_f32_bf16).
__device__ inline float sum8(bf16x8 v, float acc) {
  const uint4 w = __builtin_bit_cast(uint4, v);
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), one, acc, false);
}
__device__ inline float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// V^T element (row = head-dim index, col = permuted key slot 0..63).  The
// 16-byte chunks of a row are XOR-swizzled by (row / 16) % 8.  With 64 LDS
// banks and a 144-byte row stride:
//  - an operand read (16 lanes = 16 consecutive rows, one chunk) keeps one
//    swizzle value per 16 rows, so the rows land on disjoint bank quads;
//  - a transposed write (16 rows 8 apart x the 4 dwords of one chunk, see
//    unpack_v) spreads over all 64 banks.
__device__ inline int vt_index(int row, int col) {
  return row * VS + ((((col >> 3) ^ (row >> 4)) & 7) << 3) + (col & 7);
}

// 8 codes of BITS bits (LSB first) in the low 8*BITS bits of w -> floats.
template <int BITS>
__device__ inline void codes8(uint32_t w, float (&c)[8]) {
  if (BITS == 4) {
    const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;  // even / odd codes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = static_cast<float>((lo >> (8 * i)) & 0xffu);
      c[2 * i + 1] = static_cast<float>((hi >> (8 * i)) & 0xffu);
    }
  } else {
    // byte k of (w >> 2j) & 0x0303 holds code 4k + j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = (w >> (2 * j)) & 0x0303u;
      c[j] = static_cast<float>(m & 0xffu);
      c[4 + j] = static_cast<float>((m >> 8) & 0xffu);
    }
  }
}

// 16 codes of 2 bits (LSB first) in w -> floats, a byte lane at a time.
__device__ inline void codes16_int2(uint32_t w, float (&c)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t m = (w >> (2 * j)) & 0x03030303u;  // byte k holds code 4k + j
#pragma unroll
    for (int k = 0; k < 4; ++k) c[4 * k + j] = static_cast<float>((m >> (8 * k)) & 0xffu);
  }
}

// Query-side operands of one lane (one query row, half of its head dimension).
struct QState {
  bf16x8 q[D / 16];
  bf16x8 qext;
};

// Packed data of one tile held in registers between the fetch and the unpack.
struct Fetch {
  uint32_t kw[8];   // K: codes of 16 values (cached) or 16 bf16 values (current)
  uint32_t vw[8];   // V: codes of 2 keys x 8 values (cached) or 2 x 8 bf16 (current)
  float kstep, kzero;
  float gstep[4];   // all group steps of the key (the correction slots)
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
  int beg, end;  // key range of the segment
};

// Thread roles in fetch / unpack (every wave does both):
//  K: key kk = tid / 8, values d0 = (tid % 8) * 16 .. +16
//  V: wave w writes the permuted slots 8w .. 8w+7 (one 16-byte chunk of every
//     V^T row); lane j = lane / 16 takes slots 8w + 2j, 8w + 2j + 1, i.e.
//     keys vkey(w, j), vkey(w, j) + 1, and values 8*vq .. +8, vq = lane % 16.
__device__ inline int vkey(int w, int j) { return 16 * (w >> 1) + 4 * (w & 1) + 2 * (j & 1) + 8 * (j >> 1); }
// Rows past the end of the segment clamp to its last row (always in bounds).
template <bool CACHED, int KBITS>
__device__ inline void fetch_k(const Ctx &c, int k0, int tid, Fetch &f) {
  const int last = c.end - 1;
  const int kk = tid >> 3, d0 = (tid & 7) * 16;
  const uint32_t krow = static_cast<uint32_t>(k0 + kk <= last ? k0 + kk : last);
  if (CACHED) {
    const uint8_t *ks = c.kc_codes + (krow * (D * KBITS / 8) + static_cast<uint32_t>(d0 * KBITS / 8));
    if (KBITS == 4) {
      const uint2 w = *reinterpret_cast<const uint2 *>(ks);
      f.kw[0] = w.x;
      f.kw[1] = w.y;
    } else {
      f.kw[0] = *reinterpret_cast<const uint32_t *>(ks);
    }
    const uint32_t km = krow * static_cast<uint32_t>(c.ng);
    const uint32_t kg = km + static_cast<uint32_t>(d0 >> c.group_shift);
    f.kstep = c.kc_scale[kg];
    f.kzero = c.kc_zero[kg];
    if ((tid & 7) == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) f.gstep[g] = g < c.ng ? c.kc_scale[km + static_cast<uint32_t>(g)] : 0.f;
    }
  } else {
    const uint4 *ks = reinterpret_cast<const uint4 *>(c.k_cur + (krow * D + static_cast<uint32_t>(d0)));
    const uint4 a = ks[0], b = ks[1];
    f.kw[0] = a.x; f.kw[1] = a.y; f.kw[2] = a.z; f.kw[3] = a.w;
    f.kw[4] = b.x; f.kw[5] = b.y; f.kw[6] = b.z; f.kw[7] = b.w;
  }
}

template <bool CACHED, int VBITS>
__device__ inline void fetch_v(const Ctx &c, int k0, int tid, Fetch &f) {
  const int last = c.end - 1;
  const int vq = tid & 15, k2 = vkey(tid >> 6, (tid >> 4) & 3);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t vrow = static_cast<uint32_t>(k0 + k2 + j <= last ? k0 + k2 + j : last);
    if (CACHED) {
      const uint8_t *vs = c.vc_codes + (vrow * (D * VBITS / 8) + static_cast<uint32_t>(vq * VBITS));
      f.vw[j] = VBITS == 4 ? *reinterpret_cast<const uint32_t *>(vs)
                           : static_cast<uint32_t>(*reinterpret_cast<const uint16_t *>(vs));
      const uint32_t vm = vrow * static_cast<uint32_t>(c.ng) + static_cast<uint32_t>((8 * vq) >> c.group_shift);
      f.vstep[j] = c.vc_scale[vm];
      f.vzero[j] = c.vc_zero[vm];
    } else {
      const uint4 v = *reinterpret_cast<const uint4 *>(c.v_cur + (vrow * D + static_cast<uint32_t>(8 * vq)));
      f.vw[4 * j] = v.x; f.vw[4 * j + 1] = v.y; f.vw[4 * j + 2] = v.z; f.vw[4 * j + 3] = v.w;
    }
  }
}

template <bool CACHED, bool TAYLOR, int KBITS>
__device__ inline void unpack_k(const Ctx &c, int tid, const Fetch &f, uint16_t *Kb) {
  const int kk = tid >> 3, d0 = (tid & 7) * 16;
  uint4 *hi = reinterpret_cast<uint4 *>(Kb + kk * KS + d0);
  if (CACHED) {
    uint4 *lo = reinterpret_cast<uint4 *>(Kb + kk * KS + KLO + d0);
    float cv[16];
    if (KBITS == 4) {
      float c0[8], c1[8];
      codes8<4>(f.kw[0], c0);
      codes8<4>(f.kw[1], c1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cv[e] = c0[e];
        cv[8 + e] = c1[e];
      }
    } else {
      codes16_int2(f.kw[0], cv);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // 8 values per 16-byte store
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        split2(fmaf(f.kstep, cv[8 * i + 2 * e], f.kzero), fmaf(f.kstep, cv[8 * i + 2 * e + 1], f.kzero), wh[e],
               wl[e]);
      hi[i] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
      lo[i] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    }
    if (TAYLOR && (tid & 7) == 0) {
      // correction slots 3g+{0,1,2} = -D_g^2 split hi, lo, hi
      float e[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) e[s] = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float sq = g < c.ng ? f.gstep[g] * f.gstep[g] : 0.f;
        const float hsq = __uint_as_float(static_cast<uint32_t>(bf16_bits(sq)) << 16);
        e[3 * g] = -hsq;
        e[3 * g + 1] = -(sq - hsq);
        e[3 * g + 2] = -hsq;
      }
      uint4 *x = reinterpret_cast<uint4 *>(Kb + kk * KS + KEXT);
      x[0] = make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
      x[1] = make_uint4(pack2(e[8], e[9]), pack2(e[10], e[11]), pack2(e[12], e[13]), pack2(e[14], e[15]));
    }
  } else {
    hi[0] = make_uint4(f.kw[0], f.kw[1], f.kw[2], f.kw[3]);
    hi[1] = make_uint4(f.kw[4], f.kw[5], f.kw[6], f.kw[7]);
  }
}

template <bool CACHED, int VBITS>
__device__ inline void unpack_v(int tid, const Fetch &f, uint16_t *Vb) {
  // keys vkey(w, j), +1 sit in the permuted slots 8w + 2j, 8w + 2j + 1
  const int vq = tid & 15;
  const int slot = 8 * (tid >> 6) + 2 * ((tid >> 4) & 3);
  float v[2][8];
  if (CACHED) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float cv[8];
      codes8<VBITS>(f.vw[j], cv);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = fmaf(f.vstep[j], cv[e], f.vzero[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[j][2 * e] = lo_f(f.vw[4 * j + e]);
        v[j][2 * e + 1] = hi_f(f.vw[4 * j + e]);
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<uint32_t *>(Vb + vt_index(8 * vq + e, slot)) = pack2(v[0][e], v[1][e]);
}

// Running softmax state of one lane.
struct Soft {
  f32x16 o[D / 32];
  float m, l;
};

// One segment (cached or current keys) of the tile loop, ping-pong schedule.
// Each tile is two barrier-separated phases:
//   X: S^T = K Q^T on the matrix cores; dequantise K of the next tile
//   Y: softmax, O^T += V^T P^T; dequantise V of the next tile
// Waves 4-7 run one phase behind waves 0-3, so on every SIMD (which hosts
// waves i and i+4) one wave is in its MFMA-heavy phase X while the other is
// in its VALU-heavy phase Y.  LDS hazards: K of tile t+1 is written in
// phases where only K(t) / V(t-1) are read, V of tile t+1 where only
// V(t) / K(t) are read (double buffer indexed by tile parity).
template <bool CACHED, bool TAYLOR, int KBITS, int VBITS>
__device__ inline void segment(const Ctx &c, const QState &qs, Soft &st, uint16_t *Kl, uint16_t *Vl, int tid,
                               bool lagging, float alpha) {
  const int lane = tid & 63, qc = lane & 31, h = lane >> 5;
  const int nt = c.end > c.beg ? (c.end - c.beg + BN - 1) / BN : 0;
  if (nt == 0) return;
  Fetch f;
  fetch_k<CACHED, KBITS>(c, c.beg, tid, f);
  fetch_v<CACHED, VBITS>(c, c.beg, tid, f);
  unpack_k<CACHED, TAYLOR, KBITS>(c, tid, f, Kl);
  unpack_v<CACHED, VBITS>(tid, f, Vl);
  fetch_k<CACHED, KBITS>(c, c.beg + BN, tid, f);
  fetch_v<CACHED, VBITS>(c, c.beg + BN, tid, f);
  __syncthreads();
  if (lagging) __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int cb = t & 1;
    const uint16_t *Kb = Kl + cb * KBUF;
    const uint16_t *Vb = Vl + cb * VBUF;
    const int k0 = c.beg + t * BN;
    const int count = c.end - k0 < BN ? c.end - k0 : BN;

    // ================= phase X =================
    f32x16 acc[2];
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8 *>(Kb + (kb * 32 + qc) * KS + 8 * h + 16 * s), qs.q[s], acc[kb], 0, 0, 0);
    if (CACHED) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8 *>(Kb + (kb * 32 + qc) * KS + 8 * h + KLO + 16 * s), qs.q[s], acc[kb],
              0, 0, 0);
      if (TAYLOR) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8 *>(Kb + (kb * 32 + qc) * KS + 8 * h + KEXT), qs.qext, acc[kb], 0, 0, 0);
      }
    }
    // next tile's K (stale past the end: nothing reads it before a refill)
    unpack_k<CACHED, TAYLOR, KBITS>(c, tid, f, Kl + (cb ^ 1) * KBUF);
    fetch_k<CACHED, KBITS>(c, k0 + 2 * BN, tid, f);
    constexpr int NX = CACHED ? (TAYLOR ? 34 : 32) : 16;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, CACHED ? 3 : 1, 0);
    }
    __syncthreads();

    // ================= phase Y =================
    if (count < BN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3) >= count) acc[kb][i] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, acc[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * alpha;
    const bool grow = mt > st.m + kLazy;
    if (__any(grow)) {
      const float m_new = grow ? mt : st.m;
      const float sc = exp2f(st.m - m_new);
      st.l *= sc;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) st.o[db] *= sc;
      st.m = m_new;
    }
    bf16x8 pk[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float e[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(acc[kb][i], alpha, -st.m));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        pk[2 * kb + hf] = __builtin_bit_cast(
            bf16x8, make_uint4(pack2(e[8 * hf], e[8 * hf + 1]), pack2(e[8 * hf + 2], e[8 * hf + 3]),
                               pack2(e[8 * hf + 4], e[8 * hf + 5]), pack2(e[8 * hf + 6], e[8 * hf + 7])));
        // the row sum uses the rounded P that the value product uses
        st.l = sum8(pk[2 * kb + hf], st.l);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8 *>(Vb + vt_index(32 * db + qc, 16 * ks + 8 * h)), pk[ks], st.o[db], 0, 0,
            0);
    unpack_v<CACHED, VBITS>(tid, f, Vl + (cb ^ 1) * VBUF);
    fetch_v<CACHED, VBITS>(c, k0 + 2 * BN, tid, f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
    }
    __syncthreads();
  }
  if (!lagging) __syncthreads();
}

template <int KBITS, int VBITS, bool TAYLOR, bool SPLIT>
__global__ __launch_bounds__(THREADS, 1) void attn_fast_kernel(AttnLaunch p, int32_t group_shift,
                                                                int64_t rows_per_kvhead, int64_t split_keys) {
  __shared__ __attribute__((aligned(16))) uint16_t Kl[2 * KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t Vl[2 * VBUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qc = lane & 31, h = lane >> 5;
  const int ng = D >> group_shift;

  const int64_t bkv = blockIdx.y;
  const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
  const int64_t gq = p.Hq / p.Hkv;

  // ---- this lane's query row, Q operand and the correction operand ----
  const int64_t r = static_cast<int64_t>(blockIdx.x) * BM + wave * 32 + qc;
  const bool row_ok = r < rows_per_kvhead;
  const int64_t rr = row_ok ? r : rows_per_kvhead - 1;
  const int64_t qrow = (b * p.Hq + hk * gq + rr / p.Nq) * p.Nq + rr % p.Nq;
  const uint16_t *qptr = p.q + qrow * D;
  QState qs;
  float nsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint4 w = *reinterpret_cast<const uint4 *>(qptr + 16 * s + 8 * h);
    qs.q[s] = __builtin_bit_cast(bf16x8, w);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += lo_f(u[i]) * lo_f(u[i]) + hi_f(u[i]) * hi_f(u[i]);
    const int gs = (16 * s + 8 * h) >> group_shift;
#pragma unroll
    for (int g = 0; g < 4; ++g) nsum[g] += g == gs ? acc : 0.f;
  }
  {
    float nh[4], nl[4], e[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float n = (nsum[g] + __shfl_xor(nsum[g], 32, 64)) * (p.tau / 24.0f);
      nh[g] = __uint_as_float(static_cast<uint32_t>(bf16_bits(n)) << 16);
      nl[g] = n - nh[g];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // slot 8h+j holds group (8h+j)/3, part (8h+j)%3 (hi, hi, lo)
      float v0 = 0.f, v1 = 0.f;
      const int s0 = j, s1 = 8 + j;
      if (s0 / 3 < ng) v0 = s0 % 3 == 2 ? nl[s0 / 3] : nh[s0 / 3];
      if (s1 / 3 < 4 && s1 / 3 < ng) v1 = s1 % 3 == 2 ? nl[s1 / 3] : nh[s1 / 3];
      e[j] = TAYLOR ? (h ? v1 : v0) : 0.f;
    }
    qs.qext = __builtin_bit_cast(bf16x8, make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]),
                                                    pack2(e[6], e[7])));
  }

  // ---- key ranges ----
  int64_t kbeg = 0, kend = p.Nc + p.Ncur;
  if (SPLIT) {
    kbeg = static_cast<int64_t>(blockIdx.z) * split_keys;
    kend = kbeg + split_keys < kend ? kbeg + split_keys : kend;
  }
  Ctx c{};
  c.ng = ng;
  c.group_shift = group_shift;

  Soft st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float alpha = p.tau * kLog2e;

  const bool lagging = __builtin_amdgcn_readfirstlane(wave) >= 4;
  if (p.Nc > 0) {
    const int64_t hrow = bkv * p.cap;  // first cache row of this head
    c.kc_codes = p.kc_codes + hrow * (D * KBITS / 8);
    c.vc_codes = p.vc_codes + hrow * (D * VBITS / 8);
    c.kc_scale = p.kc_scale + hrow * ng;
    c.kc_zero = p.kc_zero + hrow * ng;
    c.vc_scale = p.vc_scale + hrow * ng;
    c.vc_zero = p.vc_zero + hrow * ng;
  }
  c.beg = static_cast<int>(kbeg < p.Nc ? kbeg : p.Nc);
  c.end = static_cast<int>(kend < p.Nc ? kend : p.Nc);
  segment<true, TAYLOR, KBITS, VBITS>(c, qs, st, Kl, Vl, tid, lagging, alpha);
  if (p.Ncur > 0) {
    c.k_cur = p.k_cur + bkv * p.Ncur * D;
    c.v_cur = p.v_cur + bkv * p.Ncur * D;
  }
  c.beg = static_cast<int>((kbeg > p.Nc ? kbeg : p.Nc) - p.Nc);
  c.end = static_cast<int>((kend > p.Nc ? kend : p.Nc) - p.Nc);
  segment<false, TAYLOR, KBITS, VBITS>(c, qs, st, Kl, Vl, tid, lagging, alpha);

  const float l_tot = st.l + __shfl_xor(st.l, 32, 64);
  if (SPLIT) {
    if (row_ok) {
      float *w = static_cast<float *>(p.workspace) +
                 (static_cast<int64_t>(blockIdx.z) * (p.B * p.Hq * p.Nq) + qrow) * kPartialStride(D);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<float4 *>(w + 32 * db + 8 * g4 + 4 * h) =
              make_float4(st.o[db][4 * g4], st.o[db][4 * g4 + 1], st.o[db][4 * g4 + 2], st.o[db][4 * g4 + 3]);
      if (h == 0) {
        w[D] = st.m;
        w[D + 1] = l_tot;
      }
    }
    return;
  }
  if (row_ok) {
    const float inv = 1.0f / l_tot;
    uint16_t *optr = p.out + qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<uint2 *>(optr + 32 * db + 8 * g4 + 4 * h) =
            make_uint2(pack2(st.o[db][4 * g4] * inv, st.o[db][4 * g4 + 1] * inv),
                       pack2(st.o[db][4 * g4 + 2] * inv, st.o[db][4 * g4 + 3] * inv));
  }
}

template <int KB, int VB, bool SPLIT>
hipError_t launch_bits(const AttnLaunch &p, hipStream_t stream) {
  const int64_t rows = p.Nq * (p.Hq / p.Hkv);
  const int splits = SPLIT ? p.splits : 1;
  int64_t split_keys = (p.Nc + p.Ncur + splits - 1) / splits;
  split_keys = (split_keys + BN - 1) / BN * BN;
  const dim3 grid(static_cast<uint32_t>((rows + BM - 1) / BM), static_cast<uint32_t>(p.B * p.Hkv),
                  static_cast<uint32_t>(splits));
  const int32_t gshift = __builtin_ctz(static_cast<unsigned>(p.group));
  if (p.corr == KV_CORR_TAYLOR)
    attn_fast_kernel<KB, VB, true, SPLIT><<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows, split_keys);
  else
    attn_fast_kernel<KB, VB, false, SPLIT><<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows, split_keys);
  return hipGetLastError();
}

}  // namespace

bool fast_path_supported(const AttnLaunch &p) { return p.d == D && p.corr != KV_CORR_EXACT; }

hipError_t launch_attention_fast(const AttnLaunch &p, hipStream_t stream, bool split) {
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (split) {
    if (kb == 2 && vb == 2) return launch_bits<2, 2, true>(p, stream);
    if (kb == 2 && vb == 4) return launch_bits<2, 4, true>(p, stream);
    if (kb == 4 && vb == 2) return launch_bits<4, 2, true>(p, stream);
    return launch_bits<4, 4, true>(p, stream);
  }
  if (kb == 2 && vb == 2) return launch_bits<2, 2, false>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4, false>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2, false>(p, stream);
  return launch_bits<4, 4, false>(p, stream);
}

}  // namespace kvq
