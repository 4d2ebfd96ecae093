// Throughput kernel of the corrected attention for gfx950 (head dim 128,
// correction off or Taylor): the computation of attn_tile_kernel in
// attention.hip, reorganised for MI355X.
//
// Work split: one workgroup = 4 waves = 256 query rows of one KV head (GQA
// rows of all its query heads packed together); each wave owns 64 rows as
// two 32-row blocks A and B.  One wave per SIMD, so a wave has the whole
// register file (up to 512 VGPR+AGPR): room for the O accumulators of both
// blocks and for MFMA operands fetched from LDS ahead of their use.
//
// Per 64-key tile, software-pipelined inside the wave so that each stretch
// pairs matrix-core work with independent VALU work:
//   1. S_A = K Q_A^T            with  dequantise K of the next tile
//   2. S_B = K Q_B^T            with  softmax of block A
//   3. O_A += V^T P_A^T         with  softmax of block B
//   4. O_B += V^T P_B^T         with  dequantise V of the next tile, fetch
//                                     the packed tile after that from HBM
// Double-buffered LDS, one barrier per tile.  Cached and current segments
// run in separate loops.  Keys past the end of a segment are fetched as
// copies of its last key: their scores equal that key's, so the tile max is
// unchanged, and only their probabilities are zeroed (last tile only).
//
// Jensen-bias correction ("量化鍵值偷走注意力…" (agents-report.net), §方法:
// b = (1/(24 d)) sum_c q_c^2 D_{i,c}^2; §為何校正有效: subtracted from the
// quantised keys' scores before softmax): one extra K=16 MFMA step per 32x32
// score block with operands [tau/24 * ||q_g||^2] per query and [-D_g^2] per
// cached key, each split into bf16 hi and lo parts.  Cached keys are kept as
// hi + lo bf16 pairs (two MFMA chains): a single bf16 rounding of the
// dequantised key moves the scores of large-step groups too much.
//
// MFMA lane layouts (32x32x16 bf16, wave64): A operand lane l holds row l%32
// and k-slots 8*(l/32)..+7, B operand column l%32 and the same k-slots, the
// fp32 result column l%32 and rows 8*(i/4) + 4*(l/32) + i%4.  With S^T
// (keys as rows) each lane owns one query: row max and sum are local plus
// one exchange with lane l^32, and the P operand is the score accumulator
// itself; V^T is stored in LDS in the matching permuted key order.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int BM = 256;        // query rows per workgroup
constexpr int BN = 64;         // keys per tile
constexpr int THREADS = 256;   // 4 waves, 64 rows each
constexpr int KS = 2 * D + 16 + 8;  // K row in LDS: hi[128] lo[128] corr[16] pad[8] (bf16)
constexpr int KLO = D;
constexpr int KEXT = 2 * D;
constexpr int VS = BN + 8;     // V^T row in LDS (bf16)
constexpr int KBUF = BN * KS;  // bf16 elements per K buffer
constexpr int VBUF = D * VS;   // bf16 elements per V buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // rescale threshold (exp2 domain)

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// (x, y) -> the bf16 pair h = (bf16(x), bf16(y)) and the pair of residuals
// (bf16(x - h.x), bf16(y - h.y)).  Each residual is one v_dot2_f32_bf16:
// h.x * -1 + h.y * 0 + x = x - h.x, exact in fp32.  The weight pair
// (-1, -0.0) is written so that it is emitted as the 32-bit literal
// 0x8000bf80: the pair (-1, 0) gets encoded as the inline constant -1.0,
// which the hardware reads as the fp32 bit pattern 0xbf800000, i.e. the bf16
// pair (0, -1).
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

// V^T element (row = head-dim index, col = permuted key slot 0..63).  The
// 16-byte chunks of a row are XOR-swizzled by (row / 16) % 8.  With 64 LDS
// banks and a 144-byte row stride an operand read (16 lanes = 16
// consecutive rows, one chunk) lands on disjoint bank quads.
__device__ inline int vt_index(int row, int col) {
  return row * VS + ((((col >> 3) ^ (row >> 4)) & 7) << 3) + (col & 7);
}

// 8 codes of BITS bits (LSB first) in the low 8*BITS bits of w -> floats.
template <int BITS>
__device__ inline void codes8(uint32_t w, float *c) {
  if (BITS == 4) {
    const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;  // even / odd codes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = static_cast<float>((lo >> (8 * i)) & 0xffu);
      c[2 * i + 1] = static_cast<float>((hi >> (8 * i)) & 0xffu);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // byte k of (w >> 2j) & 0x0303 holds code 4k + j
      const uint32_t m = (w >> (2 * j)) & 0x0303u;
      c[j] = static_cast<float>(m & 0xffu);
      c[4 + j] = static_cast<float>((m >> 8) & 0xffu);
    }
  }
}

// Query-side operands of one lane: blocks A and B, its half of each k-step.
struct QState {
  bf16x8 q[2][D / 16];
  bf16x8 qext[2];
};

// Packed data of one tile held in registers between the fetch and the unpack.
struct Fetch {
  uint32_t kw[16];  // K: codes of 32 values (cached) or 32 bf16 values (current)
  uint32_t vw[16];  // V: codes of 4 keys x 8 values (cached) or 4 x 8 bf16 (current)
  float kstep, kzero;
  float gstep;      // step of group tid % 4 of the key (its correction slots)
  float vstep[4], vzero[4];
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

// Thread roles in fetch / unpack:
//  K: key tid / 4, values 32 * (tid % 4) .. +32
//  V: keys 4*kq .. 4*kq+3 with kq = tid / 16, values 8 * (tid % 16) .. +8
// Rows past the end of the segment clamp to its last row (always in bounds).
template <bool CACHED, int KBITS>
__device__ inline void fetch_k(const Ctx &c, int k0, int tid, Fetch &f) {
  const int last = c.end - 1;
  const int kk = tid >> 2, d0 = (tid & 3) * 32;
  const uint32_t krow = static_cast<uint32_t>(k0 + kk <= last ? k0 + kk : last);
  if (CACHED) {
    const uint8_t *ks = c.kc_codes + (krow * (D * KBITS / 8) + static_cast<uint32_t>(d0 * KBITS / 8));
    if (KBITS == 4) {
      const uint4 w = *reinterpret_cast<const uint4 *>(ks);
      f.kw[0] = w.x; f.kw[1] = w.y; f.kw[2] = w.z; f.kw[3] = w.w;
    } else {
      const uint2 w = *reinterpret_cast<const uint2 *>(ks);
      f.kw[0] = w.x; f.kw[1] = w.y;
    }
    const uint32_t km = krow * static_cast<uint32_t>(c.ng);
    const int gj = (tid & 3) < c.ng ? (tid & 3) : c.ng - 1;
    f.kstep = c.kc_scale[km + static_cast<uint32_t>(d0 >> c.group_shift)];
    f.kzero = c.kc_zero[km + static_cast<uint32_t>(d0 >> c.group_shift)];
    f.gstep = c.kc_scale[km + static_cast<uint32_t>(gj)];
  } else {
    const uint4 *ks = reinterpret_cast<const uint4 *>(c.k_cur + (krow * D + static_cast<uint32_t>(d0)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 a = ks[i];
      f.kw[4 * i] = a.x; f.kw[4 * i + 1] = a.y; f.kw[4 * i + 2] = a.z; f.kw[4 * i + 3] = a.w;
    }
  }
}

// Key j (0..3) of the thread's V quad.
template <bool CACHED, int VBITS>
__device__ inline void fetch_v(const Ctx &c, int k0, int tid, int j, Fetch &f) {
  const int last = c.end - 1;
  const int dq = tid & 15, kq = tid >> 4;
  const uint32_t vrow = static_cast<uint32_t>(k0 + 4 * kq + j <= last ? k0 + 4 * kq + j : last);
  if (CACHED) {
    const uint8_t *vs = c.vc_codes + (vrow * (D * VBITS / 8) + static_cast<uint32_t>(dq * VBITS));
    f.vw[j] = VBITS == 4 ? *reinterpret_cast<const uint32_t *>(vs)
                         : static_cast<uint32_t>(*reinterpret_cast<const uint16_t *>(vs));
    const uint32_t vm = vrow * static_cast<uint32_t>(c.ng) + static_cast<uint32_t>((8 * dq) >> c.group_shift);
    f.vstep[j] = c.vc_scale[vm];
    f.vzero[j] = c.vc_zero[vm];
  } else {
    const uint4 v = *reinterpret_cast<const uint4 *>(c.v_cur + (vrow * D + static_cast<uint32_t>(8 * dq)));
    f.vw[4 * j] = v.x; f.vw[4 * j + 1] = v.y; f.vw[4 * j + 2] = v.z; f.vw[4 * j + 3] = v.w;
  }
}

// ---- work items ----------------------------------------------------------
// The VALU work of a tile is cut into items of a few instructions each, and
// every item is issued right after one MFMA (see the regions below), so the
// matrix core and the vector ALU of the SIMD stay busy together.

// Scratch of the K dequantisation between items.
struct KWork {
  float cv[8];
  uint32_t wh[4], wl[4];
};

// K tile row: hi[d] and lo[d] of the dequantised key, and for the Taylor
// correction the slots 4g+{0,1,2,3} = (-D_g^2 split hi, lo, hi; 0), zero for
// g >= d/group, each thread writing the slots of group tid % 4.  Writes:
// 16 lanes = 4 keys x 4 quarter-rows, a 560-byte row stride puts them on
// 16 disjoint bank quads.  Item p: cached p < 16 is the value pair p, p = 16
// the correction slots; current p < 4 copies 8 bf16 values.
template <bool CACHED, bool TAYLOR, int KBITS>
constexpr int kItemsK = CACHED ? (TAYLOR ? 17 : 16) : 4;

template <bool CACHED, bool TAYLOR, int KBITS>
__device__ inline void unpack_k_item(int p, const Ctx &c, int tid, const Fetch &f, uint16_t *Kb, KWork &u) {
  const int kk = tid >> 2, d0 = (tid & 3) * 32;
  if (CACHED) {
    if (p < 16) {
      const int i = p >> 2, e = p & 3;
      if (e == 0) codes8<KBITS>(KBITS == 4 ? f.kw[i] : (f.kw[i >> 1] >> (16 * (i & 1))), u.cv);
      split2(fmaf(f.kstep, u.cv[2 * e], f.kzero), fmaf(f.kstep, u.cv[2 * e + 1], f.kzero), u.wh[e], u.wl[e]);
      if (e == 3) {
        *reinterpret_cast<uint4 *>(Kb + kk * KS + d0 + 8 * i) = make_uint4(u.wh[0], u.wh[1], u.wh[2], u.wh[3]);
        *reinterpret_cast<uint4 *>(Kb + kk * KS + KLO + d0 + 8 * i) = make_uint4(u.wl[0], u.wl[1], u.wl[2], u.wl[3]);
      }
    } else if (TAYLOR) {
      const float sq = (tid & 3) < c.ng ? f.gstep * f.gstep : 0.f;
      const float hsq = lo_f(pack2(sq, 0.f));
      *reinterpret_cast<uint2 *>(Kb + kk * KS + KEXT + 4 * (tid & 3)) =
          make_uint2(pack2(-hsq, -(sq - hsq)), pack2(-hsq, 0.f));
    }
  } else {
    *reinterpret_cast<uint4 *>(Kb + kk * KS + d0 + 8 * p) =
        make_uint4(f.kw[4 * p], f.kw[4 * p + 1], f.kw[4 * p + 2], f.kw[4 * p + 3]);
  }
}

// Scratch of the V dequantisation between items.
struct VWork {
  float v[4][8];
};

// V^T tile: the thread's 4 keys form a run of 4 permuted slots (key r of a
// 16-key step sits at slot (r&3) + 4*(r>>3) + 8*((r>>2)&1)), so each of its
// 8 head-dim rows gets one 8-byte store.  Item p < 4 dequantises key p,
// item 4 + e stores row e.
constexpr int kItemsV = 12;

template <bool CACHED, int VBITS>
__device__ inline void unpack_v_item(int p, int tid, const Fetch &f, uint16_t *Vb, VWork &u) {
  const int dq = tid & 15, kq = tid >> 4;
  if (p < 4) {
    if (CACHED) {
      float cv[8];
      codes8<VBITS>(f.vw[p], cv);
#pragma unroll
      for (int e = 0; e < 8; ++e) u.v[p][e] = fmaf(f.vstep[p], cv[e], f.vzero[p]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u.v[p][2 * e] = lo_f(f.vw[4 * p + e]);
        u.v[p][2 * e + 1] = hi_f(f.vw[4 * p + e]);
      }
    }
  } else {
    const int e = p - 4, a = kq & 3;
    const int slot = 16 * (kq >> 2) + ((a >> 1) << 2) + ((a & 1) << 3);
    *reinterpret_cast<uint2 *>(Vb + vt_index(8 * dq + e, slot)) =
        make_uint2(pack2(u.v[0][e], u.v[1][e]), pack2(u.v[2][e], u.v[3][e]));
  }
}

// Running softmax state of one lane, per query block.
struct Soft {
  f32x16 o[2][D / 32];
  float m[2], l[2];
};

// Tile max of a score block in 4 items (8 scores each), then the update.
__device__ inline void max_item(int r, const f32x16 (&acc)[2], float &mt) {
  const int kb = r >> 1, i0 = 8 * (r & 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) mt = fmaxf(mt, acc[kb][i0 + i]);
}

// Lazy rescale: the running max only moves when the tile max exceeds it by
// more than kLazy, so p <= 2^kLazy.
__device__ inline void max_update(float mt, float alpha, float &m, float &l, f32x16 (&o)[D / 32]) {
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * alpha;
  const bool grow = mt > m + kLazy;
  if (__any(grow)) {
    const float m_new = grow ? mt : m;
    const float sc = exp2f(m - m_new);
    l *= sc;
    // In place on the accumulator registers, one element at a time: written
    // as plain code the multiply makes the register allocator keep O in
    // VGPRs, which then no longer fit beside the operands.
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = o[db][i], t;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32_e32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(t)
                     : "v"(sc));
        o[db][i] = x;
      }
    m = m_new;
  }
}

// p = exp2(s * alpha - m) for scores 2k, 2k+1 of the block (k = 0..15); every
// fourth item packs 8 of them into a bf16 P operand and adds the rounded p to
// the row sum.  MASK zeroes keys at or past `count`.
template <bool MASK>
__device__ inline void exp_item(int k, const f32x16 (&acc)[2], float alpha, float m, float &l, int count, int h,
                                float (&e)[8], bf16x8 (&pk)[4]) {
  const int kb = k >> 3;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = 2 * (k & 7) + u;
    float x = __builtin_amdgcn_exp2f(fmaf(acc[kb][i], alpha, -m));
    if (MASK && kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3) >= count) x = 0.f;
    e[(2 * k + u) & 7] = x;
  }
  if ((k & 3) == 3) {
    pk[k >> 2] = __builtin_bit_cast(bf16x8, make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]),
                                                       pack2(e[6], e[7])));
    l = sum8(pk[k >> 2], l);
  }
}

// ---- MFMA sequences ------------------------------------------------------
// S^T of one block: MFMA j uses the K fragment at offset qk_off(j) from the
// lane's base (kb = j % 2 alternates the two accumulators): j < 16 the hi
// chain, j < 32 the lo chain, then the correction step.
template <bool CACHED, bool TAYLOR>
constexpr int kNqk = CACHED ? (TAYLOR ? 34 : 32) : 16;

__device__ constexpr int qk_off(int j) {
  return (j & 1) * 32 * KS + (j < 16 ? 16 * (j >> 1) : j < 32 ? KLO + 16 * ((j - 16) >> 1) : KEXT);
}

// O^T += V^T P^T: MFMA j = (k-step j / 4, head-dim block j % 4).  With the
// swizzle of vt_index the fragment of (row 32 db + qc, slot 16 ks + 8 h)
// sits at the lane's base (qc * VS + 8 * (h ^ (qc / 16))) plus a constant.
__device__ constexpr int pv_off(int j) {
  return 32 * (j & 3) * VS + 16 * ((j >> 2) ^ (j & 3));
}

__device__ inline bf16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

#define KVQ_MFMA(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0)
#define KVQ_FENCE() __builtin_amdgcn_sched_barrier(0)

// One 64-key tile (keys k0 .. k0 + count - 1 of the segment), reading LDS
// buffer cb, filling buffer cb ^ 1 with the next tile from f, and fetching
// the tile after that into f (K early in the tile, V at its end, so each
// fetch has most of a tile to arrive).
template <bool CACHED, bool TAYLOR, bool MASK, int KBITS, int VBITS>
__device__ inline void tile(const Ctx &c, const QState &qs, Soft &st, Fetch &f, uint16_t *Kl, uint16_t *Vl, int cb,
                            int k0, int count, int tid, float alpha) {
  const int lane = tid & 63, qc = lane & 31, h = lane >> 5;
  const uint16_t *Kb = Kl + cb * KBUF + qc * KS + 8 * h;
  const uint16_t *Vb = Vl + cb * VBUF + qc * VS + 8 * (h ^ (qc >> 4));
  uint16_t *Kn = Kl + (cb ^ 1) * KBUF;
  uint16_t *Vn = Vl + (cb ^ 1) * VBUF;
  constexpr int NQK = kNqk<CACHED, TAYLOR>;
  constexpr int NK = kItemsK<CACHED, TAYLOR, KBITS>;
  f32x16 sa[2], sb[2];
  bf16x8 pa[4], pb[4];
  bf16x8 buf[4];
  float ev[8];

  // 1. S_A, with the next tile's K dequantised into LDS (items on odd MFMAs)
  {
    KWork u;
    sa[0] = f32x16{};
    sa[1] = f32x16{};
#pragma unroll
    for (int j = 0; j < 4; ++j) buf[j] = lds8(Kb + qk_off(j));
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      sa[j & 1] = KVQ_MFMA(buf[j & 3], j < 32 ? qs.q[0][(j & 15) >> 1] : qs.qext[0], sa[j & 1]);
      if (j + 4 < NQK) buf[j & 3] = lds8(Kb + qk_off(j + 4));
      if ((j & 1) && (j >> 1) < NK) unpack_k_item<CACHED, TAYLOR, KBITS>(j >> 1, c, tid, f, Kn, u);
      KVQ_FENCE();
    }
  }

  // 2. S_B: its first MFMAs cover the max of block A, the rest the
  //    probabilities of block A; the fetch of K two tiles ahead goes first
  {
    float mt = -INFINITY;
    sb[0] = f32x16{};
    sb[1] = f32x16{};
#pragma unroll
    for (int j = 0; j < 4; ++j) buf[j] = lds8(Kb + qk_off(j));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sb[j & 1] = KVQ_MFMA(buf[j & 3], qs.q[1][(j & 15) >> 1], sb[j & 1]);
      buf[j & 3] = lds8(Kb + qk_off(j + 4));
      if (j == 0) fetch_k<CACHED, KBITS>(c, k0 + 2 * BN, tid, f);
      max_item(j, sa, mt);
      KVQ_FENCE();
    }
    max_update(mt, alpha, st.m[0], st.l[0], st.o[0]);
#pragma unroll
    for (int j = 4; j < NQK; ++j) {
      sb[j & 1] = KVQ_MFMA(buf[j & 3], j < 32 ? qs.q[1][(j & 15) >> 1] : qs.qext[1], sb[j & 1]);
      if (j + 4 < NQK) buf[j & 3] = lds8(Kb + qk_off(j + 4));
      if (j - 4 < 16) exp_item<MASK>(j - 4, sa, alpha, st.m[0], st.l[0], count, h, ev, pa);
      KVQ_FENCE();
    }
#pragma unroll
    for (int k = NQK - 4; k < 16; ++k) exp_item<MASK>(k, sa, alpha, st.m[0], st.l[0], count, h, ev, pa);
    asm volatile("" ::"v"(pa[0]), "v"(pa[1]), "v"(pa[2]), "v"(pa[3]));  // keep P_A above the branch
  }

  // 3. O_A: its first MFMAs cover the max of block B, the rest the
  //    probabilities of block B
  {
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) buf[j] = lds8(Vb + pv_off(j));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st.o[0][j & 3] = KVQ_MFMA(buf[j & 3], pa[j >> 2], st.o[0][j & 3]);
      buf[j & 3] = lds8(Vb + pv_off(j + 4));
      max_item(j, sb, mt);
      KVQ_FENCE();
    }
    max_update(mt, alpha, st.m[1], st.l[1], st.o[1]);
#pragma unroll
    for (int j = 4; j < 16; ++j) {
      st.o[0][j & 3] = KVQ_MFMA(buf[j & 3], pa[j >> 2], st.o[0][j & 3]);
      if (j + 4 < 16) buf[j & 3] = lds8(Vb + pv_off(j + 4));
      exp_item<MASK>(j - 4, sb, alpha, st.m[1], st.l[1], count, h, ev, pb);
      KVQ_FENCE();
    }
  }

  // 4. O_B, with the rest of block B's probabilities, the next tile's V
  //    into LDS, and the fetch of V two tiles ahead
  {
    VWork u;
#pragma unroll
    for (int j = 0; j < 4; ++j) buf[j] = lds8(Vb + pv_off(j));
#pragma unroll
    for (int k = 12; k < 16; ++k) exp_item<MASK>(k, sb, alpha, st.m[1], st.l[1], count, h, ev, pb);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      st.o[1][j & 3] = KVQ_MFMA(buf[j & 3], pb[j >> 2], st.o[1][j & 3]);
      if (j + 4 < 16) buf[j & 3] = lds8(Vb + pv_off(j + 4));
      if (j < kItemsV) unpack_v_item<CACHED, VBITS>(j, tid, f, Vn, u);
      else fetch_v<CACHED, VBITS>(c, k0 + 2 * BN, tid, j - kItemsV, f);
      KVQ_FENCE();
    }
  }
  __syncthreads();
}

#undef KVQ_MFMA
#undef KVQ_FENCE

// One segment (cached or current keys) of the key range.
template <bool CACHED, bool TAYLOR, int KBITS, int VBITS>
__device__ inline void segment(const Ctx &c, const QState &qs, Soft &st, uint16_t *Kl, uint16_t *Vl, int tid,
                               float alpha) {
  const int nt = c.end > c.beg ? (c.end - c.beg + BN - 1) / BN : 0;
  if (nt == 0) return;
  constexpr int NK = kItemsK<CACHED, TAYLOR, KBITS>;
  Fetch f;
  {
    KWork uk;
    VWork uv;
    fetch_k<CACHED, KBITS>(c, c.beg, tid, f);
#pragma unroll
    for (int j = 0; j < 4; ++j) fetch_v<CACHED, VBITS>(c, c.beg, tid, j, f);
#pragma unroll
    for (int p = 0; p < NK; ++p) unpack_k_item<CACHED, TAYLOR, KBITS>(p, c, tid, f, Kl, uk);
#pragma unroll
    for (int p = 0; p < kItemsV; ++p) unpack_v_item<CACHED, VBITS>(p, tid, f, Vl, uv);
    fetch_k<CACHED, KBITS>(c, c.beg + BN, tid, f);
#pragma unroll
    for (int j = 0; j < 4; ++j) fetch_v<CACHED, VBITS>(c, c.beg + BN, tid, j, f);
  }
  __syncthreads();
  const int tail = c.end - c.beg - (nt - 1) * BN;  // keys in the last tile
  for (int t = 0; t < nt - 1; ++t)
    tile<CACHED, TAYLOR, false, KBITS, VBITS>(c, qs, st, f, Kl, Vl, t & 1, c.beg + t * BN, BN, tid, alpha);
  const int k0 = c.beg + (nt - 1) * BN;
  if (tail == BN)
    tile<CACHED, TAYLOR, false, KBITS, VBITS>(c, qs, st, f, Kl, Vl, (nt - 1) & 1, k0, BN, tid, alpha);
  else
    tile<CACHED, TAYLOR, true, KBITS, VBITS>(c, qs, st, f, Kl, Vl, (nt - 1) & 1, k0, tail, tid, alpha);
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

  // ---- the lane's two query rows: Q operands and correction operands ----
  QState qs;
  int64_t qrow[2];
  bool row_ok[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * BM + wave * 64 + blk * 32 + qc;
    row_ok[blk] = r < rows_per_kvhead;
    const int64_t rr = row_ok[blk] ? r : rows_per_kvhead - 1;
    qrow[blk] = (b * p.Hq + hk * gq + rr / p.Nq) * p.Nq + rr % p.Nq;
    const uint16_t *qptr = p.q + qrow[blk] * D;
    float nsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint4 w = *reinterpret_cast<const uint4 *>(qptr + 16 * s + 8 * h);
      qs.q[blk][s] = __builtin_bit_cast(bf16x8, w);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += lo_f(u[i]) * lo_f(u[i]) + hi_f(u[i]) * hi_f(u[i]);
      const int gs = (16 * s + 8 * h) >> group_shift;
#pragma unroll
      for (int g = 0; g < 4; ++g) nsum[g] += g == gs ? acc : 0.f;
    }
    // N_g = tau/24 * ||q_g||^2 in slots 4g+{0,1,2,3} as (hi, hi, lo, 0); the
    // lane holds slots 8h .. 8h+7, i.e. groups 2h and 2h+1
    float nh[4], nl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float n = TAYLOR && g < ng ? (nsum[g] + __shfl_xor(nsum[g], 32, 64)) * (p.tau / 24.0f) : 0.f;
      nh[g] = lo_f(pack2(n, 0.f));
      nl[g] = n - nh[g];
    }
    const float n0h = h ? nh[2] : nh[0], n0l = h ? nl[2] : nl[0];
    const float n1h = h ? nh[3] : nh[1], n1l = h ? nl[3] : nl[1];
    qs.qext[blk] = __builtin_bit_cast(bf16x8, make_uint4(pack2(n0h, n0h), pack2(n0l, 0.f),
                                                         pack2(n1h, n1h), pack2(n1l, 0.f)));
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
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[blk][db] = f32x16{};
    st.m[blk] = -INFINITY;
    st.l[blk] = 0.f;
  }
  const float alpha = p.tau * kLog2e;

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
  segment<true, TAYLOR, KBITS, VBITS>(c, qs, st, Kl, Vl, tid, alpha);
  if (p.Ncur > 0) {
    c.k_cur = p.k_cur + bkv * p.Ncur * D;
    c.v_cur = p.v_cur + bkv * p.Ncur * D;
  }
  c.beg = static_cast<int>((kbeg > p.Nc ? kbeg : p.Nc) - p.Nc);
  c.end = static_cast<int>((kend > p.Nc ? kend : p.Nc) - p.Nc);
  segment<false, TAYLOR, KBITS, VBITS>(c, qs, st, Kl, Vl, tid, alpha);

#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float l_tot = st.l[blk] + __shfl_xor(st.l[blk], 32, 64);
    if (!row_ok[blk]) continue;
    if (SPLIT) {
      float *w = static_cast<float *>(p.workspace) +
                 (static_cast<int64_t>(blockIdx.z) * (p.B * p.Hq * p.Nq) + qrow[blk]) * kPartialStride(D);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<float4 *>(w + 32 * db + 8 * g4 + 4 * h) =
              make_float4(st.o[blk][db][4 * g4], st.o[blk][db][4 * g4 + 1], st.o[blk][db][4 * g4 + 2],
                          st.o[blk][db][4 * g4 + 3]);
      if (h == 0) {
        w[D] = st.m[blk];
        w[D + 1] = l_tot;
      }
    } else {
      const float inv = 1.0f / l_tot;
      uint16_t *optr = p.out + qrow[blk] * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<uint2 *>(optr + 32 * db + 8 * g4 + 4 * h) =
              make_uint2(pack2(st.o[blk][db][4 * g4] * inv, st.o[blk][db][4 * g4 + 1] * inv),
                         pack2(st.o[blk][db][4 * g4 + 2] * inv, st.o[blk][db][4 * g4 + 3] * inv));
    }
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
