// Short-query kernel of the corrected attention for gfx950 (head dim 128,
// correction off or Taylor, at most 32 query rows per KV head per row
// group): the regime where the packed cache read bounds the run.
//
// The work per cached key is its dequantisation (shared by few query rows),
// so the cache is split over many workgroups and, inside a workgroup, over
// its 4 waves: each wave streams its own 32-key blocks of the workgroup's
// key range and keeps its own running max, sum and output for all 32 rows
// of the row group, with private LDS tiles (no barrier inside the loop).
// The waves merge at the end (log-sum-exp), and the splits are merged by
// attn_combine_kernel.  Keys are fp16 (magic-code dequantisation) with a
// per-row query scale as in the throughput kernel, and the Taylor correction
// of the cached scores is one extra bf16 MFMA step ("量化鍵值偷走注意力…"
// (agents-report.net), §方法 and §為何校正有效).  Values and probabilities
// are fp16 here (values rounded once from an fp32 fma, as the keys): the
// value dequantisation is the largest share of the work per key, and the
// fp16 form needs no conversion after it.
//
// Power-of-two scales, chosen per 32-key block from that block's own steps
// and zero points (or values), keep the fp16 operands in range; no pass over
// the whole cache is needed.  Keys are stored as k 2^-ek, folded into the
// softmax scale of the block.  Values are stored as v 2^-ev and their
// probabilities as p 2^ev: the running max follows s alpha + ev, so every
// probability stays at most 2^8 (the lazy threshold) and O = sum p v is
// unchanged; l accumulates p 2^ev 2^-ev.
//
// Per block (per wave): dequantise K (rows = keys) and V^T (rows = head
// dimension, keys in the permuted order of the P operand) into LDS, fetch
// the next block, S^T = K Q^T (8 fp16 MFMA + 1 correction step), mask the
// ragged block, lazy max, exponentials, O^T += V^T P^T (8 fp16 MFMA).
//
// Caches grouped along the tokens (KVQ_SHORT_TOK units, fp32 metadata): as in
// the 16-row kernel, keys along the tokens fold each token group's steps into
// the query (q' = q D 2^-ed, rebuilt per group from the workgroup's fp16
// query tile in LDS) and take their raw codes as the fp16 subnormals c 2^-24,
// with q.z and the per-channel Taylor bias as one term per row; values along
// the tokens dequantise with per-channel operands staged per token group.
// Each wave then walks a contiguous range of blocks.
//
// Paged caches and 16-bit metadata: the instances for them are built from
// this file in translation units of their own (attention_short_paged.hip,
// attention_short_m16*.hip and attention_short_mb16*.hip define
// KVQ_SHORT_PAGED and KVQ_SHORT_META16 = 1 binary16 / 2 bfloat16), so that
// they cannot change how the default ones are compiled.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "quant_device.h"
#include "short_common.h"

#ifndef KVQ_SHORT_PAGED
#define KVQ_SHORT_PAGED 0
#endif
#ifndef KVQ_SHORT_TOK
#define KVQ_SHORT_TOK 0
#endif
#ifndef KVQ_SHORT_META16
#define KVQ_SHORT_META16 0
#endif

namespace kvq {
namespace {

using namespace dev;
using namespace sk;

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int VS = BK + 8;      // V^T row in LDS: fp16 keys[32], pad[8] (80 bytes)
constexpr int VT = D * VS;      // 16-bit elements of a wave's V^T tile
constexpr int OS = D + 4;       // fp32 row of the merge buffer
constexpr int MERGE = 32 * OS + 64;  // floats of a wave's merge buffer (O rows, then m and l)
constexpr int LDS_BYTES = WAVES * VT * 2 > WAVES * MERGE * 4 ? WAVES * VT * 2 : WAVES * MERGE * 4;
// groups along the tokens, inside the merge buffer's span (used only after
// the block loop): the workgroup's fp16 query tile [32][D] after the V^T
// tiles, then each wave's token-group staging of K and of V (2 D floats each)
constexpr int LQ = WAVES * VT;       // 16-bit offset of the query tile
constexpr int GSTAGE = LQ + 32 * D;  // 16-bit offset of the staging areas
static_assert((GSTAGE + WAVES * 4 * D * 2) * 2 <= LDS_BYTES, "token-group staging fits the merge buffer's span");

// V^T element (row = head-dim index, col = permuted key slot 0..31); the
// 16-byte chunks of a row are XOR-swizzled by (row / 16) % 4 so that the
// transposed 8-byte stores of 16 consecutive rows spread over the banks.
__device__ inline int vts(int row, int col) {
  return row * VS + ((((col >> 3) ^ (row >> 4)) & 3) << 3) + (col & 7);
}

// Registers of one prefetched cached block.
struct Fetch {
  uint32_t kw[8];      // K codes of d in [64h, 64h+64): INT4 8 words, INT2 4
  float kstep[2];      // step and zero point of the groups of d = 64h + 32j, j = 0, 1
  float kzero[2];
  uint32_t vw[4];      // V codes of keys 4kq+j at d in [16dq, 16dq+16): INT4 words
  uint32_t vw2[4];     //   d 16dq..+7 in vw, +8..+15 in vw2; INT2 all 16 in vw
  float vstep[4], vzero[4];
  uint32_t gd[2], gz[2], vgd[2], vgz[2];  // groups along the tokens: two steps / zero points of the
                                          // block's token group per lane (K, then V; fp32 bits)
};

// Lane roles (per wave):
//  K: key kr = lane % 32 of the block, head-dim half h = lane / 32
//     (d in [64h, 64h+64), i.e. whole groups for group >= 64)
//  V: keys 4kq..4kq+3 with kq = lane % 8, d in [16dq, 16dq+16), dq = lane / 8
// Byte offsets of the lane's data from the block's first cache row; NG is
// the number of quantisation groups per row (128 / group).
struct Lanes {
  uint32_t kc, km, vc, vm;
};
template <int KBITS, int VBITS, int NG, int MT>
__device__ inline Lanes lane_offsets(int lane) {
  constexpr uint32_t KROW = D * KBITS / 8, VROW = D * VBITS / 8, ES = MT ? 2 : 4;
  const uint32_t kr = lane & 31, h = lane >> 5, kq = lane & 7, dq = lane >> 3;
  Lanes o;
  o.kc = kr * KROW + h * (KROW / 2);
  o.km = kr * NG * ES;
  o.vc = 4 * kq * VROW + 16 * dq * VBITS / 8;
  o.vm = (4 * kq * NG + (16 * dq * NG) / D) * ES;  // the group of d = 16dq
  return o;
}

// Loads one cached block (rows [k0, k0 + 32)); rows at or past the segment
// end read as zero (their scores are masked).  Paged: the buffer range stops
// at the block's end, inside its page.
// Two fp32 steps and two zero points of a token group (at metadata row
// r0 >> gshift of the arrays s and z, one row of D per group) for the lane.
__device__ inline void fetch_group(const float *s, const float *z, size_t r0, int gshift, uint32_t (&gd)[2],
                                   uint32_t (&gz)[2]) {
  const size_t mrow = r0 >> gshift;
  const Buf bs = buffer_at(s + mrow * D, D * 4), bz = buffer_at(z + mrow * D, D * 4);
  const uint32_t off = static_cast<uint32_t>(__lane_id()) * 8;
  const u32x2 a = ld64(bs, off), b = ld64(bz, off);
  gd[0] = a.x; gd[1] = a.y;
  gz[0] = b.x; gz[1] = b.y;
}

template <int KBITS, int VBITS, int NG, bool PAGED, int MT, bool KTOK = false, bool VTOK = false>
__device__ inline void fetch_cached(const Ctx &c, int k0, const Lanes &o, int h, Fetch &f, size_t pool_row = 0,
                                    int gshift = 0, bool newg = false) {
  constexpr uint32_t KROW = D * KBITS / 8, VROW = D * VBITS / 8, ES = MT ? 2 : 4;
  const uint32_t rows = static_cast<uint32_t>(PAGED ? min(c.nc - k0, BK) : c.nc - k0);
  const size_t r0 = PAGED ? pool_row : block_row<false>(c, k0);  // paged: looked up a block earlier
  if (newg) {  // groups along the tokens: the block starts the wave's next token group
    if (KTOK) fetch_group(c.kc_scale, c.kc_zero, r0, gshift, f.gd, f.gz);
    if (VTOK) fetch_group(c.vc_scale, c.vc_zero, r0, gshift, f.vgd, f.vgz);
  }
  {
    const Buf kc = buffer_at(c.kc_codes + r0 * KROW, rows * KROW);
    const u32x4 a = ld128(kc, o.kc);
    f.kw[0] = a.x; f.kw[1] = a.y; f.kw[2] = a.z; f.kw[3] = a.w;
    if (KBITS == 4) {
      const u32x4 b = ld128(kc, o.kc + 16);
      f.kw[4] = b.x; f.kw[5] = b.y; f.kw[6] = b.z; f.kw[7] = b.w;
    }
  }
  if (!KTOK) {
    const Buf ks = buffer_at(meta_adv<MT>(c.kc_scale, r0 * NG), rows * NG * ES);
    const Buf kz = buffer_at(meta_adv<MT>(c.kc_zero, r0 * NG), rows * NG * ES);
    // the groups of d = 64h + 32j, j = 0, 1 (the lane's own values)
    if (NG == 1) {
      const float st = ld_meta1<MT>(ks, o.km), z = ld_meta1<MT>(kz, o.km);
      f.kstep[0] = f.kstep[1] = st;
      f.kzero[0] = f.kzero[1] = z;
    } else if (NG == 2) {
      const float st = ld_meta1<MT>(ks, o.km + ES * h), z = ld_meta1<MT>(kz, o.km + ES * h);
      f.kstep[0] = f.kstep[1] = st;
      f.kzero[0] = f.kzero[1] = z;
    } else {
      const float2 st = ld_meta2<MT>(ks, o.km + 2 * ES * h), z = ld_meta2<MT>(kz, o.km + 2 * ES * h);
      f.kstep[0] = st.x;
      f.kstep[1] = st.y;
      f.kzero[0] = z.x;
      f.kzero[1] = z.y;
    }
  }
  {
    const Buf vc = buffer_at(c.vc_codes + r0 * VROW, rows * VROW);
    const Buf vs = buffer_at(meta_adv<MT>(c.vc_scale, r0 * NG), rows * NG * ES);
    const Buf vz = buffer_at(meta_adv<MT>(c.vc_zero, r0 * NG), rows * NG * ES);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (VBITS == 4) {
        const u32x2 w = ld64(vc, o.vc + j * VROW);
        f.vw[j] = w.x;
        f.vw2[j] = w.y;
      } else {
        f.vw[j] = ld32(vc, o.vc + j * VROW);
      }
      if (!VTOK) {
        f.vstep[j] = ld_meta1<MT>(vs, o.vm + j * NG * ES);
        f.vzero[j] = ld_meta1<MT>(vz, o.vm + j * NG * ES);
      }
    }
  }
}

// ---- groups along the tokens (fp32 metadata) --------------------------------

// K operands of a cached block whose keys group along the tokens: the lane's
// codes (key kr, d = 64h + 8i .. +7 in k[i]), each in the low bits of a
// 16-bit field (the fp16 subnormal c 2^-24), word e holding dims e and e + 4.
template <int KBITS>
__device__ inline void unpack_k_codes(const Ctx &c, const Fetch &f, f16x8 (&k)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = KBITS == 4 ? f.kw[i] : (f.kw[i >> 1] >> (16 * (i & 1)));
    const uint32_t x = KBITS == 4 ? w : (w & 0xffffu) | ((w & 0xffffu) << 8);  // INT2: code e + 4 next to e
    uint32_t m[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = (x >> (KBITS * e)) & c.kmask;
    k[i] = __builtin_bit_cast(f16x8, make_uint4(m[0], m[1], m[2], m[3]));
  }
}

// Query terms of a token group for keys along the tokens: the group's steps
// D_c and zero points z_c (two each per lane in f, staged through the wave's
// area Gm) and the workgroup's query tile Lq (row qc: fp16 q 2^-eq) give
// qk[i] word e = fp16(q_c D_c 2^-ed) of d = 64h + 8i + e and + 4 (2^ed above
// the group's largest step), the block scale alpha_g = alpha_q 2^(ed + 24)
// and the row's term sadd = q.z - (tau/24) sum_c q_c^2 D_c^2 in the scores'
// units 2^-(eq + ed + 24) (qun = 2^eq).
template <bool TAYLOR>
__device__ inline void ktok_group(const Fetch &f, int lane, float *Gm, const uint16_t *Lq, float tau, float alpha_q,
                                  float qun, f16x8 (&qk)[8], float &sadd, float &alpha_g) {
  *reinterpret_cast<float2 *>(Gm + 2 * lane) = make_float2(__uint_as_float(f.gd[0]), __uint_as_float(f.gd[1]));
  *reinterpret_cast<float2 *>(Gm + D + 2 * lane) = make_float2(__uint_as_float(f.gz[0]), __uint_as_float(f.gz[1]));
  const float dmax = wave_max(fmaxf(__uint_as_float(f.gd[0]), __uint_as_float(f.gd[1])));
  const int ed = dmax > 0.f ? ilog2_pos(dmax) + 1 : 0;
  const float ds = ldexpf(1.0f, -ed);
  const int qc = lane & 31, h = lane >> 5;
  float s2 = 0.f, sz = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d0 = 64 * h + 8 * i;
    const float4 a0 = *reinterpret_cast<const float4 *>(Gm + d0), a1 = *reinterpret_cast<const float4 *>(Gm + d0 + 4);
    const float4 b0 = *reinterpret_cast<const float4 *>(Gm + D + d0);
    const float4 b1 = *reinterpret_cast<const float4 *>(Gm + D + d0 + 4);
    const float dd[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float zz[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const uint4 qw = *reinterpret_cast<const uint4 *>(Lq + qc * D + d0);  // word e: dims 2e, 2e + 1
    const uint32_t u[4] = {qw.x, qw.y, qw.z, qw.w};
    float qv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16x2 hh = __builtin_bit_cast(f16x2, u[e]);
      qv[2 * e] = static_cast<float>(hh.x);
      qv[2 * e + 1] = static_cast<float>(hh.y);
    }
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 a = static_cast<_Float16>(qv[e] * (dd[e] * ds));
      const _Float16 b = static_cast<_Float16>(qv[e + 4] * (dd[e + 4] * ds));
      w[e] = pair_h(a, b);
      s2 = fmaf(static_cast<float>(a), static_cast<float>(a), s2);
      s2 = fmaf(static_cast<float>(b), static_cast<float>(b), s2);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sz = fmaf(qv[e], zz[e], sz);
    qk[i] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  s2 += __shfl_xor(s2, 32, 64);
  sz += __shfl_xor(sz, 32, 64);
  const float bias = TAYLOR ? (tau / 24.0f) * qun * ldexpf(s2, ed) : 0.f;
  sadd = ldexpf(sz * ds - bias, -24);
  alpha_g = ldexpf(alpha_q, ed + 24);
}

// Values along the tokens: the largest |v| the lane's two channels of the
// token group can dequantise to, and their staged operands in the wave's
// area Gv (channel c: d_c = D_c vsc 2^-p, z_c vsc - 1024 d_c, p = 0 for even
// channels and the odd field's position 4 (INT4) or 2 (INT2) for odd ones).
template <int VBITS>
__device__ inline float vtok_bound(const Fetch &f) {
  float b = 0.f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float d = __uint_as_float(f.vgd[e]), z = __uint_as_float(f.vgz[e]);
    b = fmaxf(b, fmaxf(fabsf(z), fabsf(fmaf(d, static_cast<float>((1 << VBITS) - 1), z))));
  }
  return b;
}
template <int VBITS>
__device__ inline void vtok_stage(const Fetch &f, int lane, float vsc, float *Gv) {
  constexpr int P1 = VBITS == 4 ? 4 : 2;
  const float d0 = __uint_as_float(f.vgd[0]) * vsc, d1 = __uint_as_float(f.vgd[1]) * vsc * (1.0f / (1 << P1));
  *reinterpret_cast<float2 *>(Gv + 2 * lane) = make_float2(d0, d1);
  *reinterpret_cast<float2 *>(Gv + D + 2 * lane) =
      make_float2(fmaf(-1024.0f, d0, __uint_as_float(f.vgz[0]) * vsc), fmaf(-1024.0f, d1, __uint_as_float(f.vgz[1]) * vsc));
}

// Largest |k| (|v|) a lane's share of a cached block can dequantise to:
// the values of a group lie between z and z + (2^bits - 1) D.
// With at most two groups per row the cached keys are centred (see
// group_centre), and the bound is that of k - centre.
template <int KBITS, int NG>
__device__ inline float k_bound(const Fetch &f) {
  float b = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float z = NG <= 2 ? f.kzero[j] - group_centre<KBITS>(f.kzero[j], f.kstep[j]) : f.kzero[j];
    b = fmaxf(b, fmaxf(fabsf(z), fabsf(fmaf(f.kstep[j], static_cast<float>((1 << KBITS) - 1), z))));
  }
  return b;
}
template <int VBITS>
__device__ inline float v_bound(const Fetch &f) {
  float b = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b = fmaxf(b, fmaxf(fabsf(f.vzero[j]), fabsf(fmaf(f.vstep[j], static_cast<float>((1 << VBITS) - 1), f.vzero[j]))));
  return b;
}

// The cached keys are centred per group (group_centre) when a row has at
// most two groups: the extra bf16 step then has free slots 8 + 4g, 9 + 4g
// (lane half 1) for centre x query group sum.
template <int NG>
constexpr bool kCentre = NG <= 2;

// K operand of a cached block, straight into the MFMA A-operand registers
// of S^T = K Q^T: the lane (key kr = lane % 32, half h = lane / 32) holds
// its key's values d = 64h + 8s .. +7 in k[s] (k-step s, slots 8h .. 8h+7;
// the query uses the same order), as fp16 (k - c_g) 2^-ek (magic codes, one
// v_fma_mix each; c_g the group's centre, 0 with 4 groups), and in its
// extra-step slots 8h .. 8h+7, scaled like the keys, terms of its own
// groups only: with four groups (2h, 2h+1) the Taylor terms (-D_g^2 split
// hi, lo, hi; 0) of each; with two groups (group h), or one (half 0), the
// Taylor terms of the group, then (c_g, c_g, 0, 0) (the query side holds the
// group sums against the centres); zero Taylor terms without the correction.
template <bool TAYLOR, int KBITS, int NG>
__device__ inline void unpack_k_cached(const Ctx &c, int lane, const Fetch &f, float kscale, f16x8 (&k)[8],
                                       bf16x8 &kext) {
  const int h = lane >> 5;
  float sj[2], zj[2], cj[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    cj[j] = kCentre<NG> ? group_centre<KBITS>(f.kzero[j], f.kstep[j]) : 0.f;
    sj[j] = f.kstep[j] * kscale;
    zj[j] = fmaf(-1024.0f, f.kstep[j], f.kzero[j] - cj[j]) * kscale;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // values d = 64h + 8i .. +7, in the group of d = 64h + 32 (i / 4)
    uint32_t m[4];
    magic8<KBITS>(KBITS == 4 ? f.kw[i] : (f.kw[i >> 1] >> (16 * (i & 1))), c.kmask, m);
    const float st = sj[i >> 2], z = zj[i >> 2];
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = pair_h(dequant_h(magic_code(m, 2 * e), st, z), dequant_h(magic_code(m, 2 * e + 1), st, z));
    k[i] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  uint32_t x[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // Taylor terms of group j (four groups) or of the lane's group (j = 0)
    const float sq = TAYLOR ? f.kstep[j] * f.kstep[j] * kscale : 0.f;
    const float hsq = lo_f(pack2(sq, 0.f));
    x[2 * j] = pack2(-hsq, -(sq - hsq));
    x[2 * j + 1] = pack2(-hsq, 0.f);
  }
  if (kCentre<NG>) {
    const float cs = cj[0] * kscale;
    x[2] = pack2(cs, cs);
    x[3] = 0u;
    if (NG == 1 && h == 1) x[0] = x[1] = x[2] = 0u;  // one group: its terms sit in half 0
  }
  kext = __builtin_bit_cast(bf16x8, make_uint4(x[0], x[1], x[2], x[3]));
}

// V^T tile of a cached block: fp16 values v 2^-ev of keys 4kq..4kq+3
// (adjacent permuted slots: key r of a 16-key step sits at slot (r&3) +
// 4*(r>>3) + 8*((r>>2)&1)) at head-dim rows 16dq .. 16dq+15, one 8-byte store
// per row.  One v_perm gathers the same code byte of two keys
// (bits 0..7 and 16..23); one v_and_or turns a code field at bit p of both
// into the fp16 magic numbers 1024 + c 2^p (exact: the fp16 spacing at 1024
// is 1); then v 2^-ev = fma(1024 + c 2^p, D 2^-(p+ev), (z - 1024 D 2^-p) 2^-ev)
// with fp32 operands, one v_fma_mix per value rounded once to fp16.
// INT4 fields sit at p = 0 and 4; INT2 fields at p = 0 and 2 of the byte
// and of the byte shifted right by 4.
template <int VBITS>
__device__ inline void unpack_v_cached(const Ctx &c, int lane, const Fetch &f, float vsc, uint16_t *Vt) {
  constexpr int P1 = VBITS == 4 ? 4 : 2;
  const int kq = lane & 7, dq = lane >> 3;
  const int a = kq & 3;
  const int slot = 16 * (kq >> 2) + 4 * (a >> 1) + 8 * (a & 1);
  float dd[4][2], zz[4][2];  // per key: operands of the fields at p = 0 and p = P1
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float d0 = f.vstep[j] * vsc, z0 = f.vzero[j] * vsc;
    dd[j][0] = d0;
    dd[j][1] = d0 * (1.0f / (1 << P1));
    zz[j][0] = fmaf(-1024.0f, dd[j][0], z0);
    zz[j][1] = fmaf(-1024.0f, dd[j][1], z0);
  }
  auto field = [&](uint32_t r, int k, uint32_t (&x)[2], int jp) {  // k: 0 (p = 0) or 1 (p = P1)
    const uint32_t m = (r & (k ? c.vmask1 : c.vmask0)) | 0x64006400u;
    const f16x2 h = __builtin_bit_cast(f16x2, m);
    x[jp] = pair_h(dequant_h(static_cast<float>(h.x), dd[2 * jp][k], zz[2 * jp][k]),
                   dequant_h(static_cast<float>(h.y), dd[2 * jp + 1][k], zz[2 * jp + 1][k]));
  };
#pragma unroll
  for (int byte = 0; byte < (VBITS == 4 ? 8 : 4); ++byte) {
    // INT4: d = 16dq + 2byte + {0, 1} (bytes 4.. from vw2); INT2: d = 16dq + 4byte + {0, 1, 2, 3}
    const int bw = byte & 3;
    const uint32_t sel = static_cast<uint32_t>(bw) | 0x0c00u | (static_cast<uint32_t>(4 + bw) << 16) | 0x0c000000u;
    uint32_t r[2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const uint32_t w0 = byte >= 4 ? f.vw2[2 * jp] : f.vw[2 * jp];
      const uint32_t w1 = byte >= 4 ? f.vw2[2 * jp + 1] : f.vw[2 * jp + 1];
      r[jp] = __builtin_amdgcn_perm(w1, w0, sel);
    }
    constexpr int NF = 8 / VBITS;
    uint32_t x[NF][2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      field(r[jp], 0, x[0], jp);
      field(r[jp], 1, x[1], jp);
      if (VBITS == 2) {
        field(r[jp] >> 4, 0, x[NF - 2], jp);
        field(r[jp] >> 4, 1, x[NF - 1], jp);
      }
    }
#pragma unroll
    for (int fl = 0; fl < NF; ++fl)
      *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + NF * byte + fl, slot)) = make_uint2(x[fl][0], x[fl][1]);
  }
}

// unpack_v_cached with values along the tokens: the operands of channel
// c = 16dq + NF byte + fl come from the staged token group (area Gv), the
// same for the four keys.
template <int VBITS>
__device__ inline void unpack_v_tok(const Ctx &c, int lane, const Fetch &f, const float *Gv, uint16_t *Vt) {
  constexpr int NF = 8 / VBITS;
  const int kq = lane & 7, dq = lane >> 3;
  const int a = kq & 3;
  const int slot = 16 * (kq >> 2) + 4 * (a >> 1) + 8 * (a & 1);
  float dc[16], zc[16];
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 x = *reinterpret_cast<const float4 *>(Gv + 16 * dq + e);
    const float4 y = *reinterpret_cast<const float4 *>(Gv + D + 16 * dq + e);
    dc[e] = x.x; dc[e + 1] = x.y; dc[e + 2] = x.z; dc[e + 3] = x.w;
    zc[e] = y.x; zc[e + 1] = y.y; zc[e + 2] = y.z; zc[e + 3] = y.w;
  }
  auto field = [&](uint32_t r, int k, int e) {  // both keys of r at channel e, field k (0: p = 0, 1: p = P1)
    const uint32_t m = (r & (k ? c.vmask1 : c.vmask0)) | 0x64006400u;
    const f16x2 hh = __builtin_bit_cast(f16x2, m);
    return pair_h(dequant_h(static_cast<float>(hh.x), dc[e], zc[e]), dequant_h(static_cast<float>(hh.y), dc[e], zc[e]));
  };
#pragma unroll
  for (int byte = 0; byte < (VBITS == 4 ? 8 : 4); ++byte) {
    const int bw = byte & 3;
    const uint32_t sel = static_cast<uint32_t>(bw) | 0x0c00u | (static_cast<uint32_t>(4 + bw) << 16) | 0x0c000000u;
    uint32_t r[2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const uint32_t w0 = byte >= 4 ? f.vw2[2 * jp] : f.vw[2 * jp];
      const uint32_t w1 = byte >= 4 ? f.vw2[2 * jp + 1] : f.vw[2 * jp + 1];
      r[jp] = __builtin_amdgcn_perm(w1, w0, sel);
    }
    uint32_t x[NF][2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      x[0][jp] = field(r[jp], 0, NF * byte);
      x[1][jp] = field(r[jp], 1, NF * byte + 1);
      if (VBITS == 2) {
        x[NF - 2][jp] = field(r[jp] >> 4, 0, NF * byte + 2);
        x[NF - 1][jp] = field(r[jp] >> 4, 1, NF * byte + 3);
      }
    }
#pragma unroll
    for (int fl = 0; fl < NF; ++fl)
      *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + NF * byte + fl, slot)) = make_uint2(x[fl][0], x[fl][1]);
  }
}

// Current-chunk block (bf16 keys and values): the lane's raw rows (same
// lane roles as the cached blocks; rows past the end clamp to the last one,
// their scores are masked) and the largest |k| and |v| among them.
struct Cur {
  uint4 k[8];      // key kr, d = 64h .. 64h+63
  uint32_t v[4][8];  // keys 4kq+j, bf16 pairs of d = 16dq + 2i, +1
};
__device__ inline void load_current(const Ctx &c, int k0, int lane, Cur &x, float &kb, float &vb) {
  const int last = c.ncur - 1;
  kb = vb = 0.f;
  {
    const int kr = lane & 31, h = lane >> 5;
    const uint32_t row = static_cast<uint32_t>(k0 + kr <= last ? k0 + kr : last);
    const uint4 *ks = reinterpret_cast<const uint4 *>(c.k_cur + (row * D + 64u * h));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x.k[i] = ks[i];
      const uint32_t u[4] = {x.k[i].x, x.k[i].y, x.k[i].z, x.k[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) kb = fmaxf(kb, fmaxf(fabsf(lo_f(u[e])), fabsf(hi_f(u[e]))));
    }
  }
  {
    const int kq = lane & 7, dq = lane >> 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t row = static_cast<uint32_t>(k0 + 4 * kq + j <= last ? k0 + 4 * kq + j : last);
      const uint4 *vs = reinterpret_cast<const uint4 *>(c.v_cur + (row * D + 16u * dq));
      const uint4 y0 = vs[0], y1 = vs[1];
      x.v[j][0] = y0.x; x.v[j][1] = y0.y; x.v[j][2] = y0.z; x.v[j][3] = y0.w;
      x.v[j][4] = y1.x; x.v[j][5] = y1.y; x.v[j][6] = y1.z; x.v[j][7] = y1.w;
#pragma unroll
      for (int i = 0; i < 8; ++i) vb = fmaxf(vb, fmaxf(fabsf(lo_f(x.v[j][i])), fabsf(hi_f(x.v[j][i]))));
    }
  }
}

// Keys to MFMA operand registers (as unpack_k_cached, no correction) and
// values to the V^T tile (as unpack_v_cached), both rescaled to fp16.
__device__ inline void unpack_current(int lane, const Cur &x, float kscale, float vsc, f16x8 (&k)[8], uint16_t *Vt) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t u[4] = {x.k[i].x, x.k[i].y, x.k[i].z, x.k[i].w};
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack2h(lo_f(u[e]) * kscale, hi_f(u[e]) * kscale);
    k[i] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  const int kq = lane & 7, dq = lane >> 3;
  const int a = kq & 3;
  const int slot = 16 * (kq >> 2) + 4 * (a >> 1) + 8 * (a & 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + 2 * i, slot)) =
        make_uint2(pack2h(lo_f(x.v[0][i]) * vsc, lo_f(x.v[1][i]) * vsc), pack2h(lo_f(x.v[2][i]) * vsc, lo_f(x.v[3][i]) * vsc));
    *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + 2 * i + 1, slot)) =
        make_uint2(pack2h(hi_f(x.v[0][i]) * vsc, hi_f(x.v[1][i]) * vsc), pack2h(hi_f(x.v[2][i]) * vsc, hi_f(x.v[3][i]) * vsc));
  }
}

struct Soft {
  f32x16 o[D / 32];
  float m, l, alpha;
};

// Scores, softmax and value product of one block: K operand registers,
// the wave's V^T tile, the block's score scale alpha (scores are
// q.k 2^-(eq+ek)) and value exponent ev.  count < BK marks a ragged block;
// CORR adds the correction step.  CAUSAL: count is the lane's own (possibly
// <= 0), and a row may have seen no key yet (m = -inf).  ADD: the row's
// scores add sadd.
template <bool CORR, bool CAUSAL = false, bool ADD = false>
__device__ inline void block_compute(const f16x8 (&k)[8], bf16x8 kext, const uint16_t *Vt, const f16x8 (&q)[8],
                                     bf16x8 qext, int count, float alpha, int ev, int lane, Soft &st,
                                     float sadd = 0.f) {
  const float fev = static_cast<float>(ev);
  const int qc = lane & 31, h = lane >> 5;
  f32x16 s = f32x16{};
#pragma unroll
  for (int j = 0; j < 8; ++j) s = __builtin_amdgcn_mfma_f32_32x32x16_f16(k[j], q[j], s, 0, 0, 0);
  if (CORR) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kext, qext, s, 0, 0, 0);
  if (ADD) s += sadd;
  if (CAUSAL || count < BK) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + 4 * h + (i & 3) >= count) s[i] = -INFINITY;
  }
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[i]);
  mt = fmaf(xor32_max(mt), alpha, fev);
  const bool grow = mt > st.m + kLazy;
  if (__any(grow)) {
    const float m_new = grow ? mt : st.m;
    const float sc = CAUSAL && !grow ? 1.f : exp2f(st.m - m_new);
    st.l *= sc;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] *= sc;
    st.m = m_new;
  }
  f16x8 pk[2];
  const float shift = fev - st.m;
  float lb = 0.f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = __builtin_amdgcn_exp2f(fmaf(s[8 * hf + i], alpha, shift));
      if (CAUSAL && s[8 * hf + i] == -INFINITY) e[i] = 0.f;  // shift is +inf while m = -inf
    }
    pk[hf] = __builtin_bit_cast(f16x8, make_uint4(pack2h(e[0], e[1]), pack2h(e[2], e[3]), pack2h(e[4], e[5]),
                                                  pack2h(e[6], e[7])));
    lb = sum8h(pk[hf], lb);
  }
  st.l = fmaf(lb, ldexpf(1.0f, -ev), st.l);
  // O^T += V^T P^T: k-step ks (keys 16ks..16ks+15), head-dim block db
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int row = 32 * db + qc;
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          *reinterpret_cast<const f16x8 *>(Vt + vts(row, 16 * ks + 8 * h)), pk[ks], st.o[db], 0, 0, 0);
    }
}

// KTOK / VTOK: keys / values grouped along the tokens (fp32 metadata; p.group
// is then also their token group).
template <int KBITS, int VBITS, bool TAYLOR, int NG, bool CAUSAL, bool PAGED, int MT, bool KTOK = false,
          bool VTOK = false>
__global__ __launch_bounds__(THREADS, 2) void attn_short_kernel(AttnLaunch p, int64_t rows_per_kvhead,
                                                                int32_t row_groups, int32_t nsplit, float *ws) {
  constexpr bool TOK = KTOK || VTOK;
  __shared__ __attribute__((aligned(16))) uint16_t L[LDS_BYTES / 2];

  const int tid = threadIdx.x;
  if (blockIdx.x >= p.app.wg0) {  // the chunk append's workgroups
    qdev::append_workgroup<MT>(p, blockIdx.x - p.app.wg0, tid, THREADS);
    return;
  }
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block loop control stays scalar
  const int qc = lane & 31, h = lane >> 5;
  constexpr int ng = NG;
  constexpr int group_shift = NG == 1 ? 7 : NG == 2 ? 6 : 5;

  // Workgroups are dealt to the 8 XCDs round-robin by id; renumber so that
  // consecutive ids (the splits and row groups of one KV head) share an XCD.
  const uint32_t nwg = static_cast<uint32_t>(p.app.wg0), wg = blockIdx.x;
  const uint32_t per = nwg >> 3, extra = nwg & 7, xcd = wg & 7, slotw = wg >> 3;
  const uint32_t lin = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + slotw;
  const int64_t split = lin % static_cast<uint32_t>(nsplit);
  const int64_t rest = lin / static_cast<uint32_t>(nsplit);
  const int64_t rg = rest % row_groups;
  const int64_t bkv = rest / row_groups;
  const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
  const int64_t gq = p.Hq / p.Hkv;

  // the lane's query row (all 4 waves hold the same 32 rows)
  const int64_t r = rg * 32 + qc;
  const bool row_ok = r < rows_per_kvhead;
  const int64_t rr = row_ok ? r : rows_per_kvhead - 1;
  const int64_t qrow = (b * p.Hq + hk * gq + rr / p.Nq) * p.Nq + rr % p.Nq;
  f16x8 q[8];
  bf16x8 qext;
  Soft st;
  float qun = 1.f;
  load_query<TAYLOR, true>(p.q + qrow * D, h, group_shift, p.tau, 0, q, qext, st.alpha, &qun);
  const uint16_t *Lq = L + LQ;
  if (KTOK) {  // the workgroup's query tile for the token groups' query terms (every wave holds it)
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<f16x8 *>(L + LQ + qc * D + 64 * h + 8 * i) = q[i];
    }
    __syncthreads();
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;

  const int gshift = TOK ? __builtin_ctz(static_cast<unsigned>(p.group)) : 0;
  Ctx c{};
  c.nc = static_cast<int>(p.Nc);
  c.ncur = static_cast<int>(p.Ncur);
  c.kmask = opaque_u32(kCodeMask<KBITS>);
  c.vmask0 = opaque_u32(VBITS == 4 ? 0x000f000fu : 0x00030003u);
  c.vmask1 = opaque_u32(VBITS == 4 ? 0x00f000f0u : 0x000c000cu);
  c.layout = p.layout;
  c.cap = p.cap;
  c.H = p.Hkv;
  c.b = b;
  c.hk = hk;
  if (p.Nc > 0) {
    const int64_t hrow = PAGED ? 0 : bkv * p.cap;  // paged: the pointers stay at the pool
    c.kc_codes = p.kc_codes + hrow * (D * KBITS / 8);
    c.vc_codes = p.vc_codes + hrow * (D * VBITS / 8);
    // groups along the tokens: one metadata row of D per token group
    c.kc_scale = meta_adv<MT>(p.kc_scale, KTOK ? (hrow >> gshift) * D : hrow * ng);
    c.kc_zero = meta_adv<MT>(p.kc_zero, KTOK ? (hrow >> gshift) * D : hrow * ng);
    c.vc_scale = meta_adv<MT>(p.vc_scale, VTOK ? (hrow >> gshift) * D : hrow * ng);
    c.vc_zero = meta_adv<MT>(p.vc_zero, VTOK ? (hrow >> gshift) * D : hrow * ng);
  }
  if (p.Ncur > 0) {
    c.k_cur = p.k_cur + bkv * p.Ncur * D;
    c.v_cur = p.v_cur + bkv * p.Ncur * D;
  }

  // key blocks: cached [0, nbc), current [nbc, nbt); this split's range,
  // dealt to the waves round-robin
  const int nbc = (c.nc + BK - 1) / BK, nbt = nbc + (c.ncur + BK - 1) / BK;
  const int bps = (nbt + nsplit - 1) / nsplit;
  const int bbeg = static_cast<int>(split) * bps;
  int bend = bbeg + bps < nbt ? bbeg + bps : nbt;
  // causal mask: current keys below climit are visible to the lane's row
  // (query j of Nq, aligned to the chunk's end); the workgroup stops at the
  // largest limit of its 32 rows
  const int climit = static_cast<int>(rr % p.Nq + p.Ncur - p.Nq + 1);
  if (CAUSAL) {
    const int64_t r0 = rg * 32, r1 = min(r0 + 32, rows_per_kvhead) - 1;
    const int64_t wlim = (r0 / p.Nq == r1 / p.Nq ? r1 % p.Nq : p.Nq - 1) + p.Ncur - p.Nq + 1;
    const int cb = nbc + static_cast<int>(wlim > 0 ? (wlim + BK - 1) / BK : 0);
    if (bend > cb) bend = cb;
  }
  uint16_t *Vt = L + wave * VT;
  float *Gm = reinterpret_cast<float *>(L + GSTAGE) + wave * 4 * D;  // token-group staging of K
  float *Gv = Gm + 2 * D;                                             // and of V

  // blocks dealt round-robin, or (groups along the tokens) in contiguous
  // ranges per wave
  int blk = bbeg + wave, wend = bend, bstep = WAVES;
  if (TOK) {
    const int per = (bend - bbeg + WAVES - 1) / WAVES;
    blk = bbeg + wave * per;
    wend = blk + per < bend ? blk + per : bend;
    bstep = 1;
  }
  const int cend = wend < nbc ? wend : nbc;
  const Lanes lo = lane_offsets<KBITS, VBITS, NG, MT>(lane);
  Scales sc;
  // with the caches' running bounds the exponents of the cached blocks are
  // fixed once, from bounds that cover every cached block (a block's own
  // check is then skipped); the current chunk's blocks still check theirs
  const bool cache_bounds = p.Nc > 0 && p.kc_bound != nullptr && p.vc_bound != nullptr;
  if (cache_bounds) sc.update(p.kc_bound[bkv], p.vc_bound[bkv], st.alpha);
  f16x8 kreg[8];
  bf16x8 kext = {};
  Fetch f;
  // groups along the tokens: the wave's current token group and, for keys
  // along the tokens, its query terms
  f16x8 qk[8];
  float sadd = 0.f, alpha_g = 0.f;
  int gcur = -1;
  if (blk < cend)
    fetch_cached<KBITS, VBITS, NG, PAGED, MT, KTOK, VTOK>(c, blk * BK, lo, h, f, block_row<PAGED>(c, blk * BK),
                                                          gshift, TOK);
  // paged: the pool row of the next block to fetch, looked up one block ahead
  // so that its scalar load has completed when the fetch needs it
  size_t prn = PAGED && blk + bstep < cend ? block_row<PAGED>(c, (blk + bstep) * BK) : 0;
  for (; blk < cend; blk += bstep) {
    const int k0 = blk * BK;
    const int count = c.nc - k0 < BK ? c.nc - k0 : BK;
    const bool newg = TOK && (k0 >> gshift) != gcur;  // the block starts the wave's next token group
    const float vb = VTOK ? (newg ? vtok_bound<VBITS>(f) : 0.f) : v_bound<VBITS>(f);
    if (KTOK) {
      if (!cache_bounds) sc.update(0.f, vb, st.alpha);
      if (newg) ktok_group<TAYLOR>(f, lane, Gm, Lq, p.tau, st.alpha, qun, qk, sadd, alpha_g);
      unpack_k_codes<KBITS>(c, f, kreg);
    } else {
      if (!cache_bounds) sc.update(k_bound<KBITS, NG>(f), vb, st.alpha);
      unpack_k_cached<TAYLOR, KBITS, NG>(c, lane, f, sc.kscale, kreg, kext);
    }
    if (VTOK) {
      if (newg) vtok_stage<VBITS>(f, lane, sc.vscale, Gv);
      unpack_v_tok<VBITS>(c, lane, f, Gv, Vt);
    } else {
      unpack_v_cached<VBITS>(c, lane, f, sc.vscale, Vt);
    }
    if (newg) gcur = k0 >> gshift;
    if (blk + bstep < cend) {
      const int kn = (blk + bstep) * BK;
      fetch_cached<KBITS, VBITS, NG, PAGED, MT, KTOK, VTOK>(c, kn, lo, h, f, prn, gshift,
                                                            TOK && (kn >> gshift) != (k0 >> gshift));
    }
    if (KTOK)
      block_compute<false, false, true>(kreg, kext, Vt, qk, qext, count, alpha_g, sc.ev, lane, st, sadd);
    else
      block_compute<TAYLOR || kCentre<NG>>(kreg, kext, Vt, q, qext, count, sc.alpha, sc.ev, lane, st);
    if (PAGED && blk + 2 * bstep < cend) prn = block_row<PAGED>(c, (blk + 2 * bstep) * BK);
  }
  for (; blk < wend; blk += bstep) {
    const int k0 = (blk - nbc) * BK;
    int count = c.ncur - k0 < BK ? c.ncur - k0 : BK;
    if (CAUSAL) count = min(count, climit - k0);
    Cur x;
    float kb, vb;
    load_current(c, k0, lane, x, kb, vb);
    sc.update(kb, vb, st.alpha);
    unpack_current(lane, x, sc.kscale, sc.vscale, kreg, Vt);
    block_compute<false, CAUSAL>(kreg, kext, Vt, q, qext, count, sc.alpha, sc.ev, lane, st);
  }

  // ---- merge the 4 waves (log-sum-exp), then the split partial or output ----
  const float l_tot = st.l + __shfl_xor(st.l, 32, 64);
  __syncthreads();  // every wave is done with its tiles
  float *Ob = reinterpret_cast<float *>(L) + wave * MERGE;
  float *ml = Ob + 32 * OS;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<float4 *>(Ob + qc * OS + 32 * db + 8 * g4 + 4 * h) =
          make_float4(st.o[db][4 * g4], st.o[db][4 * g4 + 1], st.o[db][4 * g4 + 2], st.o[db][4 * g4 + 3]);
  if (h == 0) {
    ml[2 * qc] = st.m;
    ml[2 * qc + 1] = l_tot;
  }
  __syncthreads();
  {
    const int row = tid >> 3, d0 = (tid & 7) * 16;  // 32 rows x 8 chunks of 16
    const int64_t rrow = rg * 32 + row;
    if (rrow < rows_per_kvhead) {
      float mw[WAVES], m = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        mw[w] = reinterpret_cast<const float *>(L)[w * MERGE + 32 * OS + 2 * row];
        m = fmaxf(m, mw[w]);
      }
      float acc[16], l = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float *base = reinterpret_cast<const float *>(L) + w * MERGE;
        const float fw = mw[w] == -INFINITY ? 0.f : exp2f(mw[w] - m);
        l += fw * base[32 * OS + 2 * row + 1];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += fw * base[row * OS + d0 + e];
      }
      const int64_t orow = (b * p.Hq + hk * gq + rrow / p.Nq) * p.Nq + rrow % p.Nq;
      if (nsplit > 1) {
        float *w = ws + (split * (p.B * p.Hq * p.Nq) + orow) * kPartialStride(D);
#pragma unroll
        for (int e = 0; e < 16; e += 4)
          *reinterpret_cast<float4 *>(w + d0 + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
        if ((tid & 7) == 0) {
          w[D] = m;
          w[D + 1] = l;
        }
      } else {
        const float inv = 1.0f / l;
        uint16_t *o = p.out + orow * D + d0;
#pragma unroll
        for (int e = 0; e < 16; e += 4)
          *reinterpret_cast<uint2 *>(o + e) =
              make_uint2(pack2(acc[e] * inv, acc[e + 1] * inv), pack2(acc[e + 2] * inv, acc[e + 3] * inv));
      }
    }
  }
}

template <int KB, int VB, int NG, bool KT, bool VT>
void launch_kernel_t(const AttnLaunch &p, hipStream_t stream, dim3 grid, int64_t rows, int32_t row_groups,
                     float *partials) {
  constexpr bool PG = KVQ_SHORT_PAGED != 0;
  constexpr int MH = KVQ_SHORT_META16;
  auto kernel = p.corr == KV_CORR_TAYLOR ? (p.causal ? attn_short_kernel<KB, VB, true, NG, true, PG, MH, KT, VT>
                                                     : attn_short_kernel<KB, VB, true, NG, false, PG, MH, KT, VT>)
                                         : (p.causal ? attn_short_kernel<KB, VB, false, NG, true, PG, MH, KT, VT>
                                                     : attn_short_kernel<KB, VB, false, NG, false, PG, MH, KT, VT>);
  kernel<<<grid, dim3(THREADS), 0, stream>>>(p, rows, row_groups, p.splits, partials);
}

// The unit's instances: caches along the head dimension, or (KVQ_SHORT_TOK)
// K, V or both grouped along the tokens.
template <int KB, int VB, int NG>
void launch_kernel(const AttnLaunch &p, hipStream_t stream, dim3 grid, int64_t rows, int32_t row_groups,
                   float *partials) {
  if constexpr (KVQ_SHORT_TOK != 0) {
    if (p.ktok && p.vtok)
      launch_kernel_t<KB, VB, NG, true, true>(p, stream, grid, rows, row_groups, partials);
    else if (p.ktok)
      launch_kernel_t<KB, VB, NG, true, false>(p, stream, grid, rows, row_groups, partials);
    else
      launch_kernel_t<KB, VB, NG, false, true>(p, stream, grid, rows, row_groups, partials);
  } else {
    launch_kernel_t<KB, VB, NG, false, false>(p, stream, grid, rows, row_groups, partials);
  }
}

template <int KB, int VB>
hipError_t launch_bits(const AttnLaunch &p, hipStream_t stream) {
  const int64_t rows = p.Nq * (p.Hq / p.Hkv);
  const int32_t row_groups = static_cast<int32_t>((rows + 31) / 32);
  const int64_t nrows = p.B * p.Hq * p.Nq;
  float *partials = static_cast<float *>(p.workspace);
  // attention workgroups, then those of the chunk append (about 64 rows of
  // K and of V each)
  AttnLaunch pa = p;
  pa.app.wg0 = static_cast<int64_t>(p.splits) * row_groups * p.B * p.Hkv;
  const int64_t append_wgs = (p.B * p.Hkv * p.Ncur + 63) / 64;
  pa.app.wgs = p.app.on ? static_cast<int32_t>(append_wgs < 4096 ? append_wgs : 4096) : 0;
  const dim3 grid(static_cast<uint32_t>(pa.app.wg0 + pa.app.wgs));
  if (p.group == 128)
    launch_kernel<KB, VB, 1>(pa, stream, grid, rows, row_groups, partials);
  else if (p.group == 64)
    launch_kernel<KB, VB, 2>(pa, stream, grid, rows, row_groups, partials);
  else
    launch_kernel<KB, VB, 4>(pa, stream, grid, rows, row_groups, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_combine(partials, p.out, nrows, p.splits, p.d, stream);
}

}  // namespace

#if KVQ_SHORT_TOK
#if KVQ_SHORT_PAGED
hipError_t launch_attention_short_tok_paged(const AttnLaunch &p, hipStream_t stream) {
#else
hipError_t launch_attention_short_tok(const AttnLaunch &p, hipStream_t stream) {
#endif
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<2, 2>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2>(p, stream);
  return launch_bits<4, 4>(p, stream);
}
#elif KVQ_SHORT_PAGED || KVQ_SHORT_META16
#if KVQ_SHORT_PAGED && KVQ_SHORT_META16 == 2
hipError_t launch_attention_short_fast_mb16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT_META16 == 2
hipError_t launch_attention_short_fast_mb16(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT_PAGED && KVQ_SHORT_META16
hipError_t launch_attention_short_fast_m16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT_PAGED
hipError_t launch_attention_short_fast_paged(const AttnLaunch &p, hipStream_t stream) {
#else
hipError_t launch_attention_short_fast_m16(const AttnLaunch &p, hipStream_t stream) {
#endif
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<2, 2>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2>(p, stream);
  return launch_bits<4, 4>(p, stream);
}
#else
// d = 128, correction off or Taylor, groups along the head dimension, and
// (paged) pages that hold whole 32-key blocks.
bool short_fast_supported(int32_t d, int corr, bool tokens_axis, int32_t page_size) {
  return d == D && corr != KV_CORR_EXACT && !tokens_axis && (page_size == 0 || page_size >= BK);
}

// Caches grouped along the tokens on the 32-row tiles: as short_fast_supported
// with fp32 metadata (K, V or both along the tokens).
bool short_tok_supported(int32_t d, int corr, bool ktok, bool vtok, int32_t page_size, int meta) {
  return d == D && corr != KV_CORR_EXACT && (ktok || vtok) && (page_size == 0 || page_size >= BK) &&
         meta == kMetaF32;
}

int short_fast_splits(int64_t B, int64_t Hkv, int64_t rows_per_kvhead, int64_t Nc, int64_t Ncur, int cu_count) {
  const int64_t groups = B * Hkv * ((rows_per_kvhead + 31) / 32);
  const int64_t blocks = (Nc + BK - 1) / BK + (Ncur + BK - 1) / BK;
  // at most one round of resident workgroups (two fit a CU), each wave with
  // as many blocks as possible to spread its fixed costs (query load,
  // merge, partials) over.  Rounding the split count up instead put a few
  // workgroups into a second round: 24 KV heads at one row group, 22
  // splits (528 workgroups) took 108 us on a 61k cache, 21 splits 80 us.
  int64_t s = 2 * static_cast<int64_t>(cu_count) / groups;
  const int64_t max_s = (blocks + 4 * WAVES - 1) / (4 * WAVES);              // >= 4 blocks per wave
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 1024) s = 1024;
  return static_cast<int>(s);
}

hipError_t launch_attention_short_fast(const AttnLaunch &p, hipStream_t stream) {
  if (p.Nq * (p.Hq / p.Hkv) <= 16) {  // one 16-row query tile per KV head (attention_short16.hip)
    if (p.meta == kMetaBF16)
      return p.layout.page_table ? launch_attention_short16_mb16_paged(p, stream) : launch_attention_short16_mb16(p, stream);
    if (p.meta == kMetaF16)
      return p.layout.page_table ? launch_attention_short16_m16_paged(p, stream) : launch_attention_short16_m16(p, stream);
    return p.layout.page_table ? launch_attention_short16_paged(p, stream) : launch_attention_short16(p, stream);
  }
  if (p.meta == kMetaBF16)
    return p.layout.page_table ? launch_attention_short_fast_mb16_paged(p, stream)
                               : launch_attention_short_fast_mb16(p, stream);
  if (p.meta == kMetaF16)
    return p.layout.page_table ? launch_attention_short_fast_m16_paged(p, stream) : launch_attention_short_fast_m16(p, stream);
  if (p.layout.page_table) return launch_attention_short_fast_paged(p, stream);
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<2, 2>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2>(p, stream);
  return launch_bits<4, 4>(p, stream);
}
#endif

}  // namespace kvq
