// Device side of the group-wise asymmetric quantizer, shared by kv_quantize
// (quantize.hip) and the chunk append fused into the attention call, so that
// both write the same bytes for the same input.
//
// The pages: "量化鍵值偷走注意力…" (agents-report.net), section 方法 -- one
// step size per group enters the correction; "QuantWM：…" (pchao.org),
// section 方法概览 -- each cache block is quantised once after it is built.
// The exact formula (step = range / (2^bits - 1), zero point = group
// minimum, codes rounded half to even and clamped) is this library's
// reading, stated in include/kvq.h.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace qdev {

template <int LANES>
__device__ inline float group_min(float v) {
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

template <int LANES>
__device__ inline float group_max(float v) {
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <typename T>
__device__ inline void load8(const T *p, float (&v)[8]);

template <>
__device__ inline void load8<uint16_t>(const uint16_t *p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4 *>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

template <>
__device__ inline void load8<float>(const float *p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Code of value v: rne((v - zp) / step) clamped to [0, TOP], with the IEEE
// quotient of the definition.  The product with the reciprocal (v_rcp_f32,
// 1 ulp; then one rounding) lies within 2^-21 |q| of that quotient, so when
// it is farther than 2^-19 |q| + 2^-20 from every half-integer the two round
// to the same integer; otherwise, or when step is outside [2^-120, 2^120]
// (reciprocal not a normal number), the division itself is taken.
template <int TOP>
__device__ inline uint32_t code_of(float v, float zp, float step, float inv, bool fast) {
#pragma clang fp contract(off)
  const float num = v - zp;
  float r;
  const float q = num * inv;
  const float frac = q - floorf(q);
  if (fast && fabsf(frac - 0.5f) > fmaf(fabsf(q), 0x1p-19f, 0x1p-20f))
    r = rintf(q);
  else
    r = rintf(num / step);  // IEEE division
  return static_cast<uint32_t>(fminf(fmaxf(r, 0.0f), static_cast<float>(TOP)));
}

__device__ inline bool reciprocal_ok(float step) { return step >= 0x1p-120f && step <= 0x1p120f; }

// Codes of one lane's 8 consecutive values of a group that LANES adjacent,
// aligned lanes hold (every lane of the group must execute this), packed
// LSB-first; step and zp are the group's step and zero point as stored (with
// 16-bit metadata of kind MT, rounded to it before the codes are taken, so
// that z + D c uses exactly the stored pair).
template <int BITS, int LANES, int MT>
__device__ inline uint32_t quantize8(const float (&v)[8], float &step, float &zp) {
#pragma clang fp contract(off)
  constexpr int TOP = (1 << BITS) - 1;
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = v[i] < mn ? v[i] : mn;
    mx = v[i] > mx ? v[i] : mx;
  }
  mn = group_min<LANES>(mn) + 0.0f;  // + 0.0f: a zero extreme is +0
  mx = group_max<LANES>(mx) + 0.0f;
  const float range = mx - mn;
  step = range / static_cast<float>(TOP);  // IEEE division
  zp = mn;
  if (MT != kMetaF32) {
    step = meta_round(step, MT);
    zp = meta_round(mn, MT);
  }
  uint32_t packed = 0;
  if (step > 0.0f) {
    const bool fast = reciprocal_ok(step);
    const float inv = fast ? __builtin_amdgcn_rcpf(step) : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= code_of<TOP>(v[i], zp, step, inv, fast) << (i * BITS);
  }
  return packed;
}

// Bound of a group's dequantised values from its stored step and zero
// point: the values lie between z and z + (2^bits - 1) D.  The attention
// pre-passes use the same rule when they scan the metadata themselves.
template <int BITS>
__device__ inline float group_bound(float step, float zp) {
  return fmaxf(fabsf(zp), fabsf(fmaf(step, static_cast<float>((1 << BITS) - 1), zp)));
}

// Raise entry i of a running bound to b (b >= 0, so the order of the float
// bits is that of the integers: one atomic max), only when b exceeds the
// value read first.  The bound never falls, so a stale read can only be
// lower than the entry: it may cost a needless atomic, never a lost raise;
// and the many waves that write one entry (a long append) stop contending
// for it once it holds their group's maximum.
__device__ inline void bound_max(float *bound, int64_t i, float b) {
  if (b > 0.f && b > __builtin_nontemporal_load(bound + i)) atomicMax(reinterpret_cast<int *>(bound) + i, __float_as_int(b));
}

// Raise the running bound of (b, h) = entry i to b.  Every lane of the wave
// must call this together: when all lanes name the same entry the wave
// maximum goes in from one lane, otherwise each lane raises its own.
__device__ inline void raise_bound(float *bound, int64_t i, float b) {
  if (!bound) return;
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(i));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(i) >> 32));
  const int64_t i0 = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  if (__all(i == i0)) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) b = fmaxf(b, __shfl_xor(b, o, 64));
    if (__lane_id() == 0) bound_max(bound, i0, b);
  } else {
    bound_max(bound, i, b);
  }
}

// Stores one lane's packed codes of token row `orow` (lane `chunk` of the
// row's d/8) and, from the first lane of each group, the group's step and
// zero point.
template <int BITS, int LANES, int MT>
__device__ inline void store8(uint8_t *codes, float *scale, float *zero, int64_t orow, int32_t lanes_per_row,
                              int32_t chunk, uint32_t packed, float step, float zp) {
  uint8_t *dst = codes + orow * (static_cast<int64_t>(lanes_per_row) * BITS) + static_cast<int64_t>(chunk) * BITS;
  if (BITS == 2)
    *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(packed);
  else
    *reinterpret_cast<uint32_t *>(dst) = packed;
  if ((chunk % LANES) == 0) {
    const int64_t m = orow * (lanes_per_row / LANES) + chunk / LANES;
    if (MT != kMetaF32) {  // step and zp already hold 16-bit values: the patterns are exact
      reinterpret_cast<uint16_t *>(scale)[m] = meta16_bits(step, MT);
      reinterpret_cast<uint16_t *>(zero)[m] = meta16_bits(zp, MT);
    } else {
      scale[m] = step;
      zero[m] = zp;
    }
  }
}

// ---- the append fused into an attention call --------------------------------

// Codes of one lane's 8 values with `bits` chosen at run time (uniform).
template <int LANES, int MT>
__device__ inline uint32_t quantize8_bits(int bits, const float (&v)[8], float &step, float &zp) {
  return bits == 2 ? quantize8<2, LANES, MT>(v, step, zp) : quantize8<4, LANES, MT>(v, step, zp);
}

template <int LANES, int MT>
__device__ inline void store8_bits(int bits, uint8_t *codes, float *scale, float *zero, int64_t orow,
                                   int32_t lanes_per_row, int32_t chunk, uint32_t packed, float step, float zp) {
  if (bits == 2)
    store8<2, LANES, MT>(codes, scale, zero, orow, lanes_per_row, chunk, packed, step, zp);
  else
    store8<4, LANES, MT>(codes, scale, zero, orow, lanes_per_row, chunk, packed, step, zp);
}

// Token rows [r0, r1) of the bf16 current chunk ([B][Hkv][Ncur][d], rows
// flattened), K and V together: with `write`, their codes, steps and zero
// points go to cache rows Nc + t of the same (b, KV head), t the row's token
// index, as kv_quantize(k_cur / v_cur, ..., tok_offset = Nc) writes them.
// The workgroup's nthr threads (a multiple of d/8) take d/8 lanes per row,
// row r0 + tid / (d/8) first, then every nthr / (d/8) rows, K and V of a row
// loaded together.  kb, vb: raised to the largest |k| and |v| over the
// lane's values (the pre-passes' bounds).
// The running bounds the rows raise: on a row's first lane, those of its
// rows in (b, KV head) entry `cur` (earlier entries already raised); zero on
// the other lanes.
struct RowBounds {
  float k = 0.f, v = 0.f;
  int64_t cur = 0;
};

template <int LANES, int MT>
__device__ void append_rows_t(const AttnLaunch &p, int64_t r0, int64_t r1, bool write, int tid, int nthr, float &kb,
                              float &vb, RowBounds &rb) {
  const AppendLaunch &a = p.app;
  const int32_t lanes_per_row = p.d >> 3;
  const int32_t chunk = tid & (lanes_per_row - 1);
  const int32_t per_pass = nthr / lanes_per_row;
  const int64_t lane_row = tid / lanes_per_row;
  // (KV head, token) of row r0; rows past it by less than 2^31 are found in
  // 32-bit arithmetic (a workgroup's range is far shorter)
  const int64_t bkv0 = r0 / p.Ncur;
  const uint32_t tok0 = static_cast<uint32_t>(r0 - bkv0 * p.Ncur), ncur = static_cast<uint32_t>(p.Ncur);
  const uint32_t hkv = static_cast<uint32_t>(p.Hkv);
  // running bounds of the rows' groups, per (b, KV head) entry; a lane whose
  // rows move to the next entry hands the finished one over first
  float kbnd = 0.f, vbnd = 0.f;
  int64_t cur = bkv0;
  auto load = [&](int64_t base, float (&k)[8], float (&v)[8]) {
    const int64_t r = base + lane_row;
    const int64_t rr = (r < r1 ? r : r1 - 1) * p.d + chunk * 8;  // dead rows (whole groups) repeat the last one
    load8<uint16_t>(p.k_cur + rr, k);
    load8<uint16_t>(p.v_cur + rr, v);
  };
  for (int64_t base = r0; base < r1; base += per_pass) {
    float k[8], v[8];
    load(base, k, v);
    const int64_t r = base + lane_row;
    const bool live = r < r1;
    if (live) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kb = fmaxf(kb, fabsf(k[i]));
        vb = fmaxf(vb, fabsf(v[i]));
      }
    }
    if (write) {
      float ks, kz, vs, vz;
      const uint32_t kp = quantize8_bits<LANES, MT>(a.bits[0], k, ks, kz);
      const uint32_t vp = quantize8_bits<LANES, MT>(a.bits[1], v, vs, vz);
      if (live) {
        const uint32_t o = tok0 + static_cast<uint32_t>(r - r0);  // < 2^23 + 2^31
        const uint32_t dq = o / ncur, tok = o - dq * ncur;
        const uint32_t bkv = static_cast<uint32_t>(bkv0) + dq;  // < 65536
        const uint32_t b = bkv / hkv, h = bkv - b * hkv;
        const int64_t orow = a.layout.row(a.cap, p.Hkv, b, h, p.Nc + tok);
        store8_bits<LANES, MT>(a.bits[0], a.codes[0], a.scale[0], a.zero[0], orow, lanes_per_row, chunk, kp, ks, kz);
        store8_bits<LANES, MT>(a.bits[1], a.codes[1], a.scale[1], a.zero[1], orow, lanes_per_row, chunk, vp, vs, vz);
        // the row's bound over its lanes (a row's lanes are live together),
        // kept by its first lane
        float kr = a.bits[0] == 2 ? group_bound<2>(ks, kz) : group_bound<4>(ks, kz);
        float vr = a.bits[1] == 2 ? group_bound<2>(vs, vz) : group_bound<4>(vs, vz);
        for (int o = LANES; o < lanes_per_row; o <<= 1) {
          kr = fmaxf(kr, __shfl_xor(kr, o, 64));
          vr = fmaxf(vr, __shfl_xor(vr, o, 64));
        }
        if (chunk == 0) {
          if (bkv != cur) {  // the lane's rows crossed into the next (b, KV head): hand the last one over
            if (a.bound[0]) bound_max(a.bound[0], cur, kbnd);
            if (a.bound[1]) bound_max(a.bound[1], cur, vbnd);
            cur = bkv;
            kbnd = vbnd = 0.f;
          }
          kbnd = fmaxf(kbnd, kr);
          vbnd = fmaxf(vbnd, vr);
        }
      }
    }
  }
  rb.k = kbnd;
  rb.v = vbnd;
  rb.cur = cur;
}

// append_rows_t with the caches' group and metadata kind MT (which must be
// p.app.meta; bounds only, no group reduction and nothing stored, without
// `write`).  kb, vb are raised to the bounds of the rows; rb receives the
// rows' running bounds for the caller to raise (its workgroup's rows may
// share one entry).
template <int MT>
__device__ inline void append_rows(const AttnLaunch &p, int64_t r0, int64_t r1, bool write, int tid, int nthr,
                                   float &kb, float &vb, RowBounds &rb) {
  if (!write) return append_rows_t<4, kMetaF32>(p, r0, r1, false, tid, nthr, kb, vb, rb);
  const int g = p.app.group;
  if (g == 32) return append_rows_t<4, MT>(p, r0, r1, true, tid, nthr, kb, vb, rb);
  if (g == 64) return append_rows_t<8, MT>(p, r0, r1, true, tid, nthr, kb, vb, rb);
  return append_rows_t<16, MT>(p, r0, r1, true, tid, nthr, kb, vb, rb);
}

// The same with the metadata kind read from p.app.meta.
__device__ inline void append_rows_any(const AttnLaunch &p, int64_t r0, int64_t r1, bool write, int tid, int nthr,
                                       float &kb, float &vb, RowBounds &rb) {
  if (p.app.meta == kMetaBF16) return append_rows<kMetaBF16>(p, r0, r1, write, tid, nthr, kb, vb, rb);
  if (p.app.meta == kMetaF16) return append_rows<kMetaF16>(p, r0, r1, write, tid, nthr, kb, vb, rb);
  return append_rows<kMetaF32>(p, r0, r1, write, tid, nthr, kb, vb, rb);
}

// Body of the append workgroups of a launch (ids p.app.wg0 .. + p.app.wgs)
// over caches of metadata kind MT: workgroup a takes an equal share of the
// B*Hkv*Ncur rows of K and V (its rows may span two entries of the running
// bounds: raised per wave).
template <int MT>
__device__ inline void append_workgroup(const AttnLaunch &p, int64_t a, int tid, int nthr) {
  const int64_t n = p.B * p.Hkv * p.Ncur, w = p.app.wgs;
  float kb = 0.f, vb = 0.f;
  RowBounds rb;
  append_rows<MT>(p, n * a / w, n * (a + 1) / w, true, tid, nthr, kb, vb, rb);
  raise_bound(p.app.bound[0], rb.cur, rb.k);
  raise_bound(p.app.bound[1], rb.cur, rb.v);
}

}  // namespace qdev
}  // namespace kvq
