// Device helpers shared by the gfx950 attention kernels (attention_fast.hip,
// attention_short.hip): vector types, bf16/fp16 packing, code unpacking and
// the power-of-two range scaling of the fp16 operands.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace kvq {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));


constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // rescale threshold (exp2 domain)
constexpr int kFp16Exp = 14;   // scaled magnitudes stay below 2^(kFp16Exp+1)

// Two floats -> two bf16 / fp16 (round to nearest even) in one instruction.
__device__ inline uint32_t pack2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline uint32_t pack2h(float lo, float hi) {
  const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Max / sum of x over lanes l and l ^ 32 (l ^ 16), in the vector ALU: with
// both operands holding x, v_permlane32_swap (v_permlane16_swap) leaves a
// lane's own value in one result and its partner's in the other, so each
// lane combines the same two values; an LDS permute (ds_bpermute) would
// put an LDS round trip on the path of every key block.
__device__ inline float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Sum of the 8 fp16 values of v, added to acc (two per v_dot2_f32_f16).
__device__ inline float sum8h(f16x8 v, float acc) {
  const uint4 w = __builtin_bit_cast(uint4, v);
  const f16x2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.z), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.w), one, acc, false);
}

// Centre of a cached key group for the fp16 key operand.  When the group's
// code range [z, z + (2^bits - 1) D] lies on one side of zero (its values
// share an offset), the centre is the range's midpoint truncated to bf16,
// else 0.  The kernels round z - centre + D c (not z + D c) to fp16, so that
// the rounding error of offset groups scales with their half range rather
// than with |k|, and add the centre back through the extra bf16 MFMA step as
// centre x (sum of the query over the group): a bf16 centre times the bf16
// (hi, lo) parts of the query sum is exact in the fp32 accumulator.  Keys
// far from zero (a large shared mean, logits far from zero) would otherwise
// lose the scores' low bits to fp16 rounding.  A range around zero keeps
// centre 0: a group mixing small channels with large ones would have its
// small values moved away from zero by a midpoint.
template <int BITS>
__device__ inline float group_centre(float z, float step) {
  const float half = static_cast<float>((1 << BITS) - 1) * 0.5f;
  const float mid = fmaf(half, step, z);
  // the range lies on one side of zero iff |mid| > half range; the centre is
  // mid truncated to bf16 (any bf16 value near mid serves)
  return fabsf(mid) > half * step ? __uint_as_float(__float_as_uint(mid) & 0xffff0000u) : 0.f;
}

// Codes as fp16 "magic" values 1024 + c (exact: the fp16 spacing at 1024 is
// 1): the integer-to-fp16 conversion by OR-ing the integer into the mantissa
// of 1024 (0x6400) and folding the 1024 offset into the following affine
// step, as published for INT4/INT8 weight dequantisation by Kim et al.,
// "Who Says Elephants Can't Run: Bringing Large Scale MoE Models into Cloud
// Scale Production" (2022).  Built here two at a time: m[j] holds codes j (low half) and j + 4 (high
// half) of 8 codes of BITS bits stored LSB first in the low 8*BITS bits of
// w.  A value z + D c is then fma(1024 + c, D, z - 1024 D) in fp32, which
// v_fma_mix evaluates straight from the fp16 half and rounds to fp16.
// The code mask is held in a vector register (`mask`, from opaque_u32) so
// that each pair is one v_and_or_b32: gfx950's VOP3 encodings take no
// literal, and with both constants literal the compiler emits and + or.
__device__ inline uint32_t opaque_u32(uint32_t x) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "s"(x));
  return r;
}
template <int BITS>
__device__ inline void magic8(uint32_t w, uint32_t mask, uint32_t (&m)[4]) {
  if (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = ((w >> (4 * j)) & mask) | 0x64006400u;
  } else {
    const uint32_t x = (w & 0xffffu) | ((w & 0xffffu) << 8);  // code j + 4 now also at bit 2j + 16
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = ((x >> (2 * j)) & mask) | 0x64006400u;
  }
}
__device__ inline float magic_code(const uint32_t (&m)[4], int e) {  // 1024 + code e
  const f16x2 h = __builtin_bit_cast(f16x2, m[e & 3]);
  return static_cast<float>((e >> 2) ? h.y : h.x);
}
template <int BITS>
constexpr uint32_t kCodeMask = BITS == 4 ? 0x000f000fu : 0x00030003u;

// fma(1024 + code, s, z) rounded to fp16 (one v_fma_mix per value).
__device__ inline _Float16 dequant_h(float magic, float s, float z) { return static_cast<_Float16>(fmaf(magic, s, z)); }
__device__ inline uint32_t pair_h(_Float16 lo, _Float16 hi) {
  const f16x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, v);
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

// Exponent e with |x| * 2^-e in [2^kFp16Exp, 2^(kFp16Exp+1)) for the
// largest |x| = bound (0 for a zero bound).
__device__ inline int scale_exponent(float bound) {
  return bound > 0.f ? ilogbf(bound) - kFp16Exp : 0;
}

// Scheduling fences do not hold pure arithmetic in place (instruction
// selection may sink it next to its use), so the results of a work item
// pass through an empty volatile asm that claims to rewrite them: that
// orders the item before the next fence.
template <typename T>
__device__ inline void pin(T &x) {
  asm volatile("" : "+v"(x));
}

// The lane's query row for the fp16 Q K^T product (lane half h holds
// dimensions 16 s + 8 h .. +7 of k-step s, or with HALVES the contiguous
// 64 h + 8 s .. +7, so that each lane half covers one half of the head
// dimension): the row scaled by its own power
// of two 2^-eq (largest |q| to [2^14, 2^15)), the softmax scale of the
// resulting scores (alpha = tau log2(e) 2^(eq+ek) for keys scaled by 2^-ek),
// and the Taylor correction operands N_g = tau/24 ||q_g||^2 2^-(eq+ek) in
// slots 4g+{0,1,2,3} as (hi, hi, lo, 0) split into bf16 (the lane holds
// slots 8h .. 8h+7, i.e. groups 2h and 2h+1; zero when not TAYLOR).  With
// at most two groups (and HALVES), lane half h holds group h only:
// (N_hi, N_hi, N_lo, 0, S_hi, S_lo, 0, 0) with the group sum
// S_g = sum_{c in g} q_c 2^-eq, which the centres of centred cached keys
// multiply (see group_centre); half 1 is zero with one group.  The row's
// other half sits in lane l^32.  qun (when given) receives 2^eq.
template <bool TAYLOR, bool HALVES = false>
__device__ inline void load_query(const uint16_t *qptr, int h, int group_shift, float tau, int ek, f16x8 (&q)[8],
                                  bf16x8 &qext, float &alpha, float *qun = nullptr) {
  const int ng = 128 >> group_shift;
  uint4 qw[8];
  float nsum[4] = {0.f, 0.f, 0.f, 0.f}, qsum[2] = {0.f, 0.f};
  float qmax = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int d0 = HALVES ? 64 * h + 8 * s : 16 * s + 8 * h;
    qw[s] = *reinterpret_cast<const uint4 *>(qptr + d0);
    const uint32_t u[4] = {qw[s].x, qw[s].y, qw[s].z, qw[s].w};
    float acc = 0.f, sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += lo_f(u[i]) * lo_f(u[i]) + hi_f(u[i]) * hi_f(u[i]);
      sum += lo_f(u[i]) + hi_f(u[i]);
      qmax = fmaxf(qmax, fmaxf(fabsf(lo_f(u[i])), fabsf(hi_f(u[i]))));
    }
    const int gs = d0 >> group_shift;
#pragma unroll
    for (int g = 0; g < 4; ++g) nsum[g] += g == gs ? acc : 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g) qsum[g] += g == gs ? sum : 0.f;
  }
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
  const int eq = scale_exponent(qmax);
  const float qs_scale = ldexpf(1.0f, -eq);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t u[4] = {qw[s].x, qw[s].y, qw[s].z, qw[s].w};
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack2h(lo_f(u[i]) * qs_scale, hi_f(u[i]) * qs_scale);
    q[s] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  const float unscale = ldexpf(1.0f, eq + ek);
  alpha = tau * kLog2e * unscale;
  if (qun) *qun = ldexpf(1.0f, eq);
  float nh[4], nl[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float n = TAYLOR && g < ng ? (nsum[g] + __shfl_xor(nsum[g], 32, 64)) * (tau / 24.0f) / unscale : 0.f;
    nh[g] = lo_f(pack2(n, 0.f));
    nl[g] = n - nh[g];
  }
  float sh[2], sl[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float t = (qsum[g] + __shfl_xor(qsum[g], 32, 64)) * qs_scale;
    sh[g] = g < ng ? lo_f(pack2(t, 0.f)) : 0.f;
    sl[g] = g < ng ? t - sh[g] : 0.f;
  }
  if (ng <= 2) {
    const bool on = h < ng;
    const float gh = on ? (h ? nh[1] : nh[0]) : 0.f, gl = on ? (h ? nl[1] : nl[0]) : 0.f;
    const float th = on ? (h ? sh[1] : sh[0]) : 0.f, tl = on ? (h ? sl[1] : sl[0]) : 0.f;
    qext = __builtin_bit_cast(bf16x8, make_uint4(pack2(gh, gh), pack2(gl, 0.f), pack2(th, tl), 0u));
    return;
  }
  const float n0h = h ? nh[2] : nh[0], n0l = h ? nl[2] : nl[0];
  const float n1h = h ? nh[3] : nh[1], n1l = h ? nl[3] : nl[1];
  qext = __builtin_bit_cast(bf16x8, make_uint4(pack2(n0h, n0h), pack2(n0l, 0.f), pack2(n1h, n1h), pack2(n1l, 0.f)));
}

}  // namespace dev
}  // namespace kvq
