// Helpers shared by the short-query kernels (attention_short.hip: 32-row
// tiles; attention_short16.hip: 16-row tiles): the per-(b, KV head)
// context, buffer loads that read zero past a bound, metadata loads, wave
// reductions and the per-block power-of-two scales.
#pragma once

#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace sk {

using namespace dev;

constexpr int D = 128;
constexpr int BK = 32;  // keys per block

struct Ctx {
  const uint8_t *kc_codes, *vc_codes;  // the (b, KV head)'s cache rows
  const float *kc_scale, *kc_zero, *vc_scale, *vc_zero;
  const uint16_t *k_cur, *v_cur;
  int nc, ncur;     // segment lengths
  CacheLayout layout;         // paged caches: the pool rows of (b, hk)
  int64_t cap, H, b, hk;
  uint32_t kmask;   // code mask of magic8 (vector register)
  uint32_t vmask0, vmask1;  // value code fields of unpack_v_cached (vector registers)
};

// Largest x over the wave, returned uniform: DPP steps (within quads,
// half rows, rows, then across rows) leave the maximum in lane 63.
template <int CTRL, int ROWS>
__device__ inline float dpp_max(float x) {
  const int v = __float_as_int(x);
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false)));
}
__device__ inline float wave_max(float x) {
  x = dpp_max<0xb1, 0xf>(x);   // quad_perm [1,0,3,2]
  x = dpp_max<0x4e, 0xf>(x);   // quad_perm [2,3,0,1]
  x = dpp_max<0x141, 0xf>(x);  // row_half_mirror
  x = dpp_max<0x140, 0xf>(x);  // row_mirror
  x = dpp_max<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_max<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Raw buffer descriptor over `bytes` bytes at p (stride 0): loads at byte
// offsets past `bytes` return zero instead of touching memory.
typedef __amdgpu_buffer_rsrc_t Buf;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline Buf buffer_at(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ inline uint32_t ld32(Buf b, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(b, off, 0, 0); }
__device__ inline u32x2 ld64(Buf b, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(b, off, 0, 0); }
__device__ inline u32x4 ld128(Buf b, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, 0); }

// Step / zero-point elements of kind MT (fp32, binary16 or bfloat16) at a
// byte offset: one element, or two consecutive ones.
template <int MT>
__device__ inline float ld_meta1(Buf b, uint32_t off) {
  if (MT != kMetaF32) return meta16_value(__builtin_amdgcn_raw_buffer_load_b16(b, off, 0, 0), MT);
  return __uint_as_float(ld32(b, off));
}
template <int MT>
__device__ inline float2 ld_meta2(Buf b, uint32_t off) {
  if (MT == kMetaBF16) {  // a bfloat16 pair is the upper halves of two fp32 values
    const uint32_t w = ld32(b, off);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  }
  if (MT == kMetaF16) {
    const uint32_t w = ld32(b, off);
    return make_float2(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w))),
                       static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16))));
  }
  const u32x2 w = ld64(b, off);
  return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
}
// A step or zero-point array advanced by n elements.
template <int MT>
__device__ inline const float *meta_adv(const float *p, int64_t n) {
  return reinterpret_cast<const float *>(reinterpret_cast<const char *>(p) + n * (MT ? 2 : 4));
}

// floor(log2 x) for x > 0 (one v_frexp_exp_i32_f32).
__device__ inline int ilog2_pos(float x) { return __builtin_amdgcn_frexp_expf(x) - 1; }

// Exponent ev of a block's values: |v| 2^-ev in [2^13, 2^14) for the largest
// |v| of the block (0 for an all-zero block), the fp16 range with the most
// precision.  Every block, cached or current, uses this rule, so the factor
// 2^(ev - running max) that a probability carries only reflects real
// differences of magnitude between blocks.
__device__ inline int value_exponent(float vmax) { return vmax > 0.f ? ilog2_pos(vmax) - 13 : 0; }

// First row of the cached block at token k0: relative to the head's first
// row (contiguous: the context's pointers are at that row), or the pool row
// (paged: the context's pointers are at the pool; a 32-key block never
// crosses a page).
template <bool PAGED>
__device__ inline size_t block_row(const Ctx &c, int k0) {
  if (!PAGED) return static_cast<size_t>(k0);
  return static_cast<size_t>(c.layout.row(c.cap, c.H, c.b, c.hk, k0));
}

// Block exponents of a wave (uniform).  A block keeps the previous block's
// exponent while all its values fit the fp16 headroom of it (|k| 2^-ek below
// 2^15, |v| 2^-ev below 2^14): fp16 precision is relative, so an exponent
// chosen for larger values costs nothing until values fall 2^28 below them.
// Otherwise the exponent is recomputed from the block's largest magnitude
// (one wave reduction): |k| 2^-ek in [2^14, 2^15), |v| 2^-ev in [2^13, 2^14).
struct Scales {
  int ek = 0, ev = 0;
  float klim = 0.f, vlim = 0.f;    // 2^(15+ek), 2^(14+ev); 0 before the first block
  float kscale = 1.f, vscale = 1.f;  // 2^-ek, 2^-ev
  float alpha = 0.f;               // softmax scale of the block's scores (exp2 domain)
  __device__ void update(float kb, float vb, float alpha_q) {
    if (!__all(kb < klim)) {
      const float m = wave_max(kb);
      ek = m > 0.f ? ilog2_pos(m) - kFp16Exp : 0;
      klim = ldexpf(32768.0f, ek);
      kscale = ldexpf(1.0f, -ek);
      alpha = ldexpf(alpha_q, ek);
    }
    if (!__all(vb < vlim)) {
      ev = value_exponent(wave_max(vb));
      vlim = ldexpf(16384.0f, ev);
      vscale = ldexpf(1.0f, -ev);
    }
  }
};

}  // namespace sk
}  // namespace kvq
