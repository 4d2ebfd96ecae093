// Quantize/pack kernel for gfx950: group-wise asymmetric INT2/INT4 along the
// head dimension, one step D and zero-point z (the group minimum) per
// (token, group), codes packed LSB-first.
//
// The pages: "量化鍵值偷走注意力…" (agents-report.net), section 方法 -- one
// step size per group (or channel) enters the correction; "QuantWM：…"
// (pchao.org), section 方法概览 -- each cache block is quantised once after
// it is built.  The exact formula (range / (2^bits - 1), zero = min, round
// half to even) is this library's reading, stated in include/kvq.h.
//
// Mapping: one lane owns 8 consecutive values of a token row (16 B of bf16 or
// 32 B of fp32, so a wave reads 1-2 KB contiguous), group/8 adjacent lanes
// own one group and reduce min/max with cross-lane shuffles.  Each lane
// writes its 8 codes as one 16-bit (INT2) or 32-bit (INT4) store, so a wave
// writes a contiguous run of packed rows.  Pure streaming, HBM-bound.
//
// Groups along the tokens (per channel, the other grouping the method's
// description names): one thread owns 8 consecutive channels of one token
// group of one head.  It streams the group's rows once for the per-channel
// minimum and maximum, then again (from cache) for the codes, which it
// writes per token row in the same packed format.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

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

// T: uint16_t (bf16 bits) or float.  LANES = group / 8.  M16: the step and
// zero point are stored as binary16, rounded (nearest, ties to even) before
// the codes are taken so that z + D c uses exactly what is stored.
// Grid: x over the N * d/8 lanes of one (b, h) = (blockIdx.z, blockIdx.y).
template <typename T, int BITS, int LANES, bool M16>
__global__ __launch_bounds__(kThreads) void quantize_pack(
    const T *__restrict__ x, int32_t lane_shift, int64_t N,
    uint8_t *__restrict__ codes, float *__restrict__ scale, float *__restrict__ zero,
    int64_t cap, int64_t off, int32_t groups_per_row, CacheLayout layout, int64_t H) {
#pragma clang fp contract(off)
  constexpr int TOP = (1 << BITS) - 1;
  const int64_t gl = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t bh = static_cast<int64_t>(blockIdx.z) * H + blockIdx.y;
  const int32_t lanes_per_row = 1 << lane_shift;
  const bool live = gl < (N << lane_shift);
  // dead lanes (whole groups past the last token) shadow the last token
  const int64_t n = live ? (gl >> lane_shift) : N - 1;
  const int32_t chunk = static_cast<int32_t>(gl & (lanes_per_row - 1));

  float v[8];
  load8<T>(x + ((bh * N + n) << (lane_shift + 3)) + chunk * 8, v);

  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = v[i] < mn ? v[i] : mn;
    mx = v[i] > mx ? v[i] : mx;
  }
  mn = group_min<LANES>(mn) + 0.0f;  // + 0.0f: a zero extreme is +0
  mx = group_max<LANES>(mx) + 0.0f;
  const float range = mx - mn;
  float step = range / static_cast<float>(TOP);  // IEEE division
  float zp = mn;
  if (M16) {
    step = static_cast<float>(static_cast<_Float16>(step));
    zp = static_cast<float>(static_cast<_Float16>(mn));
  }

  uint32_t packed = 0;
  if (step > 0.0f) {
    const bool fast = reciprocal_ok(step);
    const float inv = fast ? __builtin_amdgcn_rcpf(step) : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= code_of<TOP>(v[i], zp, step, inv, fast) << (i * BITS);
  }

  if (!live) return;
  const int64_t orow = layout.row(cap, H, blockIdx.z, blockIdx.y, off + n);  // the cache row of token off + n
  const int64_t row_bytes = static_cast<int64_t>(lanes_per_row) * BITS;  // 8 codes * BITS / 8 per lane
  uint8_t *dst = codes + orow * row_bytes + static_cast<int64_t>(chunk) * BITS;
  if (BITS == 2) {
    *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(packed);
  } else {
    *reinterpret_cast<uint32_t *>(dst) = packed;
  }
  if ((chunk % LANES) == 0) {
    const int64_t m = orow * groups_per_row + chunk / LANES;
    if (M16) {
      reinterpret_cast<_Float16 *>(scale)[m] = static_cast<_Float16>(step);
      reinterpret_cast<_Float16 *>(zero)[m] = static_cast<_Float16>(zp);
    } else {
      scale[m] = step;
      zero[m] = mn;
    }
  }
}

template <typename T, int BITS, bool M16>
hipError_t launch_t(const QuantizeLaunch &p, hipStream_t stream) {
  const int32_t lane_shift = __builtin_ctz(static_cast<unsigned>(p.d / 8));  // d/8 lanes per token row
  const int64_t blocks = ((p.N << lane_shift) + kThreads - 1) / kThreads;
  const dim3 grid(static_cast<uint32_t>(blocks), static_cast<uint32_t>(p.H), static_cast<uint32_t>(p.B));
  const T *x = static_cast<const T *>(p.x);
  const int32_t gpr = p.d / p.group;
  switch (p.group) {
    case 32:
      quantize_pack<T, BITS, 4, M16><<<grid, dim3(kThreads), 0, stream>>>(
          x, lane_shift, p.N, p.codes, p.scale, p.zero, p.cap, p.off, gpr, p.layout, p.H);
      break;
    case 64:
      quantize_pack<T, BITS, 8, M16><<<grid, dim3(kThreads), 0, stream>>>(
          x, lane_shift, p.N, p.codes, p.scale, p.zero, p.cap, p.off, gpr, p.layout, p.H);
      break;
    default:
      quantize_pack<T, BITS, 16, M16><<<grid, dim3(kThreads), 0, stream>>>(
          x, lane_shift, p.N, p.codes, p.scale, p.zero, p.cap, p.off, gpr, p.layout, p.H);
      break;
  }
  return hipGetLastError();
}

// Groups along the tokens.  Thread = (b, h, token group j of the call,
// channel octet); octets fastest, so a wave reads whole token rows.  The
// call's tokens [off, off + N) start at a multiple of G; the last group may
// be shorter.  Metadata row of a group = cache row of its first token >> log2 G.
template <typename T, int BITS, bool M16>
__global__ __launch_bounds__(kThreads) void quantize_tokens_pack(
    const T *__restrict__ x, int64_t total, int32_t octets, int64_t groups, int64_t N, int32_t gshift,
    uint8_t *__restrict__ codes, float *__restrict__ scale, float *__restrict__ zero, int64_t cap, int64_t off,
    CacheLayout layout, int64_t H) {
#pragma clang fp contract(off)
  constexpr int TOP = (1 << BITS) - 1;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (id >= total) return;
  const int32_t oc = static_cast<int32_t>(id % octets);
  const int64_t rest = id / octets;
  const int64_t j = rest % groups;
  const int64_t bh = rest / groups;
  const int64_t t0 = j << gshift;
  const int64_t G = int64_t(1) << gshift;
  const int cnt = static_cast<int>(N - t0 < G ? N - t0 : G);
  const int32_t d = octets * 8;
  const T *src = x + (bh * N + t0) * d + oc * 8;

  float v[8], mn[8], mx[8];
  load8<T>(src, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) mn[e] = mx[e] = v[e];
  for (int i = 1; i < cnt; ++i) {
    load8<T>(src + static_cast<int64_t>(i) * d, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = v[e] < mn[e] ? v[e] : mn[e];
      mx[e] = v[e] > mx[e] ? v[e] : mx[e];
    }
  }
  float step[8], zp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = mn[e] + 0.0f;  // a zero extreme is +0
    mx[e] = mx[e] + 0.0f;
    step[e] = (mx[e] - mn[e]) / static_cast<float>(TOP);  // IEEE division
    zp[e] = mn[e];
    if (M16) {
      step[e] = static_cast<float>(static_cast<_Float16>(step[e]));
      zp[e] = static_cast<float>(static_cast<_Float16>(mn[e]));
    }
  }
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t mrow = layout.row(cap, H, b, h, off + t0) >> gshift;
  const int64_t m = mrow * d + oc * 8;
  if (M16) {
    _Float16 *ps = reinterpret_cast<_Float16 *>(scale) + m;
    _Float16 *pz = reinterpret_cast<_Float16 *>(zero) + m;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ps[e] = static_cast<_Float16>(step[e]);
      pz[e] = static_cast<_Float16>(zp[e]);
    }
  } else {
    *reinterpret_cast<float4 *>(scale + m) = make_float4(step[0], step[1], step[2], step[3]);
    *reinterpret_cast<float4 *>(scale + m + 4) = make_float4(step[4], step[5], step[6], step[7]);
    *reinterpret_cast<float4 *>(zero + m) = make_float4(zp[0], zp[1], zp[2], zp[3]);
    *reinterpret_cast<float4 *>(zero + m + 4) = make_float4(zp[4], zp[5], zp[6], zp[7]);
  }

  float inv[8];
  bool fast[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    fast[e] = reciprocal_ok(step[e]);
    inv[e] = fast[e] ? __builtin_amdgcn_rcpf(step[e]) : 0.f;
  }
  const int64_t row_bytes = static_cast<int64_t>(octets) * BITS;
  for (int i = 0; i < cnt; ++i) {
    load8<T>(src + static_cast<int64_t>(i) * d, v);
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (step[e] > 0.0f) packed |= code_of<TOP>(v[e], zp[e], step[e], inv[e], fast[e]) << (e * BITS);
    const int64_t orow = layout.row(cap, H, b, h, off + t0 + i);
    uint8_t *dst = codes + orow * row_bytes + static_cast<int64_t>(oc) * BITS;
    if (BITS == 2)
      *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(packed);
    else
      *reinterpret_cast<uint32_t *>(dst) = packed;
  }
}

template <typename T, int BITS, bool M16>
hipError_t launch_tokens(const QuantizeLaunch &p, hipStream_t stream) {
  const int32_t gshift = __builtin_ctz(static_cast<unsigned>(p.group));
  const int64_t groups = (p.N + p.group - 1) / p.group;
  const int32_t octets = p.d / 8;
  const int64_t total = p.B * p.H * groups * octets;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  quantize_tokens_pack<T, BITS, M16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream>>>(
      static_cast<const T *>(p.x), total, octets, groups, p.N, gshift, p.codes, p.scale, p.zero, p.cap, p.off,
      p.layout, p.H);
  return hipGetLastError();
}

template <typename T, bool M16>
hipError_t launch_tokens_bits(const QuantizeLaunch &p, hipStream_t stream) {
  return p.bits == 2 ? launch_tokens<T, 2, M16>(p, stream) : launch_tokens<T, 4, M16>(p, stream);
}

}  // namespace

hipError_t launch_quantize(const QuantizeLaunch &p, hipStream_t stream) {
  if (p.B * p.H * p.N == 0) return hipSuccess;
  if (p.tokens) {
    if (p.xdt == KV_BF16)
      return p.meta16 ? launch_tokens_bits<uint16_t, true>(p, stream) : launch_tokens_bits<uint16_t, false>(p, stream);
    return p.meta16 ? launch_tokens_bits<float, true>(p, stream) : launch_tokens_bits<float, false>(p, stream);
  }
  if (p.meta16) {
    if (p.xdt == KV_BF16)
      return p.bits == 2 ? launch_t<uint16_t, 2, true>(p, stream) : launch_t<uint16_t, 4, true>(p, stream);
    return p.bits == 2 ? launch_t<float, 2, true>(p, stream) : launch_t<float, 4, true>(p, stream);
  }
  if (p.xdt == KV_BF16)
    return p.bits == 2 ? launch_t<uint16_t, 2, false>(p, stream) : launch_t<uint16_t, 4, false>(p, stream);
  return p.bits == 2 ? launch_t<float, 2, false>(p, stream) : launch_t<float, 4, false>(p, stream);
}

}  // namespace kvq
