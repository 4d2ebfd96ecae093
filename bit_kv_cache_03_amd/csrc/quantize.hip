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
#include "quant_device.h"

namespace kvq {
namespace {

using namespace qdev;

constexpr int kThreads = 256;

// T: uint16_t (bf16 bits) or float.  LANES = group / 8.  MT: the kind of the
// step and zero-point arrays; with 16 bits (binary16 or bfloat16) they are
// rounded (nearest, ties to even) before the codes are taken so that z + D c
// uses exactly what is stored.
// Grid: x over the N * d/8 lanes of one (b, h) = (blockIdx.z, blockIdx.y).
template <typename T, int BITS, int LANES, int MT>
__global__ __launch_bounds__(kThreads) void quantize_pack(
    const T *__restrict__ x, int32_t lane_shift, int64_t N,
    uint8_t *__restrict__ codes, float *__restrict__ scale, float *__restrict__ zero,
    int64_t cap, int64_t off, CacheLayout layout, int64_t H, float *__restrict__ bound) {
  const int64_t gl = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t bh = static_cast<int64_t>(blockIdx.z) * H + blockIdx.y;
  const int32_t lanes_per_row = 1 << lane_shift;
  const bool live = gl < (N << lane_shift);
  // dead lanes (whole groups past the last token) shadow the last token
  const int64_t n = live ? (gl >> lane_shift) : N - 1;
  const int32_t chunk = static_cast<int32_t>(gl & (lanes_per_row - 1));

  float v[8];
  load8<T>(x + ((bh * N + n) << (lane_shift + 3)) + chunk * 8, v);

  float step, zp;
  const uint32_t packed = quantize8<BITS, LANES, MT>(v, step, zp);
  if (bound) {  // the workgroup's largest group bound (all its lanes are of (b, h)), raised once
    __shared__ float red[kThreads / 64];
    float gb = live ? group_bound<BITS>(step, zp) : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) gb = fmaxf(gb, __shfl_xor(gb, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = gb;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = red[0];
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
      bound_max(bound, bh, m);
    }
  }

  if (!live) return;
  const int64_t orow = layout.row(cap, H, blockIdx.z, blockIdx.y, off + n);  // the cache row of token off + n
  store8<BITS, LANES, MT>(codes, scale, zero, orow, lanes_per_row, chunk, packed, step, zp);
}

template <typename T, int BITS, int MT>
hipError_t launch_t(const QuantizeLaunch &p, hipStream_t stream) {
  const int32_t lane_shift = __builtin_ctz(static_cast<unsigned>(p.d / 8));  // d/8 lanes per token row
  const int64_t blocks = ((p.N << lane_shift) + kThreads - 1) / kThreads;
  const dim3 grid(static_cast<uint32_t>(blocks), static_cast<uint32_t>(p.H), static_cast<uint32_t>(p.B));
  const T *x = static_cast<const T *>(p.x);
  switch (p.group) {
    case 32:
      quantize_pack<T, BITS, 4, MT><<<grid, dim3(kThreads), 0, stream>>>(
          x, lane_shift, p.N, p.codes, p.scale, p.zero, p.cap, p.off, p.layout, p.H, p.bound);
      break;
    case 64:
      quantize_pack<T, BITS, 8, MT><<<grid, dim3(kThreads), 0, stream>>>(
          x, lane_shift, p.N, p.codes, p.scale, p.zero, p.cap, p.off, p.layout, p.H, p.bound);
      break;
    default:
      quantize_pack<T, BITS, 16, MT><<<grid, dim3(kThreads), 0, stream>>>(
          x, lane_shift, p.N, p.codes, p.scale, p.zero, p.cap, p.off, p.layout, p.H, p.bound);
      break;
  }
  return hipGetLastError();
}

// Groups along the tokens.  Thread = (b, h, token group j of the call,
// channel octet); octets fastest, so a wave reads whole token rows.  The
// call's tokens [off, off + N) start at a multiple of G; the last group may
// be shorter.  Metadata row of a group = cache row of its first token >> log2 G.
// The body for one live thread; returns the bound of its channels' groups.
template <typename T, int BITS, int MT>
__device__ inline float quantize_token_group(const T *__restrict__ x, int64_t id, int32_t octets, int64_t groups,
                                             int64_t N, int32_t gshift, uint8_t *__restrict__ codes,
                                             float *__restrict__ scale, float *__restrict__ zero, int64_t cap,
                                             int64_t off, CacheLayout layout, int64_t H) {
#pragma clang fp contract(off)
  constexpr int TOP = (1 << BITS) - 1;
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
    if (MT != kMetaF32) {
      step[e] = meta_round(step[e], MT);
      zp[e] = meta_round(mn[e], MT);
    }
  }
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t mrow = layout.row(cap, H, b, h, off + t0) >> gshift;
  const int64_t m = mrow * d + oc * 8;
  if (MT != kMetaF32) {
    uint16_t *ps = reinterpret_cast<uint16_t *>(scale) + m;
    uint16_t *pz = reinterpret_cast<uint16_t *>(zero) + m;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ps[e] = meta16_bits(step[e], MT);
      pz[e] = meta16_bits(zp[e], MT);
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
  float bnd = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) bnd = fmaxf(bnd, group_bound<BITS>(step[e], zp[e]));
  return bnd;
}

// The kernel: every lane of a wave, dead ones too, takes part in raising
// the running bound.
template <typename T, int BITS, int MT>
__global__ __launch_bounds__(kThreads) void quantize_tokens_pack(
    const T *__restrict__ x, int64_t total, int32_t octets, int64_t groups, int64_t N, int32_t gshift,
    uint8_t *__restrict__ codes, float *__restrict__ scale, float *__restrict__ zero, int64_t cap, int64_t off,
    CacheLayout layout, int64_t H, float *__restrict__ bound) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const bool live = id < total;
  float bnd = 0.f;
  if (live) bnd = quantize_token_group<T, BITS, MT>(x, id, octets, groups, N, gshift, codes, scale, zero, cap, off,
                                                     layout, H);
  // every lane of the wave takes part (dead lanes with 0): the group's (b, h)
  raise_bound(bound, live ? id / octets / groups : total / octets / groups - 1, bnd);
}


template <typename T, int BITS, int MT>
hipError_t launch_tokens(const QuantizeLaunch &p, hipStream_t stream) {
  const int32_t gshift = __builtin_ctz(static_cast<unsigned>(p.group));
  const int64_t groups = (p.N + p.group - 1) / p.group;
  const int32_t octets = p.d / 8;
  const int64_t total = p.B * p.H * groups * octets;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  quantize_tokens_pack<T, BITS, MT><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream>>>(
      static_cast<const T *>(p.x), total, octets, groups, p.N, gshift, p.codes, p.scale, p.zero, p.cap, p.off,
      p.layout, p.H, p.bound);
  return hipGetLastError();
}

template <typename T, int MT>
hipError_t launch_tokens_bits(const QuantizeLaunch &p, hipStream_t stream) {
  return p.bits == 2 ? launch_tokens<T, 2, MT>(p, stream) : launch_tokens<T, 4, MT>(p, stream);
}

template <int MT>
hipError_t launch_meta(const QuantizeLaunch &p, hipStream_t stream) {
  if (p.tokens)
    return p.xdt == KV_BF16 ? launch_tokens_bits<uint16_t, MT>(p, stream) : launch_tokens_bits<float, MT>(p, stream);
  if (p.xdt == KV_BF16)
    return p.bits == 2 ? launch_t<uint16_t, 2, MT>(p, stream) : launch_t<uint16_t, 4, MT>(p, stream);
  return p.bits == 2 ? launch_t<float, 2, MT>(p, stream) : launch_t<float, 4, MT>(p, stream);
}

}  // namespace

hipError_t launch_quantize(const QuantizeLaunch &p, hipStream_t stream) {
  if (p.B * p.H * p.N == 0) return hipSuccess;
  if (p.meta == kMetaBF16) return launch_meta<kMetaBF16>(p, stream);
  if (p.meta == kMetaF16) return launch_meta<kMetaF16>(p, stream);
  return launch_meta<kMetaF32>(p, stream);
}

}  // namespace kvq
