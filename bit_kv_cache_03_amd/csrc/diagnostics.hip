// Attention-balance diagnostics for gfx950: for every query row, the
// softmax over the cached keys before quantisation is compared with the one
// the corrected attention uses ("量化鍵值偷走注意力…" (agents-report.net),
// §問題: the rounding noise of cached keys raises their share of the softmax
// through the exponential's convexity and takes attention from the current
// chunk; §為何校正有效: subtracting b restores the balance).
//
// One workgroup = 4 waves x 32 query rows of one KV head (GQA rows packed as
// on the attention paths), 64-key tiles over [cache ; current chunk].  Per
// tile two score sets come out of bf16 MFMA (S^T = K Q^T, keys as rows):
//   q:   the quantised keys dequantised in fp32 and kept as a bf16 hi + lo
//        pair (~16 significant bits), with the Taylor correction as one extra
//        K = 16 step or the exact form as a per-score epilogue;
//   ref: the unquantised bf16 keys (exact products); current keys give the
//        same scores in both sets.
// Each lane owns one query row and half of each tile's keys; it keeps, for
// both sets, a running max, sum, current-chunk sum and its 5 largest scores
// (with indices), plus sum p_ref (s_ref - s_q) for the KL divergence.  The
// two halves of a row merge at the end.  No value product: scores only.
// Caches grouped along the tokens (per channel) are dequantised channel by
// channel, and their bias is one value per row and 32-key half of a tile
// (one token group), as in the general attention kernel.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int THREADS = 256;
constexpr int TOPK = 5;

template <int D>
struct DTile {
  static constexpr int kLo = D;                // lo half of a quantised key row
  static constexpr int kExt = 2 * D;           // 16 correction slots
  static constexpr int kStride = 2 * D + 24;   // hi, lo, slots, pad (16-bit elements)
  static constexpr int rStride = D + 8;        // reference key row
};

__device__ inline uint32_t bf16_pair(float lo, float hi) { return pack2(lo, hi); }
__device__ inline float bf16_round(float x) { return lo_f(pack2(x, 0.f)); }

// log(sinh x / x) in fp32: series to x^10 below 0.5, else
// log(sinh a / a) = a - log(2a) + log1p(-exp(-2a)).
__device__ inline float log_sinhc(float x) {
  const float a = fabsf(x);
  if (a < 0.5f) {
    const float y = a * a;
    return y * (1.0f / 6.0f +
                y * (-1.0f / 180.0f + y * (1.0f / 2835.0f + y * (-1.0f / 37800.0f + y * (1.0f / 467775.0f)))));
  }
  return a - logf(2.0f * a) + log1pf(-expf(-2.0f * a));
}

template <int BITS>
__device__ inline float code_at(uint32_t w, int j) {
  return static_cast<float>((w >> (j * BITS)) & ((1u << BITS) - 1u));
}

// Running statistics of one score set for the lane's half of a row.
struct Side {
  float m, l, lc;       // max, sum of exp(s - m), the same over current keys
  float v[TOPK];        // largest scores, descending (ties: lower index first)
  int idx[TOPK];
};

__device__ inline void side_init(Side &s) {
  s.m = -INFINITY;
  s.l = s.lc = 0.f;
#pragma unroll
  for (int r = 0; r < TOPK; ++r) {
    s.v[r] = -INFINITY;
    s.idx[r] = -1;
  }
}

// Candidates reach a lane in increasing key order, so a strict comparison
// keeps the lower index ahead among equal scores.
__device__ inline void top_insert(Side &s, float x, int t) {
  s.v[TOPK - 1] = x;
  s.idx[TOPK - 1] = t;
#pragma unroll
  for (int r = TOPK - 1; r > 0; --r) {
    const bool up = s.v[r] > s.v[r - 1];
    const float tv = s.v[r - 1];
    const int ti = s.idx[r - 1];
    s.v[r - 1] = up ? s.v[r] : tv;
    s.idx[r - 1] = up ? s.idx[r] : ti;
    s.v[r] = up ? tv : s.v[r];
    s.idx[r] = up ? ti : s.idx[r];
  }
}

// a before b in (score descending, index ascending) order; empty (-1) last.
__device__ inline bool before(float va, int ia, float vb, int ib) {
  if (ib < 0) return ia >= 0;
  if (ia < 0) return false;
  return va > vb || (va == vb && ia < ib);
}

template <int D, int KBITS, int CORR>
__global__ __launch_bounds__(THREADS) void attn_diag_kernel(DiagLaunch p, int32_t group_shift,
                                                            int64_t rows_per_kvhead) {
  constexpr int KS = DTile<D>::kStride;
  constexpr int RS = DTile<D>::rStride;
  constexpr int NS = D / 16;
  constexpr bool EXACT = CORR == KV_CORR_EXACT;
  constexpr bool TAYLOR = CORR == KV_CORR_TAYLOR;
  __shared__ __attribute__((aligned(16))) uint16_t Kq[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Kr[BN * RS];
  __shared__ float Dk[EXACT ? BN * 4 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[EXACT ? BM * (D + 8) : 1];
  __shared__ __attribute__((aligned(16))) float Dt[2 * D];  // token groups: steps of each 32-key half

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qc = lane & 31, h = lane >> 5;
  const int group = 1 << group_shift;
  const int ng = D >> group_shift;

  const int64_t bkv = blockIdx.y;
  const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
  const int64_t gq = p.Hq / p.Hkv;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * BM + wave * 32 + qc;
  const bool row_ok = r < rows_per_kvhead;
  const int64_t rr = row_ok ? r : rows_per_kvhead - 1;
  const int64_t qj = rr % p.Nq;
  const int64_t qrow = (b * p.Hq + hk * gq + rr / p.Nq) * p.Nq + qj;
  const uint16_t *qptr = p.q + qrow * D;

  // the lane's query operand (bf16) and the correction operand: slots
  // 3g+{0,1,2} = N_hi, N_hi, N_lo with N_g = tau/24 ||q_g||^2 (units of q.k)
  bf16x8 qreg[NS];
  float nsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint4 w = *reinterpret_cast<const uint4 *>(qptr + 16 * s + 8 * h);
    qreg[s] = __builtin_bit_cast(bf16x8, w);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += lo_f(u[i]) * lo_f(u[i]) + hi_f(u[i]) * hi_f(u[i]);
    const int gs = (16 * s + 8 * h) >> group_shift;
#pragma unroll
    for (int g = 0; g < 4; ++g) nsum[g] += g == gs ? acc : 0.f;
  }
  bf16x8 qext;
  {
    float nh[4], nl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float n = (nsum[g] + __shfl_xor(nsum[g], 32, 64)) * (p.tau / 24.0f);
      nh[g] = bf16_round(n);
      nl[g] = n - nh[g];
    }
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slot = 8 * h + j, g = slot / 3, part = slot % 3;
      e[j] = TAYLOR && g < ng ? (part == 2 ? nl[g] : nh[g]) : 0.f;
    }
    qext = __builtin_bit_cast(bf16x8, make_uint4(bf16_pair(e[0], e[1]), bf16_pair(e[2], e[3]),
                                                 bf16_pair(e[4], e[5]), bf16_pair(e[6], e[7])));
  }
  if (EXACT) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      *reinterpret_cast<uint4 *>(&Qs[(wave * 32 + qc) * (D + 8) + 16 * s + 8 * h]) =
          __builtin_bit_cast(uint4, qreg[s]);
  }

  Side R, Q;
  side_init(R);
  side_init(Q);
  float kla = 0.f;  // sum over the lane's keys of exp(s_ref - R.m) (s_ref - s_q)
  const int climit = static_cast<int>(p.causal ? qj + p.Ncur - p.Nq + 1 : p.Ncur);

  const int ntc = static_cast<int>((p.Nc + BN - 1) / BN), ntu = static_cast<int>((p.Ncur + BN - 1) / BN);
  constexpr int KROW = D * KBITS / 8;
  for (int t = 0; t < ntc + ntu; ++t) {
    const bool cached = t < ntc;
    const int k0 = cached ? t * BN : (t - ntc) * BN;
    const int seg = static_cast<int>(cached ? p.Nc : p.Ncur);
    const int count = seg - k0 < BN ? seg - k0 : BN;
    const int base = cached ? k0 : static_cast<int>(p.Nc) + k0;  // key index of the tile's first key

    __syncthreads();  // the previous tile is consumed
    {
      // thread: key tid / 4, head-dim values [d0, d0 + D/4)
      constexpr int DPT = D / 4;
      const int key = tid >> 2, d0 = (tid & 3) * DPT;
      const bool ok = key < count;
      uint32_t hi[DPT / 2];
      if (cached) {
        const int64_t row = p.layout.row(p.cap, p.Hkv, b, hk, k0 + (ok ? key : 0));  // cache row of the key
        // one step / zero point for the thread's values (a group of the row),
        // or one per channel (groups along the tokens)
        const int64_t m0 = p.ktok ? (row >> group_shift) * D + d0 : row * ng + (d0 >> group_shift);
        const int mstep = p.ktok ? 1 : 0;
        constexpr int WORDS = DPT * KBITS / 32;
        constexpr int PER = 32 / KBITS;
        uint32_t w[WORDS];
        const uint8_t *src = p.kc_codes + row * KROW + d0 * KBITS / 8;
#pragma unroll
        for (int i = 0; i < WORDS; ++i) w[i] = ok ? reinterpret_cast<const uint32_t *>(src)[i] : 0u;
        uint32_t lo[DPT / 2];
#pragma unroll
        for (int e = 0; e < DPT; e += 2) {
          const float sa = meta_at(p.kc_scale, m0 + mstep * e, p.meta);
          const float za = meta_at(p.kc_zero, m0 + mstep * e, p.meta);
          const float sc = meta_at(p.kc_scale, m0 + mstep * (e + 1), p.meta);
          const float zc = meta_at(p.kc_zero, m0 + mstep * (e + 1), p.meta);
          const float a = fmaf(sa, code_at<KBITS>(w[e / PER], e % PER), za);
          const float c = fmaf(sc, code_at<KBITS>(w[(e + 1) / PER], (e + 1) % PER), zc);
          hi[e / 2] = ok ? bf16_pair(a, c) : 0u;
          lo[e / 2] = ok ? bf16_pair(a - lo_f(hi[e / 2]), c - hi_f(hi[e / 2])) : 0u;
        }
#pragma unroll
        for (int i = 0; i < DPT / 8; ++i)
          *reinterpret_cast<uint4 *>(&Kq[key * KS + DTile<D>::kLo + d0 + 8 * i]) =
              make_uint4(lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]);
        // reference keys of the same rows
        const int64_t rrow = bkv * p.Nc + k0 + (ok ? key : 0);
        const uint4 *rs = reinterpret_cast<const uint4 *>(p.k_ref + rrow * D + d0);
#pragma unroll
        for (int i = 0; i < DPT / 8; ++i)
          *reinterpret_cast<uint4 *>(&Kr[key * RS + d0 + 8 * i]) = ok ? rs[i] : make_uint4(0, 0, 0, 0);
        if (p.ktok && !(CORR == KV_CORR_OFF) && tid < 2 * D) {
          const int hk0 = 32 * (tid / D);  // first key of the half
          const bool okh = hk0 < count;
          const int64_t hrow = p.layout.row(p.cap, p.Hkv, b, hk, k0 + (okh ? hk0 : 0));
          Dt[tid] = okh ? meta_at(p.kc_scale, (hrow >> group_shift) * D + tid % D, p.meta) : 0.f;
        }
        if ((tid & 3) == 0 && !p.ktok) {
          // correction slots 3g+{0,1,2} = -D^2 split (hi, lo, hi)
          float e16[16];
          float dsh[4] = {0.f, 0.f, 0.f, 0.f}, dsl[4] = {0.f, 0.f, 0.f, 0.f};
          for (int gg = 0; gg < ng; ++gg) {
            const float s = ok ? meta_at(p.kc_scale, row * ng + gg, p.meta) : 0.f;
            dsh[gg] = bf16_round(s * s);
            dsl[gg] = s * s - dsh[gg];
            if (EXACT) Dk[key * 4 + gg] = s;
          }
#pragma unroll
          for (int slot = 0; slot < 16; ++slot) {
            const int gg = slot / 3, part = slot % 3;
            e16[slot] = TAYLOR && gg < ng ? -(part == 1 ? dsl[gg] : dsh[gg]) : 0.f;
          }
          uint4 *dst = reinterpret_cast<uint4 *>(&Kq[key * KS + DTile<D>::kExt]);
          dst[0] = make_uint4(bf16_pair(e16[0], e16[1]), bf16_pair(e16[2], e16[3]), bf16_pair(e16[4], e16[5]),
                              bf16_pair(e16[6], e16[7]));
          dst[1] = make_uint4(bf16_pair(e16[8], e16[9]), bf16_pair(e16[10], e16[11]),
                              bf16_pair(e16[12], e16[13]), bf16_pair(e16[14], e16[15]));
        }
      } else {
        const int64_t row = bkv * p.Ncur + k0 + (ok ? key : 0);
        const uint4 *src = reinterpret_cast<const uint4 *>(p.k_cur + row * D + d0);
#pragma unroll
        for (int i = 0; i < DPT / 8; ++i) {
          const uint4 v = ok ? src[i] : make_uint4(0, 0, 0, 0);
          hi[4 * i] = v.x; hi[4 * i + 1] = v.y; hi[4 * i + 2] = v.z; hi[4 * i + 3] = v.w;
        }
      }
#pragma unroll
      for (int i = 0; i < DPT / 8; ++i)
        *reinterpret_cast<uint4 *>(&Kq[key * KS + d0 + 8 * i]) =
            make_uint4(hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]);
    }
    __syncthreads();

    // groups along the tokens: the bias of each 32-key half (one token
    // group) for the lane's row, in logit units
    float tokb[2] = {0.f, 0.f};
    if (cached && p.ktok && CORR != KV_CORR_OFF) {
      const float half_tau = 0.5f * p.tau;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint4 w = __builtin_bit_cast(uint4, qreg[s]);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float qv = (i & 1) ? hi_f(u[i >> 1]) : lo_f(u[i >> 1]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const float st = Dt[kb * D + 16 * s + 8 * h + i];
            tokb[kb] += TAYLOR ? qv * qv * (st * st) : log_sinhc(half_tau * qv * st);
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float tot = tokb[kb] + __shfl_xor(tokb[kb], 32, 64);
        tokb[kb] = TAYLOR ? tot * (p.tau * p.tau / 24.0f) : tot;
      }
    }

    // S^T of both sets: lane (query qc) gets keys kb*32 + 8(i/4) + 4h + i%4
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 aq = f32x16{}, ar = f32x16{};
      const uint16_t *kq = &Kq[(kb * 32 + qc) * KS + 8 * h];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        aq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(kq + 16 * s), qreg[s], aq,
                                                     0, 0, 0);
      if (cached) {
        const uint16_t *kr = &Kr[(kb * 32 + qc) * RS + 8 * h];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          aq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8 *>(kq + DTile<D>::kLo + 16 * s), qreg[s], aq, 0, 0, 0);
          ar = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(kr + 16 * s), qreg[s],
                                                       ar, 0, 0, 0);
        }
        if (TAYLOR && !p.ktok)
          aq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(kq + DTile<D>::kExt),
                                                       qext, aq, 0, 0, 0);
      }
      float sq[16], sr[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sq[i] = aq[i] * p.tau - tokb[kb];
        sr[i] = cached ? ar[i] * p.tau : sq[i];
      }
      if (EXACT && cached && !p.ktok) {
        const uint16_t *qs = &Qs[(wave * 32 + qc) * (D + 8)];
        const float half_tau = 0.5f * p.tau;
        for (int g = 0; g < ng; ++g) {
          float st[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) st[i] = Dk[(kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3)) * 4 + g];
          for (int c = g * group; c < (g + 1) * group; ++c) {
            const float ac = half_tau * lo_f(static_cast<uint32_t>(qs[c]));
#pragma unroll
            for (int i = 0; i < 16; ++i) sq[i] -= log_sinhc(ac * st[i]);
          }
        }
      }
      // visibility: inside the segment and, on current keys, the mask
      bool vis[16];
      float mr = -INFINITY, mq = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        vis[i] = key < count && (cached || k0 + key < climit);
        if (vis[i]) {
          mr = fmaxf(mr, sr[i]);
          mq = fmaxf(mq, sq[i]);
        }
      }
      // running sums (natural exponentials through exp2)
      const float nmr = fmaxf(R.m, mr), nmq = fmaxf(Q.m, mq);
      if (nmr != -INFINITY) {
        const float f = R.m == -INFINITY ? 0.f : exp2f((R.m - nmr) * kLog2e);
        R.l *= f;
        R.lc *= f;
        kla *= f;
        R.m = nmr;
      }
      if (nmq != -INFINITY) {
        const float f = Q.m == -INFINITY ? 0.f : exp2f((Q.m - nmq) * kLog2e);
        Q.l *= f;
        Q.lc *= f;
        Q.m = nmq;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!vis[i]) continue;
        const float pr = exp2f((sr[i] - R.m) * kLog2e), pq = exp2f((sq[i] - Q.m) * kLog2e);
        R.l += pr;
        Q.l += pq;
        kla = fmaf(pr, sr[i] - sq[i], kla);
        if (!cached) {
          R.lc += pr;
          Q.lc += pq;
        }
      }
      // top-5 of both sets
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t_idx = base + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool ir = vis[i] && sr[i] > R.v[TOPK - 1], iq = vis[i] && sq[i] > Q.v[TOPK - 1];
        if (__any(ir)) {
          if (ir) top_insert(R, sr[i], t_idx);
        }
        if (__any(iq)) {
          if (iq) top_insert(Q, sq[i], t_idx);
        }
      }
    }
  }

  // ---- merge the two halves of each row (lanes l and l^32) ----
  auto merge_side = [&](Side &s, float *extra) {
    const float om = __shfl_xor(s.m, 32, 64), ol = __shfl_xor(s.l, 32, 64), olc = __shfl_xor(s.lc, 32, 64);
    const float oe = extra ? __shfl_xor(*extra, 32, 64) : 0.f;
    const float M = fmaxf(s.m, om);
    const float fa = s.m == -INFINITY ? 0.f : exp2f((s.m - M) * kLog2e);
    const float fb = om == -INFINITY ? 0.f : exp2f((om - M) * kLog2e);
    s.l = s.l * fa + ol * fb;
    s.lc = s.lc * fa + olc * fb;
    if (extra) *extra = *extra * fa + oe * fb;
    s.m = M;
    float ov[TOPK];
    int oi[TOPK];
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
      ov[k] = __shfl_xor(s.v[k], 32, 64);
      oi[k] = __shfl_xor(s.idx[k], 32, 64);
    }
    float mv[TOPK];
    int mi[TOPK];
    int a = 0, c = 0;
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
      // a + c == k; each list has at least TOPK - k entries left
      float va = s.v[0], vb = ov[0];
      int ia = s.idx[0], ib = oi[0];
#pragma unroll
      for (int j = 1; j < TOPK; ++j) {
        if (a == j) { va = s.v[j]; ia = s.idx[j]; }
        if (c == j) { vb = ov[j]; ib = oi[j]; }
      }
      const bool takea = before(va, ia, vb, ib);
      mv[k] = takea ? va : vb;
      mi[k] = takea ? ia : ib;
      a += takea ? 1 : 0;
      c += takea ? 0 : 1;
    }
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
      s.v[k] = mv[k];
      s.idx[k] = mi[k];
    }
  };
  merge_side(R, &kla);
  merge_side(Q, nullptr);

  if (row_ok && h == 0) {
    const float lse_r = R.m + logf(R.l), lse_q = Q.m + logf(Q.l);
    kv_diag_row o;
    o.lse_ref = lse_r;
    o.lse_q = lse_q;
    o.mass_ref = R.lc / R.l;
    o.mass_q = Q.lc / Q.l;
    o.kl = kla / R.l - lse_r + lse_q;
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
      o.top_ref[k] = R.idx[k];
      o.top_q[k] = Q.idx[k];
    }
    o.reserved = 0;
    p.out[qrow] = o;
  }
}

template <int D, int KB>
hipError_t launch_d(const DiagLaunch &p, hipStream_t stream) {
  const int64_t rows = p.Nq * (p.Hq / p.Hkv);
  const dim3 grid(static_cast<uint32_t>((rows + BM - 1) / BM), static_cast<uint32_t>(p.B * p.Hkv));
  const int32_t gshift = __builtin_ctz(static_cast<unsigned>(p.group));
  if (p.corr == KV_CORR_TAYLOR)
    attn_diag_kernel<D, KB, KV_CORR_TAYLOR><<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows);
  else if (p.corr == KV_CORR_EXACT)
    attn_diag_kernel<D, KB, KV_CORR_EXACT><<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows);
  else
    attn_diag_kernel<D, KB, KV_CORR_OFF><<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diagnostics(const DiagLaunch &p, hipStream_t stream) {
  if (p.d == 64) return p.kbits == 4 ? launch_d<64, 4>(p, stream) : launch_d<64, 2>(p, stream);
  return p.kbits == 4 ? launch_d<128, 4>(p, stream) : launch_d<128, 2>(p, stream);
}

}  // namespace kvq
