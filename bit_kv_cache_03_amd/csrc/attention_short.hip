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
// attn_combine_kernel.  Numerics match the throughput kernel: keys in fp16
// (magic-code dequantisation), per-row query scale, probabilities and values
// in bf16, the Taylor correction of the cached scores as one extra bf16
// MFMA step ("量化鍵值偷走注意力…" (agents-report.net), §方法 and §為何校正有效).
// The keys' power-of-two fp16 scale is chosen per 32-key block from that
// block's own steps and zero points (or values), and folded into the
// softmax scale of the block, so no pass over the whole cache is needed.
//
// Per block (per wave): dequantise K (rows = keys) and V^T (rows = head
// dimension, keys in the permuted order of the P operand) into LDS, fetch
// the next block, S^T = K Q^T (8 fp16 MFMA + 1 correction step), mask the
// ragged block, lazy max, exponentials, O^T += V^T P^T (8 bf16 MFMA).
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int D = 128;
constexpr int BK = 32;          // keys per block
constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int KS = D + 16 + 8;  // K row in LDS: fp16 values[128], bf16 corr[16], pad[8]
constexpr int KEXT = D;
constexpr int VS = BK + 8;      // V^T row in LDS: bf16 keys[32], pad[8] (80 bytes)
constexpr int KT = BK * KS;     // 16-bit elements of a wave's K tile
constexpr int VT = D * VS;      // 16-bit elements of a wave's V^T tile
constexpr int WLDS = KT + VT;
constexpr int OS = D + 4;       // fp32 row of the merge buffer

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
  float gstep[2];      // steps of groups 2h, 2h+1 (correction slots; clamped index)
  uint32_t vw[4];      // V codes of keys 4kq+j at d in [16dq, 16dq+16): INT4 words
  uint32_t vw2[4];     //   d 16dq..+7 in vw, +8..+15 in vw2; INT2 all 16 in vw
  float vstep[4], vzero[4];
};

struct Ctx {
  const uint8_t *kc_codes, *vc_codes;
  const float *kc_scale, *kc_zero, *vc_scale, *vc_zero;
  const uint16_t *k_cur, *v_cur;
  int ng, group_shift;
  int nc, ncur;     // segment lengths
  uint32_t kmask;   // code mask of magic8 (vector register)
};

// Largest of x over the wave.
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Lane roles (per wave):
//  K: key kr = lane % 32 of the block, head-dim half h = lane / 32
//     (d in [64h, 64h+64), i.e. whole groups for group >= 64)
//  V: keys 4kq..4kq+3 with kq = lane % 8, d in [16dq, 16dq+16), dq = lane / 8
// Cached rows past the segment end clamp to its last row (in bounds; the
// scores of those keys are masked).
template <int KBITS, int VBITS>
__device__ inline void fetch_cached(const Ctx &c, int k0, int lane, Fetch &f) {
  const int last = c.nc - 1;
  {
    const int kr = lane & 31, h = lane >> 5;
    const uint32_t row = static_cast<uint32_t>(k0 + kr <= last ? k0 + kr : last);
    const uint4 *ks = reinterpret_cast<const uint4 *>(c.kc_codes + (row * (D * KBITS / 8) + 32u * KBITS / 4 * h));
    const uint4 a = ks[0];
    f.kw[0] = a.x; f.kw[1] = a.y; f.kw[2] = a.z; f.kw[3] = a.w;
    if (KBITS == 4) {
      const uint4 b = ks[1];
      f.kw[4] = b.x; f.kw[5] = b.y; f.kw[6] = b.z; f.kw[7] = b.w;
    }
    const uint32_t km = row * static_cast<uint32_t>(c.ng);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t g = static_cast<uint32_t>((64 * h + 32 * j) >> c.group_shift);
      f.kstep[j] = c.kc_scale[km + g];
      f.kzero[j] = c.kc_zero[km + g];
      const int gg = 2 * h + j < c.ng ? 2 * h + j : c.ng - 1;
      f.gstep[j] = c.kc_scale[km + static_cast<uint32_t>(gg)];
    }
  }
  {
    const int kq = lane & 7, dq = lane >> 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t row = static_cast<uint32_t>(k0 + 4 * kq + j <= last ? k0 + 4 * kq + j : last);
      const uint8_t *vs = c.vc_codes + (row * (D * VBITS / 8) + static_cast<uint32_t>(16 * dq * VBITS / 8));
      if (VBITS == 4) {
        const uint2 w = *reinterpret_cast<const uint2 *>(vs);
        f.vw[j] = w.x;
        f.vw2[j] = w.y;
      } else {
        f.vw[j] = *reinterpret_cast<const uint32_t *>(vs);
      }
      const uint32_t vm = row * static_cast<uint32_t>(c.ng) + static_cast<uint32_t>((16 * dq) >> c.group_shift);
      f.vstep[j] = c.vc_scale[vm];
      f.vzero[j] = c.vc_zero[vm];
    }
  }
}

// K tile of a cached block: fp16 values (magic codes, one v_fma_mix each)
// and, for the Taylor correction, the slots 4g+{0,1,2,3} = (-D_g^2 split
// hi, lo, hi; 0) in bf16 (zero for g >= d/group); lane h writes slots
// 8h .. 8h+7 (groups 2h, 2h+1).
// Returns the block's key exponent e (keys stored as k * 2^-e): the
// dequantised values lie between z and z + (2^bits - 1) D of their group.
template <bool TAYLOR, int KBITS>
__device__ inline int unpack_k_cached(const Ctx &c, int lane, const Fetch &f, uint16_t *Kt) {
  const int kr = lane & 31, h = lane >> 5;
  uint16_t *row = Kt + kr * KS;
  float bound = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    bound = fmaxf(bound, fmaxf(fabsf(f.kzero[j]), fabsf(fmaf(f.kstep[j], static_cast<float>((1 << KBITS) - 1), f.kzero[j]))));
  const int e = scale_exponent(wave_max(bound));
  const float kscale = ldexpf(1.0f, -e);
  float sj[2], zj[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    sj[j] = f.kstep[j] * kscale;
    zj[j] = fmaf(-1024.0f, f.kstep[j], f.kzero[j]) * kscale;
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
    *reinterpret_cast<uint4 *>(row + 64 * h + 8 * i) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (TAYLOR) {
    uint32_t x[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int g = 2 * h + j;
      const float sq = g < c.ng ? f.gstep[j] * f.gstep[j] * kscale : 0.f;
      const float hsq = lo_f(pack2(sq, 0.f));
      x[2 * j] = pack2(-hsq, -(sq - hsq));
      x[2 * j + 1] = pack2(-hsq, 0.f);
    }
    *reinterpret_cast<uint4 *>(row + KEXT + 8 * h) = make_uint4(x[0], x[1], x[2], x[3]);
  }
  return e;
}

// V^T tile of a cached block: bf16 values of keys 4kq..4kq+3 (adjacent
// permuted slots: key r of a 16-key step sits at slot (r&3) + 4*(r>>3) +
// 8*((r>>2)&1)) at head-dim rows 16dq .. 16dq+15, one 8-byte store per row.
template <int VBITS>
__device__ inline void unpack_v_cached(int lane, const Fetch &f, uint16_t *Vt) {
  const int kq = lane & 7, dq = lane >> 3;
  const int a = kq & 3;
  const int slot = 16 * (kq >> 2) + 4 * (a >> 1) + 8 * (a & 1);
#pragma unroll
  for (int half = 0; half < 2; ++half) {  // d = 16dq + 8half .. +7
    float v[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float cv[8];
      codes8<VBITS>(VBITS == 4 ? (half ? f.vw2[j] : f.vw[j]) : (f.vw[j] >> (16 * half)), cv);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = fmaf(f.vstep[j], cv[e], f.vzero[j]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + 8 * half + e, slot)) =
          make_uint2(pack2(v[0][e], v[1][e]), pack2(v[2][e], v[3][e]));
  }
}

// Current-chunk block (bf16 keys and values, loaded and written directly);
// returns the block's key exponent like unpack_k_cached.
__device__ inline int unpack_current(const Ctx &c, int k0, int lane, uint16_t *Kt, uint16_t *Vt) {
  const int last = c.ncur - 1;
  int ek;
  {
    const int kr = lane & 31, h = lane >> 5;
    const uint32_t row = static_cast<uint32_t>(k0 + kr <= last ? k0 + kr : last);
    const uint4 *ks = reinterpret_cast<const uint4 *>(c.k_cur + (row * D + 64u * h));
    uint4 x[8];
    float bound = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = ks[i];
      const uint32_t u[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) bound = fmaxf(bound, fmaxf(fabsf(lo_f(u[e])), fabsf(hi_f(u[e]))));
    }
    ek = scale_exponent(wave_max(bound));
    const float kscale = ldexpf(1.0f, -ek);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack2h(lo_f(u[e]) * kscale, hi_f(u[e]) * kscale);
      *reinterpret_cast<uint4 *>(Kt + kr * KS + 64 * h + 8 * i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  {
    const int kq = lane & 7, dq = lane >> 3;
    const int a = kq & 3;
    const int slot = 16 * (kq >> 2) + 4 * (a >> 1) + 8 * (a & 1);
    uint4 x[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t row = static_cast<uint32_t>(k0 + 4 * kq + j <= last ? k0 + 4 * kq + j : last);
      const uint4 *vs = reinterpret_cast<const uint4 *>(c.v_cur + (row * D + 16u * dq));
      x[j][0] = vs[0];
      x[j][1] = vs[1];
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {  // bf16 pair (8half + 2e2, +1) of each key
        uint32_t u[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 y = x[j][half];
          u[j] = e2 == 0 ? y.x : e2 == 1 ? y.y : e2 == 2 ? y.z : y.w;
        }
        // row d = 16dq + 8half + 2e2 (low halves) and +1 (high halves)
        *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + 8 * half + 2 * e2, slot)) =
            make_uint2(__builtin_amdgcn_perm(u[1], u[0], 0x05040100u), __builtin_amdgcn_perm(u[3], u[2], 0x05040100u));
        *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + 8 * half + 2 * e2 + 1, slot)) =
            make_uint2(__builtin_amdgcn_perm(u[1], u[0], 0x07060302u), __builtin_amdgcn_perm(u[3], u[2], 0x07060302u));
      }
  }
  return ek;
}

struct Soft {
  f32x16 o[D / 32];
  float m, l, alpha;
};

// Scores, softmax and value product of one block from the wave's tiles.
// count < BK marks a ragged block; CORR adds the correction step.
template <bool CORR>
__device__ inline void block_compute(const uint16_t *Kt, const uint16_t *Vt, const f16x8 (&q)[8], bf16x8 qext,
                                     int count, int ek, int lane, Soft &st) {
  const float alpha = ldexpf(st.alpha, ek);  // scores of this block are q.k * 2^-(eq+ek)
  const int qc = lane & 31, h = lane >> 5;
  f32x16 s = f32x16{};
  const uint16_t *kb = Kt + qc * KS + 8 * h;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    s = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8 *>(kb + 16 * j), q[j], s, 0, 0, 0);
  if (CORR)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(kb + KEXT), qext, s, 0, 0, 0);
  if (count < BK) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + 4 * h + (i & 3) >= count) s[i] = -INFINITY;
  }
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[i]);
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
  bf16x8 pk[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(s[8 * hf + i], alpha, -st.m));
    pk[hf] = __builtin_bit_cast(bf16x8, make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]),
                                                   pack2(e[6], e[7])));
    st.l = sum8(pk[hf], st.l);
  }
  // O^T += V^T P^T: k-step ks (keys 16ks..16ks+15), head-dim block db
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int row = 32 * db + qc;
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8 *>(Vt + vts(row, 16 * ks + 8 * h)), pk[ks], st.o[db], 0, 0, 0);
    }
}

template <int KBITS, int VBITS, bool TAYLOR>
__global__ __launch_bounds__(THREADS, 2) void attn_short_kernel(AttnLaunch p, int32_t group_shift,
                                                                int64_t rows_per_kvhead, int32_t row_groups,
                                                                int32_t nsplit, float *ws) {
  __shared__ __attribute__((aligned(16))) uint16_t L[WAVES * WLDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qc = lane & 31, h = lane >> 5;
  const int ng = D >> group_shift;

  // Workgroups are dealt to the 8 XCDs round-robin by id; renumber so that
  // consecutive ids (the splits and row groups of one KV head) share an XCD.
  const uint32_t nwg = gridDim.x, wg = blockIdx.x;
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
  load_query<TAYLOR>(p.q + qrow * D, h, group_shift, p.tau, 0, q, qext, st.alpha);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;

  Ctx c{};
  c.ng = ng;
  c.group_shift = group_shift;
  c.nc = static_cast<int>(p.Nc);
  c.ncur = static_cast<int>(p.Ncur);
  c.kmask = opaque_u32(kCodeMask<KBITS>);
  if (p.Nc > 0) {
    const int64_t hrow = bkv * p.cap;
    c.kc_codes = p.kc_codes + hrow * (D * KBITS / 8);
    c.vc_codes = p.vc_codes + hrow * (D * VBITS / 8);
    c.kc_scale = p.kc_scale + hrow * ng;
    c.kc_zero = p.kc_zero + hrow * ng;
    c.vc_scale = p.vc_scale + hrow * ng;
    c.vc_zero = p.vc_zero + hrow * ng;
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
  const int bend = bbeg + bps < nbt ? bbeg + bps : nbt;
  uint16_t *Kt = L + wave * WLDS;
  uint16_t *Vt = Kt + KT;

  int blk = bbeg + wave;
  Fetch f;
  if (blk < bend && blk < nbc) fetch_cached<KBITS, VBITS>(c, blk * BK, lane, f);
  for (; blk < bend; blk += WAVES) {
    int count;
    if (blk < nbc) {
      const int k0 = blk * BK;
      count = c.nc - k0 < BK ? c.nc - k0 : BK;
      const int ek = unpack_k_cached<TAYLOR, KBITS>(c, lane, f, Kt);
      unpack_v_cached<VBITS>(lane, f, Vt);
      const int nb = blk + WAVES;
      if (nb < bend && nb < nbc) fetch_cached<KBITS, VBITS>(c, nb * BK, lane, f);
      block_compute<TAYLOR>(Kt, Vt, q, qext, count, ek, lane, st);
    } else {
      const int k0 = (blk - nbc) * BK;
      count = c.ncur - k0 < BK ? c.ncur - k0 : BK;
      const int ek = unpack_current(c, k0, lane, Kt, Vt);
      block_compute<false>(Kt, Vt, q, qext, count, ek, lane, st);
    }
  }

  // ---- merge the 4 waves (log-sum-exp), then the split partial or output ----
  const float l_tot = st.l + __shfl_xor(st.l, 32, 64);
  __syncthreads();  // every wave is done with its tiles
  float *Ob = reinterpret_cast<float *>(L) + wave * (32 * OS + 64);
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
        mw[w] = reinterpret_cast<const float *>(L)[w * (32 * OS + 64) + 32 * OS + 2 * row];
        m = fmaxf(m, mw[w]);
      }
      float acc[16], l = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float *base = reinterpret_cast<const float *>(L) + w * (32 * OS + 64);
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

template <int KB, int VB>
hipError_t launch_bits(const AttnLaunch &p, hipStream_t stream) {
  const int64_t rows = p.Nq * (p.Hq / p.Hkv);
  const int32_t row_groups = static_cast<int32_t>((rows + 31) / 32);
  const int32_t gshift = __builtin_ctz(static_cast<unsigned>(p.group));
  const int64_t nrows = p.B * p.Hq * p.Nq;
  float *partials = static_cast<float *>(p.workspace);
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.splits) * row_groups * p.B * p.Hkv));
  if (p.corr == KV_CORR_TAYLOR)
    attn_short_kernel<KB, VB, true><<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows, row_groups, p.splits, partials);
  else
    attn_short_kernel<KB, VB, false><<<grid, dim3(THREADS), 0, stream>>>(p, gshift, rows, row_groups, p.splits,
                                                                         partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_combine(partials, p.out, nrows, p.splits, p.d, stream);
}

}  // namespace

bool short_fast_supported(int32_t d, int corr) { return d == D && corr != KV_CORR_EXACT; }

int short_fast_splits(int64_t B, int64_t Hkv, int64_t rows_per_kvhead, int64_t Nc, int64_t Ncur, int cu_count) {
  const int64_t groups = B * Hkv * ((rows_per_kvhead + 31) / 32);
  const int64_t blocks = (Nc + BK - 1) / BK + (Ncur + BK - 1) / BK;
  int64_t s = (4 * static_cast<int64_t>(cu_count) + groups - 1) / groups;  // ~4 workgroups per CU
  const int64_t max_s = (blocks + 4 * WAVES - 1) / (4 * WAVES);              // >= 4 blocks per wave
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 1024) s = 1024;
  return static_cast<int>(s);
}

hipError_t launch_attention_short_fast(const AttnLaunch &p, hipStream_t stream) {
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<2, 2>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2>(p, stream);
  return launch_bits<4, 4>(p, stream);
}

}  // namespace kvq
