// Short-query kernel for at most 16 query rows per KV head (decode and
// small chunks of GQA heads) on gfx950: head dim 128, correction off or
// Taylor.
//
// The same split of the cache as attention_short.hip (many workgroups per
// KV head; inside one, 4 waves that stream their own 32-key blocks and
// merge at the end), but on 16 x 16 x 32 MFMA tiles: one 16-row query tile
// instead of a 32-row one, so a block's scores are 8 per lane instead of 16
// (half the exponentials, maxima and packing) and the accumulators take half
// the registers.  The scores of the cached keys carry the Taylor correction
// in extra bf16 MFMA steps ("量化鍵值偷走注意力…" (agents-report.net), §方法
// and §為何校正有效), with the current chunk's keys left alone; everything
// goes through one online softmax.
//
// Caches grouped along the head dimension with at most two groups per row
// (the common case) take the staged, raw-operand form: each wave streams its
// blocks through two LDS stages filled by direct-to-LDS buffer loads (two
// blocks in flight, no registers held; see "staged fetch"), the keys enter
// the score MFMAs as raw codes with one accumulator per group (stage_k_raw),
// and the value operands are built in registers from the staged codes on a
// permuted head-dim order (v_operand), the codes multiplying p D carried as
// fp16 hi + lo.  Other caches dequantise keys into fp16 MFMA operands and
// values into a V^T tile in LDS, with a one-block register prefetch.
//
// Lane roles of the dequantising form (r = lane % 16, j = lane / 16):
//  K (A operand of S^T = K Q^T): keys 16t + r of the block (t = 0, 1), head
//    dims 32j .. 32j+31 (k-step s: 32j + 8s .. +7) -- one group per lane;
//  Q (B operand): query row r of the tile, the same dims;
//  S^T (16 x 16 per key tile): query r, keys 16t + 4j + i (i = 0..3);
//  P^T (B operand of O^T = V^T P^T, 32 keys in one k-step): query r, k-slots
//    8j .. 8j+7 = keys 4j .. 4j+3, then 16+4j .. 16+4j+3 -- the lane's own
//    probabilities, so the V^T tile in LDS takes its keys in that order;
//  V (dequantisation): keys 4kq .. 4kq+3 (kq = lane % 8), dims 16dq .. 16dq+15
//    (dq = lane / 8), written transposed into the V^T tile;
//  O^T (16 x 16 per head-dim tile dt): query r, dims 16dt + 4j + i.
// The raw-operand form changes the K and Q dims of k-step i to
// 32i + 8j .. +7 (kraw_dim0) and the O^T rows to vrow<true>.
//
// Keys grouped along the tokens (KVQ_SHORT16_KTOK: one step D_c and zero
// point z_c per channel c and token group, the page's per-channel reading of
// D_{i,c}; values along the head dimension): a 32-key block lies in one token
// group, so D folds into the query instead of the keys.  Per group a lane
// forms q'_c = q_c D_c 2^-ed for its 32 dims (fp16, in the order of the code
// words below) and one per-row term, q.z - (tau/24) sum_c q_c^2 D_c^2 (the
// Taylor bias of "量化鍵值偷走注意力…" (agents-report.net) §方法 with per-channel
// steps); the key operand is then the raw codes themselves, each in the low
// bits of its 16-bit field, i.e. the fp16 subnormal c 2^-24 (exact: the MFMA
// takes subnormal inputs as they are).  Each wave walks a contiguous range of
// blocks so that consecutive blocks share their group's query terms.
//
// Values grouped along the tokens (KVQ_SHORT16_VTOK, with keys either way):
// the values are dequantised as above, with per-channel operands instead of
// per-key ones, staged per token group in the wave's LDS area.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "quant_device.h"
#include "short_common.h"

#ifndef KVQ_SHORT16_PAGED
#define KVQ_SHORT16_PAGED 0
#endif
#ifndef KVQ_SHORT16_META16
#define KVQ_SHORT16_META16 0
#endif
#ifndef KVQ_SHORT16_KTOK
#define KVQ_SHORT16_KTOK 0
#endif
#ifndef KVQ_SHORT16_VTOK
#define KVQ_SHORT16_VTOK 0
#endif

namespace kvq {
namespace {

using namespace dev;
using namespace sk;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int ROWS = 16;             // query rows of the tile
constexpr int VS = BK + 8;           // V^T row in LDS: fp16 key slots[32], pad[8] (80 bytes)
constexpr int VT = D * VS;           // 16-bit elements of a wave's V^T tile
constexpr int OS = D + 4;            // fp32 row of the merge buffer
constexpr int MERGE = ROWS * OS + 2 * ROWS;  // floats of a wave's merge buffer (O rows, then m and l)
constexpr int LDS_BYTES = WAVES * VT * 2 > WAVES * MERGE * 4 ? WAVES * VT * 2 : WAVES * MERGE * 4;
constexpr int GM = 2 * D;  // floats of a wave's token-group staging of K or of V (two per channel)
// Cached values as raw codes (groups along the head dimension): a wave's
// per-key steps Ds (4 groups x 32 keys, as fp16 hi then lo) and zero-point
// operand Zs (16
// rows x ZS fp16: rows g and NG + g the hi and lo parts of group g's zero
// points, the rest zero; 80-byte rows keep the 16 rows' reads on distinct
// banks).  kVcodeScale keeps p D 2^-ev kVcodeScale < 2^15.42 for p <= 2^8
// and |v| 2^-ev < 2^14 (D <= 2^15 / 3), inside the fp16 range.
constexpr int ZS = 40;
constexpr int VCODE_HALVES = 2 * 4 * 32 + 16 * ZS;
constexpr float kVcodeScale = 1.0f / 64.0f;

// V^T element (row = head-dim index, col = key slot 0..31); the 16-byte
// chunks of a row are XOR-swizzled by (row / 16) % 4 so that the transposed
// 8-byte stores of 16 consecutive rows spread over the banks.
__device__ inline int vts(int row, int col) {
  return row * VS + ((((col >> 3) ^ (row >> 4)) & 3) << 3) + (col & 7);
}

// Key slot of the four keys 4kq .. 4kq+3 (consecutive slots): keys below 16
// sit at 8 (k / 4) + k % 4, keys 16 + k at 8 (k / 4) + 4 + k % 4.
__device__ inline int vslot4(int kq) { return kq < 4 ? 8 * kq : 8 * (kq - 4) + 4; }

// Registers of one prefetched cached block.
struct Fetch {
  uint32_t kw[2][4];  // K codes of keys 16t + r, dims [32j, 32j+32): INT4 4 words, INT2 2
  float kstep[2];     // their group's step and zero point
  float kzero[2];
  uint32_t vw[4];     // V codes of keys 4kq+i at d in [16dq, 16dq+16): INT4 words
  uint32_t vw2[4];    //   d 16dq..+7 in vw, +8..+15 in vw2; INT2 all 16 in vw
  float vstep[4], vzero[4];
  uint32_t gd[2], gz[2];  // keys along the tokens: two steps / zero points of the block's token group, as stored
  uint32_t vgd[2], vgz[2];  // values along the tokens: the same for V
};

// Byte offsets of the lane's data from the block's first cache row; NG is
// the number of quantisation groups per row (128 / group).
struct Lanes {
  uint32_t kc, km, vc, vm;
};
template <int KBITS, int VBITS, int NG, int MT>
__device__ inline Lanes lane_offsets(int lane) {
  constexpr uint32_t KROW = D * KBITS / 8, VROW = D * VBITS / 8, ES = MT ? 2 : 4;
  const uint32_t r = lane & 15, j = lane >> 4, kq = lane & 7, dq = lane >> 3;
  Lanes o;
  o.kc = r * KROW + j * (32 * KBITS / 8);
  o.km = (r * NG + (32 * j * NG) / D) * ES;  // the group of d = 32j
  o.vc = 4 * kq * VROW + 16 * dq * VBITS / 8;
  o.vm = (4 * kq * NG + (16 * dq * NG) / D) * ES;  // the group of d = 16dq
  return o;
}

// Loads one cached block (rows [k0, k0 + 32)); rows at or past the segment
// end read as zero (their scores are masked).  Paged: the buffer range stops
// at the block's end, inside its page.
template <int KBITS, int VBITS, int NG, bool PAGED, int MT, bool KTOK = false, bool VTOK = false>
__device__ inline void fetch_cached(const Ctx &c, int k0, const Lanes &o, Fetch &f, size_t pool_row = 0,
                                    int gshift = 0, bool newg = false) {
  constexpr uint32_t KROW = D * KBITS / 8, VROW = D * VBITS / 8, ES = MT ? 2 : 4;
  const uint32_t rows = static_cast<uint32_t>(PAGED ? min(c.nc - k0, BK) : c.nc - k0);
  const size_t r0 = PAGED ? pool_row : block_row<false>(c, k0);  // paged: looked up a block earlier
  {
    const Buf kc = buffer_at(c.kc_codes + r0 * KROW, rows * KROW);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (KBITS == 4) {
        const u32x4 a = ld128(kc, o.kc + t * 16 * KROW);
        f.kw[t][0] = a.x; f.kw[t][1] = a.y; f.kw[t][2] = a.z; f.kw[t][3] = a.w;
      } else {
        const u32x2 a = ld64(kc, o.kc + t * 16 * KROW);
        f.kw[t][0] = a.x; f.kw[t][1] = a.y;
      }
    }
    if (KTOK) {
      // the token group's D row of steps and of zero points (at metadata row
      // r0 >> gshift): two of each per lane, when the block starts a group
      if (newg) {
        const size_t mrow = r0 >> gshift;
        const Buf ks = buffer_at(meta_adv<MT>(c.kc_scale, mrow * D), D * ES);
        const Buf kz = buffer_at(meta_adv<MT>(c.kc_zero, mrow * D), D * ES);
        const uint32_t off = static_cast<uint32_t>(__lane_id()) * 2 * ES;
        if (MT == kMetaF32) {
          const u32x2 a = ld64(ks, off), b = ld64(kz, off);
          f.gd[0] = a.x; f.gd[1] = a.y; f.gz[0] = b.x; f.gz[1] = b.y;
        } else {
          f.gd[0] = ld32(ks, off);
          f.gz[0] = ld32(kz, off);
        }
      }
    } else {
      const Buf ks = buffer_at(meta_adv<MT>(c.kc_scale, r0 * NG), rows * NG * ES);
      const Buf kz = buffer_at(meta_adv<MT>(c.kc_zero, r0 * NG), rows * NG * ES);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f.kstep[t] = ld_meta1<MT>(ks, o.km + t * 16 * NG * ES);
        f.kzero[t] = ld_meta1<MT>(kz, o.km + t * 16 * NG * ES);
      }
    }
  }
  {
    const Buf vc = buffer_at(c.vc_codes + r0 * VROW, rows * VROW);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (VBITS == 4) {
        const u32x2 w = ld64(vc, o.vc + i * VROW);
        f.vw[i] = w.x;
        f.vw2[i] = w.y;
      } else {
        f.vw[i] = ld32(vc, o.vc + i * VROW);
      }
    }
    if (VTOK) {
      if (newg) {  // as for the keys: the token group's rows of steps and zero points
        const size_t mrow = r0 >> gshift;
        const Buf vs = buffer_at(meta_adv<MT>(c.vc_scale, mrow * D), D * ES);
        const Buf vz = buffer_at(meta_adv<MT>(c.vc_zero, mrow * D), D * ES);
        const uint32_t off = static_cast<uint32_t>(__lane_id()) * 2 * ES;
        if (MT == kMetaF32) {
          const u32x2 a = ld64(vs, off), b = ld64(vz, off);
          f.vgd[0] = a.x; f.vgd[1] = a.y; f.vgz[0] = b.x; f.vgz[1] = b.y;
        } else {
          f.vgd[0] = ld32(vs, off);
          f.vgz[0] = ld32(vz, off);
        }
      }
    } else {
      const Buf vs = buffer_at(meta_adv<MT>(c.vc_scale, r0 * NG), rows * NG * ES);
      const Buf vz = buffer_at(meta_adv<MT>(c.vc_zero, r0 * NG), rows * NG * ES);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f.vstep[i] = ld_meta1<MT>(vs, o.vm + i * NG * ES);
        f.vzero[i] = ld_meta1<MT>(vz, o.vm + i * NG * ES);
      }
    }
  }
}

// ---- staged fetch: cached blocks through per-wave LDS stages ----------------
// A register prefetch keeps one block in flight per wave, and only while the
// block before it is being multiplied: too few bytes in flight to cover the
// HBM latency with two waves per SIMD.  Instead each wave streams its blocks
// through two LDS stages filled by buffer loads that write LDS directly
// (buffer_load ... lds: lane l of a 16-byte load lands at 16 l past the
// address in M0, of a 4-byte load at 4 l), so two blocks are in flight
// while a third is unpacked and multiplied, and no registers are held for
// them.  A stage mirrors the block's bytes in HBM: K codes, V codes, then
// the four step / zero-point arrays (each padded to 256 bytes, the span of
// one 4-byte load); rows past the segment end read as zero.
//
// The loads are issued from inline assembly, so the compiler's wait
// counting does not see them (it would otherwise wait for every load into
// LDS before any LDS read it cannot tell apart from the stages, the V^T
// tile's included); the kernel waits for a stage itself (s_waitcnt vmcnt
// with the count of the loads issued after the stage's own, which every
// step issues in the same number, past-the-end blocks as empty ranges).
// Each asm block saves and restores M0, keeps the 5 wait states between an
// SGPR written by the VALU and a memory instruction reading it, and the one
// between writing M0 and a load into LDS.
template <int KBITS, int VBITS, int NG, int MT>
struct StageLayout {
  static constexpr uint32_t KROW = D * KBITS / 8, VROW = D * VBITS / 8, ES = MT ? 2 : 4;
  static constexpr uint32_t KC = BK * KROW, VC = BK * VROW;     // code bytes (multiples of 1 KB)
  static constexpr uint32_t MB = BK * NG * ES;                  // bytes of one metadata array
  static constexpr uint32_t MR = MB < 256 ? 256 : MB;           // its region
  static constexpr uint32_t KS = KC + VC, KZ = KS + MR, VSC = KZ + MR, VZ = VSC + MR;
  static constexpr uint32_t BYTES = VZ + MR;
  static constexpr int LOADS = (KC + VC) / 1024 + 4 * (MR / 256);  // load instructions per block
};

// Buffer descriptor words over `bytes` bytes at p (stride 0, the same flags
// as buffer_at).
__device__ inline u32x4 rsrc_words(const void *p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
__device__ inline uint32_t lds_addr(const uint8_t *p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const void *)(p)));
}
// One load into LDS at lds (wave-uniform), lane offset voff.  WAIT: first
// wait for the wave's outstanding LDS reads (the stage being refilled was
// just read).
#define KVQ_DMA_ASM(WAITSTR, LOAD)                                                                              \
  asm volatile(WAITSTR "s_mov_b32 %[t], m0\n\ts_nop 4\n\ts_mov_b32 m0, %[a]\n\ts_nop 0\n\t" LOAD            \
                       " %[v], %[r], 0 offen lds\n\ts_nop 0\n\ts_mov_b32 m0, %[t]"                                 \
               : [t] "=&s"(saved)                                                                               \
               : [a] "s"(a), [v] "v"(voff), [r] "s"(rs)                                                         \
               : "memory")
template <int BYTES, bool WAIT>
__device__ inline void dma(u32x4 rs, const uint8_t *lds, uint32_t voff) {
  static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte loads");
  uint32_t saved;
  const uint32_t a = lds_addr(lds);
  if (BYTES == 16 && WAIT) KVQ_DMA_ASM("s_waitcnt lgkmcnt(0)\n\t", "buffer_load_dwordx4");
  if (BYTES == 16 && !WAIT) KVQ_DMA_ASM("", "buffer_load_dwordx4");
  if (BYTES == 4 && WAIT) KVQ_DMA_ASM("s_waitcnt lgkmcnt(0)\n\t", "buffer_load_dword");
  if (BYTES == 4 && !WAIT) KVQ_DMA_ASM("", "buffer_load_dword");
}
#undef KVQ_DMA_ASM

// Starts the loads of the cached block at rows [r0, r0 + 32) (rows: rows
// left in the segment from r0, 0 for an empty range) into the wave's stage
// st, after the wave's outstanding LDS reads.
template <int KBITS, int VBITS, int NG, int MT>
__device__ inline void stage_issue(const Ctx &c, size_t r0, uint32_t rows, const uint8_t *st, int lane) {
  using SL = StageLayout<KBITS, VBITS, NG, MT>;
  const uint32_t l16 = static_cast<uint32_t>(lane) * 16, l4 = static_cast<uint32_t>(lane) * 4;
  const u32x4 kc = rsrc_words(c.kc_codes + r0 * SL::KROW, rows * SL::KROW);
  dma<16, true>(kc, st, l16);
#pragma unroll
  for (uint32_t i = 1; i < SL::KC / 1024; ++i) dma<16, false>(kc, st + 1024 * i, l16 + 1024 * i);
  const u32x4 vc = rsrc_words(c.vc_codes + r0 * SL::VROW, rows * SL::VROW);
#pragma unroll
  for (uint32_t i = 0; i < SL::VC / 1024; ++i) dma<16, false>(vc, st + SL::KC + 1024 * i, l16 + 1024 * i);
  const uint32_t mbytes = rows * NG * SL::ES;
  const u32x4 m[4] = {rsrc_words(meta_adv<MT>(c.kc_scale, r0 * NG), mbytes),
                      rsrc_words(meta_adv<MT>(c.kc_zero, r0 * NG), mbytes),
                      rsrc_words(meta_adv<MT>(c.vc_scale, r0 * NG), mbytes),
                      rsrc_words(meta_adv<MT>(c.vc_zero, r0 * NG), mbytes)};
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (uint32_t i = 0; i < SL::MR / 256; ++i) dma<4, false>(m[a], st + SL::KS + a * SL::MR + 256 * i, l4 + 256 * i);
}

template <int MT>
__device__ inline float lds_meta(const uint8_t *p) {
  if (MT != kMetaF32) return meta16_value(*reinterpret_cast<const uint16_t *>(p), MT);
  return *reinterpret_cast<const float *>(p);
}

// The lane's share of a staged block, at the offsets fetch_cached loads it
// from HBM.
template <int KBITS, int VBITS, int NG, int MT, bool VCODES = true, bool KCODES = true>
__device__ inline void stage_read(const uint8_t *st, const Lanes &o, Fetch &f) {
  using SL = StageLayout<KBITS, VBITS, NG, MT>;
#pragma unroll
  for (int t = 0; t < 2 && KCODES; ++t) {
    const uint8_t *k = st + o.kc + t * 16 * SL::KROW;
    if (KBITS == 4) {
      const uint4 a = *reinterpret_cast<const uint4 *>(k);
      f.kw[t][0] = a.x; f.kw[t][1] = a.y; f.kw[t][2] = a.z; f.kw[t][3] = a.w;
    } else {
      const uint2 a = *reinterpret_cast<const uint2 *>(k);
      f.kw[t][0] = a.x; f.kw[t][1] = a.y;
    }
    f.kstep[t] = lds_meta<MT>(st + SL::KS + o.km + t * 16 * NG * SL::ES);
    f.kzero[t] = lds_meta<MT>(st + SL::KZ + o.km + t * 16 * NG * SL::ES);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t *v = st + SL::KC + o.vc + i * SL::VROW;
    if (!VCODES) {
    } else if (VBITS == 4) {
      const uint2 w = *reinterpret_cast<const uint2 *>(v);
      f.vw[i] = w.x;
      f.vw2[i] = w.y;
    } else {
      f.vw[i] = *reinterpret_cast<const uint32_t *>(v);
    }
    f.vstep[i] = lds_meta<MT>(st + SL::VSC + o.vm + i * NG * SL::ES);
    f.vzero[i] = lds_meta<MT>(st + SL::VZ + o.vm + i * NG * SL::ES);
  }
}

// The cached keys are centred per group (group_centre) when a row has at
// most two groups; the extra bf16 steps carry centre x query group sum.
template <int NG>
constexpr bool kCentre = NG <= 2;

// Largest |k - centre| (|v|) a lane's share of a cached block can
// dequantise to: the values of a group lie between z and z + (2^bits - 1) D.
template <int KBITS, int NG>
__device__ inline float k_bound(const Fetch &f) {
  float b = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float z = kCentre<NG> ? f.kzero[t] - group_centre<KBITS>(f.kzero[t], f.kstep[t]) : f.kzero[t];
    b = fmaxf(b, fmaxf(fabsf(z), fabsf(fmaf(f.kstep[t], static_cast<float>((1 << KBITS) - 1), z))));
  }
  return b;
}
template <int VBITS>
__device__ inline float v_bound(const Fetch &f) {
  float b = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    b = fmaxf(b, fmaxf(fabsf(f.vzero[i]), fabsf(fmaf(f.vstep[i], static_cast<float>((1 << VBITS) - 1), f.vzero[i]))));
  return b;
}

// Is the lane's quarter j the first of its group (the one that carries the
// group's terms in the extra step)?
template <int NG>
__device__ inline bool group_owner(int j) {
  return NG == 4 ? true : NG == 2 ? (j & 1) == 0 : j == 0;
}

// K operands of a cached block: k[t][s] = fp16 (k - c_g) 2^-ek of key 16t + r
// at dims 32j + 8s .. +7 (magic codes, one v_fma_mix each; c_g the group's
// centre, 0 with 4 groups), and the extra step's slots 8j .. 8j+7, scaled
// like the keys, on the first quarter of each group only: the Taylor terms
// (-D^2 split hi, lo, hi; 0), then (c_g, c_g, 0, 0) with centring (the query
// side holds N_g and the group sum against them); zero elsewhere.
template <bool TAYLOR, int KBITS, int NG>
__device__ inline void unpack_k_cached(const Ctx &c, int lane, const Fetch &f, float kscale, f16x8 (&k)[2][4],
                                       bf16x8 (&kext)[2]) {
  const bool owner = group_owner<NG>(lane >> 4);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float cg = kCentre<NG> ? group_centre<KBITS>(f.kzero[t], f.kstep[t]) : 0.f;
    const float st = f.kstep[t] * kscale;
    const float z = fmaf(-1024.0f, f.kstep[t], f.kzero[t] - cg) * kscale;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t m[4];
      magic8<KBITS>(KBITS == 4 ? f.kw[t][s] : (f.kw[t][s >> 1] >> (16 * (s & 1))), c.kmask, m);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pair_h(dequant_h(magic_code(m, 2 * e), st, z), dequant_h(magic_code(m, 2 * e + 1), st, z));
      k[t][s] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
    const float sq = TAYLOR ? f.kstep[t] * f.kstep[t] * kscale : 0.f;
    const float hsq = lo_f(pack2(sq, 0.f));
    const float cs = cg * kscale;
    uint4 x = make_uint4(pack2(-hsq, -(sq - hsq)), pack2(-hsq, 0.f), kCentre<NG> ? pack2(cs, cs) : 0u, 0u);
    if (!owner) x = make_uint4(0u, 0u, 0u, 0u);
    kext[t] = __builtin_bit_cast(bf16x8, x);
  }
}

// K operands of a cached block whose keys group along the tokens: the codes
// of key 16t + r at dims 32j + 8s .. +7, each in the low bits of a 16-bit
// field (the fp16 subnormal c 2^-24), word e holding dims e and e + 4 (the
// query side takes the same order).
template <int KBITS>
__device__ inline void unpack_k_codes(const Ctx &c, const Fetch &f, f16x8 (&k)[2][4]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w = KBITS == 4 ? f.kw[t][s] : (f.kw[t][s >> 1] >> (16 * (s & 1)));
      // INT2: code e + 4 of the 16-bit chunk moves next to code e, 16 bits up
      const uint32_t x = KBITS == 4 ? w : (w & 0xffffu) | ((w & 0xffffu) << 8);
      uint32_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = (x >> (KBITS * e)) & c.kmask;
      k[t][s] = __builtin_bit_cast(f16x8, make_uint4(m[0], m[1], m[2], m[3]));
    }
}

// Two stored steps or zero points of a token group (one 32-bit word each in
// fp32, both in one word with 16 bits) as fp32.
template <int MT>
__device__ inline void meta_pair(const uint32_t (&w)[2], float (&v)[2]) {
  if (MT == kMetaF32) {
    v[0] = __uint_as_float(w[0]);
    v[1] = __uint_as_float(w[1]);
  } else {
    v[0] = meta16_value(static_cast<uint16_t>(w[0]), MT);
    v[1] = meta16_value(static_cast<uint16_t>(w[0] >> 16), MT);
  }
}

// Query terms of a token group (keys along the tokens), from the group's
// steps D_c and zero points z_c in f (staged through the wave's LDS area Gm):
// qk[s] word e = fp16(q_c D_c 2^-ed) of dims c = 32j + 8s + e and + 4, with
// 2^ed above the group's largest step; the scores of the codes then read
// sum_c q'_c c_c 2^-24 (units of 2^-(eq + ed + 24)), so the block's softmax
// scale is alpha_g = alpha_q 2^(ed + 24) and the row adds
// sadd = q.z - (tau/24) sum_c q_c^2 D_c^2 in those units (q.z over the
// unscaled z; the bias from the rounded q').
// qun = 2^eq undoes the query's scaling (q holds q 2^-eq).
template <bool TAYLOR, int MT>
__device__ inline void ktok_group(const Fetch &f, int lane, float *Gm, const f16x8 (&q)[4], float tau, float alpha_q,
                                  float qun, f16x8 (&qk)[4], float &sadd, float &alpha_g) {
  float dv[2], zv[2];
  meta_pair<MT>(f.gd, dv);
  meta_pair<MT>(f.gz, zv);
  *reinterpret_cast<float2 *>(Gm + 2 * lane) = make_float2(dv[0], dv[1]);
  *reinterpret_cast<float2 *>(Gm + D + 2 * lane) = make_float2(zv[0], zv[1]);
  const float dmax = wave_max(fmaxf(dv[0], dv[1]));
  const int ed = dmax > 0.f ? ilog2_pos(dmax) + 1 : 0;
  const float ds = ldexpf(1.0f, -ed);
  const int j = lane >> 4;
  float s2 = 0.f, sz = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float *gd = Gm + 32 * j + 8 * s, *gz = Gm + D + 32 * j + 8 * s;
    const float4 d0 = *reinterpret_cast<const float4 *>(gd), d1 = *reinterpret_cast<const float4 *>(gd + 4);
    const float4 z0 = *reinterpret_cast<const float4 *>(gz), z1 = *reinterpret_cast<const float4 *>(gz + 4);
    const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
    const uint4 qw = __builtin_bit_cast(uint4, q[s]);  // word e: dims 2e, 2e + 1
    const uint32_t u[4] = {qw.x, qw.y, qw.z, qw.w};
    float qv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16x2 h = __builtin_bit_cast(f16x2, u[e]);
      qv[2 * e] = static_cast<float>(h.x);
      qv[2 * e + 1] = static_cast<float>(h.y);
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
    qk[s] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  s2 += __shfl_xor(s2, 16, 64);
  sz += __shfl_xor(sz, 16, 64);
  s2 += __shfl_xor(s2, 32, 64);
  sz += __shfl_xor(sz, 32, 64);
  // in units of q' c: q.z 2^-eq 2^-ed = sz ds; bias (tau/24) 2^(eq+ed) s2
  const float bias = TAYLOR ? (tau / 24.0f) * qun * ldexpf(s2, ed) : 0.f;
  sadd = ldexpf(sz * ds - bias, -24);
  alpha_g = ldexpf(alpha_q, ed + 24);
}

// Values along the tokens: the largest |v| the lane's two channels of the
// block's token group can dequantise to.
template <int VBITS, int MT>
__device__ inline float vtok_bound(const Fetch &f) {
  float dv[2], zv[2];
  meta_pair<MT>(f.vgd, dv);
  meta_pair<MT>(f.vgz, zv);
  float b = 0.f;
#pragma unroll
  for (int e = 0; e < 2; ++e)
    b = fmaxf(b, fmaxf(fabsf(zv[e]), fabsf(fmaf(dv[e], static_cast<float>((1 << VBITS) - 1), zv[e]))));
  return b;
}

// Stages a token group's value operands in the wave's LDS area Gv: for
// channel c, d_c = D_c vsc 2^-p and z_c = (z_c vsc) - 1024 d_c, p the
// position of its code field in the byte pair the dequantisation reads (0
// for even channels, 4 (INT4) or 2 (INT2) for odd ones); the lane writes
// channels 2 lane and 2 lane + 1.
template <int VBITS, int MT>
__device__ inline void vtok_stage(const Fetch &f, int lane, float vsc, float *Gv) {
  constexpr int P1 = VBITS == 4 ? 4 : 2;
  float dv[2], zv[2];
  meta_pair<MT>(f.vgd, dv);
  meta_pair<MT>(f.vgz, zv);
  const float d0 = dv[0] * vsc, d1 = dv[1] * vsc * (1.0f / (1 << P1));
  *reinterpret_cast<float2 *>(Gv + 2 * lane) = make_float2(d0, d1);
  *reinterpret_cast<float2 *>(Gv + D + 2 * lane) =
      make_float2(fmaf(-1024.0f, d0, zv[0] * vsc), fmaf(-1024.0f, d1, zv[1] * vsc));
}

// V^T tile of a cached block as raw codes, and the block's per-key value
// operands.  The value product then needs no dequantisation per value:
//   sum_i p_i (z_ig + D_ig c_i) = sum_i (p_i D_ig) c_i + sum_i p_i z_ig,
// so the codes enter the MFMA as they are and each group's step D_ig rides
// on the probabilities (one B operand per group), the zero points on one
// extra MFMA step per block.
//  - Codes: one v_perm gathers the same code byte of two keys (bits 0..7 and
//    16..23), one AND keeps a code field at bit p of both: the fp16
//    subnormals c 2^(p-24), exact.  INT4 fields sit at p = 0 and 4, INT2 at
//    p = 0 and 2 of the byte and of the byte shifted right by 4; head-dim row
//    16dq + NF byte + fl holds field fl, so odd rows carry 2^P1.
//  - Per key (slots vslot4(kq) .. +3, from the first lane of each group):
//    Ds rows 2g, 2g + 1 = D 2^-ev kVcodeScale and Zs rows g, NG + g =
//    z 2^-ev, each split into hi + lo, all fp16 (the other rows of Zs stay
//    zero).
template <int VBITS, int NG, bool TILE = true>
__device__ inline void unpack_v_raw(const Ctx &c, int lane, const Fetch &f, float vsc, uint16_t *Vt, uint16_t *Ds,
                                    uint16_t *Zs) {
  const int kq = lane & 7, dq = lane >> 3;
  const int slot = vslot4(kq);
  constexpr int DQG = 8 / NG;  // lanes' dq values per group (16 dims each)
  if (dq % DQG == 0) {
    const int g = dq / DQG;
    const float ds = vsc * kVcodeScale;
    _Float16 zh[4], zl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = f.vzero[i] * vsc;
      zh[i] = static_cast<_Float16>(z);
      zl[i] = static_cast<_Float16>(z - static_cast<float>(zh[i]));
    }
    _Float16 dh[4], dl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = f.vstep[i] * ds;
      dh[i] = static_cast<_Float16>(d);
      dl[i] = static_cast<_Float16>(d - static_cast<float>(dh[i]));
    }
    *reinterpret_cast<uint2 *>(Ds + 64 * g + slot) = make_uint2(pair_h(dh[0], dh[1]), pair_h(dh[2], dh[3]));
    *reinterpret_cast<uint2 *>(Ds + 64 * g + 32 + slot) = make_uint2(pair_h(dl[0], dl[1]), pair_h(dl[2], dl[3]));
    *reinterpret_cast<uint2 *>(Zs + ZS * g + slot) = make_uint2(pair_h(zh[0], zh[1]), pair_h(zh[2], zh[3]));
    *reinterpret_cast<uint2 *>(Zs + ZS * (NG + g) + slot) = make_uint2(pair_h(zl[0], zl[1]), pair_h(zl[2], zl[3]));
  }
  if (!TILE) return;  // the value operands come from registers (v_operands)
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
      x[0][jp] = r[jp] & c.vmask0;
      x[1][jp] = r[jp] & c.vmask1;
      if (VBITS == 2) {
        x[NF - 2][jp] = (r[jp] >> 4) & c.vmask0;
        x[NF - 1][jp] = (r[jp] >> 4) & c.vmask1;
      }
    }
#pragma unroll
    for (int fl = 0; fl < NF; ++fl)
      *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + NF * byte + fl, slot)) = make_uint2(x[fl][0], x[fl][1]);
  }
}

// Value operands in registers (staged caches, at most two groups per row):
// the A operand of the value product for head-dim tile dt is built by the
// lane from the staged codes instead of a V^T tile in LDS, which saves the
// transposed LDS stores and their reads on every block.  The tile's rows are
// a permutation of the head dimension chosen so that a lane's eight tiles
// cover dims 4r .. 4r+3 and 64 + 4r .. 64 + 4r+3 (r = lane % 16), i.e. two
// 16-bit (INT4) or 8-bit (INT2) pieces of each code row, and every tile lies
// in one quantisation group: row r of tile dt is dim vrow<true>(dt, r).
// A lane's k-slots 8j .. 8j+7 (j = lane / 16) are the keys of its P^T
// operand, 4j .. 4j+3 and 16 + 4j .. 16 + 4j+3.
template <bool PERM>
__device__ inline int vrow(int dt, int r) {
  return PERM ? 64 * (dt >> 2) + 4 * r + (dt & 3) : 16 * dt + r;
}

// The lane's code words of its eight keys from the stage: y[i][0] the
// 4-byte word holding the piece of dims 4r .. 4r+3 of key i (INT4: bytes
// 2 (r % 2), +1 of it; INT2: byte r % 4), y[i][1] the word holding the piece of
// dims 64 + 4r .. +3 (the same bytes, half a code row further).
template <int VBITS>
__device__ inline void stage_read_vcodes(const uint8_t *vc, int lane, uint32_t (&y)[8][2]) {
  constexpr uint32_t VROW = D * VBITS / 8;
  const int r = lane & 15, j = lane >> 4;
  const uint32_t off = VBITS == 4 ? 4 * (r >> 1) : 4 * (r >> 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = i < 4 ? 4 * j + i : 16 + 4 * j + (i - 4);
    const uint8_t *row = vc + key * VROW + off;
    y[i][0] = *reinterpret_cast<const uint32_t *>(row);
    y[i][1] = *reinterpret_cast<const uint32_t *>(row + VROW / 2);
  }
}

// Byte selector of v_operand for code byte fb of the lane's piece (INT4:
// fb = 0, 1; INT2: 0): that byte of two keys' words to bits 0..7 and
// 16..23.
template <int VBITS>
__device__ inline uint32_t vcode_sel(int lane, int fb) {
  const int r = lane & 15;
  const uint32_t b = static_cast<uint32_t>(VBITS == 4 ? 2 * (r & 1) + fb : (r & 3));
  return b | 0x0c00u | ((4 + b) << 16) | 0x0c000000u;
}

// Tile dt's operand from the code words: word w holds keys of slots 2w,
// 2w+1, each as the fp16 subnormal of its code field (dim 4r + f of the
// tile's half h, f = dt % 4) at bit p: odd f sits at p = P1, like the odd
// rows of unpack_v_raw.  sel[fb]: vcode_sel.
template <int VBITS>
__device__ inline f16x8 v_operand(const Ctx &c, const uint32_t (&y)[8][2], const uint32_t (&sel)[2], int dt) {
  const int h = dt >> 2, f = dt & 3;
  const uint32_t sl = sel[VBITS == 4 ? (f >> 1) : 0];
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t x = __builtin_amdgcn_perm(y[2 * e + 1][h], y[2 * e][h], sl);
    if (VBITS == 2 && f >= 2) x >>= 4;
    w[e] = x & ((f & 1) ? c.vmask1 : c.vmask0);
  }
  return __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// Key operands as raw codes (staged caches, at most two groups per row).
// The score of a cached key is split by quantisation group,
//   s = sum_g D_g (q_g . c_g) + sum_g z_g S_g - tau/24 sum_g D_g^2 ||q_g||^2
// (S_g the query's group sum), so the codes enter the score MFMAs as they
// are, one accumulator per group, each group's step multiplies its
// accumulator per score, and the zero points and the Taylor term
// ("量化鍵值偷走注意力…" (agents-report.net), §方法) come from the extra bf16
// step.  The keys are never rounded to fp16.  For that the MFMA k-steps
// must not mix groups: k-step i covers dims 32i .. 32i+31 (the lane's eight
// of them 32i + 8j .. +7, j = lane / 16), and a 16-bit word e of an operand
// holds dims e and e + 4 of the lane's eight.  The query and the current
// chunk's keys use the same order (kraw_dims).
//
// The lane's dims of k-step i: 32 i + 8 j + (e, e + 4) in word e.
__device__ inline uint32_t kraw_dim0(int i, int j) { return static_cast<uint32_t>(32 * i + 8 * j); }
// Unit of a raw code in its fp16 field, and so of the code products: INT4
// codes sit at bits 0..3 (c 2^-24), INT2 codes at bits 8..9 (c 2^-16: one
// byte permute and a mask per two codes, see stage_k_raw).
template <int KBITS>
constexpr float kRawUnit = KBITS == 4 ? 0x1p-24f : 0x1p-16f;
// Eight bf16 values (one uint4, consecutive dims) to an fp16 operand in the
// (e, e + 4) word order, scaled by sc.
__device__ inline f16x8 kraw_pack(uint4 w, float sc) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t a = u[e >> 1], b = u[2 + (e >> 1)];
    o[e] = (e & 1) ? pack2h(hi_f(a) * sc, hi_f(b) * sc) : pack2h(lo_f(a) * sc, lo_f(b) * sc);
  }
  return __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// The lane's query operands in that order (query row r of the tile), q
// scaled by its own power of two 2^-eq; the extra step's slots on quarter
// j < NG carry group j: N_j = tau/24 ||q_j||^2 2^-eq as (hi, hi, lo, 0) (zero
// without the correction), then S_j = sum q 2^-eq as (hi, lo, hi, 0), both
// times kRawUnit, the unit of the code products (the scores' softmax scale
// is alpha / kRawUnit).
template <bool TAYLOR, int NG, int KBITS>
__device__ inline void load_query_kraw(const uint16_t *qptr, int lane, float tau, f16x8 (&q)[4], bf16x8 &qext,
                                       float &alpha, float &qun) {
  const int j = lane >> 4;
  uint4 qw[4];
  float nsum[NG], qsum[NG], qmax = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) nsum[g] = qsum[g] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qw[i] = *reinterpret_cast<const uint4 *>(qptr + kraw_dim0(i, j));
    const uint32_t u[4] = {qw[i].x, qw[i].y, qw[i].z, qw[i].w};
    const int g = (32 * i * NG) / D;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      nsum[g] += lo_f(u[e]) * lo_f(u[e]) + hi_f(u[e]) * hi_f(u[e]);
      qsum[g] += lo_f(u[e]) + hi_f(u[e]);
      qmax = fmaxf(qmax, fmaxf(fabsf(lo_f(u[e])), fabsf(hi_f(u[e]))));
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {  // over the four quarters
    nsum[g] += __shfl_xor(nsum[g], 16, 64);
    nsum[g] += __shfl_xor(nsum[g], 32, 64);
    qsum[g] += __shfl_xor(qsum[g], 16, 64);
    qsum[g] += __shfl_xor(qsum[g], 32, 64);
  }
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
  const int eq = scale_exponent(qmax);
  const float qs_scale = ldexpf(1.0f, -eq);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = kraw_pack(qw[i], qs_scale);
  qun = ldexpf(1.0f, eq);
  alpha = tau * kLog2e * qun;
  float ns = 0.f, ts = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    ns = j == g ? nsum[g] : ns;
    ts = j == g ? qsum[g] : ts;
  }
  const float n = TAYLOR ? ns * (tau / 24.0f) * qs_scale * kRawUnit<KBITS> : 0.f;
  const float nh = lo_f(pack2(n, 0.f)), nl = n - nh;
  const float t = ts * qs_scale * kRawUnit<KBITS>;
  const float th = lo_f(pack2(t, 0.f)), tl = t - th;
  uint4 x = make_uint4(pack2(nh, nh), pack2(nl, 0.f), pack2(th, tl), pack2(th, 0.f));
  if (j >= NG) x = make_uint4(0u, 0u, 0u, 0u);
  qext = __builtin_bit_cast(bf16x8, x);
}

// A cached block's key operands from the stage (codes at sk, steps at ks,
// zero points at kz): k[t][i] = the codes of key 16t + r at the lane's dims
// of k-step i as fp16 subnormals c kRawUnit (exact); kext[t] on quarter j < NG
// = group j's (-D^2 split hi, lo, hi; 0; z split into its bf16 truncation
// z_h twice and z - z_h; 0) for the key; dk[t][g][i] = D of key 16t + 4j + i
// in group g (the scores' layout).  The scores come out in units of kRawUnit.
template <bool TAYLOR, int KBITS, int NG, int MT>
__device__ inline void stage_k_raw(const Ctx &c, const uint8_t *sk, const uint8_t *ks, const uint8_t *kz, int lane,
                                   f16x8 (&k)[2][4], bf16x8 (&kext)[2], float (&dk)[2][NG][4]) {
  constexpr uint32_t KROW = D * KBITS / 8, ES = MT ? 2 : 4;
  const int r = lane & 15, j = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint8_t *row = sk + (16 * t + r) * KROW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x;
      if (KBITS == 4) {
        x = *reinterpret_cast<const uint32_t *>(row + kraw_dim0(i, j) / 2);
      } else {
        // the lane's 16-bit chunk (half j % 2 of the word): its low byte (codes
        // 0..3) to byte 1, its high byte (codes 4..7) to byte 3, so that code e
        // sits at bit 8 + 2e and code e + 4 at bit 24 + 2e
        const uint32_t w = *reinterpret_cast<const uint32_t *>(row + 8 * i + 4 * (j >> 1));
        const uint32_t b = 2u * static_cast<uint32_t>(j & 1);
        x = __builtin_amdgcn_perm(w, w, 0x0cu | (b << 8) | (0x0cu << 16) | ((b + 1) << 24));
      }
      uint32_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = (x >> (KBITS * e)) & (KBITS == 4 ? c.kmask : c.kmask << 8);
      k[t][i] = __builtin_bit_cast(f16x8, make_uint4(m[0], m[1], m[2], m[3]));
    }
    const int g = j < NG ? j : 0;
    const float d = lds_meta<MT>(ks + ((16 * t + r) * NG + g) * ES);
    const float z = lds_meta<MT>(kz + ((16 * t + r) * NG + g) * ES);
    // bf16 hi parts by truncation (exact bf16 values; the remainder is exact in fp32)
    const float sq = TAYLOR ? d * d : 0.f;
    const float hsq = __uint_as_float(__float_as_uint(sq) & 0xffff0000u);
    const float zh = __uint_as_float(__float_as_uint(z) & 0xffff0000u);
    uint4 x = make_uint4(pack2(-hsq, -(sq - hsq)), pack2(-hsq, 0.f), pack2(zh, zh), pack2(z - zh, 0.f));
    if (j >= NG) x = make_uint4(0u, 0u, 0u, 0u);
    kext[t] = __builtin_bit_cast(bf16x8, x);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int gg = 0; gg < NG; ++gg)
        dk[t][gg][i] = lds_meta<MT>(ks + ((16 * t + 4 * j + i) * NG + gg) * ES);
  }
}

// The same with values along the tokens: the operands of channel c =
// 16dq + NF byte + fl (fl: the field within the byte) come from the staged
// token group, the same for the four keys.
template <int VBITS>
__device__ inline void unpack_v_tok(const Ctx &c, int lane, const Fetch &f, const float *Gv, uint16_t *Vt) {
  constexpr int NF = 8 / VBITS;
  const int kq = lane & 7, dq = lane >> 3;
  const int slot = vslot4(kq);
  float dc[16], zc[16];
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 a = *reinterpret_cast<const float4 *>(Gv + 16 * dq + e);
    const float4 b = *reinterpret_cast<const float4 *>(Gv + D + 16 * dq + e);
    dc[e] = a.x; dc[e + 1] = a.y; dc[e + 2] = a.z; dc[e + 3] = a.w;
    zc[e] = b.x; zc[e + 1] = b.y; zc[e + 2] = b.z; zc[e + 3] = b.w;
  }
  auto field = [&](uint32_t r, int k, int e) {  // both keys of r at channel e, field k (0: p = 0, 1: p = P1)
    const uint32_t m = (r & (k ? c.vmask1 : c.vmask0)) | 0x64006400u;
    const f16x2 h = __builtin_bit_cast(f16x2, m);
    return pair_h(dequant_h(static_cast<float>(h.x), dc[e], zc[e]), dequant_h(static_cast<float>(h.y), dc[e], zc[e]));
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
  uint4 k[2][4];     // keys 16t + r, d = 32j + 8s .. +7
  uint32_t v[4][8];  // keys 4kq+i, bf16 pairs of d = 16dq + 2e, +1
};
template <bool KRAW = false>
__device__ inline void load_current(const Ctx &c, int k0, int lane, Cur &x, float &kb, float &vb) {
  const int last = c.ncur - 1;
  kb = vb = 0.f;
  {
    const int r = lane & 15, j = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t row = static_cast<uint32_t>(k0 + 16 * t + r <= last ? k0 + 16 * t + r : last);
      const uint16_t *ks = c.k_cur + row * D;
#pragma unroll
      for (int s = 0; s < 4; ++s) {  // KRAW: the dims of k-step s in kraw_dim0's order
        x.k[t][s] = *reinterpret_cast<const uint4 *>(ks + (KRAW ? kraw_dim0(s, j) : 32u * j + 8u * s));
        const uint32_t u[4] = {x.k[t][s].x, x.k[t][s].y, x.k[t][s].z, x.k[t][s].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) kb = fmaxf(kb, fmaxf(fabsf(lo_f(u[e])), fabsf(hi_f(u[e]))));
      }
    }
  }
  {
    const int kq = lane & 7, dq = lane >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row = static_cast<uint32_t>(k0 + 4 * kq + i <= last ? k0 + 4 * kq + i : last);
      const uint4 *vs = reinterpret_cast<const uint4 *>(c.v_cur + (row * D + 16u * dq));
      const uint4 y0 = vs[0], y1 = vs[1];
      x.v[i][0] = y0.x; x.v[i][1] = y0.y; x.v[i][2] = y0.z; x.v[i][3] = y0.w;
      x.v[i][4] = y1.x; x.v[i][5] = y1.y; x.v[i][6] = y1.z; x.v[i][7] = y1.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) vb = fmaxf(vb, fmaxf(fabsf(lo_f(x.v[i][e])), fabsf(hi_f(x.v[i][e]))));
    }
  }
}

// Keys to MFMA operand registers (no correction) and values to the V^T
// tile, both rescaled to fp16.
template <bool KRAW = false>
__device__ inline void unpack_current(int lane, const Cur &x, float kscale, float vsc, f16x8 (&k)[2][4],
                                      uint16_t *Vt) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (KRAW) {
        k[t][s] = kraw_pack(x.k[t][s], kscale);
        continue;
      }
      const uint32_t u[4] = {x.k[t][s].x, x.k[t][s].y, x.k[t][s].z, x.k[t][s].w};
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack2h(lo_f(u[e]) * kscale, hi_f(u[e]) * kscale);
      k[t][s] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  const int kq = lane & 7, dq = lane >> 3;
  const int slot = vslot4(kq);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + 2 * e, slot)) =
        make_uint2(pack2h(lo_f(x.v[0][e]) * vsc, lo_f(x.v[1][e]) * vsc), pack2h(lo_f(x.v[2][e]) * vsc, lo_f(x.v[3][e]) * vsc));
    *reinterpret_cast<uint2 *>(Vt + vts(16 * dq + 2 * e + 1, slot)) =
        make_uint2(pack2h(hi_f(x.v[0][e]) * vsc, hi_f(x.v[1][e]) * vsc), pack2h(hi_f(x.v[2][e]) * vsc, hi_f(x.v[3][e]) * vsc));
  }
}

// The lane's query operands (query row r of the tile, dims 32j + 8s .. +7 in
// q[s]): the row scaled by its own power of two 2^-eq (largest |q| to
// [2^14, 2^15)), the softmax scale of the resulting scores (alpha = tau
// log2(e) 2^eq for keys not yet scaled), and the extra step's slots 8j ..
// 8j+7 on the first quarter of each group: N_g = tau/24 ||q_g||^2 2^-eq as
// (hi, hi, lo, 0) split into bf16 (zero without the correction), then the
// group sum S_g = sum_{c in g} q_c 2^-eq as (hi, lo, 0, 0) with centring;
// qun = 2^eq.
template <bool TAYLOR, int NG>
__device__ inline void load_query(const uint16_t *qptr, int lane, float tau, f16x8 (&q)[4], bf16x8 &qext,
                                  float &alpha, float &qun) {
  const int j = lane >> 4;
  uint4 qw[4];
  float nsum = 0.f, qsum = 0.f, qmax = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qw[s] = *reinterpret_cast<const uint4 *>(qptr + 32 * j + 8 * s);
    const uint32_t u[4] = {qw[s].x, qw[s].y, qw[s].z, qw[s].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      nsum += lo_f(u[e]) * lo_f(u[e]) + hi_f(u[e]) * hi_f(u[e]);
      qsum += lo_f(u[e]) + hi_f(u[e]);
      qmax = fmaxf(qmax, fmaxf(fabsf(lo_f(u[e])), fabsf(hi_f(u[e]))));
    }
  }
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
  // group sums: one quarter per group (4 groups), two (2), four (1)
  if (NG <= 2) {
    nsum += __shfl_xor(nsum, 16, 64);
    qsum += __shfl_xor(qsum, 16, 64);
  }
  if (NG == 1) {
    nsum += __shfl_xor(nsum, 32, 64);
    qsum += __shfl_xor(qsum, 32, 64);
  }
  const int eq = scale_exponent(qmax);
  const float qs_scale = ldexpf(1.0f, -eq);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t u[4] = {qw[s].x, qw[s].y, qw[s].z, qw[s].w};
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack2h(lo_f(u[e]) * qs_scale, hi_f(u[e]) * qs_scale);
    q[s] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  qun = ldexpf(1.0f, eq);
  alpha = tau * kLog2e * qun;
  const float n = TAYLOR ? nsum * (tau / 24.0f) * qs_scale : 0.f;
  const float nh = lo_f(pack2(n, 0.f)), nl = n - nh;
  const float t = qsum * qs_scale;
  const float th = lo_f(pack2(t, 0.f)), tl = t - th;
  uint4 x = make_uint4(pack2(nh, nh), pack2(nl, 0.f), kCentre<NG> ? pack2(th, tl) : 0u, 0u);
  if (!group_owner<NG>(j)) x = make_uint4(0u, 0u, 0u, 0u);
  qext = __builtin_bit_cast(bf16x8, x);
}

struct Soft {
  f32x4 o[D / 16];
  f32x4 oz;  // raw-code values: the zero points' sums (rows: Zs rows), query r
  float m, l, alpha;
};

// Scores, softmax and value product of one block: K operand registers, the
// wave's V^T tile, the block's score scale alpha (scores are q.k 2^-(eq+ek))
// and value exponent ev.  count < BK marks a ragged block; CORR adds the
// correction steps.  CAUSAL: count is the lane's own (possibly <= 0), and a
// row may have seen no key yet (m = -inf).  ADD: the row's scores add sadd.
// VCODE: the V^T tile holds raw codes (unpack_v_raw), with the block's steps
// in Ds and zero points in Zs.
template <bool CORR, bool CAUSAL = false, bool ADD = false, bool VCODE = false, int NG = 1, bool PERM = false,
          int VREG = 0, bool KRAW = false>
__device__ inline void block_compute(const f16x8 (&k)[2][4], const bf16x8 (&kext)[2], const uint16_t *Vt,
                                     const f16x8 (&q)[4], bf16x8 qext, int count, float alpha, int ev, int lane,
                                     Soft &st, float sadd = 0.f, const uint16_t *Ds = nullptr,
                                     const uint16_t *Zs = nullptr, const Ctx *c = nullptr,
                                     const uint32_t (*vy)[8][2] = nullptr, const float *dk = nullptr) {
  const float fev = static_cast<float>(ev);
  const uint32_t vsel[2] = {VREG ? vcode_sel<VREG ? VREG : 4>(lane, 0) : 0u, VREG ? vcode_sel<VREG ? VREG : 4>(lane, 1) : 0u};
  const int r = lane & 15, j = lane >> 4;
  f32x4 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (KRAW) {  // raw codes: one accumulator per group, scaled per score by the keys' steps dk (t, g, element)
      f32x4 a[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) a[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = (32 * i * NG) / D;
        a[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k[t][i], q[i], a[g], 0, 0, 0);
      }
      s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kext[t], qext, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int g = 0; g < NG; ++g) s[t][e] = fmaf(dk[(t * NG + g) * 4 + e], a[g][e], s[t][e]);
      continue;
    }
    s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) s[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k[t][i], q[i], s[t], 0, 0, 0);
    if (CORR) s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kext[t], qext, s[t], 0, 0, 0);
    if (ADD) s[t] += sadd;
  }
  if (CAUSAL || count < BK) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * t + 4 * j + i >= count) s[t][i] = -INFINITY;
  }
  float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  mt = fmaf(xor32_max(xor16_max(mt)), alpha, fev);
  const bool grow = mt > st.m + kLazy;
  if (__any(grow)) {
    const float m_new = grow ? mt : st.m;
    const float sc = CAUSAL && !grow ? 1.f : exp2f(st.m - m_new);
    st.l *= sc;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st.o[dt] *= sc;
    if (VCODE) st.oz *= sc;
    st.m = m_new;
  }
  const float shift = fev - st.m;
  float e[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[t][i] = __builtin_amdgcn_exp2f(fmaf(s[t][i], alpha, shift));
      if (CAUSAL && s[t][i] == -INFINITY) e[t][i] = 0.f;  // shift is +inf while m = -inf
    }
  const f16x8 pk = __builtin_bit_cast(
      f16x8, make_uint4(pack2h(e[0][0], e[0][1]), pack2h(e[0][2], e[0][3]), pack2h(e[1][0], e[1][1]),
                        pack2h(e[1][2], e[1][3])));
  // O^T += V^T P^T: head-dim tile dt, the block's 32 keys in one k-step
  if (VCODE) {
    // The raw codes multiply p D, and nothing averages its rounding when a
    // row sees few keys (one cached key: the output is that key's value), so
    // p D is carried as fp16 hi + lo: hi = p D_hi rounded, lo = its exact
    // rounding error (one fp16 fma) plus p D_lo, with p the fp16 p of the row
    // sum and the zero points; two MFMAs per tile.
    st.l = fmaf(sum8h(pk, 0.f), ldexpf(1.0f, -ev), st.l);
    // group g's operand: the probabilities times the keys' steps (the slots
    // 8j .. 8j+7 of Ds row g, the same for the 16 lanes of a quarter)
    f16x8 pgh[NG], pgl[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const f16x8 dh = *reinterpret_cast<const f16x8 *>(Ds + 64 * g + 8 * j);
      const f16x8 dl = *reinterpret_cast<const f16x8 *>(Ds + 64 * g + 32 + 8 * j);
      pgh[g] = pk * dh;
      pgl[g] = __builtin_elementwise_fma(pk, dl, __builtin_elementwise_fma(pk, dh, -pgh[g]));
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f16x8 a;
      if (VREG)
        a = v_operand<VREG>(*c, *vy, vsel, dt);
      else
        a = *reinterpret_cast<const f16x8 *>(Vt + vts(vrow<PERM>(dt, r), 8 * j));
      const int g = (vrow<PERM>(dt, 0) * NG) / D;
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pgh[g], st.o[dt], 0, 0, 0);
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pgl[g], st.o[dt], 0, 0, 0);
    }
    const f16x8 za = *reinterpret_cast<const f16x8 *>(Zs + ZS * r + 8 * j);
    st.oz = __builtin_amdgcn_mfma_f32_16x16x32_f16(za, pk, st.oz, 0, 0, 0);
  } else {
    st.l = fmaf(sum8h(pk, 0.f), ldexpf(1.0f, -ev), st.l);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          *reinterpret_cast<const f16x8 *>(Vt + vts(vrow<PERM>(dt, r), 8 * j)), pk, st.o[dt], 0, 0, 0);
  }
}

// Raw-code values: the accumulators of the cached blocks back to the units
// of dequantised values, o = o_codes 2^(24-p) / kVcodeScale + the group's
// zero-point sum (p = P1 on odd head-dim rows), before the current chunk's
// blocks add to them.
template <int VBITS, int NG, bool PERM = false>
__device__ inline void vcode_finish(Soft &st, int lane) {
  constexpr int P1 = VBITS == 4 ? 4 : 2;
  const int r = lane & 15;
  float zs[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    // rows g (hi) and NG + g (lo) of the query's column: lane 16 (row / 4) + r, element row % 4
    const int hrow = g, lrow = NG + g;
    zs[g] = __shfl(st.oz[hrow & 3], 16 * (hrow >> 2) + r, 64) + __shfl(st.oz[lrow & 3], 16 * (lrow >> 2) + r, 64);
  }
  const float f0 = 16777216.0f / kVcodeScale, f1 = f0 * (1.0f / (1 << P1));
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)  // element i: dim vrow<PERM>(dt, 4 (lane / 16) + i); odd dims at 2^P1
      st.o[dt][i] = fmaf(st.o[dt][i], ((PERM ? dt : i) & 1) ? f1 : f0, zs[(vrow<PERM>(dt, 0) * NG) / D]);
}

// KTOK / VTOK: keys / values grouped along the tokens (p.group is then also
// their token group; NG counts the groups per row of a cache grouped along
// the head dimension).
template <int KBITS, int VBITS, bool TAYLOR, int NG, bool CAUSAL, bool PAGED, int MT, bool KTOK = false,
          bool VTOK = false>
__global__ __launch_bounds__(THREADS, 2) void attn_short16_kernel(AttnLaunch p, int64_t rows_per_kvhead,
                                                                  int32_t nsplit, float *ws) {
  constexpr bool TOK = KTOK || VTOK;
  constexpr bool VCODE = !VTOK;  // cached values as raw codes
  constexpr int TOK_BYTES = TOK ? WAVES * 2 * GM * 4 : 0;
  using SL = StageLayout<KBITS, VBITS, NG, MT>;
  constexpr int STAGE_BYTES = 2 * WAVES * SL::BYTES;  // two stages per wave
  // Caches with head-dimension groups, at most two per row and metadata rows
  // of whole 4-byte words (the range check of a 4-byte load that straddles
  // the segment's end zeroes the whole word) are staged and take raw-code
  // operands (PERM: value operands from registers on permuted head-dim rows;
  // KRAW: keys as raw codes).  Their V^T tiles (current chunk) and merge
  // buffer are used only after the cached blocks, so they share one array
  // with the stages (a barrier between the two uses).
  constexpr int ALIAS_BYTES = STAGE_BYTES > LDS_BYTES ? STAGE_BYTES : LDS_BYTES;
  constexpr bool PERM = !TOK && NG <= 2 && (NG * SL::ES) % 4 == 0 &&
                        WAVES * VCODE_HALVES * 2 + ALIAS_BYTES <= 80 * 1024;
  constexpr bool KRAW = PERM;
  constexpr int BASE_BYTES =
      PERM ? WAVES * VCODE_HALVES * 2 : LDS_BYTES + TOK_BYTES + (VCODE ? WAVES * VCODE_HALVES * 2 : 0);
  __shared__ __attribute__((aligned(16))) uint16_t L[BASE_BYTES / 2];
  // other head-dimension caches (four groups per row) stage where the stages
  // still leave room for two workgroups per CU
  constexpr bool STAGED = PERM || (!TOK && (NG * SL::ES) % 4 == 0 && BASE_BYTES + STAGE_BYTES <= 80 * 1024);
  __shared__ __attribute__((aligned(16))) uint8_t S[PERM ? ALIAS_BYTES : STAGED ? STAGE_BYTES : 16];
  uint16_t *const T = PERM ? reinterpret_cast<uint16_t *>(S) : L;  // V^T tiles and merge buffer

  const int tid = threadIdx.x;
  if (blockIdx.x >= p.app.wg0) {  // the chunk append's workgroups
    qdev::append_workgroup<MT>(p, blockIdx.x - p.app.wg0, tid, THREADS);
    return;
  }
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block loop control stays scalar
  const int r = lane & 15;

  // Workgroups are dealt to the 8 XCDs round-robin by id; renumber so that
  // consecutive ids (the splits of one KV head) share an XCD.
  const uint32_t nwg = static_cast<uint32_t>(p.app.wg0), wg = blockIdx.x;
  const uint32_t per = nwg >> 3, extra = nwg & 7, xcd = wg & 7, slotw = wg >> 3;
  const uint32_t lin = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + slotw;
  const int64_t split = lin % static_cast<uint32_t>(nsplit);
  const int64_t bkv = lin / static_cast<uint32_t>(nsplit);
  const int64_t b = bkv / p.Hkv, hk = bkv - b * p.Hkv;
  const int64_t gq = p.Hq / p.Hkv;

  // the lane's query row (every quarter and every wave holds the 16 rows)
  const bool row_ok = r < rows_per_kvhead;
  const int64_t rr = row_ok ? r : rows_per_kvhead - 1;
  const int64_t qrow = (b * p.Hq + hk * gq + rr / p.Nq) * p.Nq + rr % p.Nq;
  f16x8 q[4];
  bf16x8 qext;
  Soft st;
  float qun;
  if (KRAW)
    load_query_kraw<TAYLOR, NG, KBITS>(p.q + qrow * D, lane, p.tau, q, qext, st.alpha, qun);
  else
    load_query<TAYLOR, NG>(p.q + qrow * D, lane, p.tau, q, qext, st.alpha, qun);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.oz = f32x4{0.f, 0.f, 0.f, 0.f};
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
    // keys along the tokens: one metadata row of D per token group
    c.kc_scale = meta_adv<MT>(p.kc_scale, KTOK ? (hrow >> gshift) * D : hrow * NG);
    c.kc_zero = meta_adv<MT>(p.kc_zero, KTOK ? (hrow >> gshift) * D : hrow * NG);
    c.vc_scale = meta_adv<MT>(p.vc_scale, VTOK ? (hrow >> gshift) * D : hrow * NG);
    c.vc_zero = meta_adv<MT>(p.vc_zero, VTOK ? (hrow >> gshift) * D : hrow * NG);
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
  // largest limit of its rows
  const int climit = static_cast<int>(rr % p.Nq + p.Ncur - p.Nq + 1);
  if (CAUSAL) {
    const int64_t r1 = rows_per_kvhead - 1;
    const int64_t wlim = (r1 / p.Nq == 0 ? r1 % p.Nq : p.Nq - 1) + p.Ncur - p.Nq + 1;
    const int cb = nbc + static_cast<int>(wlim > 0 ? (wlim + BK - 1) / BK : 0);
    if (bend > cb) bend = cb;
  }
  uint16_t *Vt = T + wave * VT;
  float *Gm = reinterpret_cast<float *>(L + WAVES * VT) + wave * 2 * GM;  // token-group staging of K
  float *Gv = Gm + GM;                                                     // and of V
  uint16_t *Ds = (PERM ? L : L + (LDS_BYTES + TOK_BYTES) / 2) + wave * VCODE_HALVES;
  uint16_t *Zs = Ds + 2 * 4 * 32;
  if (VCODE) {  // rows 2 NG .. 15 of Zs stay zero (16 rows x 80 bytes: 80 chunks of 16)
    for (int ch = lane; ch < 16 * ZS / 8; ch += 64) *reinterpret_cast<uint4 *>(Zs + 8 * ch) = make_uint4(0u, 0u, 0u, 0u);
  }

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
  f16x8 kreg[2][4];
  bf16x8 kext[2] = {};
  Fetch f;
  // keys along the tokens: the query terms of the wave's current token group
  f16x8 qk[4];
  float sadd = 0.f, alpha_g = 0.f;
  int gcur = -1;
  if constexpr (STAGED) {
    uint8_t *const s0 = S + wave * SL::BYTES, *const s1 = S + (WAVES + wave) * SL::BYTES;
    // both stages start zeroed, so that a byte no load writes is a finite zero
    for (uint32_t o = static_cast<uint32_t>(lane) * 16; o < SL::BYTES; o += 1024) {
      *reinterpret_cast<uint4 *>(s0 + o) = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4 *>(s1 + o) = make_uint4(0u, 0u, 0u, 0u);
    }
    // every step issues one block's loads (an empty range past the wave's
    // last block), so a stage is ready once at most one block's loads are
    // outstanding
    // paged: pr is the block's pool row (a 32-key block lies in one page),
    // looked up a step before its loads are issued
    auto issue = [&](const uint8_t *stg, int bk, size_t pr) {
      const int k0 = bk * BK;
      const bool in = bk < cend;
      const uint32_t rows = static_cast<uint32_t>(PAGED ? min(c.nc - k0, BK) : c.nc - k0);
      stage_issue<KBITS, VBITS, NG, MT>(c, in ? (PAGED ? pr : static_cast<size_t>(k0)) : 0, in ? rows : 0u, stg,
                                        lane);
    };
    auto lookup = [&](int bk) -> size_t { return PAGED && bk < cend ? block_row<PAGED>(c, bk * BK) : 0; };
    issue(s0, blk, lookup(blk));
    issue(s1, blk + bstep, lookup(blk + bstep));
    size_t prn = lookup(blk + 2 * bstep);
    // one block from stage stg: read the lane's share, refill the stage with
    // the block two steps on, then unpack and multiply
    auto body = [&](const uint8_t *stg) {
      const int k0 = blk * BK;
      const int count = c.nc - k0 < BK ? c.nc - k0 : BK;
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(SL::LOADS) : "memory");
      stage_read<KBITS, VBITS, NG, MT, !PERM, !KRAW>(stg, lo, f);
      uint32_t vy[8][2];
      if (PERM) stage_read_vcodes<VBITS>(stg + SL::KC, lane, vy);
      float dk[2][NG][4];
      if (KRAW) stage_k_raw<TAYLOR, KBITS, NG, MT>(c, stg, stg + SL::KS, stg + SL::KZ, lane, kreg, kext, dk);
      issue(stg, blk + 2 * bstep, prn);
      prn = lookup(blk + 3 * bstep);
      if (!cache_bounds) sc.update(KRAW ? 0.f : k_bound<KBITS, NG>(f), v_bound<VBITS>(f), st.alpha);
      if (!KRAW) unpack_k_cached<TAYLOR, KBITS, NG>(c, lane, f, sc.kscale, kreg, kext);
      unpack_v_raw<VBITS, NG, !PERM>(c, lane, f, sc.vscale, Vt, Ds, Zs);
      block_compute<TAYLOR || kCentre<NG> || KRAW, false, false, true, NG, PERM, PERM ? VBITS : 0, KRAW>(
          kreg, kext, Vt, q, qext, count, KRAW ? st.alpha / kRawUnit<KBITS> : sc.alpha, sc.ev, lane, st, 0.f, Ds, Zs, &c, &vy,
          &dk[0][0][0]);
    };
    for (;;) {
      if (blk >= cend) break;
      body(s0);
      blk += bstep;
      if (blk >= cend) break;
      body(s1);
      blk += bstep;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load into LDS outlives the loop
    if (PERM) __syncthreads();  // every wave is done with its stages before any V^T tile reuses them
  }
  if (!STAGED && blk < cend)
    fetch_cached<KBITS, VBITS, NG, PAGED, MT, KTOK, VTOK>(c, blk * BK, lo, f, block_row<PAGED>(c, blk * BK), gshift,
                                                          true);
  // paged: the pool row of the next block to fetch, looked up one block ahead
  // so that its scalar load has completed when the fetch needs it
  size_t prn = PAGED && blk + bstep < cend ? block_row<PAGED>(c, (blk + bstep) * BK) : 0;
  for (; !STAGED && blk < cend; blk += bstep) {
    const int k0 = blk * BK;
    const int count = c.nc - k0 < BK ? c.nc - k0 : BK;
    const bool newg = TOK && (k0 >> gshift) != gcur;  // the block starts the wave's next token group
    // values along the tokens: their bound per token group, checked when one starts
    const float vb = VTOK ? (newg ? vtok_bound<VBITS, MT>(f) : 0.f) : v_bound<VBITS>(f);
    if (KTOK) {
      if (!cache_bounds) sc.update(0.f, vb, st.alpha);
      if (newg) ktok_group<TAYLOR, MT>(f, lane, Gm, q, p.tau, st.alpha, qun, qk, sadd, alpha_g);
      unpack_k_codes<KBITS>(c, f, kreg);
    } else {
      if (!cache_bounds) sc.update(k_bound<KBITS, NG>(f), vb, st.alpha);
      unpack_k_cached<TAYLOR, KBITS, NG>(c, lane, f, sc.kscale, kreg, kext);
    }
    if (VTOK) {
      if (newg) vtok_stage<VBITS, MT>(f, lane, sc.vscale, Gv);
      unpack_v_tok<VBITS>(c, lane, f, Gv, Vt);
    } else {
      unpack_v_raw<VBITS, NG>(c, lane, f, sc.vscale, Vt, Ds, Zs);
    }
    if (newg) gcur = k0 >> gshift;
    if (blk + bstep < cend) {
      const int kn = (blk + bstep) * BK;
      fetch_cached<KBITS, VBITS, NG, PAGED, MT, KTOK, VTOK>(c, kn, lo, f, prn, gshift,
                                                            (kn >> gshift) != (k0 >> gshift));
    }
    if (KTOK)
      block_compute<false, false, true, VCODE, NG>(kreg, kext, Vt, qk, qext, count, alpha_g, sc.ev, lane, st, sadd,
                                                   Ds, Zs);
    else
      block_compute<TAYLOR || kCentre<NG>, false, false, VCODE, NG>(kreg, kext, Vt, q, qext, count, sc.alpha, sc.ev,
                                                                      lane, st, 0.f, Ds, Zs);
    if (PAGED && blk + 2 * bstep < cend) prn = block_row<PAGED>(c, (blk + 2 * bstep) * BK);
  }
  if (VCODE) vcode_finish<VBITS, NG, PERM>(st, lane);
  for (; blk < wend; blk += bstep) {
    const int k0 = (blk - nbc) * BK;
    int count = c.ncur - k0 < BK ? c.ncur - k0 : BK;
    if (CAUSAL) count = min(count, climit - k0);
    Cur x;
    float kb, vb;
    load_current<KRAW>(c, k0, lane, x, kb, vb);
    sc.update(kb, vb, st.alpha);
    unpack_current<KRAW>(lane, x, sc.kscale, sc.vscale, kreg, Vt);
    block_compute<false, CAUSAL, false, false, 1, PERM>(kreg, kext, Vt, q, qext, count, sc.alpha, sc.ev, lane, st);
  }

  // ---- merge the 4 waves (log-sum-exp), then the split partial or output ----
  float l_tot = st.l + __shfl_xor(st.l, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  __syncthreads();  // every wave is done with its tiles
  float *Ob = reinterpret_cast<float *>(T) + wave * MERGE;
  float *ml = Ob + ROWS * OS;
  const int j = lane >> 4;
  if (PERM) {  // element i of tile dt: dim 64 (dt / 4) + 16 j + 4 i + dt % 4
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4 *>(Ob + r * OS + 64 * h + 16 * j + 4 * i) =
            make_float4(st.o[4 * h][i], st.o[4 * h + 1][i], st.o[4 * h + 2][i], st.o[4 * h + 3][i]);
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4 *>(Ob + r * OS + 16 * dt + 4 * j) =
          make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
  }
  if (j == 0) {
    ml[2 * r] = st.m;
    ml[2 * r + 1] = l_tot;
  }
  __syncthreads();
  {
    const int row = tid >> 4, d0 = (tid & 15) * 8;  // 16 rows x 16 chunks of 8
    if (row < rows_per_kvhead) {
      float mw[WAVES], m = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        mw[w] = reinterpret_cast<const float *>(T)[w * MERGE + ROWS * OS + 2 * row];
        m = fmaxf(m, mw[w]);
      }
      float acc[8], l = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float *base = reinterpret_cast<const float *>(T) + w * MERGE;
        const float fw = mw[w] == -INFINITY ? 0.f : exp2f(mw[w] - m);
        l += fw * base[ROWS * OS + 2 * row + 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += fw * base[row * OS + d0 + e];
      }
      const int64_t orow = (b * p.Hq + hk * gq + row / p.Nq) * p.Nq + row % p.Nq;
      if (nsplit > 1) {
        float *w = ws + (split * (p.B * p.Hq * p.Nq) + orow) * kPartialStride(D);
#pragma unroll
        for (int e = 0; e < 8; e += 4)
          *reinterpret_cast<float4 *>(w + d0 + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
        if ((tid & 15) == 0) {
          w[D] = m;
          w[D + 1] = l;
        }
      } else {
        const float inv = 1.0f / l;
        uint16_t *o = p.out + orow * D + d0;
        *reinterpret_cast<uint4 *>(o) = make_uint4(pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv),
                                                   pack2(acc[4] * inv, acc[5] * inv), pack2(acc[6] * inv, acc[7] * inv));
      }
    }
  }
}

template <int KB, int VB, int NG, bool KT, bool VT>
void launch_kernel_t(const AttnLaunch &p, hipStream_t stream, dim3 grid, int64_t rows, float *partials) {
  constexpr bool PG = KVQ_SHORT16_PAGED != 0;
  constexpr int MH = KVQ_SHORT16_META16;
  auto kernel = p.corr == KV_CORR_TAYLOR ? (p.causal ? attn_short16_kernel<KB, VB, true, NG, true, PG, MH, KT, VT>
                                                     : attn_short16_kernel<KB, VB, true, NG, false, PG, MH, KT, VT>)
                                         : (p.causal ? attn_short16_kernel<KB, VB, false, NG, true, PG, MH, KT, VT>
                                                     : attn_short16_kernel<KB, VB, false, NG, false, PG, MH, KT, VT>);
  kernel<<<grid, dim3(THREADS), 0, stream>>>(p, rows, p.splits, partials);
}

// The unit's instances: keys along the tokens (KVQ_SHORT16_KTOK), values
// along the tokens with keys either way (KVQ_SHORT16_VTOK), or neither.
template <int KB, int VB, int NG>
void launch_kernel(const AttnLaunch &p, hipStream_t stream, dim3 grid, int64_t rows, float *partials) {
  if constexpr (KVQ_SHORT16_VTOK != 0) {
    if (p.ktok)
      launch_kernel_t<KB, VB, NG, true, true>(p, stream, grid, rows, partials);
    else
      launch_kernel_t<KB, VB, NG, false, true>(p, stream, grid, rows, partials);
  } else {
    launch_kernel_t<KB, VB, NG, KVQ_SHORT16_KTOK != 0, false>(p, stream, grid, rows, partials);
  }
}

template <int KB, int VB>
hipError_t launch_bits(const AttnLaunch &p, hipStream_t stream) {
  const int64_t rows = p.Nq * (p.Hq / p.Hkv);
  const int64_t nrows = p.B * p.Hq * p.Nq;
  float *partials = static_cast<float *>(p.workspace);
  // attention workgroups, then those of the chunk append (about 64 rows of
  // K and of V each)
  AttnLaunch pa = p;
  pa.app.wg0 = static_cast<int64_t>(p.splits) * p.B * p.Hkv;
  const int64_t append_wgs = (p.B * p.Hkv * p.Ncur + 63) / 64;
  pa.app.wgs = p.app.on ? static_cast<int32_t>(append_wgs < 4096 ? append_wgs : 4096) : 0;
  const dim3 grid(static_cast<uint32_t>(pa.app.wg0 + pa.app.wgs));
  if (p.group == 128)
    launch_kernel<KB, VB, 1>(pa, stream, grid, rows, partials);
  else if (p.group == 64)
    launch_kernel<KB, VB, 2>(pa, stream, grid, rows, partials);
  else
    launch_kernel<KB, VB, 4>(pa, stream, grid, rows, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_combine(partials, p.out, nrows, p.splits, p.d, stream);
}

}  // namespace

#if KVQ_SHORT16_VTOK
#if KVQ_SHORT16_PAGED
hipError_t launch_attention_short16_vtok_paged(const AttnLaunch &p, hipStream_t stream) {
#else
hipError_t launch_attention_short16_vtok(const AttnLaunch &p, hipStream_t stream) {
#endif
#elif KVQ_SHORT16_KTOK
#if KVQ_SHORT16_PAGED && KVQ_SHORT16_META16 == 2
hipError_t launch_attention_short16_ktok_mb16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_PAGED && KVQ_SHORT16_META16
hipError_t launch_attention_short16_ktok_m16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_PAGED
hipError_t launch_attention_short16_ktok_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_META16 == 2
hipError_t launch_attention_short16_ktok_mb16(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_META16
hipError_t launch_attention_short16_ktok_m16(const AttnLaunch &p, hipStream_t stream) {
#else
hipError_t launch_attention_short16_ktok(const AttnLaunch &p, hipStream_t stream) {
#endif
#elif KVQ_SHORT16_PAGED && KVQ_SHORT16_META16 == 2
hipError_t launch_attention_short16_mb16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_META16 == 2
hipError_t launch_attention_short16_mb16(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_PAGED && KVQ_SHORT16_META16
hipError_t launch_attention_short16_m16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_PAGED
hipError_t launch_attention_short16_paged(const AttnLaunch &p, hipStream_t stream) {
#elif KVQ_SHORT16_META16
hipError_t launch_attention_short16_m16(const AttnLaunch &p, hipStream_t stream) {
#else
hipError_t launch_attention_short16(const AttnLaunch &p, hipStream_t stream) {
#endif
  const int kb = p.Nc > 0 ? p.kbits : 2, vb = p.Nc > 0 ? p.vbits : 2;
  if (kb == 2 && vb == 2) return launch_bits<2, 2>(p, stream);
  if (kb == 2 && vb == 4) return launch_bits<2, 4>(p, stream);
  if (kb == 4 && vb == 2) return launch_bits<4, 2>(p, stream);
  return launch_bits<4, 4>(p, stream);
}

#if !KVQ_SHORT16_PAGED && !KVQ_SHORT16_META16 && !KVQ_SHORT16_KTOK && !KVQ_SHORT16_VTOK
// Caches grouped along the tokens: d = 128, correction off or Taylor, at most
// 16 query rows per KV head, (paged) pages that hold whole 32-key blocks,
// and with values along the tokens fp32 metadata.
bool short16_tok_supported(int32_t d, int corr, bool ktok, bool vtok, int32_t page_size, int meta,
                           int64_t rows_per_kvhead) {
  return d == D && corr != KV_CORR_EXACT && (ktok || vtok) && rows_per_kvhead <= ROWS &&
         (page_size == 0 || page_size >= BK) && (!vtok || meta == kMetaF32);
}

hipError_t launch_attention_short16_tok(const AttnLaunch &p, hipStream_t stream) {
  const bool paged = p.layout.page_table != nullptr;
  if (p.vtok) return paged ? launch_attention_short16_vtok_paged(p, stream) : launch_attention_short16_vtok(p, stream);
  if (p.meta == kMetaBF16)
    return paged ? launch_attention_short16_ktok_mb16_paged(p, stream) : launch_attention_short16_ktok_mb16(p, stream);
  if (p.meta == kMetaF16)
    return paged ? launch_attention_short16_ktok_m16_paged(p, stream) : launch_attention_short16_ktok_m16(p, stream);
  return paged ? launch_attention_short16_ktok_paged(p, stream) : launch_attention_short16_ktok(p, stream);
}
#endif

}  // namespace kvq
