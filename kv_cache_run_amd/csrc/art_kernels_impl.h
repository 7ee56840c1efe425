// gfx950 kernels for ART paged decode attention (templates; instantiated in
// kern_<kernel>_<type>.hip).
//
// Method: "ART: Attention Run-time Termination for Efficient Large Language
// Model Decoding" (gist.science explainer), Technical Summary 2.1-2.4.
//
// Both kernels share one per-block datapath, entirely in registers:
//  * QK: v_mfma_f32_16x16x32_bf16 (fp8 K converted to bf16 exactly; f32 uses
//    v_mfma_f32_16x16x4_f32) with K tile rows as the A operand and the query
//    group as the B operand (one head per column);
//  * block softmax on the 16x16 score tile (row reductions with the gfx950
//    permlane swaps);
//  * PV: v_mfma_f32_16x16x4_f32 with V^T as the A operand and P as the B
//    operand.  Each lane supplies one element of each operand, so P is used
//    straight from the score registers (column = head, k = token) and V is
//    loaded with coalesced 16-byte loads in the A-operand layout; products and
//    sums are fp32.
//
//  * art_sched_kernel -- the terminating path, one launch.  Scanner
//    workgroups (one per stream = (sequence, kv-head), NWA waves) fold the
//    stream's blocks in visit order, C blocks per step: per-block partials
//    (m_b, l_b, a_b), then one wave per query head folds them, forms
//    O_t = A_t / L_t for every t of the chunk, reduces ‖O_t‖² and
//    ‖O_t - O_{t-1}‖² for all t at once (transposed butterfly) and evaluates
//    both statistics and the patience rule for all t in parallel (one lane per
//    t, bit masks).  A head that stops writes O_t and is frozen; the stream
//    stops fetching when every head of its group stopped.  Helper workgroups
//    compute the partials of chunks ahead of the scanners (see the
//    scheduler notes below); chunks nobody claimed are computed by the
//    scanner itself, with their KV loads issued one chunk ahead.
//
//  * full_split_kernel -- full attention (no detector).  Each workgroup owns
//    a contiguous slice of one stream's blocks; each wave keeps its own
//    online-softmax state with the next block's loads in flight; waves merge
//    through LDS; the last slice of a stream to finish merges the slices.
//
// Data layout (HBM): k_pages/v_pages [page][kv_head][B][D], the (page, kvh)
// tile contiguous, so one block of one stream is B*D*es contiguous bytes.
//
// Lane layouts inside a wave (64 lanes, q = lane >> 4, c = lane & 15):
//  * K (QK A operand): 16 B of token row c of each 16-row tile at byte
//    q * 16 + 64 * i; the q operand uses the same byte -> d map.
//  * Scores / P: lane holds head c, tokens 16 t + 4 q + r (r = 0..3).
//  * V (PV A operand): lane holds, for each row 16 t + 4 q + r, the DT = D/16
//    elements d = DT * c .. DT * c + DT - 1 (R/16 contiguous bytes).
//  * PV accumulator O^T: lane holds head c, d = DT * (4 q + i) + dt for
//    i = 0..3, dt = 0..DT-1, i.e. the 4*DT consecutive d from 4*DT*q.
#pragma once
#include <math.h>

#include <type_traits>

#include "art_internal.h"

namespace art {
namespace kern {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr float NEG_INF = -__builtin_inff();
constexpr int NW = 4;        // waves per workgroup, full-attention kernel
constexpr int WG = 64 * NW;  // threads per workgroup, full-attention kernel
#ifndef FULL_PREFETCH
#define FULL_PREFETCH 2  // blocks in the full kernel's register ring
#endif

template <int KV> struct ElemSize;
template <> struct ElemSize<KV_F32> { static constexpr int v = 4; };
template <> struct ElemSize<KV_BF16> { static constexpr int v = 2; };
template <> struct ElemSize<KV_FP8> { static constexpr int v = 1; };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int KV_, int D_, int B_, int GM_>
struct Cfg {
  static constexpr int KV = KV_, D = D_, B = B_, GM = GM_;
  static constexpr int ES = ElemSize<KV>::v;
  static constexpr int R = D * ES;                    // bytes per token row
  static constexpr int NKL = R / 64;                  // 16-B K chunks per lane per 16-row tile
  static constexpr int T = B / 16;                    // 16-row tiles per block
  static constexpr int DT = D / 16;                   // V elements per lane per row (PV d-tiles)
  static constexpr int VBL = R / 16;                  // V bytes per lane per row
  static constexpr int VWD = VBL / 4;                 // V dwords per lane per row
  static constexpr int QF = KV == KV_FP8 ? 2 * NKL : NKL;  // 16-B q fragments
  // ART chunk: C blocks (8, fewer when the per-block partials [C][GM][D]
  // fp32 would pass 32 KiB)
  static constexpr int C = art_chunk_blocks(GM, D);
  static constexpr int NS = 4;                        // scanner: scan waves
  static constexpr int NBW = C;                       // scanner: block waves (one block of each chunk)
  static constexpr int NWA = NS + NBW;                // waves per workgroup, ART kernel
  static constexpr int BPB = 1;                       // blocks per block wave per chunk
  static constexpr int HPS = (GM + NS - 1) / NS;      // scanner: query heads per scan wave
  static constexpr int HWV = C;                       // helper: waves computing blocks (one each)
  // register ring depth of a block wave (chunks held): two while the ring
  // fits its VGPR budget (96 per lane, less for 8-head groups, fp8
  // conversion and 32-token blocks, whose math needs more registers), else
  // one.  (A third chunk in flight was measured: no faster on one CU, whose
  // steps are bound by the VALU/MFMA work, and a longer start.)
  static constexpr int TILE_VGPRS = 2 * B * R / 256;
  static constexpr int RING_BUDGET = 96 - (GM > 4 ? 32 : 0) - (KV == KV_FP8 ? 32 : 0) - (B == 32 ? 32 : 0);
  static constexpr int PFD = cmax(1, cmin(2, RING_BUDGET / TILE_VGPRS));
  // the farthest chunk a block wave issues at step c is c + IA
  static constexpr int IA = PFD == 3 ? 3 : 2;
  static constexpr int DPL = D / 64;                  // d per lane in the scan
  static constexpr int SH = 6 - ilog2(2 * C);         // stat reduction: lane >> SH = value index
  static constexpr int SLOT_A = C * GM * D;           // partials of one chunk: a[C][GM][D], m[C][GM], l[C][GM]
  static constexpr int SLOT = art_slot_floats(GM, D);
  // PV on v_mfma_f32_4x4x1_16b_f32 for query groups of up to 8 heads:
  // V in a lane-owns-d layout (each 256-B load covers RPL token rows, LPR
  // lanes per row, EPL consecutive d per lane), P broadcast per head from LDS.
  static constexpr bool PV4 = GM <= 8;
  static constexpr int RPL = R >= 256 ? 1 : 256 / R;  // token rows per V load
  static constexpr int BPL = R >= 256 ? R / 64 : 4;   // V bytes per lane per load
  static constexpr int LPR = 64 / RPL;                // lanes per token row
  static constexpr int NLD = B / RPL;                 // V loads per block
  static constexpr int VW = BPL / 4;                  // dwords per lane per load
  static constexpr int EPL = BPL / ES;                // d per lane per load
  static constexpr int HG = PV4 ? GM / 4 : 1;         // groups of 4 heads
  static constexpr int CH = EPL >= 4 ? 1 : 2;         // independent accumulator chains
  static constexpr int VN = B * R / 256;              // V dwords per lane per block (either layout)
  static constexpr int NACC = PV4 ? HG * CH * EPL : DT;
  // Full attention with fp8 V: P V on v_mfma_f32_16x16x16_bf16 instead of
  // the fp32 4x4x1 product (fp8 values are exact in bf16; P goes in as two
  // bf16 parts, hi + lo, so the products keep about 16 bits of P), with V
  // loaded four token rows per lane and transposed in registers.
  static constexpr bool PVB = KV == KV_FP8 && PV4 && D == 128;
  static constexpr int NACCF = PVB ? D / 16 : NACC;   // accumulators of the full-attention kernel
  static_assert(BPB * NBW == C && HWV <= NWA, "one block wave per block of a chunk");
  static_assert(!PV4 || NLD % 4 == 0, "P is read four tokens at a time");
  static_assert(2 * C <= 64, "stat reduction holds at most 64 values");
  static_assert(VWD >= 1, "a lane reads at least one dword of each V row");
};

template <class Cf>
struct BlockRegs {
  uint4 k[Cf::T][Cf::NKL];
  uint32_t v[Cf::VN];  // PV4: [NLD][VW]; otherwise [T][4][VWD]
};

// PV accumulator: PV4: [HG][CH][EPL] tiles, lane l holds O[4hg + r][d(l, e)]
// in component r; otherwise the 16x16 O^T tiles (lane = head column).
template <class Cf>
struct PvAcc {
  f32x4 a[Cf::NACC];
};

// ---------------------------------------------------------------------------
// Cross-lane primitives (VALU only: DPP and the gfx950 permlane swaps)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __uint_as_float(x); }

constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane ^ 7 within each 8
constexpr int DPP_ROW_MIRROR = 0x140;   // lane ^ 15 within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bitsf(__builtin_amdgcn_update_dpp(0u, fbits(x), CTRL, 0xF, 0xF, true));
}

// v_permlane32_swap: lanes 32..63 of a <-> lanes 0..31 of b.
__device__ __forceinline__ void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(fbits(a), fbits(b), false, false);
  a = bitsf(r[0]);
  b = bitsf(r[1]);
}
// v_permlane16_swap: odd 16-lane rows of a <-> even 16-lane rows of b.
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(fbits(a), fbits(b), false, false);
  a = bitsf(r[0]);
  b = bitsf(r[1]);
}

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_max(float x) {
  float y = x;
  swap32(x, y);
  x = fmaxf(x, y);
  y = x;
  swap16(x, y);
  return fmaxf(x, y);
}
__device__ __forceinline__ float rows_sum(float x) {
  float y = x;
  swap32(x, y);
  x += y;
  y = x;
  swap16(x, y);
  return x + y;
}
__device__ __forceinline__ float xor32_sum(float x) {
  float y = x;
  swap32(x, y);
  return x + y;
}
__device__ __forceinline__ float xor16_sum(float x) {
  float y = x;
  swap16(x, y);
  return x + y;
}

// One transposed-butterfly stage inside a 16-lane row: lanes with `up` keep
// the upper half of the live values, the partner lane (given by CTRL) the lower.
template <int CTRL, int HALF, int K>
__device__ __forceinline__ void xstage(float (&v)[K], bool up) {
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float send = up ? v[i] : v[i + HALF];
    const float keep = up ? v[i + HALF] : v[i];
    v[i] = keep + dpp<CTRL>(send);
  }
}

// Transposed butterfly over 64 lanes: every lane returns the 64-lane sum of
// v[lane >> (6 - log2 K)].  Pairings per stage: l^32, l^16 (permlane swaps),
// l^15, l^7 (row / half-row mirrors), l^2, l^1 (quad permutes); together they
// generate all 64 lanes, so each value is summed over every lane once.
template <int K>
__device__ __forceinline__ float xreduce(float (&v)[K], int lane) {
  constexpr int LOGK = ilog2(K);
  static_assert((1 << LOGK) == K && K <= 64, "K must be a power of two <= 64");
  if constexpr (LOGK >= 1) {
#pragma unroll
    for (int i = 0; i < K / 2; ++i) { swap32(v[i], v[i + K / 2]); v[i] += v[i + K / 2]; }
  } else {
    v[0] = xor32_sum(v[0]);
  }
  if constexpr (LOGK >= 2) {
#pragma unroll
    for (int i = 0; i < K / 4; ++i) { swap16(v[i], v[i + K / 4]); v[i] += v[i + K / 4]; }
  } else {
    v[0] = xor16_sum(v[0]);
  }
  if constexpr (LOGK >= 3) xstage<DPP_ROW_MIRROR, K / 8>(v, (lane & 8) != 0); else v[0] += dpp<DPP_ROW_MIRROR>(v[0]);
  if constexpr (LOGK >= 4) xstage<DPP_HALF_MIRROR, K / 16>(v, (lane & 4) != 0); else v[0] += dpp<DPP_HALF_MIRROR>(v[0]);
  if constexpr (LOGK >= 5) xstage<DPP_XOR2, K / 32>(v, (lane & 2) != 0); else v[0] += dpp<DPP_XOR2>(v[0]);
  if constexpr (LOGK >= 6) xstage<DPP_XOR1, K / 64>(v, (lane & 1) != 0); else v[0] += dpp<DPP_XOR1>(v[0]);
  return v[0];
}

// ---------------------------------------------------------------------------
// Per-block datapath
// ---------------------------------------------------------------------------

// 4 fp8 E4M3FN bytes -> 4 floats (exact; gfx950 converts the OCP format).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float (&o)[4]) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y;
}

// 4 fp8 bytes -> 2 dwords of packed bf16 (exact: E4M3 values fit bf16), one
// v_cvt_scalef32_pk_bf16_fp8 per pair with unit scale (checked bit for bit
// against converting through f32 and truncating, for every byte value).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// One KV load of 16, 8 or 4 bytes; NT: non-temporal (streamed past the
// caches, for data read exactly once).
template <bool NT>
__device__ __forceinline__ uint4 ld_kv16(const char* a) {
  if constexpr (NT) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
    return make_uint4(x.x, x.y, x.z, x.w);
  } else {
    return *reinterpret_cast<const uint4*>(a);
  }
}
template <bool NT>
__device__ __forceinline__ uint2 ld_kv8(const char* a) {
  if constexpr (NT) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a));
    return make_uint2(x.x, x.y);
  } else {
    return *reinterpret_cast<const uint2*>(a);
  }
}
template <bool NT>
__device__ __forceinline__ uint32_t ld_kv4(const char* a) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a));
  else
    return *reinterpret_cast<const uint32_t*>(a);
}

// Load one block: K in the QK A-operand layout, V in the PV operand layout.
// Every row of the tile is read (a tile always holds B rows), so the loads
// are a base address plus immediate offsets; when the block is the partial
// last block of a sequence, the V values of rows at or past nvalid are then
// zeroed, so that every V value fed to the PV product is finite (their P is
// exactly 0; K of those rows only feeds masked scores).
// NT: non-temporal loads.  The full-attention kernel reads every tile once
// and streams them (measured: 0.82 instead of 0.73 of HBM peak on 8 KiB
// tiles); the terminating kernels keep the default, since their clamped
// re-reads of a chunk past a stream's end are meant to hit in the cache.
// VQ: V in the full-attention kernel's fp8 layout for the bf16 P V product
// (Cf::PVB): lane (c, q) holds, in v[8 t + 2 r] and v[8 t + 2 r + 1], bytes
// 8 c .. 8 c + 7 of token row 16 t + 4 q + r (one 8-byte load per row: the
// 16 lanes of a q read a whole 128-byte row).
template <class Cf, bool NT = false, bool VQ = false>
__device__ __forceinline__ void load_block(BlockRegs<Cf>& r, const char* kt, const char* vt, int lane, int nvalid) {
  const int c = lane & 15;
  const int q = lane >> 4;
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i)
      r.k[t][i] = ld_kv16<NT>(kt + (size_t)(16 * t + c) * Cf::R + q * 16 + 64 * i);
  if constexpr (VQ) {
    static_assert(Cf::PVB && Cf::R == 128 && Cf::VN == 8 * Cf::T, "fp8 rows of 128 bytes");
    const char* src = vt + (size_t)(4 * q) * Cf::R + 8 * c;
#pragma unroll
    for (int t = 0; t < Cf::T; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint2 x = ld_kv8<NT>(src + (size_t)(16 * t + rr) * Cf::R);
        r.v[8 * t + 2 * rr] = x.x;
        r.v[8 * t + 2 * rr + 1] = x.y;
      }
    if (nvalid < Cf::B) {
#pragma unroll
      for (int t = 0; t < Cf::T; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (16 * t + 4 * q + rr >= nvalid) r.v[8 * t + 2 * rr] = r.v[8 * t + 2 * rr + 1] = 0u;
    }
  } else if constexpr (Cf::PV4) {
    // load u covers token rows u*RPL .. u*RPL+RPL-1; lane: row u*RPL + lane/LPR,
    // bytes (lane % LPR) * BPL .. +BPL of it
    const int rg = lane / Cf::LPR;
    const char* src = vt + (size_t)rg * Cf::R + (lane % Cf::LPR) * Cf::BPL;
#pragma unroll
    for (int u = 0; u < Cf::NLD; ++u) {
      if constexpr (Cf::VW == 1) {
        r.v[u] = ld_kv4<NT>(src + u * Cf::RPL * Cf::R);
      } else {
        const uint2 x = ld_kv8<NT>(src + u * Cf::RPL * Cf::R);
        r.v[2 * u] = x.x; r.v[2 * u + 1] = x.y;
      }
    }
    if (nvalid < Cf::B) {
#pragma unroll
      for (int u = 0; u < Cf::NLD; ++u)
#pragma unroll
        for (int j = 0; j < Cf::VW; ++j)
          if (u * Cf::RPL + rg >= nvalid) r.v[u * Cf::VW + j] = 0u;
    }
  } else {
    const char* src = vt + (size_t)(4 * q) * Cf::R + c * Cf::VBL;
#pragma unroll
    for (int t = 0; t < Cf::T; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const char* row = src + (size_t)(16 * t + rr) * Cf::R;
        uint32_t* dst = &r.v[(t * 4 + rr) * Cf::VWD];
        if constexpr (Cf::VWD == 1) {
          dst[0] = ld_kv4<NT>(row);
        } else if constexpr (Cf::VWD == 2) {
          const uint2 x = ld_kv8<NT>(row);
          dst[0] = x.x; dst[1] = x.y;
        } else {
#pragma unroll
          for (int h = 0; h < Cf::VWD / 4; ++h) {
            const uint4 x = ld_kv16<NT>(row + 16 * h);
            dst[4 * h + 0] = x.x; dst[4 * h + 1] = x.y; dst[4 * h + 2] = x.z; dst[4 * h + 3] = x.w;
          }
        }
      }
    if (nvalid < Cf::B) {
#pragma unroll
      for (int t = 0; t < Cf::T; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int j = 0; j < Cf::VWD; ++j)
            if (16 * t + 4 * q + rr >= nvalid) r.v[(t * 4 + rr) * Cf::VWD + j] = 0u;
    }
  }
}

// q fragments for the MFMA B operand: column (lane & 15) = head of the group.
template <class Cf>
__device__ __forceinline__ void load_q(const Params& p, int s, int kvh, int lane, uint4 (&qf)[Cf::QF]) {
  const int c = lane & 15;
#pragma unroll
  for (int i = 0; i < Cf::QF; ++i) qf[i] = make_uint4(0, 0, 0, 0);
  if (c >= p.g) return;
  const int hq = kvh * p.g + c;
  const int base = (lane >> 4) * 16;
  if constexpr (Cf::KV == KV_FP8) {
    const char* row = static_cast<const char*>(p.q) + ((size_t)s * p.hq + hq) * Cf::D * 2;
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qf[2 * i + hf] = *reinterpret_cast<const uint4*>(row + 2 * (base + 64 * i + 8 * hf));
  } else {
    const char* row = static_cast<const char*>(p.q) + ((size_t)s * p.hq + hq) * Cf::R;
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i) qf[i] = *reinterpret_cast<const uint4*>(row + base + 64 * i);
  }
}

template <class Cf>
__device__ __forceinline__ void qk_scores(const BlockRegs<Cf>& r, const uint4 (&qf)[Cf::QF], f32x4 (&S)[Cf::T]) {
#pragma unroll
  for (int t = 0; t < Cf::T; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i) {
      const uint4 kk = r.k[t][i];
      if constexpr (Cf::KV == KV_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk),
                                                      __builtin_bit_cast(bf16x8, qf[i]), acc, 0, 0, 0);
      } else if constexpr (Cf::KV == KV_FP8) {
        const uint2 a = fp8x4_to_bf16x4(kk.x), b = fp8x4_to_bf16x4(kk.y);
        const uint2 c = fp8x4_to_bf16x4(kk.z), d = fp8x4_to_bf16x4(kk.w);
        const uint4 lo = make_uint4(a.x, a.y, b.x, b.y);
        const uint4 hi = make_uint4(c.x, c.y, d.x, d.y);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo),
                                                      __builtin_bit_cast(bf16x8, qf[2 * i]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi),
                                                      __builtin_bit_cast(bf16x8, qf[2 * i + 1]), acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bitsf(kk.x), bitsf(qf[i].x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bitsf(kk.y), bitsf(qf[i].y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bitsf(kk.z), bitsf(qf[i].z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bitsf(kk.w), bitsf(qf[i].w), acc, 0, 0, 0);
      }
    }
    S[t] = acc;
  }
}

// Masked, log2-scaled scores and their block maximum (per head column).
template <class Cf>
__device__ __forceinline__ float block_scores(const f32x4 (&S)[Cf::T], int nvalid, float sl2, int lane,
                                              float (&x)[Cf::T][4]) {
  const int quad = lane >> 4;
  float mb = NEG_INF;
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = 16 * t + 4 * quad + r;
      x[t][r] = tok < nvalid ? S[t][r] * sl2 : NEG_INF;
      mb = fmaxf(mb, x[t][r]);
    }
  return rows_max(mb);
}

// A lane's V row segment (DT elements) as fp32 (exact for every storage type).
template <class Cf>
__device__ __forceinline__ void v_row(const uint32_t* w, float (&f)[Cf::DT]) {
  if constexpr (Cf::KV == KV_BF16) {
#pragma unroll
    for (int i = 0; i < Cf::VWD; ++i) {
      f[2 * i] = bitsf(w[i] << 16);
      f[2 * i + 1] = bitsf(w[i] & 0xffff0000u);
    }
  } else if constexpr (Cf::KV == KV_FP8) {
#pragma unroll
    for (int i = 0; i < Cf::VWD; ++i) {
      float o[4];
      fp8x4_to_f32(w[i], o);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[4 * i + e] = o[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < Cf::VWD; ++i) f[i] = bitsf(w[i]);
  }
}

// 16x16 layout (query groups of 9..16 heads): acc[dt] += V^T P over the
// block, the 16x16 tile of O^T whose rows are d = DT * m + dt (m = 0..15)
// and whose columns are the heads of the group.
template <class Cf>
__device__ __forceinline__ void pv_mfma(const BlockRegs<Cf>& r, const float (&pq)[Cf::T][4], f32x4 (&acc)[Cf::NACC]) {
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float vf[Cf::DT];
      v_row<Cf>(&r.v[(t * 4 + rr) * Cf::VWD], vf);
#pragma unroll
      for (int dt = 0; dt < Cf::DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[dt], pq[t][rr], acc[dt], 0, 0, 0);
    }
}

// The lane's V values of load u (4x4 layout), as fp32 (exact).
template <class Cf>
__device__ __forceinline__ void v4_decode(const BlockRegs<Cf>& r, int u, float (&vf)[Cf::EPL]) {
  if constexpr (Cf::KV == KV_BF16) {
#pragma unroll
    for (int j = 0; j < Cf::VW; ++j) {
      const uint32_t w = r.v[u * Cf::VW + j];
      vf[2 * j] = bitsf(w << 16);
      vf[2 * j + 1] = bitsf(w & 0xffff0000u);
    }
  } else if constexpr (Cf::KV == KV_FP8) {
    fp8x4_to_f32(r.v[u], vf);
  } else {
#pragma unroll
    for (int j = 0; j < Cf::VW; ++j) vf[j] = bitsf(r.v[u * Cf::VW + j]);
  }
}

// 4x4 layout: acc += P V over the block on v_mfma_f32_4x4x1_16b_f32.  Output
// lane l, component r: O[4hg + r][d] with d = (l % LPR) * EPL + e; the A
// operand (lane m) is P[4hg + m%4][token of lane m's V row], read from this
// wave's LDS row buffer pbuf [GM][RPL][NLD] (token u*RPL + rg at [rg][u]).
template <class Cf>
__device__ __forceinline__ void pv4_mfma(const BlockRegs<Cf>& r, const float (&pq)[Cf::T][4], float* pbuf, int lane,
                                         f32x4 (&acc)[Cf::NACC]) {
  const int c16 = lane & 15;
  const int q = lane >> 4;
  if (c16 < Cf::GM) {
    float* row = pbuf + c16 * Cf::B;
#pragma unroll
    for (int t = 0; t < Cf::T; ++t) {
      if constexpr (Cf::RPL == 1) {
        *reinterpret_cast<f32x4*>(row + 16 * t + 4 * q) = f32x4{pq[t][0], pq[t][1], pq[t][2], pq[t][3]};
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int k = 16 * t + 4 * q + rr;
          row[(k % Cf::RPL) * Cf::NLD + k / Cf::RPL] = pq[t][rr];
        }
      }
    }
  }
  const int rg = lane / Cf::LPR;
#pragma unroll
  for (int hg = 0; hg < Cf::HG; ++hg) {
    const float* src = pbuf + (4 * hg + (lane & 3)) * Cf::B + rg * Cf::NLD;
#pragma unroll
    for (int u4 = 0; u4 < Cf::NLD / 4; ++u4) {
      const f32x4 pp = *reinterpret_cast<const f32x4*>(src + 4 * u4);
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int u = 4 * u4 + uu;
        float vf[Cf::EPL];
        v4_decode<Cf>(r, u, vf);
#pragma unroll
        for (int e = 0; e < Cf::EPL; ++e) {
          f32x4& a = acc[(hg * Cf::CH + u % Cf::CH) * Cf::EPL + e];
          a = __builtin_amdgcn_mfma_f32_4x4x1f32(pp[uu], vf[e], a, 0, 0, 0);
        }
      }
    }
  }
}

template <class Cf>
__device__ __forceinline__ void pv_zero(f32x4 (&acc)[Cf::NACC]) {
#pragma unroll
  for (int i = 0; i < Cf::NACC; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <class Cf>
__device__ __forceinline__ void pv_block(const BlockRegs<Cf>& r, const float (&pq)[Cf::T][4], float* pbuf, int lane,
                                         f32x4 (&acc)[Cf::NACC]) {
  if constexpr (Cf::PV4) pv4_mfma<Cf>(r, pq, pbuf, lane, acc);
  else pv_mfma<Cf>(r, pq, acc);
}

// Multiply each head's accumulator by that head's factor; `al` is held by
// lane h for head h (lanes 0..15 of the score layout).
template <class Cf>
__device__ __forceinline__ void pv_rescale(f32x4 (&acc)[Cf::NACC], float al) {
  if constexpr (Cf::PV4) {
#pragma unroll
    for (int hg = 0; hg < Cf::HG; ++hg) {
      float sc[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sc[rr] = bitsf(__builtin_amdgcn_readlane(fbits(al), 4 * hg + rr));
#pragma unroll
      for (int i = 0; i < Cf::CH * Cf::EPL; ++i) {
        f32x4& a = acc[hg * Cf::CH * Cf::EPL + i];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) a[rr] *= sc[rr];
      }
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < Cf::DT; ++dt) acc[dt] *= al;
  }
}

// 4x4 layout: sum the chains into chain 0 and the token-row groups of a V
// load (lanes l, l + LPR, ...) so that every lane holds the totals.
template <class Cf>
__device__ __forceinline__ void pv_finish(f32x4 (&acc)[Cf::NACC]) {
  if constexpr (Cf::PV4) {
#pragma unroll
    for (int hg = 0; hg < Cf::HG; ++hg)
#pragma unroll
      for (int e = 0; e < Cf::EPL; ++e) {
        f32x4& a = acc[(hg * Cf::CH) * Cf::EPL + e];
        if constexpr (Cf::CH == 2) a += acc[(hg * Cf::CH + 1) * Cf::EPL + e];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          if constexpr (Cf::RPL == 2) a[rr] = xor32_sum(a[rr]);
          if constexpr (Cf::RPL == 4) a[rr] = rows_sum(a[rr]);
        }
      }
  }
}

// 16x16 layout: store a lane's O^T accumulator row (head c) as D-contiguous
// floats: dst points at [head][0]; the lane writes d = DT*(4q+i) + dt.
template <class Cf>
__device__ __forceinline__ void store_acc(float* dst, int lane, const f32x4 (&acc)[Cf::NACC], float scale) {
  const int q = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* row = dst + Cf::DT * (4 * q + i);
#pragma unroll
    for (int dt = 0; dt < Cf::DT; dt += 4) {
      f32x4 o = {acc[dt][i] * scale, acc[dt + 1][i] * scale, acc[dt + 2][i] * scale, acc[dt + 3][i] * scale};
      *reinterpret_cast<f32x4*>(row + dt) = o;
    }
  }
}

// Store the (finished) accumulator as dst[h][d] (head-major, D floats per
// head) for heads h < GM, scaled by `scale`.
template <class Cf>
__device__ __forceinline__ void pv_store(float* dst, int lane, const f32x4 (&acc)[Cf::NACC], float scale) {
  if constexpr (Cf::PV4) {
    if (lane < Cf::LPR) {
#pragma unroll
      for (int hg = 0; hg < Cf::HG; ++hg)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float* o = dst + (4 * hg + rr) * Cf::D + lane * Cf::EPL;
          float v[Cf::EPL];
#pragma unroll
          for (int e = 0; e < Cf::EPL; ++e) v[e] = acc[(hg * Cf::CH) * Cf::EPL + e][rr] * scale;
          if constexpr (Cf::EPL == 4) *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
          else if constexpr (Cf::EPL == 2) *reinterpret_cast<f32x2*>(o) = f32x2{v[0], v[1]};
          else o[0] = v[0];
        }
    }
  } else {
    const int c16 = lane & 15;
    if (c16 < Cf::GM) store_acc<Cf>(dst + c16 * Cf::D, lane, acc, scale);
  }
}

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlanef(float v, int l) { return bitsf(__builtin_amdgcn_readlane(fbits(v), l)); }

// Visit positions of sequence s: n_s = ceil(L / B), or the caller's visit
// count (a pruned cache: only the first visit_lens[s] entries of the order
// are visited) clamped to [0, n_s].
__device__ __forceinline__ int visit_count_b(const Params& p, int s, int L, int B) {
  const int n = (L + B - 1) / B;
  return p.visit_lens ? min(max(p.visit_lens[s], 0), n) : n;
}
template <int B>
__device__ __forceinline__ int visit_count(const Params& p, int s, int L) {
  return visit_count_b(p, s, L, B);
}

// ---------------------------------------------------------------------------
// Terminating path: one launch = per-stream scanners + helper workgroups
// ---------------------------------------------------------------------------
//
// Workgroups [0, streams) are scanners: scanner s owns stream s, holds the
// per-head ART state (running max, sum, numerator, previous output, pass
// count, sink flag) in registers and folds the stream's blocks strictly in
// visit order, one chunk of C blocks per step.  Workgroups past that are
// helpers: they claim chunks of still-running streams ahead of the scanner,
// turn them into per-block partials and publish them through a ring of slots
// in the workspace.  The scanner folds a helper's chunk from its slot; any
// chunk nobody claimed it computes itself, so it never waits for work that has
// not been started.  When a stream stops (every head of the group fired) its
// claim word is closed and helpers move to the other streams: CUs freed by
// early-terminated streams go to the ones still running.
//
// Control words live in the workspace and carry an epoch in their upper 32
// bits; a word written by an earlier call reads as its initial value, so no
// call has to clear them.  The last workgroup to finish advances the epoch.
//   claim[s]  = FIN | number of chunks claimed (initially 1: chunk 0 is the
//               scanner's); claims are compare-and-swap, in chunk order.
//   done[s]   = chunks the scanner has consumed (helpers may claim chunk c
//               only while c < done + window, window <= ring).
//   ready[s][c % ring] = c + 1 once chunk c's partials are in its slot.
// Partials and flags are written and read with device-scope (agent) relaxed
// atomics, which are coherent across the XCDs' L2s without a cache-wide
// writeback; a helper waits for its partial stores to complete
// (s_waitcnt vmcnt(0)) before it stores the ready flag.

typedef unsigned long long u64;
constexpr uint32_t CLAIM_FIN = 0x80000000u;

__device__ __forceinline__ u64 ld_dev(const u64* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev32(const uint32_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(u64* a, u64 v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev32(uint32_t* a, uint32_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// compare-and-swap; returns the value found (== expected iff it succeeded)
__device__ __forceinline__ u64 cas_dev(u64* a, u64 expected, u64 desired) {
  __hip_atomic_compare_exchange_strong(a, &expected, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return expected;
}
__device__ __forceinline__ u64 tag_word(uint32_t E, uint32_t v) { return ((u64)E << 32) | v; }
__device__ __forceinline__ uint32_t tag_val(u64 w, uint32_t E, uint32_t init) {
  return (uint32_t)(w >> 32) == E ? (uint32_t)w : init;
}
// the epoch of this call from the stored one (never 0, the value of a cleared word)
__device__ __forceinline__ uint32_t epoch_of(uint32_t stored) { return stored + 1u == 0u ? 1u : stored + 1u; }
// every memory operation this wave issued so far has completed
__device__ __forceinline__ void wait_all_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads, so loads issued ahead (the next
// chunk's KV tiles) stay in flight across it.  (__syncthreads() carries a
// workgroup-scope fence, which on gfx950 waits for every outstanding load.)
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Lanes of one 16-lane row shifted up by K (lane i reads lane i-K); the
// first K lanes of the row get `fill`.
template <int K>
__device__ __forceinline__ float row_shr(float x, float fill) {
  return bitsf(__builtin_amdgcn_update_dpp(fbits(fill), fbits(x), 0x110 + K, 0xF, 0xF, false));
}

// Issue the KV loads of this wave's NB blocks of one chunk (blocks
// wv*NB .. wv*NB+NB-1).  Slots past the chunk end re-read its last block (a
// cache hit), so the loads are unconditional.
template <class Cf, int NB>
__device__ __forceinline__ void issue_chunk_part(BlockRegs<Cf> (&regs)[NB], const Params& p, int kvh, int L,
                                                 int ob_lane, int pg_lane, int nt, int wv, int lane) {
  const size_t tile = (size_t)Cf::B * Cf::R;
  const char* kbase = static_cast<const char*>(p.k_pages);
  const char* vbase = static_cast<const char*>(p.v_pages);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = min(wv * NB + i, nt - 1);
    const int nvalid = min(Cf::B, L - readlane(ob_lane, b) * Cf::B);
    const size_t off = ((size_t)readlane(pg_lane, b) * p.hkv + kvh) * tile;
    load_block<Cf>(regs[i], kbase + off, vbase + off, lane, nvalid);
  }
}

// Block phase: each wave turns its NB blocks of the chunk into partials
// (m_b, l_b, a_b) for every head of the group, into `part` (slot layout:
// a[C][GM][D], then m[C][GM], then l[C][GM]).  Slots past the chunk end get
// neutral partials (m = -inf, l = 0, a = 0).
template <class Cf, int NB>
__device__ __forceinline__ void block_phase(const BlockRegs<Cf> (&regs)[NB], const uint4 (&qf)[Cf::QF],
                                            int ob_lane, float ks_lane, float vs_lane, int nt, int L, float qk_log2,
                                            int wv, int lane, float* part, float* pbuf) {
  const int c16 = lane & 15;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = wv * NB + i;
    float* pa = part + (size_t)b * Cf::GM * Cf::D;
    float* pm = part + Cf::SLOT_A + b * Cf::GM;
    float* pl = pm + Cf::C * Cf::GM;
    if (b < nt) {
      const int nvalid = min(Cf::B, L - readlane(ob_lane, b) * Cf::B);
      float ksc = 1.f, vsc = 1.f;
      if constexpr (Cf::KV == KV_FP8) { ksc = readlanef(ks_lane, b); vsc = readlanef(vs_lane, b); }
      f32x4 S[Cf::T];
      qk_scores<Cf>(regs[i], qf, S);
      float x[Cf::T][4];
      const float mb = block_scores<Cf>(S, nvalid, qk_log2 * ksc, lane, x);
      float ls = 0.f;
      float pq[Cf::T][4];
#pragma unroll
      for (int t = 0; t < Cf::T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(x[t][r] - mb);
          ls += e;
          pq[t][r] = e * vsc;
        }
      ls = rows_sum(ls);
      f32x4 acc[Cf::NACC];
      pv_zero<Cf>(acc);
      pv_block<Cf>(regs[i], pq, pbuf, lane, acc);
      pv_finish<Cf>(acc);
      pv_store<Cf>(pa, lane, acc, 1.f);
      if (c16 < Cf::GM && (lane >> 4) == 0) { pm[c16] = mb; pl[c16] = ls; }
    } else {
      if (c16 < Cf::GM && (lane >> 4) == 0) { pm[c16] = NEG_INF; pl[c16] = 0.f; }
      for (int e = lane; e < Cf::GM * Cf::D; e += 64) pa[e] = 0.f;
    }
  }
}

// One head's chunk input in registers: lane holds a[t][DPL*lane + j] and, for
// lane t < C, (m_t, l_t).
template <class Cf>
struct ChunkIn {
  float a[Cf::C][Cf::DPL];
  float m, l;
};

template <class Cf>
__device__ __forceinline__ void gather_lds(ChunkIn<Cf>& in, const float* part, int h, int lane) {
#pragma unroll
  for (int t = 0; t < Cf::C; ++t) {
    const float* src = part + ((size_t)t * Cf::GM + h) * Cf::D + Cf::DPL * lane;
    if constexpr (Cf::DPL == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(src);
      in.a[t][0] = v.x; in.a[t][1] = v.y;
    } else {
      in.a[t][0] = src[0];
    }
  }
  const int t = lane < Cf::C ? lane : 0;
  in.m = lane < Cf::C ? part[Cf::SLOT_A + t * Cf::GM + h] : NEG_INF;
  in.l = lane < Cf::C ? part[Cf::SLOT_A + Cf::C * Cf::GM + t * Cf::GM + h] : 0.f;
}

// The same from a ring slot in global memory, with device-scope loads.
template <class Cf>
__device__ __forceinline__ void gather_ring(ChunkIn<Cf>& in, const float* slot, int h, int lane) {
#pragma unroll
  for (int t = 0; t < Cf::C; ++t) {
    const float* src = slot + ((size_t)t * Cf::GM + h) * Cf::D + Cf::DPL * lane;
    if constexpr (Cf::DPL == 2) {
      const u64 v = ld_dev(reinterpret_cast<const u64*>(src));
      in.a[t][0] = bitsf((uint32_t)v); in.a[t][1] = bitsf((uint32_t)(v >> 32));
    } else {
      in.a[t][0] = bitsf(ld_dev32(reinterpret_cast<const uint32_t*>(src)));
    }
  }
  const int t = lane < Cf::C ? lane : 0;
  const float m = bitsf(ld_dev32(reinterpret_cast<const uint32_t*>(slot + Cf::SLOT_A + t * Cf::GM + h)));
  const float l = bitsf(ld_dev32(reinterpret_cast<const uint32_t*>(slot + Cf::SLOT_A + Cf::C * Cf::GM + t * Cf::GM + h)));
  in.m = lane < Cf::C ? m : NEG_INF;
  in.l = lane < Cf::C ? l : 0.f;
}

// Per-head state carried across chunks.
template <class Cf>
struct HeadCarry {
  float M, L, Np;
  int cnt;
  bool alive, sink;
  float A[Cf::DPL], Op[Cf::DPL];
};

// Fold one chunk into one head and run the detector on every position of it.
//  * The scalars of the fold are computed lane-parallel (lane t = position
//    t): running maxima by a prefix max, rescale factors, and the running sums
//    L_t by a prefix scan of the affine maps L -> al_t L + be_t l_t.
//  * The vector fold A_t = al_t A_{t-1} + be_t a_t, O_t = A_t / L_t and the
//    squared norms ‖O_t‖², ‖O_t - O_{t-1}‖² are per lane; the 2C squared norms
//    are reduced together by one transposed butterfly.
//  * Lane t then evaluates both statistics and the patience/sink rule.
// Returns true if the head fired in this chunk (it wrote out/stop).
template <class Cf>
__device__ __forceinline__ bool scan_head(HeadCarry<Cf>& hc, const ChunkIn<Cf>& in, int t0, int nt,
                                          unsigned long long sinkbits, const Params& p, int lane, float* out_row,
                                          int32_t* stop_ptr) {
  constexpr int C = Cf::C, DPL = Cf::DPL, SH = Cf::SH;
  const int slot = lane < C ? lane : C - 1;

  float mx = in.m;
  if constexpr (C > 1) mx = fmaxf(mx, row_shr<1>(mx, NEG_INF));
  if constexpr (C > 2) mx = fmaxf(mx, row_shr<2>(mx, NEG_INF));
  if constexpr (C > 4) mx = fmaxf(mx, row_shr<4>(mx, NEG_INF));
  mx = fmaxf(mx, hc.M);
  const float mprev = row_shr<1>(mx, hc.M);
  const float al = __builtin_amdgcn_exp2f(mprev - mx);
  const float be = __builtin_amdgcn_exp2f(in.m - mx);
  float fa = al, fb = be * in.l;
  if constexpr (C > 1) { const float pa = row_shr<1>(fa, 1.f), pb = row_shr<1>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  if constexpr (C > 2) { const float pa = row_shr<2>(fa, 1.f), pb = row_shr<2>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  if constexpr (C > 4) { const float pa = row_shr<4>(fa, 1.f), pb = row_shr<4>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  const float Lt = fmaf(fa, hc.L, fb);
  const float rl = __builtin_amdgcn_rcpf(Lt);  // 1 ulp; the statistics need ~1e-6

  float st[2 * C];
  float oo[C][DPL];
#pragma unroll
  for (int t = 0; t < C; ++t) {
    const float at = readlanef(al, t), bt = readlanef(be, t), rt = readlanef(rl, t);
    float nn = 0.f, ee = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      hc.A[j] = fmaf(at, hc.A[j], bt * in.a[t][j]);
      const float o = hc.A[j] * rt;
      const float df = o - hc.Op[j];
      const float op = DPL * lane + j < p.probe ? o : 0.f;  // coordinates outside the probe do not count
      const float dp = DPL * lane + j < p.probe ? df : 0.f;
      nn = fmaf(op, op, nn);
      ee = fmaf(dp, dp, ee);
      hc.Op[j] = o;
      oo[t][j] = o;
    }
    st[2 * t] = nn;
    st[2 * t + 1] = ee;
  }
  float nn_t = 0.f;
  bool ps = false;
  if (!p.skip_stats) {  // uniform: off only to measure what the statistics cost
  const float v0 = xreduce<2 * C>(st, lane);
  // lane (2t) << SH holds ‖O_t‖², lane (2t+1) << SH holds ‖O_t - O_{t-1}‖²;
  // gather them so that lane t < C evaluates position t.
  nn_t = __shfl(v0, (2 * slot) << SH);
  const float ee_t = __shfl(v0, (2 * slot + 1) << SH);
  float np_t = __shfl(v0, (2 * max(slot - 1, 0)) << SH);
  if (lane == 0) np_t = hc.Np;
  if (lane < nt && t0 + lane >= 1) {
    const float a = __builtin_amdgcn_sqrtf(nn_t);
    const float bn = __builtin_amdgcn_sqrtf(np_t);
    float dm, dd;
    if (a == 0.f && bn == 0.f) {
      dm = 0.f; dd = 0.f;
    } else if (bn == 0.f) {
      dm = __builtin_inff(); dd = 1.f;
    } else {
      const float df = a - bn;
      dm = fabsf(df) * __builtin_amdgcn_rcpf(bn);
      // 1 - cos = (‖O_t - O_{t-1}‖² - (‖O_t‖ - ‖O_{t-1}‖)²) / (2 ‖O_t‖ ‖O_{t-1}‖)
      dd = (a == 0.f) ? 1.f : fmaxf(0.f, (ee_t - df * df) * __builtin_amdgcn_rcpf(2.f * a * bn));
    }
    ps = (dm < p.eps_mag) && (dd < p.eps_dir);
  }
  }
  // patience rule for every position at once: lane t counts the passes in a
  // row that end at t (carrying the count from earlier chunks when every test
  // of this chunk up to t passed) and whether block 0 has been folded by t.
  const unsigned long long pass = __ballot(ps);
  const unsigned long long upto = (2ull << slot) - 1ull;
  const unsigned long long zeros = ~pass & upto;
  const int cnt_t = zeros == 0ull ? hc.cnt + slot + 1 : slot - (63 - __builtin_clzll(zeros));
  const bool sink_t = hc.sink || (sinkbits & upto) != 0ull;
  const unsigned long long fire = __ballot(lane < nt && cnt_t >= p.patience && sink_t);
  hc.M = readlanef(mx, C - 1);
  hc.L = readlanef(Lt, C - 1);
  if (fire != 0ull) {
    const int stop_t = __builtin_ctzll(fire);
    float ov[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) ov[j] = oo[0][j];
#pragma unroll
    for (int t = 1; t < C; ++t)
      if (stop_t == t)
#pragma unroll
        for (int j = 0; j < DPL; ++j) ov[j] = oo[t][j];
#pragma unroll
    for (int j = 0; j < DPL; ++j) out_row[DPL * lane + j] = ov[j];
    if (lane == 0) *stop_ptr = t0 + stop_t + 1;
    hc.alive = false;
    return true;
  }
  hc.cnt = readlane(cnt_t, nt - 1);
  hc.sink = readlane(sink_t ? 1 : 0, nt - 1) != 0;
  hc.Np = readlanef(nn_t, nt - 1);
  return false;
}

// Scheduler workspace views (laid out by the host).
struct Sched {
  uint32_t* ctrl;   // [0] stored epoch, [1] finished workgroups, [2] error flag
  u64* claim;       // [streams]
  u64* done;        // [streams]
  u64* ready;       // [streams][ring]
  float* ring;      // [streams][ring][slot_floats]
};

// Scanner of one stream.  Waves [0, NS) are scan waves (query heads
// w, w + NS, ...); waves [NS, NWA) are block waves.  Step c: the scan waves
// fold chunk c from LDS buffer c % 2 while the block waves turn chunk c+1
// into partials in buffer (c+1) % 2 (computing it, or copying a helper's slot)
// with chunk c+2's KV loads already in flight (register ring of two chunks).
// One LDS barrier per step.  KV loads are issued unconditionally (clamped
// to valid blocks when there is nothing to fetch), so the waits the compiler
// places for a chunk's data never include younger loads.
template <class Cf>
__device__ void art_scanner(const Params& p, int stream, uint32_t E, float* part2, float* pbuf, int* sh) {
  constexpr int C = Cf::C, NS = Cf::NS, BPB = Cf::BPB, HPS = Cf::HPS, DPL = Cf::DPL;
  constexpr int NT = 64 * Cf::NWA;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scanw = w < NS;
  const int bw = scanw ? 0 : w - NS;
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  const int g = p.g;
  const int L = p.seq_lens[s];
  const int n = visit_count<Cf::B>(p, s, L);
  const int nch = (n + C - 1) / C;
  const size_t head0 = (size_t)s * p.hq + (size_t)kvh * g;
  u64* claimw = p.sched_claim + stream;
  u64* donew = p.sched_done + stream;
  u64* readyw = p.sched_ready + (size_t)stream * p.ring;
  const float* ringb = p.sched_ring + (size_t)stream * p.ring * p.slot_floats;
  const bool helped = p.helpers > 0;
  const bool claimer = w == NS && lane == 0;  // block wave 0, lane 0: the stream's claims
  int* dec = sh + 16;                         // dec[k % 8]: 1 if chunk k is computed here (sh[0..15]: wave votes)

  if (n <= 0) {
    for (int i = threadIdx.x; i < g * Cf::D; i += NT) p.out[head0 * Cf::D + i] = 0.f;
    if (threadIdx.x < g) p.stop_block[head0 + threadIdx.x] = 0;
    if (threadIdx.x == 0) {
      if (helped) {
        u64 cw = ld_dev(claimw);
        for (int k = 0; k < 64; ++k) {
          const u64 r = cas_dev(claimw, cw, tag_word(E, CLAIM_FIN | (tag_val(cw, E, 1) & ~CLAIM_FIN)));
          if (r == cw) break;
          cw = r;
        }
      }
      if (p.blocks_fetched) p.blocks_fetched[stream] = 0;
    }
    return;
  }

  const int32_t* trow = p.block_table + (size_t)s * p.max_blocks;
  const int32_t* orow = p.block_order + (size_t)s * p.max_blocks;
  const int slot = lane < C ? lane : C - 1;

  // Order and page entries: scan wave 0 keeps two lane-held windows of 64
  // visit positions, [W, W+64) and [W+64, W+128), and at step c writes chunk
  // c+4's entries (lane = slot) into the LDS ring ent[(c+4) % 8]; the other
  // waves read a chunk's entries from there.  Window 1 is re-read when the
  // windows slide (its pages one step after its order entries).
  int* ent = sh + 32;  // [8][2][8]: order entry, page
  int W = 0, ob_w0 = 0, ob_w1 = 0, pg_w0 = 0, pg_w1 = 0;
  bool pg_w1_due = false;
  auto publish_entries = [&](int k) {  // scan wave 0: chunk k (clamped) into ent[k % 4]
    const int tc = min(k, nch - 1) * C;
    if (tc >= W + 64) {
      W += 64;
      ob_w0 = ob_w1;
      pg_w0 = pg_w1;
      ob_w1 = orow[min(W + 64 + lane, n - 1)];
      pg_w1_due = true;
    }
    const int idx = tc - W + slot;
    const int ob = __shfl(ob_w0, idx);
    const int pg = __shfl(pg_w0, idx);
    if (lane < C) { ent[(k & 7) * 16 + lane] = ob; ent[(k & 7) * 16 + 8 + lane] = pg; }
  };
  auto entries = [&](int k, int& ob, int& pg) {  // lane-held entries of chunk k
    ob = ent[(k & 7) * 16 + slot];
    pg = ent[(k & 7) * 16 + 8 + slot];
  };
  if (w == 0) {
    ob_w0 = orow[min(lane, n - 1)];
    ob_w1 = orow[min(64 + lane, n - 1)];
    pg_w0 = trow[ob_w0];
    pg_w1 = trow[ob_w1];
    publish_entries(0);
    publish_entries(1);
    publish_entries(2);
    publish_entries(3);
  }

  // claims (helpers only): chunk 0 is the scanner's; chunks 1 .. IA are
  // claimed before the first step, chunk k > IA at step k-IA-1 (attempted
  // one step earlier); dec[k % 8] = 1 when chunk k is computed here
  constexpr int IA = Cf::IA;
  u64 cw = 0, exp3 = 0, ret3 = 0;
  bool tried3 = false;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) dec[k] = 1;
  }
  if (claimer && helped) {
    cw = ld_dev(claimw);
    for (int k = 1; k <= IA && k < nch; ++k) {
      bool loc = false;
      if ((tag_val(cw, E, 1) & ~CLAIM_FIN) == (uint32_t)k) {
        const u64 r = cas_dev(claimw, cw, tag_word(E, k + 1));
        loc = r == cw;
        cw = loc ? tag_word(E, k + 1) : r;
      }
      dec[k] = loc ? 1 : 0;
    }
    if (IA + 1 < nch && (tag_val(cw, E, 1) & ~CLAIM_FIN) == (uint32_t)(IA + 1)) {
      exp3 = cw;
      ret3 = cas_dev(claimw, cw, tag_word(E, IA + 2));
      tried3 = true;
    }
  }
  lds_barrier();

  bool err = false;
  int c = 0;
  // end of a step: vote, barrier, common decision (every wave runs the same
  // number of barriers)
  auto end_step = [&](int alive_vote) {
    if (lane == 0) sh[w] = alive_vote | (err ? 2 : 0);
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int ww = 0; ww < Cf::NWA; ++ww) any |= sh[ww];
    if (any & 2) err = true;
    if (threadIdx.x == 0 && helped) st_dev(donew, tag_word(E, c + 1));
    return (any & 1) && !(any & 2) && c + 1 < nch;
  };

  if (scanw) {
    // ================= scan waves: fold chunk c from buffer c % 2 =================
    lds_barrier();  // the block waves' prologue
    HeadCarry<Cf> hc[HPS];
#pragma unroll
    for (int k = 0; k < HPS; ++k) {
      hc[k].M = NEG_INF; hc[k].L = 0.f; hc[k].Np = 0.f; hc[k].cnt = 0; hc[k].sink = false;
      hc[k].alive = (w + NS * k) < g;
#pragma unroll
      for (int j = 0; j < DPL; ++j) { hc[k].A[j] = 0.f; hc[k].Op[j] = 0.f; }
    }
    for (;; ++c) {
      const int t0 = c * C;
      const int nt = min(C, n - t0);
      const float* cur = part2 + (c & 1) * Cf::SLOT;
      int ob_c, pg_c;
      entries(c, ob_c, pg_c);
      const unsigned long long sinkbits = __ballot(lane < nt && ob_c == 0);
      if (w == 0) {
        if (pg_w1_due) { pg_w1 = trow[ob_w1]; pg_w1_due = false; }
        publish_entries(c + 4);
      }
      int a = 0;
#pragma unroll
      for (int k = 0; k < HPS; ++k) {
        const int h = w + NS * k;
        if (h < g && hc[k].alive) {
          ChunkIn<Cf> in;
          gather_lds<Cf>(in, cur, h, lane);
          scan_head<Cf>(hc[k], in, t0, nt, sinkbits, p, lane, p.out + (head0 + h) * Cf::D, p.stop_block + head0 + h);
        }
        if (hc[k].alive) a = 1;
      }
      if (!end_step(a)) break;
    }
    // heads that never stopped: the output after all n blocks
#pragma unroll
    for (int k = 0; k < HPS; ++k) {
      const int h = w + NS * k;
      if (h < g && hc[k].alive) {
        float* o = p.out + (head0 + h) * Cf::D;
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[DPL * lane + j] = err ? __builtin_nanf("") : hc[k].Op[j];
        if (lane == 0) p.stop_block[head0 + h] = err ? -1 : n;
      }
    }
  } else {
    // ================= block waves: chunk c+1 into buffer (c+1) % 2 =================
    constexpr int PFD = Cf::PFD;
    uint4 qf[Cf::QF];
    load_q<Cf>(p, s, kvh, lane, qf);
    // register ring: chunk k's tiles in slot k % PFD (one slot when PFD == 1)
    BlockRegs<Cf> r0[BPB], r1[BPB], r2[BPB];
    float ks0 = 1.f, vs0 = 1.f, ks1 = 1.f, vs1 = 1.f, ks2 = 1.f, vs2 = 1.f;
    // issue chunk k's loads for this block wave (k past the end re-reads the last chunk)
    auto issue = [&](int k, BlockRegs<Cf> (&rr)[BPB], float& ks, float& vs) {
      int ob, pg;
      entries(k, ob, pg);
      const int kc = min(k, nch - 1);
      issue_chunk_part<Cf, BPB>(rr, p, kvh, L, ob, pg, min(C, n - kc * C), bw, lane);
      if constexpr (Cf::KV == KV_FP8) {
        ks = p.k_scale[(size_t)pg * p.hkv + kvh];
        vs = p.v_scale[(size_t)pg * p.hkv + kvh];
      }
    };
    // the chunk to load at step c (issue distance IA); a chunk a helper took,
    // or one past the end, re-reads chunk c+1 clamped into [0, nch) (cache
    // hits; the loads stay unconditional so the waits stay exact)
    auto target = [&](int k) { return (k < nch && dec[k & 7]) ? k : max(0, min(k - (IA - 1), nch - 1)); };
    // prologue: chunk 0 into buffer 0, chunks 1 .. PFD-1 in flight
    issue(0, r0, ks0, vs0);
    if constexpr (PFD >= 2) issue(target(1), r1, ks1, vs1);
    if constexpr (PFD >= 3) issue(target(2), r2, ks2, vs2);
    __builtin_amdgcn_sched_barrier(0);
    {
      int ob0, pg0;
      entries(0, ob0, pg0);
      block_phase<Cf, BPB>(r0, qf, ob0, ks0, vs0, min(C, n), L, p.qk_log2, bw, lane, part2, pbuf);
    }
    if constexpr (PFD == 1) issue(target(1), r0, ks0, vs0);
    lds_barrier();

    // one step: rc holds chunk c+1's tiles; rn receives chunk c+IA's
    // (before the math when PFD == 2, after it otherwise)
    auto bstep = [&](BlockRegs<Cf> (&rc)[BPB], float& ksc, float& vsc, BlockRegs<Cf> (&rn)[BPB], float& ksn,
                     float& vsn) {
      const int t0 = c * C;
      float* nxt = part2 + ((c + 1) & 1) * Cf::SLOT;
      if constexpr (PFD == 2) {
        issue(target(c + 2), rn, ksn, vsn);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c + 1 < nch) {
        if (dec[(c + 1) & 7]) {
          int ob1, pg1;
          entries(c + 1, ob1, pg1);
          block_phase<Cf, BPB>(rc, qf, ob1, ksc, vsc, min(C, n - t0 - C), L, p.qk_log2, bw, lane, nxt, pbuf);
        } else {
          // a helper's chunk: wait for its slot, copy it into the buffer
          const u64* fw = readyw + (c + 1) % p.ring;
          int spins = 0;
          while (tag_val(ld_dev(fw), E, 0) != (uint32_t)(c + 2)) {
            if (++spins > p.spin_limit) { err = true; break; }
            __builtin_amdgcn_s_sleep(1);
          }
          const u64* src = reinterpret_cast<const u64*>(ringb + (size_t)((c + 1) % p.ring) * p.slot_floats);
          u64* dst = reinterpret_cast<u64*>(nxt);
          for (int i = threadIdx.x - 64 * NS; i < Cf::SLOT / 2; i += 64 * Cf::NBW) dst[i] = ld_dev(src + i);
        }
      }
      if constexpr (PFD != 2) issue(target(c + IA), rn, ksn, vsn);
      // claims: resolve the attempt for chunk c+IA+1, attempt chunk c+IA+2
      if (claimer && helped) {
        bool loc = false;
        if (tried3) {
          loc = ret3 == exp3;
          cw = loc ? tag_word(E, c + IA + 2) : ret3;
        }
        if (c + IA + 1 < nch) dec[(c + IA + 1) & 7] = loc ? 1 : 0;
        tried3 = false;
        if (c + IA + 2 < nch && (tag_val(cw, E, 1) & ~CLAIM_FIN) == (uint32_t)(c + IA + 2)) {
          exp3 = cw;
          ret3 = cas_dev(claimw, cw, tag_word(E, c + IA + 3));
          tried3 = true;
        }
      }
      const bool more = end_step(0);
      if (more) ++c;
      return more;
    };
    for (;;) {
      if constexpr (PFD == 3) {
        if (!bstep(r1, ks1, vs1, r0, ks0, vs0)) break;  // c % 3 == 0: compute slot 1, issue into slot 0
        if (!bstep(r2, ks2, vs2, r1, ks1, vs1)) break;
        if (!bstep(r0, ks0, vs0, r2, ks2, vs2)) break;
      } else if constexpr (PFD == 2) {
        if (!bstep(r1, ks1, vs1, r0, ks0, vs0)) break;
        if (!bstep(r0, ks0, vs0, r1, ks1, vs1)) break;
      } else {
        if (!bstep(r0, ks0, vs0, r0, ks0, vs0)) break;
      }
    }

    // KV tiles fetched: chunks [0, min(nch, c+IA+1)) were loaded here or by
    // a helper; with helpers, chunks claimed later by helpers were loaded by
    // them, and chunks c+IA+1, c+IA+2 claimed here were never loaded.  Then
    // close the stream for helpers.
    if (claimer) {
      int fetched = min(n, (c + IA + 1) * C);
      if (helped) {
        bool own_last = false;
        if (tried3) {
          own_last = ret3 == exp3;
          cw = own_last ? tag_word(E, c + IA + 3) : ret3;
        }
        uint32_t cnt = 0;
        for (int k = 0; k < (1 << 20); ++k) {
          cnt = tag_val(cw, E, 1) & ~CLAIM_FIN;
          const u64 r = cas_dev(claimw, cw, tag_word(E, CLAIM_FIN | cnt));
          if (r == cw) break;
          cw = r;
        }
        fetched = min(n, (int)cnt * C);
        auto blocks = [&](int k) { return k < nch ? min(C, n - k * C) : 0; };
        if (c + IA + 1 < nch && (int)cnt > c + IA + 1 && dec[(c + IA + 1) & 7]) fetched -= blocks(c + IA + 1);
        if (own_last) fetched -= blocks(c + IA + 2);
        if (err) st_dev32(p.sched_ctrl + 2, 1u);
      }
      if (p.blocks_fetched) p.blocks_fetched[stream] = fetched;
    }
  }
}

template <class Cf>
__device__ void art_helper(const Params& p, int hid, uint32_t E, float* part, float* pbuf, int* sh) {
  constexpr int C = Cf::C, NWA = Cf::NWA;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int streams = p.batch * p.hkv;
  const int slot = lane < C ? lane : C - 1;
  int pref = hid % streams;
  BlockRegs<Cf> regs[1];
  for (int iter = 0;; ++iter) {
    // ---- wave 0 looks for a claimable chunk: 64 streams per round
    if (w == 0) {
      int got_s = -1, got_c = 0;
      bool live_any = false;
      for (int base = 0; base < streams && got_s < 0; base += 64) {
        const bool valid = base + lane < streams;
        int st = pref + base + lane;
        if (st >= streams) st -= streams;
        u64 cwv = 0, dwv = 0;
        int nchv = 0;
        if (valid) {
          cwv = ld_dev(p.sched_claim + st);
          dwv = ld_dev(p.sched_done + st);
          const int nb = visit_count<Cf::B>(p, st / p.hkv, p.seq_lens[st / p.hkv]);
          nchv = (nb + C - 1) / C;
        }
        const uint32_t cv = tag_val(cwv, E, 1);
        const uint32_t cnt = cv & ~CLAIM_FIN;
        const uint32_t dn = tag_val(dwv, E, 0);
        const bool live = valid && (cv & CLAIM_FIN) == 0u && (int)cnt < nchv;
        const uint32_t win = min((uint32_t)p.ring, (uint32_t)p.lookahead + dn);
        const bool ok = live && cnt < dn + win;
        live_any |= __ballot(live) != 0ull;
        unsigned long long m = __ballot(ok);
        while (m != 0ull) {
          const int l = __builtin_ctzll(m);
          int won = 0;
          if (lane == l) won = cas_dev(p.sched_claim + st, cwv, tag_word(E, cnt + 1)) == cwv;
          if (__ballot(won) != 0ull) {
            got_s = readlane(st, l);
            got_c = readlane((int)cnt, l);
            break;
          }
          m &= m - 1ull;
        }
      }
      if (lane == 0) { sh[0] = got_s; sh[1] = got_c; sh[2] = live_any ? 1 : 0; }
    }
    lds_barrier();
    const int st = sh[0], cc = sh[1];
    const bool live_any = sh[2] != 0;
    lds_barrier();
    if (st < 0) {
      if (!live_any || iter >= p.spin_limit) break;
      __builtin_amdgcn_s_sleep(4);
      continue;
    }
    pref = st;

    // ---- produce chunk cc of stream st into its ring slot
    const int s = st / p.hkv;
    const int kvh = st - s * p.hkv;
    const int L = p.seq_lens[s];
    const int n = visit_count<Cf::B>(p, s, L);
    const int t0 = cc * C;
    const int nt = min(C, n - t0);
    const int32_t* trow = p.block_table + (size_t)s * p.max_blocks;
    const int32_t* orow = p.block_order + (size_t)s * p.max_blocks;
    const int ob = orow[min(t0 + slot, n - 1)];
    const int pg = trow[ob];
    float ks = 1.f, vs = 1.f;
    if (w < Cf::HWV) {
      issue_chunk_part<Cf, 1>(regs, p, kvh, L, ob, pg, nt, w, lane);
      if constexpr (Cf::KV == KV_FP8) {
        ks = p.k_scale[(size_t)pg * p.hkv + kvh];
        vs = p.v_scale[(size_t)pg * p.hkv + kvh];
      }
      uint4 qf[Cf::QF];
      load_q<Cf>(p, s, kvh, lane, qf);
      block_phase<Cf, 1>(regs, qf, ob, ks, vs, nt, L, p.qk_log2, w, lane, part, pbuf);
    }
    lds_barrier();
    u64* dst = reinterpret_cast<u64*>(p.sched_ring + ((size_t)st * p.ring + cc % p.ring) * p.slot_floats);
    const u64* src = reinterpret_cast<const u64*>(part);
    for (int i = threadIdx.x; i < Cf::SLOT / 2; i += 64 * NWA) st_dev(dst + i, src[i]);
    wait_all_memory();
    lds_barrier();
    if (threadIdx.x == 0) st_dev(p.sched_ready + (size_t)st * p.ring + cc % p.ring, tag_word(E, cc + 1));
  }
}

template <int KV, int D, int B, int GM>
__global__ __launch_bounds__((64 * Cfg<KV, D, B, GM>::NWA)) void art_sched_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  __shared__ __attribute__((aligned(16))) float part[2 * Cf::SLOT];
  __shared__ __attribute__((aligned(16))) float pbuf_all[Cf::NWA][Cf::PV4 ? GM * B : 4];
  __shared__ int sh[192];
  const int streams = p.batch * p.hkv;
  // The epoch tags the scheduler words, which only calls with helpers use;
  // it is constant during the launch (advanced by the last workgroup), so
  // each role reads it where it needs it.
  const bool helped = p.helpers > 0;
  const uint32_t E = helped ? epoch_of(ld_dev32(p.sched_ctrl)) : 0u;
  if ((int)blockIdx.x < streams)
    art_scanner<Cf>(p, blockIdx.x, E, part, pbuf_all[threadIdx.x >> 6], sh);
  else
    art_helper<Cf>(p, blockIdx.x - streams, E, part, pbuf_all[threadIdx.x >> 6], sh);
  // speculative loads may still be in flight
  wait_all_memory();
  if (helped) {
    // count this workgroup out; the last one advances the epoch
    lds_barrier();
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(p.sched_ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == gridDim.x - 1) {
        st_dev32(p.sched_ctrl + 1, 0u);
        st_dev32(p.sched_ctrl, E);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Terminating path, look-back scheduler: art_lb_kernel
// ---------------------------------------------------------------------------
//
// Persistent workgroups ("workers") take items = (stream, chunk of C blocks)
// from per-stream claim counters and carry each item through a three-step
// pipeline, one item per step in each stage: the item's KV loads are issued
// (block waves), its per-block partials computed into LDS (block waves), and
// it is folded into the stream's ART state (scan waves, one query head per
// wave).  Chunks of one stream can be on many workers at once; the state
// entering chunk k comes from the records of earlier chunks (a decoupled
// look-back over an associative combine):
//   * (M, L, A): the online-softmax state is a monoid under
//     (M1, L1, A1) + (M2, L2, A2) = (M, 2^(M1-M) L1 + 2^(M2-M) L2, same for A),
//     M = max(M1, M2).  Each chunk publishes its own aggregate G_k (folded
//     from its blocks) and its inclusive state I_k = X_k + G_k; the state
//     entering chunk k is X_k = (((I_j + G_{j+1}) + G_{j+2}) + ... + G_{k-1})
//     for the nearest chunk j whose inclusive state is out (X_0 = empty).
//     Since every I_j is itself that left fold of G_0 .. G_j, the result has
//     the same bits whichever j a chunk starts from: results do not depend on
//     the timing, the number of workers or the window, and no chunk waits on
//     a chain of other chunks' look-backs -- only on aggregates.
//   * The detector's inputs at the chunk's first position need only the
//     output O = A / L entering it, so the statistics of all C positions (and
//     their pass bits) follow from that state alone.
//   * The pass count, the block-0-folded flag and whether the head still runs
//     are replayed from the nearest resolved chunk over the pass bits of the
//     chunks after it.
// A head that fires writes its output and stop; when every head of a stream
// has fired the stream's claim counter is closed, later chunks are no longer
// claimed and chunks already in flight are dropped before their fold.
//
// Forward progress: an item only waits for records of earlier chunks of its
// stream, which were claimed before it, and a worker's items are processed in
// claim order; every wait therefore points to an item claimed earlier, and
// the earliest unfinished item can always proceed -- whether or not every
// worker is resident.
//
// Claims: a worker stays on the stream of its last item while that stream
// has unclaimed chunks (waiting while its window is full), else sweeps all
// streams and takes one of those with the most unclaimed chunks (ties spread
// over the workers by a hash).  Chunk k of a stream is claimable while
// k < resolved + window, where resolved is one past the highest chunk whose
// state is final for every head; that bounds the speculative reads past a
// stop, and keeps the nearest resolved chunk of a chunk in flight within
// about `window` chunks of it (the look-back waits otherwise).
//
// Record of (stream, chunk, head): a status word tag(E, payload) with
//   bits 0-2   level: 1 aggregate, 2 inclusive state, 3 pass bits, 4 resolved
//              (a chunk can skip level 1 when its inclusive state follows at
//              once; a dropped chunk goes straight to 4)
//   bits 3-10  pass bits of the chunk's positions          (level >= 3)
//   bits 11-18 positions holding block 0                   (level >= 3)
//   bit 19     head still running after the chunk          (level 4)
//   bit 20     block 0 folded by the end of the chunk      (level 4)
//   bits 21-31 passes in a row at the chunk end, at most the patience (level 4)
// and floats: aggregate [A(D), m, l] at 0, inclusive [A(D), M, L] at D + 4.
// Data is stored with device-scope stores and the status after them
// (s_waitcnt vmcnt(0) in between); readers load the status, then the data.

constexpr uint32_t LB_AGG = 1u, LB_INCL = 2u, LB_PASS = 3u, LB_FIN = 4u;
constexpr uint32_t LB_LEVEL = 7u;
constexpr int LB_PASS_SH = 3, LB_SINK_SH = 11, LB_CNT_SH = 21;
constexpr uint32_t LB_RUNNING = 1u << 19, LB_SINKED = 1u << 20;
constexpr uint32_t LB_BEFORE = LB_FIN | LB_RUNNING;  // the state before chunk 0 (its inclusive state: empty)
constexpr int LB_CNT_MAX = 2047;
constexpr int LB_ENT = 24;                          // ints per LDS item entry: s, k, n, L, ob[8], pg[8]
constexpr int LB_BUBBLE = -1, LB_END = -2;

template <class Cf>
struct LbState {
  float M, L;
  float A[Cf::DPL];
};

template <class Cf>
__device__ __forceinline__ void lb_load(const float* r, int lane, float& m, float& l, float (&a)[Cf::DPL]) {
  if constexpr (Cf::DPL == 2) {
    const u64 v = ld_dev(reinterpret_cast<const u64*>(r + 2 * lane));
    a[0] = bitsf((uint32_t)v);
    a[1] = bitsf((uint32_t)(v >> 32));
  } else {
    a[0] = bitsf(ld_dev32(reinterpret_cast<const uint32_t*>(r + lane)));
  }
  const u64 ml = ld_dev(reinterpret_cast<const u64*>(r + Cf::D));
  m = bitsf((uint32_t)ml);
  l = bitsf((uint32_t)(ml >> 32));
}

template <class Cf>
__device__ __forceinline__ void lb_store(float* r, int lane, float m, float l, const float (&a)[Cf::DPL]) {
  if constexpr (Cf::DPL == 2)
    st_dev(reinterpret_cast<u64*>(r + 2 * lane), ((u64)fbits(a[1]) << 32) | fbits(a[0]));
  else
    st_dev32(reinterpret_cast<uint32_t*>(r + lane), fbits(a[0]));
  if (lane == 0) st_dev(reinterpret_cast<u64*>(r + Cf::D), ((u64)fbits(l) << 32) | fbits(m));
}

// x <- x (+) (m, l, a)
template <class Cf>
__device__ __forceinline__ void lb_combine(LbState<Cf>& x, float m, float l, const float (&a)[Cf::DPL]) {
  const float mn = fmaxf(x.M, m);
  const bool empty = mn == NEG_INF;
  const float fx = empty ? 0.f : __builtin_amdgcn_exp2f(x.M - mn);
  const float fy = empty ? 0.f : __builtin_amdgcn_exp2f(m - mn);
  x.L = fmaf(fx, x.L, fy * l);
#pragma unroll
  for (int j = 0; j < Cf::DPL; ++j) x.A[j] = fmaf(fx, x.A[j], fy * a[j]);
  x.M = mn;
}

// O = A / L entering a chunk (0 before any block) and the squared norm of
// its coordinates [0, probe).
template <class Cf>
__device__ __forceinline__ void lb_entering_output(const LbState<Cf>& x, int lane, int probe, float (&Op)[Cf::DPL],
                                                   float& np) {
  const float rl = x.L > 0.f ? __builtin_amdgcn_rcpf(x.L) : 0.f;
  float sq[1] = {0.f};
#pragma unroll
  for (int j = 0; j < Cf::DPL; ++j) {
    Op[j] = x.L > 0.f ? x.A[j] * rl : 0.f;
    const float op = Cf::DPL * lane + j < probe ? Op[j] : 0.f;
    sq[0] = fmaf(op, op, sq[0]);
  }
  np = xreduce<1>(sq, lane);
}

// The chunk's own aggregate from its per-block partials (positions past the
// chunk end are neutral: m = -inf, l = 0, a = 0; position 0 is a real block).
template <class Cf>
__device__ __forceinline__ void lb_aggregate(const ChunkIn<Cf>& in, float& m, float& l, float (&a)[Cf::DPL]) {
  float mx = NEG_INF;
#pragma unroll
  for (int t = 0; t < Cf::C; ++t) mx = fmaxf(mx, readlanef(in.m, t));
  l = 0.f;
#pragma unroll
  for (int j = 0; j < Cf::DPL; ++j) a[j] = 0.f;
#pragma unroll
  for (int t = 0; t < Cf::C; ++t) {
    const float e = __builtin_amdgcn_exp2f(readlanef(in.m, t) - mx);
    l = fmaf(e, readlanef(in.l, t), l);
#pragma unroll
    for (int j = 0; j < Cf::DPL; ++j) a[j] = fmaf(e, in.a[t][j], a[j]);
  }
  m = mx;
}

// Fold one chunk into the state entering it (x, with O_prev = Op and
// Np = ‖Op‖²) and evaluate both statistics at every position of the chunk
// (the same arithmetic as scan_head).  Returns the pass bits (bit t:
// position t passed both tests); x becomes the inclusive state, Op the
// output at the chunk's last position, oo[t] the output at position t.
template <class Cf>
__device__ __forceinline__ u64 lb_stats(LbState<Cf>& x, float (&Op)[Cf::DPL], float Np, const ChunkIn<Cf>& in,
                                        int t0, int nt, const Params& p, int lane, float (&oo)[Cf::C][Cf::DPL]) {
  constexpr int C = Cf::C, DPL = Cf::DPL, SH = Cf::SH;
  const int slot = lane < C ? lane : C - 1;
  float mx = in.m;
  if constexpr (C > 1) mx = fmaxf(mx, row_shr<1>(mx, NEG_INF));
  if constexpr (C > 2) mx = fmaxf(mx, row_shr<2>(mx, NEG_INF));
  if constexpr (C > 4) mx = fmaxf(mx, row_shr<4>(mx, NEG_INF));
  mx = fmaxf(mx, x.M);
  const float mprev = row_shr<1>(mx, x.M);
  const float al = mprev == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mprev - mx);
  const float be = __builtin_amdgcn_exp2f(in.m - mx);
  float fa = al, fb = be * in.l;
  if constexpr (C > 1) { const float pa = row_shr<1>(fa, 1.f), pb = row_shr<1>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  if constexpr (C > 2) { const float pa = row_shr<2>(fa, 1.f), pb = row_shr<2>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  if constexpr (C > 4) { const float pa = row_shr<4>(fa, 1.f), pb = row_shr<4>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  const float Lt = fmaf(fa, x.L, fb);
  const float rl = __builtin_amdgcn_rcpf(Lt);

  float st[2 * C];
#pragma unroll
  for (int t = 0; t < C; ++t) {
    const float at = readlanef(al, t), bt = readlanef(be, t), rt = readlanef(rl, t);
    float nn = 0.f, ee = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      x.A[j] = fmaf(at, x.A[j], bt * in.a[t][j]);
      const float o = x.A[j] * rt;
      const float df = o - Op[j];
      const float op = DPL * lane + j < p.probe ? o : 0.f;  // coordinates outside the probe do not count
      const float dp = DPL * lane + j < p.probe ? df : 0.f;
      nn = fmaf(op, op, nn);
      ee = fmaf(dp, dp, ee);
      Op[j] = o;
      oo[t][j] = o;
    }
    st[2 * t] = nn;
    st[2 * t + 1] = ee;
  }
  const float v0 = xreduce<2 * C>(st, lane);
  const float nn_t = __shfl(v0, (2 * slot) << SH);
  const float ee_t = __shfl(v0, (2 * slot + 1) << SH);
  float np_t = __shfl(v0, (2 * max(slot - 1, 0)) << SH);
  if (lane == 0) np_t = Np;
  bool ps = false;
  if (lane < nt && t0 + lane >= 1) {
    const float a = __builtin_amdgcn_sqrtf(nn_t);
    const float bn = __builtin_amdgcn_sqrtf(np_t);
    float dm, dd;
    if (a == 0.f && bn == 0.f) {
      dm = 0.f; dd = 0.f;
    } else if (bn == 0.f) {
      dm = __builtin_inff(); dd = 1.f;
    } else {
      const float df = a - bn;
      dm = fabsf(df) * __builtin_amdgcn_rcpf(bn);
      dd = (a == 0.f) ? 1.f : fmaxf(0.f, (ee_t - df * df) * __builtin_amdgcn_rcpf(2.f * a * bn));
    }
    ps = (dm < p.eps_mag) && (dd < p.eps_dir);
  }
  x.M = readlanef(mx, C - 1);
  x.L = readlanef(Lt, C - 1);
  return __ballot(ps);
}

// A wait that ran past its limit marks the call failed ([3] = this epoch,
// [2] = 1); every other wait of the call then gives up at its next check.
__device__ __forceinline__ void lb_fail(const Params& p, uint32_t E) {
  st_dev32(p.sched_ctrl + 3, E);
  st_dev32(p.sched_ctrl + 2, 1u);
}
__device__ __forceinline__ bool lb_give_up(const Params& p, uint32_t E, int spin) {
  return spin > p.spin_limit || ((spin & 63) == 63 && ld_dev32(p.sched_ctrl + 3) == E);
}

// Status words of chunks k-1-lane (lanes < window); the state before chunk 0
// for lanes that reach past it.
__device__ __forceinline__ uint32_t lb_probe(const u64* st0, int g, int k, int window, uint32_t E, int lane) {
  const int j = k - 1 - lane;
  uint32_t v = LB_BEFORE;
  if (lane < window && j >= 0) v = tag_val(ld_dev(st0 + (size_t)j * g), E, 0u);
  if (lane >= window) v = 0u;
  return v;
}

// One query head of one item: publish, look back, fold, detect, resolve.
// Returns false if a wait ran past the spin limit (the head is then marked
// stopped with stop = -1 and a NaN output).
template <class Cf>
__device__ bool lb_head(const Params& p, uint32_t E, int s, int k, int n, int h, const ChunkIn<Cf>& in,
                        uint32_t sinkb, bool dead, int lane) {
  constexpr int C = Cf::C, DPL = Cf::DPL;
  const int g = p.g;
  const int nt = min(C, n - k * C);
  const int t0 = k * C;
  const int nch = (n + C - 1) / C;
  const int lbw = min(64, 2 * p.window);  // chunks a look-back examines
  const u64* st0 = p.lb_st + (size_t)s * p.max_chunks * g + h;  // chunk stride g
  u64* stw = p.lb_st + ((size_t)s * p.max_chunks + k) * g + h;
  const size_t rstride = (size_t)g * p.rec_floats;
  const float* rec0 = p.lb_rec + ((size_t)s * p.max_chunks * g + h) * p.rec_floats;
  float* rec = p.lb_rec + (((size_t)s * p.max_chunks + k) * g + h) * p.rec_floats;
  const size_t head = (size_t)(s / p.hkv) * p.hq + (size_t)(s % p.hkv) * g + h;
  const int incl = Cf::D + 4;
  const int cap = min(p.patience, LB_CNT_MAX);
  const bool last = k == nch - 1;  // no chunk after it reads its records
  if (dead) {
    if (lane == 0) st_dev(stw, tag_word(E, LB_FIN | (sinkb << LB_SINK_SH)));
    return true;
  }

  // ---- the chunk's own aggregate
  float gm, gl, ga[DPL];
  lb_aggregate<Cf>(in, gm, gl, ga);

  // ---- state entering the chunk: nearest published inclusive state (lane f
  // examines chunk k-1-f), then the aggregates after it in chunk order; the
  // aggregate is published first unless that state can be had at once
  LbState<Cf> x;
  x.M = NEG_INF;
  x.L = 0.f;
#pragma unroll
  for (int j = 0; j < DPL; ++j) x.A[j] = 0.f;
  bool ok = true;
  int f = 0;
  if (k > 0) {
    bool published = last;
    for (int spin = 0;; ++spin) {
      const uint32_t v = lb_probe(st0, g, k, lbw, E, lane);
      const u64 inc = __ballot((v & LB_LEVEL) >= LB_INCL);
      if (inc != 0ull) {
        f = __builtin_ctzll(inc);
        const u64 need = (1ull << f) - 1ull;
        if ((__ballot((v & LB_LEVEL) >= LB_AGG) & need) == need) break;
      }
      if (!published) {
        lb_store<Cf>(rec, lane, gm, gl, ga);
        wait_all_memory();
        if (lane == 0) st_dev(stw, tag_word(E, LB_AGG));
        published = true;
      }
      if (lb_give_up(p, E, spin)) { ok = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    if (ok) {
      const int jb = k - 1 - f;
      if (jb >= 0) lb_load<Cf>(rec0 + (size_t)jb * rstride + incl, lane, x.M, x.L, x.A);
      for (int i = f - 1; i >= 0; --i) {
        float m, l, a[DPL];
        lb_load<Cf>(rec0 + (size_t)(k - 1 - i) * rstride, lane, m, l, a);
        lb_combine<Cf>(x, m, l, a);
      }
    }
  }
  // ---- publish the inclusive state X_k + G_k
  if (ok && !last) {
    LbState<Cf> xi = x;
    lb_combine<Cf>(xi, gm, gl, ga);
    lb_store<Cf>(rec + incl, lane, xi.M, xi.L, xi.A);
    wait_all_memory();
    if (lane == 0) st_dev(stw, tag_word(E, LB_INCL));
  }

  // ---- statistics of every position
  float Op[DPL];
  float np = 0.f;
  lb_entering_output<Cf>(x, lane, p.probe, Op, np);
  float oo[C][DPL];
  const u64 pass = lb_stats<Cf>(x, Op, np, in, t0, nt, p, lane, oo);
  const uint32_t passb = (uint32_t)pass & 0xFFu;
  const uint32_t bits = (passb << LB_PASS_SH) | (sinkb << LB_SINK_SH);
  if (ok && lane == 0 && !last) st_dev(stw, tag_word(E, LB_PASS | bits));

  // ---- pass count, block-0 flag and running flag entering the chunk:
  // replayed from the nearest resolved chunk over the pass bits after it
  int cnt = 0;
  bool sink = false, alive = true;
  if (ok && k > 0) {
    uint32_t v = 0;
    for (int spin = 0;; ++spin) {
      v = lb_probe(st0, g, k, lbw, E, lane);
      const u64 fin = __ballot((v & LB_LEVEL) == LB_FIN);
      if (fin != 0ull) {
        f = __builtin_ctzll(fin);
        const u64 need = (1ull << f) - 1ull;
        if ((__ballot((v & LB_LEVEL) >= LB_PASS) & need) == need) break;
      }
      if (lb_give_up(p, E, spin)) { ok = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    if (ok) {
      const uint32_t wf = (uint32_t)readlane((int)v, f);
      cnt = (int)(wf >> LB_CNT_SH);
      sink = (wf & LB_SINKED) != 0u;
      alive = (wf & LB_RUNNING) != 0u;
      for (int i = f - 1; i >= 0 && alive; --i) {
        const uint32_t wi = (uint32_t)readlane((int)v, i);
        const int ci = k - 1 - i;
        const int nti = min(C, n - ci * C);
        for (int t = 0; t < nti; ++t) {
          cnt = ((wi >> (LB_PASS_SH + t)) & 1u) ? min(cnt + 1, cap) : 0;
          sink = sink || ((wi >> (LB_SINK_SH + t)) & 1u);
          if (cnt >= p.patience && sink) { alive = false; break; }
        }
      }
    }
  }

  // ---- resolve this chunk
  const int slot = lane < C ? lane : C - 1;
  const u64 upto = (2ull << slot) - 1ull;
  const u64 zeros = ~pass & upto;
  const int cnt_t = zeros == 0ull ? min(cnt + slot + 1, cap) : slot - (63 - __builtin_clzll(zeros));
  const bool sink_t = sink || ((u64)sinkb & upto) != 0ull;
  const u64 fire = __ballot(ok && alive && lane < nt && cnt_t >= p.patience && sink_t);
  float* out_row = p.out + head * Cf::D;
  bool alive_out = ok && alive;
  if (fire != 0ull) {
    const int stop_t = __builtin_ctzll(fire);
    float ov[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) ov[j] = oo[0][j];
#pragma unroll
    for (int t = 1; t < C; ++t)
      if (stop_t == t)
#pragma unroll
        for (int j = 0; j < DPL; ++j) ov[j] = oo[t][j];
#pragma unroll
    for (int j = 0; j < DPL; ++j) out_row[DPL * lane + j] = ov[j];
    if (lane == 0) p.stop_block[head] = t0 + stop_t + 1;
    alive_out = false;
  } else if (alive_out && last) {
    // never stopped: the output after all n blocks
#pragma unroll
    for (int j = 0; j < DPL; ++j) out_row[DPL * lane + j] = Op[j];
    if (lane == 0) p.stop_block[head] = n;
  }
  if (!ok) {
#pragma unroll
    for (int j = 0; j < DPL; ++j) out_row[DPL * lane + j] = __builtin_nanf("");
    if (lane == 0) {
      p.stop_block[head] = -1;
      lb_fail(p, E);
    }
  }
  const int cnt_out = readlane(min(cnt_t, cap), nt - 1);
  const bool sink_out = readlane(sink_t ? 1 : 0, nt - 1) != 0;
  if (lane == 0) {
    st_dev(stw, tag_word(E, LB_FIN | bits | (alive_out ? LB_RUNNING : 0u) | (sink_out ? LB_SINKED : 0u) |
                                ((uint32_t)cnt_out << LB_CNT_SH)));
    if (fire != 0ull || !ok) {
      // mark the head stopped; close the stream when the whole group is
      const uint32_t bit = 1u << h;
      const uint32_t was = __hip_atomic_fetch_or(p.lb_heads + s, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((was | bit) == (1u << g) - 1u && was != (was | bit))
        __hip_atomic_fetch_or(p.lb_claim + s, CLAIM_FIN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return ok;
}

// Claim the next item into LDS entry e (whole claimer wave).  `cur` is the
// stream of this worker's last claim, `ended` becomes true once no stream has
// unclaimed chunks left.  A claim is an atomic add on the stream's counter,
// attempted only while the counter is inside the window; concurrent claims
// can pass the window or the chunk count by a few, which only makes the
// later chunk wait for its look-back, or returns nothing.
template <class Cf>
__device__ void lb_claim(const Params& p, uint32_t E, int* e, char* qdst, int& cur, bool& ended, int lane) {
  constexpr int C = Cf::C;
  constexpr int QROWB = Cf::KV == KV_FP8 ? 2 * Cf::D : Cf::R;
  const int S = p.batch * p.hkv;
  int got_s = -1, got_k = 0;
  (void)E;
  if (!ended) {
    auto nch_of = [&](int st) { return (visit_count<Cf::B>(p, st / p.hkv, p.seq_lens[st / p.hkv]) + C - 1) / C; };
    auto take = [&](int st) {  // lane 0 adds, the wave gets the chunk index (or -1)
      uint32_t k = 0;
      if (lane == 0) k = __hip_atomic_fetch_add(p.lb_claim + st, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      k = (uint32_t)readlane((int)k, 0);
      return ((k & CLAIM_FIN) || (int)k >= nch_of(st)) ? -1 : (int)k;
    };
    // the current stream while it has unclaimed chunks (waiting while its
    // window is full), so that a stream's chunks stay on a fixed set of
    // workers and an item never queues behind another stream's
    bool stay = false;
    if (cur >= 0) {
      const uint32_t cv = ld_dev32(p.lb_claim + cur);
      const uint32_t prog = ld_dev32(p.lb_prog + cur);
      stay = !(cv & CLAIM_FIN) && (int)cv < nch_of(cur);
      if (stay && cv < prog + (uint32_t)p.window) {
        const int k = take(cur);
        if (k >= 0) { got_s = cur; got_k = k; }
      }
    }
    // else a claimable stream: most unclaimed chunks first (counted up to
    // 16), ties spread over the workers
    if (got_s < 0 && !stay) {
      uint32_t best = 0u;  // (min(remaining, 16) << 24) | (hash << 16) | stream, 0 = none
      bool live_any = false;
      const uint32_t hw = (blockIdx.x * 2654435761u) >> 24;
      for (int base = 0; base < S; base += 64) {
        const int st = base + lane;
        uint32_t key = 0u;
        if (st < S) {
          const uint32_t cv = ld_dev32(p.lb_claim + st);
          const uint32_t prog = ld_dev32(p.lb_prog + st);
          const int nch = nch_of(st);
          const bool live = !(cv & CLAIM_FIN) && (int)cv < nch;
          live_any |= live;
          if (live && cv < prog + (uint32_t)p.window)
            key = ((uint32_t)min(nch - (int)cv, 16) << 24) | ((((uint32_t)st * 40503u) ^ hw) & 0xFFu) << 16 |
                  (uint32_t)st;
        }
        uint32_t mk = key;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mk = max(mk, (uint32_t)__shfl_xor((int)mk, o));
        best = max(best, mk);
      }
      live_any = __ballot(live_any) != 0ull;
      if (best != 0u) {
        const int st = (int)(best & 0xFFFFu);
        const int k = take(st);
        if (k >= 0) { got_s = st; got_k = k; }
        cur = st;
      } else if (!live_any) {
        ended = true;
      }
    }
  }
  if (got_s < 0) {
    if (lane == 0) e[0] = ended ? LB_END : LB_BUBBLE;
    return;
  }
  cur = got_s;
  // entries: visit order, pages, query rows of the group
  const int sq = got_s / p.hkv;
  const int kvh = got_s - sq * p.hkv;
  const int L = p.seq_lens[sq];
  const int n = visit_count<Cf::B>(p, sq, L);
  const int32_t* orow = p.block_order + (size_t)sq * p.max_blocks;
  const int32_t* trow = p.block_table + (size_t)sq * p.max_blocks;
  const int ob = orow[min(got_k * C + min(lane, C - 1), n - 1)];
  const char* qsrc = static_cast<const char*>(p.q) + ((size_t)sq * p.hq + (size_t)kvh * p.g) * QROWB;
  const int qwords = p.g * QROWB / 16;
  for (int i = lane; i < qwords; i += 64)
    *reinterpret_cast<uint4*>(qdst + 16 * i) = *reinterpret_cast<const uint4*>(qsrc + 16 * i);
  const int pg = trow[ob];
  if (lane == 0) { e[0] = got_s; e[1] = got_k; e[2] = n; e[3] = L; }
  if (lane < C) { e[4 + lane] = ob; e[4 + C + lane] = pg; }
}

// q fragments (as load_q) from the LDS copy of the group's query rows [GM][row bytes].
template <class Cf>
__device__ __forceinline__ void load_q_lds(const char* qs, int g, int lane, uint4 (&qf)[Cf::QF]) {
  constexpr int QROWB = Cf::KV == KV_FP8 ? 2 * Cf::D : Cf::R;
  const int c = lane & 15;
#pragma unroll
  for (int i = 0; i < Cf::QF; ++i) qf[i] = make_uint4(0, 0, 0, 0);
  if (c >= g) return;
  const char* row = qs + c * QROWB;
  const int base = (lane >> 4) * 16;
  if constexpr (Cf::KV == KV_FP8) {
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qf[2 * i + hf] = *reinterpret_cast<const uint4*>(row + 2 * (base + 64 * i + 8 * hf));
  } else {
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i) qf[i] = *reinterpret_cast<const uint4*>(row + base + 64 * i);
  }
}

template <int KV, int D, int B, int GM>
__global__ __launch_bounds__((64 * Cfg<KV, D, B, GM>::NWA)) void art_lb_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int C = Cf::C, NS = Cf::NS, HPS = Cf::HPS, PFD = Cf::PFD;
  constexpr int QROWB = KV == KV_FP8 ? 2 * D : Cf::R;
  constexpr int CLW = NS - 1;  // the scan wave that also claims
  __shared__ __attribute__((aligned(16))) float part[2 * Cf::SLOT];
  __shared__ __attribute__((aligned(16))) float pbuf_all[Cf::NWA][Cf::PV4 ? GM * B : 4];
  __shared__ __attribute__((aligned(16))) char qring[4][GM * QROWB];
  __shared__ int ent[4][LB_ENT];
  __shared__ int last_wg;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.batch * p.hkv;
  const uint32_t E = epoch_of(ld_dev32(p.sched_ctrl));
  const int slot = lane < C ? lane : C - 1;

  // streams without tokens: out = 0, stop = 0
  for (int st = blockIdx.x; st < S; st += gridDim.x) {
    const int sq = st / p.hkv;
    if (visit_count<Cf::B>(p, sq, p.seq_lens[sq]) <= 0) {
      const size_t head0 = (size_t)sq * p.hq + (size_t)(st - sq * p.hkv) * p.g;
      for (int i = threadIdx.x; i < p.g * D; i += blockDim.x) p.out[head0 * D + i] = 0.f;
      if ((int)threadIdx.x < p.g) p.stop_block[head0 + threadIdx.x] = 0;
    }
  }

  int cur = (int)(blockIdx.x % (unsigned)S);
  bool ended = false;
  if (w == CLW) {
    lb_claim<Cf>(p, E, ent[0], qring[0], cur, ended, lane);
    lb_claim<Cf>(p, E, ent[1], qring[1], cur, ended, lane);
  }
  lds_barrier();

  // Step j: the claimer takes item j+2, block waves issue item j+1's loads
  // and compute item j into buffer j % 2, scan waves fold item j-1 from
  // buffer (j-1) % 2.  One LDS barrier per step; LDS entry e % 4 and query
  // copy e % 4 hold item e from its claim (step e-2) to its fold (step e+1).
  if (w < NS) {
    bool err = false;
    int ps = -1, pk = 0;  // item folded in the previous step
    for (int j = 0;; ++j) {
      if (w == 0 && lane == 0 && ps >= 0)
        __hip_atomic_fetch_max(p.lb_prog + ps, (uint32_t)pk + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ps = -1;
      if (w == CLW) lb_claim<Cf>(p, E, ent[(j + 2) & 3], qring[(j + 2) & 3], cur, ended, lane);
      if (j >= 1) {
        const int* e = ent[(j - 1) & 3];
        const int s = e[0];
        if (s >= 0) {
          const int k = e[1], n = e[2];
          const int nt = min(C, n - k * C);
          const int ob = e[4 + slot];
          const uint32_t sinkb = (uint32_t)__ballot(lane < nt && ob == 0) & 0xFFu;
          const uint32_t stopped = ld_dev32(p.lb_heads + s);
          const float* buf = part + ((j - 1) & 1) * Cf::SLOT;
#pragma unroll
          for (int kk = 0; kk < HPS; ++kk) {
            const int h = w + NS * kk;
            if (h < p.g) {
              ChunkIn<Cf> in;
              gather_lds<Cf>(in, buf, h, lane);
              if (!lb_head<Cf>(p, E, s, k, n, h, in, sinkb, ((stopped >> h) & 1u) != 0u, lane)) err = true;
            }
          }
          ps = s;
          pk = k;
        }
      }
      lds_barrier();
      if (ent[j & 3][0] == LB_END) break;
    }
    (void)err;
  } else {
    const int bw = w - NS;
    float* pbuf = pbuf_all[w];
    BlockRegs<Cf> r0[1], r1[1];
    float ks0 = 1.f, vs0 = 1.f, ks1 = 1.f, vs1 = 1.f;
    // issue item j's loads (a bubble or the end re-reads page 0's first tile,
    // so the loads stay unconditional and the compiler's waits exact)
    auto issue = [&](int j, BlockRegs<Cf> (&rr)[1], float& ks, float& vs) {
      const int* e = ent[j & 3];
      const int s = e[0];
      if (s >= 0) {
        const int k = e[1], n = e[2], L = e[3];
        const int kvh = s % p.hkv;
        const int ob = e[4 + slot], pg = e[4 + C + slot];
        const int nt = min(C, n - k * C);
        issue_chunk_part<Cf, 1>(rr, p, kvh, L, ob, pg, nt, bw, lane);
        if constexpr (KV == KV_FP8) {
          ks = p.k_scale[(size_t)pg * p.hkv + kvh];
          vs = p.v_scale[(size_t)pg * p.hkv + kvh];
        }
        if (bw == 0 && lane == 0)
          __hip_atomic_fetch_add(p.lb_fetch + s, (uint32_t)nt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        issue_chunk_part<Cf, 1>(rr, p, 0, Cf::B, 0, 0, 1, bw, lane);
        if constexpr (KV == KV_FP8) {
          ks = p.k_scale[0];
          vs = p.v_scale[0];
        }
      }
    };
    auto compute = [&](int j, const BlockRegs<Cf> (&rr)[1], float ks, float vs) {
      const int* e = ent[j & 3];
      if (e[0] >= 0) {
        const int k = e[1], n = e[2], L = e[3];
        uint4 qf[Cf::QF];
        load_q_lds<Cf>(qring[j & 3], p.g, lane, qf);
        block_phase<Cf, 1>(rr, qf, e[4 + slot], ks, vs, min(C, n - k * C), L, p.qk_log2, bw, lane,
                           part + (j & 1) * Cf::SLOT, pbuf);
      }
    };
    auto bstep = [&](int j, BlockRegs<Cf> (&rc)[1], float& ksc, float& vsc, BlockRegs<Cf> (&rn)[1], float& ksn,
                     float& vsn) {
      if constexpr (PFD >= 2) {
        issue(j + 1, rn, ksn, vsn);
        __builtin_amdgcn_sched_barrier(0);
        compute(j, rc, ksc, vsc);
      } else {
        compute(j, rc, ksc, vsc);
        issue(j + 1, rc, ksc, vsc);
      }
      lds_barrier();
      return ent[j & 3][0] != LB_END;
    };
    issue(0, r0, ks0, vs0);
    for (int j = 0;; j += 2) {
      if constexpr (PFD >= 2) {
        if (!bstep(j, r0, ks0, vs0, r1, ks1, vs1)) break;
        if (!bstep(j + 1, r1, ks1, vs1, r0, ks0, vs0)) break;
      } else {
        if (!bstep(j, r0, ks0, vs0, r0, ks0, vs0)) break;
        if (!bstep(j + 1, r0, ks0, vs0, r0, ks0, vs0)) break;
      }
    }
  }
  // loads issued ahead may still be in flight
  wait_all_memory();
  // count this workgroup out; the last one publishes the fetched counts,
  // clears the per-stream words and advances the epoch
  lds_barrier();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(p.sched_ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_wg = prev == gridDim.x - 1 ? 1 : 0;
  }
  lds_barrier();
  if (last_wg) {
    for (int st = threadIdx.x; st < S; st += blockDim.x) {
      const uint32_t f = ld_dev32(p.lb_fetch + st);
      if (p.blocks_fetched) p.blocks_fetched[st] = (int32_t)f;
      st_dev32(p.lb_fetch + st, 0u);
      st_dev32(p.lb_claim + st, 0u);
      st_dev32(p.lb_prog + st, 0u);
      st_dev32(p.lb_heads + st, 0u);
    }
    wait_all_memory();
    lds_barrier();
    if (threadIdx.x == 0) {
      st_dev32(p.sched_ctrl + 1, 0u);
      st_dev32(p.sched_ctrl, E);
    }
  }
}

// ---------------------------------------------------------------------------
// Terminating path, windowed: art_win_part_kernel + art_win_scan_kernel
// ---------------------------------------------------------------------------
//
// A stream's chunks are processed window by window (growing windows of at
// most 64 chunks; the host picks their sizes), two launches per window;
// launch boundaries are the only waits between workgroups.
//   * art_win_part_kernel: one workgroup per (stream, chunk), one wave per
//     block, computes each chunk's per-block partials (m_b, l_b, a_b) for
//     every head of the group and each head's chunk aggregate.  Streams whose
//     heads have all stopped are skipped.
//   * art_win_scan_kernel: K workgroups per (stream, query head) (K = 1 unless asked
//     otherwise), in four phases: (1) each chunk's aggregate into LDS; (2) the
//     state entering each chunk, in chunk order, from the state carried from
//     the previous window; (3) the statistics of every position of the
//     workgroup's own chunks (the detector at a chunk needs only the state
//     entering it), whose pass bits are published; (4) in the last of the K
//     workgroups to finish (an arrival counter; nothing waits), the
//     patience/block-0 rule over the window's pass bits from the carried pass
//     count.  A head that fires writes its output (folded again at its chunk)
//     and its stop; a head that reaches the end of its stream writes the
//     output after all n blocks.
// Every combine runs in the order the look-back kernel uses, so results are
// deterministic and the same bits as that kernel's.

constexpr int WNW = art_win_waves;  // waves of art_win_scan_kernel

// The chunk's partials of head h from its slot in global memory.
template <class Cf>
__device__ __forceinline__ void win_gather(ChunkIn<Cf>& in, const float* slotp, int h, int lane) {
#pragma unroll
  for (int t = 0; t < Cf::C; ++t) {
    const float* src = slotp + ((size_t)t * Cf::GM + h) * Cf::D + Cf::DPL * lane;
    if constexpr (Cf::DPL == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(src);
      in.a[t][0] = v.x; in.a[t][1] = v.y;
    } else {
      in.a[t][0] = src[0];
    }
  }
  const int t = lane < Cf::C ? lane : 0;
  in.m = lane < Cf::C ? slotp[Cf::SLOT_A + t * Cf::GM + h] : NEG_INF;
  in.l = lane < Cf::C ? slotp[Cf::SLOT_A + Cf::C * Cf::GM + t * Cf::GM + h] : 0.f;
}

// Partials: workgroup `bid` takes one chunk of one stream of the window, one
// wave per block.  Streams that have stopped are skipped.
template <int KV, int D, int B, int GM>
__global__ __launch_bounds__((64 * Cfg<KV, D, B, GM>::C)) void art_win_part_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int C = Cf::C;
  __shared__ __attribute__((aligned(16))) float pbuf_all[C][Cf::PV4 ? GM * B : 4];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stream = blockIdx.x / p.win_n;
  const int ci = blockIdx.x - stream * p.win_n;
  const int c = p.win_c0 + ci;
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  if (p.win_idx == 0) {
    // first window: clear the stop records (read from the next launch on)
    if (ci == 0 && threadIdx.x == 0) {
      p.win_dead[stream] = 0u;
      p.win_dwin[stream] = 0u;
    }
  } else if (p.win_dwin[stream] != 0u) {
    return;
  }
  const int L = p.seq_lens[s];
  const int n = visit_count<B>(p, s, L);
  const int nch = (n + C - 1) / C;
  if (c >= nch) return;
  const int t0 = c * C;
  const int nt = min(C, n - t0);
  const int slot = lane < C ? lane : C - 1;
  const int ob = p.block_order[(size_t)s * p.max_blocks + min(t0 + slot, n - 1)];
  const int pg = p.block_table[(size_t)s * p.max_blocks + ob];
  float ks = 1.f, vs = 1.f;
  if constexpr (KV == KV_FP8) {
    ks = p.k_scale[(size_t)pg * p.hkv + kvh];
    vs = p.v_scale[(size_t)pg * p.hkv + kvh];
  }
  BlockRegs<Cf> regs[1];
  issue_chunk_part<Cf, 1>(regs, p, kvh, L, ob, pg, nt, w, lane);
  uint4 qf[Cf::QF];
  load_q<Cf>(p, s, kvh, lane, qf);
  float* dst = p.win_slots + ((size_t)stream * p.win_max + ci) * p.win_slot;
  block_phase<Cf, 1>(regs, qf, ob, ks, vs, nt, L, p.qk_log2, w, lane, dst, pbuf_all[w]);
  // each head's chunk aggregate [A(D), m, l] after the partials (the fold
  // launch reads these first)
  __syncthreads();
  for (int h = w; h < p.g; h += C) {
    ChunkIn<Cf> in;
    win_gather<Cf>(in, dst, h, lane);
    float m, l, a[Cf::DPL];
    lb_aggregate<Cf>(in, m, l, a);
    float* gq = dst + Cf::SLOT + h * (D + 4);
#pragma unroll
    for (int j = 0; j < Cf::DPL; ++j) gq[Cf::DPL * lane + j] = a[j];
    if (lane == 0) { gq[D] = m; gq[D + 1] = l; }
  }
}

// Fold: workgroup q of K of (stream, head) hs = blockIdx.x / K.
template <int KV, int D, int B, int GM, int WMAXC>
__global__ __launch_bounds__(64 * WNW) void art_win_scan_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int C = Cf::C, DPL = Cf::DPL;
  constexpr int XS = D + 4;  // floats per chunk entry: A[D], M, L
  static_assert(WMAXC <= 64, "one lane per chunk of the window");
  __shared__ __attribute__((aligned(16))) float xs[WMAXC * XS];
  __shared__ uint32_t pas[WMAXC];  // one workgroup per head: its pass words stay here
  __shared__ float4 fsc[64];        // phase 2: per-chunk scalars of the chain
  __shared__ uint32_t arrived;
  const int bid = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = p.g;
  const int K = p.win_k;
  const int hs = bid / K;  // (stream, head)
  const int q = bid - hs * K;
  const int stream = hs / g;
  const int h = hs - stream * g;
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  const int L = p.seq_lens[s];
  const int n = visit_count<B>(p, s, L);
  const int nch = (n + C - 1) / C;
  const size_t head = (size_t)s * p.hq + (size_t)kvh * g + h;
  float* st = p.win_state + (size_t)hs * (D + 8);
  const bool first = p.win_c0 == 0;
  float* out_row = p.out + head * D;
  if (n == 0) {
    if (first && q == 0) {
      for (int i = threadIdx.x; i < D; i += 64 * WNW) out_row[i] = 0.f;
      if (threadIdx.x == 0) {
        p.stop_block[head] = 0;
        if (h == 0 && p.blocks_fetched) p.blocks_fetched[stream] = 0;
        atomicOr(p.win_dead + stream, 1u << h);
      }
    }
    return;
  }
  // state entering the window (read by every workgroup of the head before
  // any of them arrives below; only the last to arrive writes it)
  int cnt = 0;
  bool sink = false, alive = true;
  LbState<Cf> x0;
  x0.M = NEG_INF;
  x0.L = 0.f;
#pragma unroll
  for (int j = 0; j < DPL; ++j) x0.A[j] = 0.f;
  if (!first) {
    alive = st[D + 4] != 0.f;
    if (!alive) return;
    x0.M = st[D];
    x0.L = st[D + 1];
#pragma unroll
    for (int j = 0; j < DPL; ++j) x0.A[j] = st[DPL * lane + j];
    cnt = (int)st[D + 2];
    sink = st[D + 3] != 0.f;
  }
  const int c0 = p.win_c0;
  const int cend = min(nch, c0 + p.win_n);
  if (c0 >= cend) return;
  const int ncw = cend - c0;
  const float* slots = p.win_slots + (size_t)stream * p.win_max * p.win_slot;
  const int32_t* orow = p.block_order + (size_t)s * p.max_blocks;
  uint32_t* pw = p.win_pass + (size_t)hs * p.win_max;

  // (1) chunk aggregates, written by the partials launch, into LDS (a
  // wave's loads go out together)
  constexpr int U = (WMAXC + WNW - 1) / WNW;
  {
    float ga[U][DPL], gml[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ci = min(wv + WNW * u, ncw - 1);
      const float* gq = slots + (size_t)ci * p.win_slot + Cf::SLOT + h * (D + 4);
#pragma unroll
      for (int j = 0; j < DPL; ++j) ga[u][j] = gq[DPL * lane + j];
      gml[u] = gq[D + (lane & 1)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ci = wv + WNW * u;
      if (ci < ncw) {
        float* e = xs + ci * XS;
#pragma unroll
        for (int j = 0; j < DPL; ++j) e[DPL * lane + j] = ga[u][j];
        if (lane < 2) e[D + lane] = gml[u];
      }
    }
  }
  __syncthreads();
  // (2) the state entering each chunk, in chunk order (every workgroup of
  // the head, for all chunks of the window).  The running max is a prefix
  // max over the chunks (lane k: chunk k) and each step's two scale factors
  // follow from it, so the sequential part is one FMA per element and step
  // -- the same operations as lb_combine, in the same order.
  LbState<Cf> xw = x0;  // wave 0: the state after the window
  if (wv == 0) {
    const float mk = lane < ncw ? xs[lane * XS + D] : NEG_INF;
    const float lk = lane < ncw ? xs[lane * XS + D + 1] : 0.f;
    float mi = mk;  // max(m_0 .. m_lane)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float v = __shfl_up(mi, o);
      if (lane >= o) mi = fmaxf(mi, v);
    }
    const float mn = fmaxf(x0.M, mi);  // the running max after chunk `lane`
    float me = __shfl_up(mn, 1);       // ... and before it
    if (lane == 0) me = x0.M;
    const bool empty = mn == NEG_INF;
    const float fxv = empty ? 0.f : __builtin_amdgcn_exp2f(me - mn);
    const float fyv = empty ? 0.f : __builtin_amdgcn_exp2f(mk - mn);
    // each step's scalars (scale factors, the chunk's sum, the running max
    // entering it), one lane per chunk, into LDS: the chain reads them back
    // as broadcasts, prefetched with the aggregates, instead of a cross-lane
    // read per scalar and step (same values, so the same bits)
    fsc[lane] = make_float4(fxv, fyv, lk, me);
    constexpr int PF = 4;  // entries read ahead of the chain
    float na[PF][DPL];
    float4 nf[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
#pragma unroll
      for (int j = 0; j < DPL; ++j) na[u][j] = xs[min(u, ncw - 1) * XS + DPL * lane + j];
      nf[u] = fsc[min(u, ncw - 1)];
    }
    for (int cb = 0; cb < ncw; cb += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int ci = cb + u;
        if (ci < ncw) {
          float* e = xs + ci * XS;
          float a[DPL];
#pragma unroll
          for (int j = 0; j < DPL; ++j) a[j] = na[u][j];
          const float4 f = nf[u];  // fx, fy, l, running max entering the chunk
          if (ci + PF < ncw) {  // read before the chain overwrites that entry
#pragma unroll
            for (int j = 0; j < DPL; ++j) na[u][j] = e[PF * XS + DPL * lane + j];
            nf[u] = fsc[ci + PF];
          }
#pragma unroll
          for (int j = 0; j < DPL; ++j) e[DPL * lane + j] = xw.A[j];
          if (lane == 0) { e[D] = f.w; e[D + 1] = xw.L; }
          xw.L = fmaf(f.x, xw.L, f.y * f.z);
#pragma unroll
          for (int j = 0; j < DPL; ++j) xw.A[j] = fmaf(f.x, xw.A[j], f.y * a[j]);
        }
      }
    }
    xw.M = readlanef(mn, ncw - 1);
  }
  __syncthreads();
  // (3) pass bits of every position of this workgroup's chunks (wave w of
  // workgroup q takes chunks (q + K u) WNW + w) and the positions holding
  // block 0, published per chunk; the partials of a wave's next chunks are
  // loaded while one is evaluated
  ChunkIn<Cf> nx1, nx2;
  {
    const int c1 = q * WNW + wv, c2 = (q + K) * WNW + wv;
    if (c1 < ncw) win_gather<Cf>(nx1, slots + (size_t)c1 * p.win_slot, h, lane);
    if (c2 < ncw) win_gather<Cf>(nx2, slots + (size_t)c2 * p.win_slot, h, lane);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ci = (q + K * u) * WNW + wv;
    if (ci >= ncw) break;
    const int c = c0 + ci;
    const int t0 = c * C;
    const int nt = min(C, n - t0);
    const ChunkIn<Cf> in = nx1;
    nx1 = nx2;
    const int c3 = (q + K * (u + 2)) * WNW + wv;
    if (c3 < ncw) win_gather<Cf>(nx2, slots + (size_t)c3 * p.win_slot, h, lane);
    const float* e = xs + ci * XS;
    LbState<Cf> x;
#pragma unroll
    for (int j = 0; j < DPL; ++j) x.A[j] = e[DPL * lane + j];
    x.M = e[D];
    x.L = e[D + 1];
    float Op[DPL], np;
    lb_entering_output<Cf>(x, lane, p.probe, Op, np);
    float oo[C][DPL];
    const u64 pass = lb_stats<Cf>(x, Op, np, in, t0, nt, p, lane, oo);
    const int ob = orow[min(t0 + (lane < C ? lane : C - 1), n - 1)];
    const u64 sb = __ballot(lane < nt && ob == 0);
    const uint32_t word = ((uint32_t)pass & 0xFFu) | (((uint32_t)sb & 0xFFu) << 8);
    if (lane == 0) {
      if (K == 1)
        pas[ci] = word;
      else
        st_dev32(pw + ci, word);
    }
  }
  if (K > 1) {
    // the last workgroup of the head to get here applies the rule; nothing
    // waits: the others leave
    wait_all_memory();
    __syncthreads();
    if (threadIdx.x == 0)
      arrived = __hip_atomic_fetch_add(p.win_cnt + hs, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (uint32_t)(K - 1)) return;
  } else {
    __syncthreads();
  }
  // (4) the patience/block-0 rule over the window: lane c holds chunk c.
  // The passes in a row after chunk c follow R_c = a_c R_{c-1} + b_c (a_c = 1
  // when every position of chunk c passed, b_c = its length then, else its
  // trailing passes), composed lane-parallel; the block-0 flag is a prefix
  // OR.  Each lane then evaluates its own chunk's positions from the state
  // entering it; the first chunk that fires decides.
  if (wv == 0) {
    if (K > 1 && lane == 0) st_dev32(p.win_cnt + hs, 0u);  // zero again for the next launch
    const int cap = min(p.patience, 1 << 24);  // the carried count is stored as a float
    const bool lv = lane < ncw;
    const uint32_t wd = !lv ? 0u : (K == 1 ? pas[lane] : ld_dev32(pw + lane));
    const int ntl = lv ? min(C, n - (c0 + lane) * C) : 0;
    const uint32_t full = (1u << ntl) - 1u;
    const uint32_t pb = wd & full;
    const uint32_t sb = (wd >> 8) & full;
    const bool allp = lv && pb == full;
    const uint32_t zeros = ~pb & full;
    const int trail = zeros == 0u ? ntl : ntl - 1 - (31 - __builtin_clz(zeros));
    // inclusive scan of (a, b): (a2, b2) after (a1, b1) = (a2 a1, a2 b1 + b2)
    int a = (!lv || allp) ? 1 : 0;
    int b = lv ? (allp ? ntl : trail) : 0;
    int so = (lv && sb != 0u) ? 1 : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int pa = __shfl_up(a, o), pbv = __shfl_up(b, o), ps = __shfl_up(so, o);
      if (lane >= o) {
        b = a * pbv + b;
        a = a * pa;
        so = so | ps;
      }
    }
    // state entering chunk `lane`: the exclusive values
    int rin = __shfl_up(a * cnt + b, 1);  // R after chunk lane-1
    int sin = __shfl_up(so, 1);
    if (lane == 0) { rin = cnt; sin = 0; }
    const bool sink_in = sink || sin != 0;
    const int cnt_in = min(rin, cap);
    // positions of this lane's chunk
    int ft = -1;
    {
      int cc = cnt_in;
      bool sk = sink_in;
#pragma unroll
      for (int t = 0; t < C; ++t) {
        if (t < ntl && ft < 0) {
          cc = ((pb >> t) & 1u) ? min(cc + 1, cap) : 0;
          sk = sk || ((sb >> t) & 1u);
          if (cc >= p.patience && sk) ft = t;
        }
      }
    }
    const u64 fires = __ballot(lv && ft >= 0);
    int fire_ci = -1, fire_t = 0;
    if (fires != 0ull) {
      fire_ci = __builtin_ctzll(fires);
      fire_t = readlane(ft, fire_ci);
    } else {
      // no stop in the window: carry the count and the flag to the next one
      const int last = ncw - 1;
      cnt = min(readlane(a * cnt + b, last), cap);
      sink = sink || readlane(so, last) != 0;
    }
    const bool ends = cend == nch;
    if (fire_ci >= 0 || ends) {
      // the output at the stop (or after the last block), folded again
      const int ci = fire_ci >= 0 ? fire_ci : ncw - 1;
      const int c = c0 + ci;
      const int t0 = c * C;
      const int nt = min(C, n - t0);
      ChunkIn<Cf> in;
      win_gather<Cf>(in, slots + (size_t)ci * p.win_slot, h, lane);
      const float* e = xs + ci * XS;
      LbState<Cf> x;
#pragma unroll
      for (int j = 0; j < DPL; ++j) x.A[j] = e[DPL * lane + j];
      x.M = e[D];
      x.L = e[D + 1];
      float Op[DPL], np;
      lb_entering_output<Cf>(x, lane, p.probe, Op, np);
      float oo[C][DPL];
      (void)lb_stats<Cf>(x, Op, np, in, t0, nt, p, lane, oo);
      float ov[DPL];
#pragma unroll
      for (int j = 0; j < DPL; ++j) ov[j] = Op[j];
      if (fire_ci >= 0) {
#pragma unroll
        for (int t = 0; t < C; ++t)
          if (fire_t == t)
#pragma unroll
            for (int j = 0; j < DPL; ++j) ov[j] = oo[t][j];
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) out_row[DPL * lane + j] = ov[j];
      if (lane == 0) p.stop_block[head] = fire_ci >= 0 ? t0 + fire_t + 1 : n;
      alive = false;
    }
    // the state carried to the next window
#pragma unroll
    for (int j = 0; j < DPL; ++j) st[DPL * lane + j] = xw.A[j];
    if (lane == 0) {
      st[D] = xw.M;
      st[D + 1] = xw.L;
      st[D + 2] = (float)cnt;
      st[D + 3] = sink ? 1.f : 0.f;
      st[D + 4] = alive ? 1.f : 0.f;
      if (!alive) {
        // the head completing the mask records the window in which the
        // stream stopped and the blocks it loaded (through this window)
        const uint32_t bit = 1u << h;
        const uint32_t was = atomicOr(p.win_dead + stream, bit);
        if ((was | bit) == (1u << g) - 1u && was != (was | bit)) {
          p.win_dwin[stream] = (uint32_t)p.win_idx + 1u;
          if (p.blocks_fetched) p.blocks_fetched[stream] = min(n, cend * C);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Full-attention split kernel
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));

// P V for one block on bf16 MFMA, V as load_block<Cf, NT, true> holds it.
// Four of a lane's dwords (token rows 4q .. 4q+3, bytes 8c + 4k .. 8c + 4k
// + 3, k = 0, 1) form a 4x4 byte matrix; two byte permutations pair the
// rows' bytes so that each bf16 conversion yields two consecutive tokens of
// one d.  So d-tile j = 4 k + e (e = 0..3) takes, in row m = c, the element
// d = 8 c + j: A = that V^T tile (lane (c, q): tokens 4q .. 4q+3), B = P^T
// (lane: head c, tokens 4q .. 4q+3: the score layout itself), P split into
// bf16 hi + lo (truncation: P = hi + lo + O(2^-16 P)).  acc[j] then holds,
// in lane (c, q) component i, head c at d = 8 (4 q + i) + j.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <class Cf>
__device__ __forceinline__ void pvb_block(const BlockRegs<Cf>& r, const float (&pq)[Cf::T][4], f32x4 (&acc)[Cf::NACCF]) {
  static_assert(Cf::NACCF == 8, "eight d-tiles of 16");
#pragma unroll
  for (int t = 0; t < Cf::T; ++t) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b = fbits(pq[t][i]);
      hi[i] = b & 0xffff0000u;
      lo[i] = fbits(pq[t][i] - bitsf(hi[i])) & 0xffff0000u;
    }
    s16x4 ph, pl;
    {
      const uint32_t h0 = (hi[0] >> 16) | hi[1], h1 = (hi[2] >> 16) | hi[3];
      const uint32_t l0 = (lo[0] >> 16) | lo[1], l1 = (lo[2] >> 16) | lo[3];
      ph = __builtin_bit_cast(s16x4, make_uint2(h0, h1));
      pl = __builtin_bit_cast(s16x4, make_uint2(l0, l1));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t w[4] = {r.v[8 * t + k], r.v[8 * t + 2 + k], r.v[8 * t + 4 + k], r.v[8 * t + 6 + k]};
      // bytes (row 0, row 1) of columns 0 and 2, of columns 1 and 3; likewise rows 2, 3
      const uint32_t a01 = __builtin_amdgcn_perm(w[1], w[0], 0x06020400u);
      const uint32_t b01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030501u);
      const uint32_t a23 = __builtin_amdgcn_perm(w[3], w[2], 0x06020400u);
      const uint32_t b23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030501u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = (e & 1) ? b01 : a01, y = (e & 1) ? b23 : a23;
        const uint2 xy = e >= 2 ? make_uint2(fp8x2_to_bf16x2<true>(x), fp8x2_to_bf16x2<true>(y))
                                : make_uint2(fp8x2_to_bf16x2<false>(x), fp8x2_to_bf16x2<false>(y));
        const s16x4 a = __builtin_bit_cast(s16x4, xy);
        f32x4& o = acc[4 * k + e];
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ph, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pl, o, 0, 0, 0);
      }
    }
  }
}

template <class Cf>
__device__ __forceinline__ void full_block(const BlockRegs<Cf>& r, int nvalid, float ksc, float vsc,
                                           const uint4 (&qf)[Cf::QF], float qk_log2, int lane, float& m_run,
                                           float& l_run, f32x4 (&acc)[Cf::NACCF], float* pbuf) {
  f32x4 S[Cf::T];
  qk_scores<Cf>(r, qf, S);
  float x[Cf::T][4];
  const float mb = block_scores<Cf>(S, nvalid, qk_log2 * ksc, lane, x);
  const float mn = fmaxf(m_run, mb);
  const float al = __builtin_amdgcn_exp2f(m_run - mn);
  float ls = 0.f;
  float pq[Cf::T][4];
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float e = __builtin_amdgcn_exp2f(x[t][rr] - mn);
      ls += e;
      pq[t][rr] = e * vsc;
    }
  ls = rows_sum(ls);
  l_run = fmaf(al, l_run, ls);
  m_run = mn;
  // Once the running maxima settle, every factor is exactly 2^0 = 1 and the
  // rescale would leave the accumulators unchanged bit for bit: it is skipped
  // unless some head's maximum moved (a wave-uniform test).
  const bool rescale = __ballot((lane & 15) < Cf::GM && al != 1.f) != 0ull;
  if constexpr (Cf::PVB) {
    if (rescale) {
#pragma unroll
      for (int j = 0; j < Cf::NACCF; ++j) acc[j] *= al;  // lane (c, q) holds head c
    }
    pvb_block<Cf>(r, pq, acc);
  } else {
    if (rescale) pv_rescale<Cf>(acc, al);
    pv_block<Cf>(r, pq, pbuf, lane, acc);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ long long wave_incl_scan(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Full attention over a balanced partition: the blocks of all streams
// (sequence, kv-head), kv-head fastest and in logical order within a
// stream, form one flattened list of W blocks; workgroup i of G folds
// positions [floor(i W / G), floor((i + 1) W / G)), whatever streams they
// belong to, so every workgroup gets the same number of blocks however
// ragged the sequences are.  Each piece (a workgroup's part of one stream)
// leaves a partial (max, sum, numerator per head) in slot s + i of the
// workspace (injective: stream s's pieces take consecutive workgroups), and
// the stream's last piece to finish merges its pieces in order.
// Waves per SIMD the full-attention kernel is compiled for: three for fp8 KV
// with 16-token blocks (the register budget then drops from 178 to 136, no
// spills; 212-243 -> 204 us on the fp8 Qwen shape, box to box), else what
// the compiler picks.
template <int KV, int B>
struct FullWaves {
  static constexpr int v = (KV == KV_FP8 && B == 16) ? 3 : 1;
};
template <int KV, int D, int B, int GM>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(FullWaves<KV, B>::v))) void full_split_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int HPW = (GM + NW - 1) / NW, DPL = Cf::DPL;
  __shared__ __attribute__((aligned(16))) float mw_a[NW][GM][D];
  __shared__ float mw_m[NW][GM];
  __shared__ float mw_l[NW][GM];
  __shared__ __attribute__((aligned(16))) float pbuf_all[NW][Cf::PV4 && !Cf::PVB ? GM * B : 4];
  __shared__ long long plan[4];  // W, first position, end position, flattened start of the first sequence
  __shared__ int plan_sq;        // the sequence holding the first position
  __shared__ int is_last;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int hkv = p.hkv;
  const int streams = p.batch * hkv;
  const int g = p.g;

  // streams without visits: out = 0, stop = 0 (no position belongs to them)
  for (int st = wg; st < streams; st += G) {
    const int sq = st / hkv;
    if (visit_count<B>(p, sq, p.seq_lens[sq]) <= 0) {
      const size_t head0 = (size_t)sq * p.hq + (size_t)(st - sq * hkv) * g;
      for (int i = threadIdx.x; i < g * D; i += blockDim.x) p.out[head0 * D + i] = 0.f;
      if ((int)threadIdx.x < g) p.stop_block[head0 + threadIdx.x] = 0;
      if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[st] = 0;
    }
  }

  // wave 0: the total W, this workgroup's range and the sequence holding its
  // first position (two sweeps over the sequences, 64 at a time)
  if (w == 0) {
    long long tot = 0;
    for (int base = 0; base < p.batch; base += 64) {
      const int sq = base + lane;
      const long long nb = sq < p.batch ? (long long)visit_count<B>(p, sq, p.seq_lens[sq]) * hkv : 0;
      tot += __shfl(wave_incl_scan(nb, lane), 63);
    }
    // with fewer blocks than workgroups, the first W workgroups take one each
    const long long Ge = tot < G ? tot : G;
    const long long a = wg < Ge ? tot * wg / Ge : 0, e = wg < Ge ? tot * (wg + 1) / Ge : 0;
    long long before = 0;
    int found = -1;
    long long fstart = 0;
    for (int base = 0; base < p.batch && found < 0 && a < e; base += 64) {
      const int sq = base + lane;
      const long long nb = sq < p.batch ? (long long)visit_count<B>(p, sq, p.seq_lens[sq]) * hkv : 0;
      const long long inc = before + wave_incl_scan(nb, lane);
      const unsigned long long hit = __ballot(sq < p.batch && nb > 0 && inc > a && inc - nb <= a);
      if (hit != 0ull) {
        const int l = __builtin_ctzll(hit);
        found = base + l;
        fstart = __shfl(inc - nb, l);
      }
      before = __shfl(inc, 63);
    }
    if (lane == 0) {
      plan[0] = tot;
      plan[1] = a;
      plan[2] = e;
      plan[3] = fstart;
      plan_sq = found;
    }
  }
  __syncthreads();
  const long long W = plan[0];
  long long pos = plan[1];
  const long long end = plan[2];
  if (pos >= end || plan_sq < 0) return;
  const long long Ge = W < G ? W : G;  // workgroups with a non-empty range
  // the workgroup holding flattened position x: the largest i with floor(i W / Ge) <= x
  auto wg_of = [&](long long x) { return (int)(((x + 1) * Ge - 1) / W); };

  int sq = plan_sq;
  int L = p.seq_lens[sq];
  int n = visit_count<B>(p, sq, L);
  int kvh = (int)((pos - plan[3]) / n);
  int off = (int)(pos - plan[3] - (long long)kvh * n);

  uint4 qf[Cf::QF];
  const size_t tile = (size_t)B * Cf::R;
  const char* kbase = static_cast<const char*>(p.k_pages);
  const char* vbase = static_cast<const char*>(p.v_pages);
  float* pbuf = pbuf_all[w];

  while (pos < end) {
    const int s = sq * hkv + kvh;
    const int len = (int)min((long long)(n - off), end - pos);
    const size_t head0 = (size_t)sq * p.hq + (size_t)kvh * g;
    const int32_t* trow = p.block_table + (size_t)sq * p.max_blocks;
    load_q<Cf>(p, sq, kvh, lane, qf);

    // ---- this wave's blocks of the piece: off + w + NW k, in sub-ranges of
    // 64 (one lane-held page table each), the state carried across them
    float m_run = NEG_INF, l_run = 0.f;
    f32x4 acc[Cf::NACCF];
#pragma unroll
    for (int jj = 0; jj < Cf::NACCF; ++jj) acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int cnt_all = w < len ? (len - w + NW - 1) / NW : 0;
    for (int k0 = 0; k0 < cnt_all; k0 += 64) {
      const int cnt = min(64, cnt_all - k0);
      int tab = 0, blk = 0;
      float ks_t = 1.f, vs_t = 1.f;
      {
        const int t = off + w + NW * (k0 + min(lane, cnt - 1));
        blk = p.visit_lens ? p.block_order[(size_t)sq * p.max_blocks + t] : t;
        tab = trow[blk];
        if constexpr (KV == KV_FP8) {
          ks_t = p.k_scale[(size_t)tab * hkv + kvh];
          vs_t = p.v_scale[(size_t)tab * hkv + kvh];
        }
      }
      auto nvalid_of = [&](int k) { return min(B, L - readlane(blk, k) * B); };
      auto tile_of = [&](int k) { return ((size_t)readlane(tab, k) * hkv + kvh) * tile; };
      auto fold = [&](const BlockRegs<Cf>& r, int k) {
        float ks = 1.f, vs = 1.f;
        if constexpr (KV == KV_FP8) { ks = readlanef(ks_t, k); vs = readlanef(vs_t, k); }
        full_block<Cf>(r, nvalid_of(k), ks, vs, qf, p.qk_log2, lane, m_run, l_run, acc, pbuf);
      };
      // Register ring of PF block buffers: while block k is folded, blocks
      // k+1 .. k+PF-1 are in flight.  Loads are unconditional (past the last
      // block they re-read that block, a cache hit), so every fold site has
      // the same PF-1 blocks of younger loads outstanding and the waits are exact.
      constexpr int PF = FULL_PREFETCH;
      BlockRegs<Cf> ring[PF];
#pragma unroll
      for (int jj = 0; jj < PF - 1; ++jj) {
        const int kk = min(jj, cnt - 1);
        const size_t o = tile_of(kk);
        load_block<Cf, true, Cf::PVB>(ring[jj], kbase + o, vbase + o, lane, nvalid_of(kk));
      }
      for (int k = 0; k < cnt; k += PF) {
#pragma unroll
        for (int jj = 0; jj < PF; ++jj) {
          const int kk = min(k + jj + PF - 1, cnt - 1);
          const size_t o = tile_of(kk);
          load_block<Cf, true, Cf::PVB>(ring[(jj + PF - 1) % PF], kbase + o, vbase + o, lane, nvalid_of(kk));
          __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
          if (k + jj < cnt) fold(ring[jj], k + jj);
        }
      }
    }

    // ---- merge the four waves
    {
      const int c = lane & 15;
      if constexpr (Cf::PVB) {
        if (c < GM) {
          const int q = lane >> 4;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 2; ++k)
              *reinterpret_cast<f32x4*>(&mw_a[w][c][8 * (4 * q + i) + 4 * k]) =
                  f32x4{acc[4 * k][i], acc[4 * k + 1][i], acc[4 * k + 2][i], acc[4 * k + 3][i]};
        }
      } else {
        pv_finish<Cf>(acc);
        pv_store<Cf>(&mw_a[w][0][0], lane, acc, 1.f);
      }
      if (c < GM && (lane >> 4) == 0) { mw_m[w][c] = m_run; mw_l[w][c] = l_run; }
    }
    __syncthreads();
    const long long sstart = pos - off;  // flattened start of stream s
    const int first = wg_of(sstart), last = wg_of(sstart + n - 1);
    const bool alone = first == last;  // the whole stream is this piece
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      const int h = w + NW * k;
      if (h >= g) continue;
      float M = NEG_INF;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mw_m[ww][h]);
      float Ls = 0.f;
      float A[DPL];
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj) A[jj] = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = mw_m[ww][h];
        const float f = (mw == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        Ls = fmaf(f, mw_l[ww][h], Ls);
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) A[jj] = fmaf(f, mw_a[ww][h][lane + 64 * jj], A[jj]);
      }
      if (alone) {
        const float rl = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) p.out[(head0 + h) * D + lane + 64 * jj] = A[jj] * rl;
        if (lane == 0) p.stop_block[head0 + h] = n;
      } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(p.ws_part + ((size_t)(s + wg) * GM + h) * (D + 2));
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) st_dev32(dst + lane + 64 * jj, __float_as_uint(A[jj]));
        if (lane == 0) { st_dev32(dst + D, __float_as_uint(M)); st_dev32(dst + D + 1, __float_as_uint(Ls)); }
      }
    }
    if (alone) {
      if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[s] = n;
    } else {
      // The stream's last piece to finish merges all of them: every piece's
      // partials are complete (device-coherent stores, waited for) before
      // its count goes in; the piece that brings the count to the number of
      // pieces resets it for the next call and folds the partials, in piece
      // order, with device-coherent loads.
      const int pieces = last - first + 1;
      wait_all_memory();
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(p.full_cnt + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == (uint32_t)(pieces - 1) ? 1 : 0;
        if (is_last) st_dev32(p.full_cnt + s, 0u);
      }
      __syncthreads();
      if (is_last) {
        const size_t sstride = (size_t)GM * (D + 2);
        for (int h = w; h < g; h += NW) {
          const uint32_t* src = reinterpret_cast<const uint32_t*>(p.ws_part + ((size_t)(s + first) * GM + h) * (D + 2));
          // common maximum over the pieces (lane-parallel, they may exceed 64)
          float M = NEG_INF;
          for (int sp = lane; sp < pieces; sp += 64) M = fmaxf(M, __uint_as_float(ld_dev32(src + sp * sstride + D)));
          M = rows_max(M);
          M = fmaxf(M, dpp<DPP_ROW_MIRROR>(M));
          M = fmaxf(M, dpp<DPP_HALF_MIRROR>(M));
          M = fmaxf(M, dpp<DPP_XOR2>(M));
          M = fmaxf(M, dpp<DPP_XOR1>(M));
          // weighted numerators: every lane owns D/64 output elements
          float Ls = 0.f;
          float A[DPL];
#pragma unroll
          for (int jj = 0; jj < DPL; ++jj) A[jj] = 0.f;
          int sp = 0;
          for (; sp + 4 <= pieces; sp += 4) {
            float ms[4], ls[4], a[4][DPL];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint32_t* q = src + (size_t)(sp + u) * sstride;
              ms[u] = __uint_as_float(ld_dev32(q + D));
              ls[u] = __uint_as_float(ld_dev32(q + D + 1));
#pragma unroll
              for (int jj = 0; jj < DPL; ++jj) a[u][jj] = __uint_as_float(ld_dev32(q + lane + 64 * jj));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float f = (ms[u] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - M);
              Ls = fmaf(f, ls[u], Ls);
#pragma unroll
              for (int jj = 0; jj < DPL; ++jj) A[jj] = fmaf(f, a[u][jj], A[jj]);
            }
          }
          for (; sp < pieces; ++sp) {
            const uint32_t* q = src + (size_t)sp * sstride;
            const float ms = __uint_as_float(ld_dev32(q + D));
            const float f = (ms == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
            Ls = fmaf(f, __uint_as_float(ld_dev32(q + D + 1)), Ls);
#pragma unroll
            for (int jj = 0; jj < DPL; ++jj) A[jj] = fmaf(f, __uint_as_float(ld_dev32(q + lane + 64 * jj)), A[jj]);
          }
          const float rl = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
          for (int jj = 0; jj < DPL; ++jj) p.out[(head0 + h) * D + lane + 64 * jj] = A[jj] * rl;
          if (lane == 0) p.stop_block[head0 + h] = n;
        }
        if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[s] = n;
      }
    }
    __syncthreads();  // mw_* are rewritten by the next piece

    // ---- the next stream (kv-head fastest; sequences without visits hold no position)
    pos += len;
    off = 0;
    if (pos >= end) break;
    if (++kvh == hkv) {
      kvh = 0;
      do {
        ++sq;
        L = p.seq_lens[sq];
        n = visit_count<B>(p, sq, L);
      } while (n <= 0);
    }
  }
}

}  // namespace kern
}  // namespace art
