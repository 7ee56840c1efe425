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
//  * art_chunk_kernel -- the terminating path.  One workgroup (NWA waves)
//    owns one stream = (sequence, kv-head) and walks its visit order in
//    chunks of C blocks.  Each wave turns one block into partials
//    (m_b, l_b, a_b) in LDS; then one wave per query head folds the partials
//    in visit order, forms O_t = A_t / L_t for every t of the chunk, reduces
//    ‖O_t‖² and ‖O_t - O_{t-1}‖² for all t at once (transposed butterfly),
//    evaluates both statistics and the patience rule for all t in parallel
//    (one lane per t, bit masks).  A head that stops writes O_t and is frozen;
//    the stream stops fetching when every head of its group stopped.  The KV
//    loads of chunk c+1 are issued before chunk c is scanned (speculatively),
//    and page entries run two chunks ahead.
//
//  * full_split_kernel -- full attention (no detector).  Each workgroup owns
//    a contiguous slice of one stream's blocks; each wave keeps its own
//    online-softmax state with the next block's loads in flight; waves merge
//    through LDS; slices are merged by full_merge_kernel (second launch).
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
#define FULL_PREFETCH 3  // blocks in the full kernel's register ring
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
  static constexpr int C = cmin(8, 8192 / (GM * D));
  static constexpr int NWA = cmin(8, C);              // waves per workgroup, ART kernel
  static constexpr int BPW = C / NWA;                 // blocks per wave per chunk
  static constexpr int HPW = (GM + NWA - 1) / NWA;    // query heads per wave in the scan
  static constexpr int DPL = D / 64;                  // d per lane in the scan
  static constexpr int SH = 6 - ilog2(2 * C);         // stat reduction: lane >> SH = value index
  static_assert(BPW >= 1 && BPW * NWA == C, "chunk must split evenly over the waves");
  static_assert(2 * C <= 64, "stat reduction holds at most 64 values");
  static_assert(VWD >= 1, "a lane reads at least one dword of each V row");
};

template <class Cf>
struct BlockRegs {
  uint4 k[Cf::T][Cf::NKL];
  uint32_t v[Cf::T][4][Cf::VWD];
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

// 4 fp8 bytes -> 2 dwords of packed bf16 (exact: E4M3 values fit bf16).
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  float f[4];
  fp8x4_to_f32(w, f);
  uint2 r;
  r.x = (__float_as_uint(f[1]) & 0xffff0000u) | (__float_as_uint(f[0]) >> 16);
  r.y = (__float_as_uint(f[3]) & 0xffff0000u) | (__float_as_uint(f[2]) >> 16);
  return r;
}

// Load one block: K in the QK A-operand layout, V in the PV A-operand layout.
// V rows at or past nvalid are read from the last valid row instead, so that
// every V value fed to the PV product is finite (their P is exactly 0).
template <class Cf>
__device__ __forceinline__ void load_block(BlockRegs<Cf>& r, const char* kt, const char* vt, int lane, int nvalid) {
  const int c = lane & 15;
  const int q = lane >> 4;
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i)
      r.k[t][i] = *reinterpret_cast<const uint4*>(kt + (size_t)(16 * t + c) * Cf::R + q * 16 + 64 * i);
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = 16 * t + 4 * q + rr;
      const char* src = vt + (size_t)min(row, nvalid - 1) * Cf::R + c * Cf::VBL;
      if constexpr (Cf::VWD == 1) {
        r.v[t][rr][0] = *reinterpret_cast<const uint32_t*>(src);
      } else if constexpr (Cf::VWD == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(src);
        r.v[t][rr][0] = x.x; r.v[t][rr][1] = x.y;
      } else {
#pragma unroll
        for (int h = 0; h < Cf::VWD / 4; ++h) {
          const uint4 x = *reinterpret_cast<const uint4*>(src + 16 * h);
          r.v[t][rr][4 * h + 0] = x.x; r.v[t][rr][4 * h + 1] = x.y;
          r.v[t][rr][4 * h + 2] = x.z; r.v[t][rr][4 * h + 3] = x.w;
        }
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
__device__ __forceinline__ void v_row(const uint32_t (&w)[Cf::VWD], float (&f)[Cf::DT]) {
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

// acc += V^T P over the block: acc[dt] is the 16x16 tile of O^T whose rows are
// d = DT * m + dt (m = 0..15) and whose columns are the heads of the group.
template <class Cf>
__device__ __forceinline__ void pv_mfma(const BlockRegs<Cf>& r, const float (&pq)[Cf::T][4], f32x4 (&acc)[Cf::DT]) {
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float vf[Cf::DT];
      v_row<Cf>(r.v[t][rr], vf);
#pragma unroll
      for (int dt = 0; dt < Cf::DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[dt], pq[t][rr], acc[dt], 0, 0, 0);
    }
}

// Store a lane's O^T accumulator row (head c) as D-contiguous floats:
// dst points at [head][0]; the lane writes d = DT*(4q+i) + dt.
template <class Cf>
__device__ __forceinline__ void store_acc(float* dst, int lane, const f32x4 (&acc)[Cf::DT], float scale) {
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

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlanef(float v, int l) { return bitsf(__builtin_amdgcn_readlane(fbits(v), l)); }

// ---------------------------------------------------------------------------
// Terminating kernel
// ---------------------------------------------------------------------------
template <int KV, int D, int B, int GM>
__global__ __launch_bounds__((64 * Cfg<KV, D, B, GM>::NWA)) void art_chunk_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int C = Cf::C, NWA = Cf::NWA, BPW = Cf::BPW, HPW = Cf::HPW, DPL = Cf::DPL, SH = Cf::SH;
  __shared__ __attribute__((aligned(16))) float part_a[C][GM][D];
  __shared__ float part_m[C][GM];
  __shared__ float part_l[C][GM];
  __shared__ int alive_lds[GM];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stream = blockIdx.x;
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  const int g = p.g;
  const int L = p.seq_lens[s];
  const int n = (L + B - 1) / B;
  const size_t head0 = (size_t)s * p.hq + (size_t)kvh * g;

  if (n <= 0) {
    for (int i = threadIdx.x; i < g * D; i += 64 * NWA) p.out[head0 * D + i] = 0.f;
    if (threadIdx.x < g) p.stop_block[head0 + threadIdx.x] = 0;
    if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[stream] = 0;
    return;
  }

  uint4 qf[Cf::QF];
  load_q<Cf>(p, s, kvh, lane, qf);

  const size_t tile = (size_t)B * Cf::R;
  const char* kbase = static_cast<const char*>(p.k_pages);
  const char* vbase = static_cast<const char*>(p.v_pages);
  const int32_t* trow = p.block_table + (size_t)s * p.max_blocks;
  const int32_t* orow = p.block_order + (size_t)s * p.max_blocks;
  const int c16 = lane & 15;
  const int slot = lane < C ? lane : C - 1;

  // Chunk entries are lane-held (lane = slot): logical block and page of the
  // current chunk (c) and of the next (n); entries of chunk c+2 are fetched
  // while chunk c is scanned, so no KV load waits on the tables.
  int ob_c = orow[min(slot, n - 1)];
  int ob_n = orow[min(C + slot, n - 1)];
  int pg_c = trow[ob_c];
  int pg_n = trow[ob_n];
  float ks_c = 1.f, vs_c = 1.f;

  BlockRegs<Cf> regs[BPW];
  auto issue_chunk = [&](int ob_lane, int pg_lane, int nt_chunk) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = min(w * BPW + i, nt_chunk - 1);  // slots past the end re-read a valid block (cache hit)
      const int nvalid = min(B, L - readlane(ob_lane, b) * B);
      const size_t off = ((size_t)readlane(pg_lane, b) * p.hkv + kvh) * tile;
      load_block<Cf>(regs[i], kbase + off, vbase + off, lane, nvalid);
    }
  };
  issue_chunk(ob_c, pg_c, min(C, n));
  if constexpr (KV == KV_FP8) {
    ks_c = p.k_scale[(size_t)pg_c * p.hkv + kvh];
    vs_c = p.v_scale[(size_t)pg_c * p.hkv + kvh];
  }

  // Per-head streaming state, carried across chunks (head h = w + NWA * k).
  float cM[HPW], cL[HPW], cNp[HPW];
  int cCnt[HPW];
  bool cAlive[HPW], cSink[HPW];
  float cA[HPW][DPL], cOp[HPW][DPL];
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    cM[k] = NEG_INF; cL[k] = 0.f; cNp[k] = 0.f; cCnt[k] = 0; cSink[k] = false;
    cAlive[k] = (w + NWA * k) < g;
#pragma unroll
    for (int j = 0; j < DPL; ++j) { cA[k][j] = 0.f; cOp[k][j] = 0.f; }
  }

  int fetched = min(C, n);
  for (int t0 = 0; t0 < n; t0 += C) {
    const int nt = min(C, n - t0);

    // ---- block phase: per-block partials (m_b, l_b, a_b) into LDS; slots past
    // the chunk end get neutral partials (m = -inf, l = 0, a = 0).
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = w * BPW + i;
      if (b < nt) {
        const int nvalid = min(B, L - readlane(ob_c, b) * B);
        float ksc = 1.f, vsc = 1.f;
        if constexpr (KV == KV_FP8) { ksc = readlanef(ks_c, b); vsc = readlanef(vs_c, b); }
        f32x4 S[Cf::T];
        qk_scores<Cf>(regs[i], qf, S);
        float x[Cf::T][4];
        const float mb = block_scores<Cf>(S, nvalid, p.qk_log2 * ksc, lane, x);
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
        f32x4 acc[Cf::DT];
#pragma unroll
        for (int dt = 0; dt < Cf::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        pv_mfma<Cf>(regs[i], pq, acc);
        if (c16 < GM) {
          store_acc<Cf>(&part_a[b][c16][0], lane, acc, 1.f);
          if ((lane >> 4) == 0) { part_m[b][c16] = mb; part_l[b][c16] = ls; }
        }
      } else {
        if (c16 < GM && (lane >> 4) == 0) { part_m[b][c16] = NEG_INF; part_l[b][c16] = 0.f; }
        for (int e = lane; e < GM * D; e += 64) (&part_a[b][0][0])[e] = 0.f;
      }
    }

    // ---- speculative fetch of the next chunk: its loads fly during the scan
    const bool has_next = t0 + C < n;
    int ob_nn = 0;
    float ks_n = 1.f, vs_n = 1.f;
    if (has_next) {
      const int nt1 = min(C, n - t0 - C);
      issue_chunk(ob_n, pg_n, nt1);
      __builtin_amdgcn_sched_barrier(0);  // the loads must leave before the scan
      if constexpr (KV == KV_FP8) {
        ks_n = p.k_scale[(size_t)pg_n * p.hkv + kvh];
        vs_n = p.v_scale[(size_t)pg_n * p.hkv + kvh];
      }
      ob_nn = orow[min(t0 + 2 * C + slot, n - 1)];
      fetched += nt1;
    }
    __syncthreads();

    // ---- scan phase: fold the chunk's partials in visit order, one wave per head
    const unsigned long long sinkbits = __ballot(lane < nt && ob_c == 0);
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      const int h = w + NWA * k;
      if (h < g && cAlive[k]) {
        // branch-free over all C slots: neutral slots leave (M, L, A) unchanged
        float st[2 * C];
#pragma unroll
        for (int t = 0; t < C; ++t) {
          const float mb = part_m[t][h];
          const float lb = part_l[t][h];
          const float Mn = fmaxf(cM[k], mb);
          const float al = __builtin_amdgcn_exp2f(cM[k] - Mn);
          const float be = __builtin_amdgcn_exp2f(mb - Mn);
          cL[k] = fmaf(al, cL[k], be * lb);
          cM[k] = Mn;
          const float rl = __builtin_amdgcn_rcpf(cL[k]);  // 1 ulp; the statistics need ~1e-6
          float nn = 0.f, ee = 0.f;
#pragma unroll
          for (int j = 0; j < DPL; ++j) {
            float* sl = &part_a[t][h][lane + 64 * j];
            cA[k][j] = fmaf(al, cA[k][j], be * *sl);
            const float o = cA[k][j] * rl;
            const float df = o - cOp[k][j];
            nn = fmaf(o, o, nn);
            ee = fmaf(df, df, ee);
            cOp[k][j] = o;
            *sl = o;  // keep O_t for the epilogue
          }
          st[2 * t] = nn;
          st[2 * t + 1] = ee;
        }
        const float v0 = xreduce<2 * C>(st, lane);
        // lane (2t) << SH holds ‖O_t‖², lane (2t+1) << SH holds ‖O_t - O_{t-1}‖²;
        // gather them so that lane t < C evaluates position t.
        const float nn_t = __shfl(v0, (2 * slot) << SH);
        const float ee_t = __shfl(v0, (2 * slot + 1) << SH);
        float np_t = __shfl(v0, (2 * max(slot - 1, 0)) << SH);
        if (lane == 0) np_t = cNp[k];
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
            // 1 - cos = (‖O_t - O_{t-1}‖² - (‖O_t‖ - ‖O_{t-1}‖)²) / (2 ‖O_t‖ ‖O_{t-1}‖)
            dd = (a == 0.f) ? 1.f : fmaxf(0.f, (ee_t - df * df) * __builtin_amdgcn_rcpf(2.f * a * bn));
          }
          ps = (dm < p.eps_mag) && (dd < p.eps_dir);
        }
        // patience rule for every position at once: lane t counts the passes
        // in a row that end at t (carrying the count from earlier chunks when
        // every test of this chunk up to t passed) and whether block 0 has
        // been folded by t.
        const unsigned long long pass = __ballot(ps);
        const unsigned long long upto = (2ull << slot) - 1ull;
        const unsigned long long zeros = ~pass & upto;
        const int cnt_t = zeros == 0ull ? cCnt[k] + slot + 1 : slot - (63 - __builtin_clzll(zeros));
        const bool sink_t = cSink[k] || (sinkbits & upto) != 0ull;
        const unsigned long long fire = __ballot(lane < nt && cnt_t >= p.patience && sink_t);
        if (fire != 0ull) {
          const int stop_t = __builtin_ctzll(fire);
          float* o = p.out + (head0 + h) * D;
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[lane + 64 * j] = part_a[stop_t][h][lane + 64 * j];
          if (lane == 0) p.stop_block[head0 + h] = t0 + stop_t + 1;
          cAlive[k] = false;
        } else {
          cCnt[k] = readlane(cnt_t, nt - 1);
          cSink[k] = readlane(sink_t ? 1 : 0, nt - 1) != 0;
          cNp[k] = readlanef(nn_t, nt - 1);
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < HPW; ++k)
        if (w + NWA * k < g) alive_lds[w + NWA * k] = cAlive[k] ? 1 : 0;
    }
    __syncthreads();
    int any = 0;
    for (int h = 0; h < g; ++h) any |= alive_lds[h];
    if (!any || !has_next) break;
    // rotate the lane-held entries; the page of chunk c+2 is looked up now
    ob_c = ob_n;
    pg_c = pg_n;
    ob_n = ob_nn;
    pg_n = trow[ob_nn];
    ks_c = ks_n;
    vs_c = vs_n;
  }

  // heads that never stopped: output after all n blocks
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = w + NWA * k;
    if (h < g && cAlive[k]) {
      float* o = p.out + (head0 + h) * D;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[lane + 64 * j] = cOp[k][j];
      if (lane == 0) p.stop_block[head0 + h] = n;
    }
  }
  if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[stream] = fetched;
  // speculative loads of a chunk that was not needed may still be in flight
  __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------------------
// Full-attention split kernel
// ---------------------------------------------------------------------------
template <class Cf>
__device__ __forceinline__ void full_block(const BlockRegs<Cf>& r, int nvalid, float ksc, float vsc,
                                           const uint4 (&qf)[Cf::QF], float qk_log2, int lane, float& m_run,
                                           float& l_run, f32x4 (&acc)[Cf::DT]) {
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
  // the lane's accumulator column is its own head: rescale in place
#pragma unroll
  for (int dt = 0; dt < Cf::DT; ++dt) acc[dt] *= al;
  pv_mfma<Cf>(r, pq, acc);
}

template <int KV, int D, int B, int GM>
__global__ __launch_bounds__(WG) void full_split_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int HPW = (GM + NW - 1) / NW, DPL = Cf::DPL;
  __shared__ __attribute__((aligned(16))) float mw_a[NW][GM][D];
  __shared__ float mw_m[NW][GM];
  __shared__ float mw_l[NW][GM];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x % p.splits;
  const int stream = blockIdx.x / p.splits;
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  const int g = p.g;
  const int L = p.seq_lens[s];
  const int n = (L + B - 1) / B;
  const size_t head0 = (size_t)s * p.hq + (size_t)kvh * g;
  const int b0 = split * p.split_blocks;
  const int b1 = min(n, b0 + p.split_blocks);
  // this wave folds blocks b0 + w + NW * k, k < cnt (cnt <= 64 by the split plan)
  const int cnt = b0 + w < b1 ? (b1 - b0 - w + NW - 1) / NW : 0;

  uint4 qf[Cf::QF];
  load_q<Cf>(p, s, kvh, lane, qf);

  const size_t tile = (size_t)B * Cf::R;
  const char* kbase = static_cast<const char*>(p.k_pages);
  const char* vbase = static_cast<const char*>(p.v_pages);
  const int32_t* trow = p.block_table + (size_t)s * p.max_blocks;

  // lane k holds the page (and fp8 scales) of the wave's k-th block
  int tab = 0;
  float ks_t = 1.f, vs_t = 1.f;
  if (cnt > 0) {
    tab = trow[b0 + w + NW * min(lane, cnt - 1)];
    if constexpr (KV == KV_FP8) {
      ks_t = p.k_scale[(size_t)tab * p.hkv + kvh];
      vs_t = p.v_scale[(size_t)tab * p.hkv + kvh];
    }
  }

  float m_run = NEG_INF, l_run = 0.f;
  f32x4 acc[Cf::DT];
#pragma unroll
  for (int dt = 0; dt < Cf::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto nvalid_of = [&](int k) { return min(B, L - (b0 + w + NW * k) * B); };
  auto tile_of = [&](int k) { return ((size_t)readlane(tab, k) * p.hkv + kvh) * tile; };
  auto fold = [&](const BlockRegs<Cf>& r, int k) {
    float ks = 1.f, vs = 1.f;
    if constexpr (KV == KV_FP8) { ks = readlanef(ks_t, k); vs = readlanef(vs_t, k); }
    full_block<Cf>(r, nvalid_of(k), ks, vs, qf, p.qk_log2, lane, m_run, l_run, acc);
  };

  // Register ring of PF block buffers: while block k is folded, blocks
  // k+1 .. k+PF-1 are in flight.  Loads are unconditional (past the wave's
  // last block they re-read that block, a cache hit), so every fold site has
  // the same PF-1 blocks of younger loads outstanding and the waits are exact.
  if (cnt > 0) {
    constexpr int PF = FULL_PREFETCH;
    BlockRegs<Cf> ring[PF];
#pragma unroll
    for (int j = 0; j < PF - 1; ++j) {
      const int kk = min(j, cnt - 1);
      const size_t o = tile_of(kk);
      load_block<Cf>(ring[j], kbase + o, vbase + o, lane, nvalid_of(kk));
    }
    for (int k = 0; k < cnt; k += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int kk = min(k + j + PF - 1, cnt - 1);
        const size_t o = tile_of(kk);
        load_block<Cf>(ring[(j + PF - 1) % PF], kbase + o, vbase + o, lane, nvalid_of(kk));
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
        if (k + j < cnt) fold(ring[j], k + j);
      }
    }
  }

  // merge the four waves
  {
    const int c = lane & 15;
    if (c < GM) {
      store_acc<Cf>(&mw_a[w][c][0], lane, acc, 1.f);
      if ((lane >> 4) == 0) { mw_m[w][c] = m_run; mw_l[w][c] = l_run; }
    }
  }
  __syncthreads();

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
    for (int j = 0; j < DPL; ++j) A[j] = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = mw_m[ww][h];
      const float f = (mw == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      Ls = fmaf(f, mw_l[ww][h], Ls);
#pragma unroll
      for (int j = 0; j < DPL; ++j) A[j] = fmaf(f, mw_a[ww][h][lane + 64 * j], A[j]);
    }
    if (p.splits == 1) {
      const float rl = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) p.out[(head0 + h) * D + lane + 64 * j] = A[j] * rl;
      if (lane == 0) p.stop_block[head0 + h] = n;
    } else {
      float* dst = p.ws_part + (((size_t)stream * p.splits + split) * GM + h) * (D + 2);
#pragma unroll
      for (int j = 0; j < DPL; ++j) dst[lane + 64 * j] = A[j];
      if (lane == 0) { dst[D] = M; dst[D + 1] = Ls; }
    }
  }
  if (p.splits == 1 && threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[stream] = n;
}

// Merge of the full-attention splits (a separate launch, so stream order
// makes the partials visible without any device-scope fence).  One 64-lane
// workgroup per (stream, query head): lanes first read the splits' (M, L) in
// parallel and reduce the common maximum and the weights; then every lane
// owns D/64 output elements and sums the weighted split numerators with
// independent loads in flight.
template <int D, int GM>
__global__ __launch_bounds__(64) void full_merge_kernel(Params p) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x;
  const int g = p.g;
  const int stream = blockIdx.x / g;
  const int h = blockIdx.x - stream * g;
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  const int n = (p.seq_lens[s] + p.block_size - 1) / p.block_size;
  const size_t head = (size_t)s * p.hq + (size_t)kvh * g + h;
  const size_t sstride = (size_t)GM * (D + 2);
  const float* src = p.ws_part + ((size_t)stream * p.splits * GM + h) * (D + 2);
  const int S = p.splits;

  // pass 1: common max over splits (lane-parallel, S may exceed 64)
  float M = NEG_INF;
  for (int sp = lane; sp < S; sp += 64) M = fmaxf(M, src[sp * sstride + D]);
  M = rows_max(M);
  M = fmaxf(M, dpp<DPP_ROW_MIRROR>(M));
  M = fmaxf(M, dpp<DPP_HALF_MIRROR>(M));
  M = fmaxf(M, dpp<DPP_XOR2>(M));
  M = fmaxf(M, dpp<DPP_XOR1>(M));
  // pass 2: weighted numerators; the weight of split sp is read by every lane
  float Ls = 0.f;
  float A[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) A[j] = 0.f;
  int sp = 0;
  for (; sp + 8 <= S; sp += 8) {
    float ms[8], ls[8], a[8][DPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* q = src + (size_t)(sp + u) * sstride;
      ms[u] = q[D];
      ls[u] = q[D + 1];
#pragma unroll
      for (int j = 0; j < DPL; ++j) a[u][j] = q[lane + 64 * j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = (ms[u] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - M);
      Ls = fmaf(f, ls[u], Ls);
#pragma unroll
      for (int j = 0; j < DPL; ++j) A[j] = fmaf(f, a[u][j], A[j]);
    }
  }
  for (; sp < S; ++sp) {
    const float* q = src + (size_t)sp * sstride;
    const float ms = q[D];
    const float f = (ms == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    Ls = fmaf(f, q[D + 1], Ls);
#pragma unroll
    for (int j = 0; j < DPL; ++j) A[j] = fmaf(f, q[lane + 64 * j], A[j]);
  }
  const float rl = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
  for (int j = 0; j < DPL; ++j) p.out[head * D + lane + 64 * j] = A[j] * rl;
  if (lane == 0) {
    p.stop_block[head] = n;
    if (h == 0 && p.blocks_fetched) p.blocks_fetched[stream] = n;
  }
}

}  // namespace kern
}  // namespace art
