// gfx950 kernels for ART paged decode attention (templates; instantiated in
// kern_<kernel>_<type>.hip).
//
// Method: "ART: Attention Run-time Termination for Efficient Large Language
// Model Decoding" (gist.science explainer), Technical Summary 2.1-2.4.
//
// Two kernels share one per-block datapath (QK on MFMA, block softmax, PV on
// the VALU in fp32):
//
//  * art_chunk_kernel -- the terminating path.  One workgroup (NWA waves)
//    owns one stream = (sequence, kv-head) and walks its visit order in
//    chunks of C blocks.  All blocks of a chunk are fetched at once
//    (speculatively) and reduced to per-block partials (m_b, l_b, a_b) in
//    LDS; then one wave per query head folds the partials in visit order,
//    forms O_t = A_t / L_t for every t of the chunk, reduces ‖O_t‖² and
//    ‖O_t - O_{t-1}‖² for all t at once (transposed butterfly), evaluates
//    both statistics for all t in parallel (one lane per t) and runs the
//    patience counter over the resulting pass bitmask.  A head that stops
//    writes O_t and is frozen; the stream stops fetching when every head of
//    its group stopped.  The page entries of chunk c+1 are fetched while
//    chunk c is computed, so a chunk's KV loads never wait on the table.
//
//  * full_split_kernel -- full attention (no detector).  Each workgroup owns
//    a contiguous slice of one stream's blocks; each wave keeps its own
//    online-softmax state with the next block's loads in flight; waves merge
//    through LDS; slices are merged by full_merge_kernel (second launch).
//
// Data layout (HBM): k_pages/v_pages [page][kv_head][B][D], the (page, kvh)
// tile contiguous, so one block of one stream is B*D*es contiguous bytes.
//
// Lane layouts inside a wave (64 lanes):
//  * K, MFMA A operand: lane l loads 16 B of token row (l & 15) of each
//    16-row tile at byte (l >> 4) * 16 + 64 * i.  The q operand (B operand,
//    column = head l & 15) uses the same byte -> d map, so the dot product
//    pairs q[d] with k[d] exactly.
//  * Scores (16x16 MFMA result): lane l holds head (l & 15), tokens
//    4 * (l >> 4) + r, r = 0..3, of each 16-row tile.
//  * V and the PV accumulator: lane l owns VB contiguous bytes of a row:
//    segment (l % LPR) of the rows j with j % RPL == l / LPR.
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

template <int KV> struct ElemSize;
template <> struct ElemSize<KV_F32> { static constexpr int v = 4; };
template <> struct ElemSize<KV_BF16> { static constexpr int v = 2; };
template <> struct ElemSize<KV_FP8> { static constexpr int v = 1; };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

template <int KV_, int D_, int B_, int GM_>
struct Cfg {
  static constexpr int KV = KV_, D = D_, B = B_, GM = GM_;
  static constexpr int ES = ElemSize<KV>::v;
  static constexpr int R = D * ES;                    // bytes per token row
  static constexpr int NKL = R / 64;                  // 16-B K chunks per lane per 16-row tile
  static constexpr int T = B / 16;                    // 16-row tiles per block
  static constexpr int VB = R >= 256 ? R / 64 : 4;    // V bytes per lane per row
  static constexpr int LPR = R / VB;                  // lanes per V row
  static constexpr int RPL = 64 / LPR;                // V rows per wave load
  static constexpr int EPL = VB / ES;                 // V elements per lane
  static constexpr int VL = B / RPL;                  // V loads per lane per block
  static constexpr int QF = KV == KV_FP8 ? 2 * NKL : NKL;  // 16-B q fragments
  // ART chunk: C blocks; the per-block partials [C][GM][D] fp32 fit 32 KiB
  static constexpr int C = cmin(256 / B, 8192 / (GM * D));
  static constexpr int NWA = cmin(8, C);              // waves per workgroup, ART kernel
  static constexpr int BPW = C / NWA;                 // blocks per wave per chunk
  static constexpr int HPW = (GM + NWA - 1) / NWA;    // query heads per wave in the scan
  static constexpr int DPL = D / 64;                  // d per lane in the scan
  static constexpr int SH = 6 - ilog2(2 * C);         // stat reduction: lane >> SH = value index
  static_assert(BPW >= 1 && BPW * NWA == C, "chunk must split evenly over the waves");
  static_assert(2 * C <= 64, "stat reduction holds at most 64 values");
  static_assert(LPR * EPL == D, "V lanes must tile a row");
  static_assert(B % (4 * RPL) == 0, "P quads must cover the lane's rows");
};

template <int VB> struct VWordT;
template <> struct VWordT<4> { using type = uint32_t; };
template <> struct VWordT<8> { using type = uint2; };

template <class Cf>
struct BlockRegs {
  uint4 k[Cf::T][Cf::NKL];
  typename VWordT<Cf::VB>::type v[Cf::VL];
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

template <class Cf>
__device__ __forceinline__ void load_block(BlockRegs<Cf>& r, const char* kt, const char* vt, int lane) {
  const int krow = lane & 15;
  const int kcol = (lane >> 4) * 16;
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int i = 0; i < Cf::NKL; ++i)
      r.k[t][i] = *reinterpret_cast<const uint4*>(kt + (size_t)(16 * t + krow) * Cf::R + kcol + 64 * i);
  const int rg = lane / Cf::LPR;
  const int sg = lane % Cf::LPR;
  using VW = typename VWordT<Cf::VB>::type;
#pragma unroll
  for (int u = 0; u < Cf::VL; ++u)
    r.v[u] = *reinterpret_cast<const VW*>(vt + (size_t)(u * Cf::RPL + rg) * Cf::R + sg * Cf::VB);
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

// Store the lane's P values (score layout) into the wave's P rows so that a
// PV lane reads its own rows contiguously: token j of head h is stored at
// h*B + (j % RPL) * (B / RPL) + j / RPL.
template <class Cf>
__device__ __forceinline__ void store_p(float* pw, int lane, const float (&pv)[Cf::T][4]) {
  const int c = lane & 15;
  const int quad = lane >> 4;
  if (c >= Cf::GM) return;
  float* row = pw + c * Cf::B;
  if constexpr (Cf::RPL == 1) {
#pragma unroll
    for (int t = 0; t < Cf::T; ++t) {
      f32x4 q4 = {pv[t][0], pv[t][1], pv[t][2], pv[t][3]};
      *reinterpret_cast<f32x4*>(row + 16 * t + 4 * quad) = q4;
    }
  } else {
#pragma unroll
    for (int t = 0; t < Cf::T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * t + 4 * quad + r;
        row[(j % Cf::RPL) * (Cf::B / Cf::RPL) + j / Cf::RPL] = pv[t][r];
      }
  }
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Decode one V word into EPL floats.
template <class Cf>
__device__ __forceinline__ void decode_v(typename VWordT<Cf::VB>::type w, float (&o)[Cf::EPL]) {
  if constexpr (Cf::KV == KV_BF16) {
    o[0] = bitsf(w << 16);
    o[1] = bitsf(w & 0xffff0000u);
  } else if constexpr (Cf::KV == KV_FP8) {
    float f[4];
    fp8x4_to_f32(w, f);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = f[e];
  } else if constexpr (Cf::VB == 4) {
    o[0] = bitsf(w);
  } else {
    o[0] = bitsf(w.x);
    o[1] = bitsf(w.y);
  }
}

// acc[h][e] += sum_j P[h][j] * V[j][d(e)] over the lane's rows of one block,
// for every head slot of the group capacity (slots >= g carry finite junk).
// Rows past the sequence end may hold any bits, so they are replaced by 0 with
// a select on every block (no branch: a branch-local redefinition of the
// decoded values has been miscompiled by the register allocator).
template <class Cf>
__device__ __forceinline__ void pv_accumulate(const BlockRegs<Cf>& r, int nvalid, const float* pw, int lane,
                                              float (&acc)[Cf::GM][Cf::EPL]) {
  const int rg = lane / Cf::LPR;
  float v[Cf::VL][Cf::EPL];
#pragma unroll
  for (int u = 0; u < Cf::VL; ++u) {
    decode_v<Cf>(r.v[u], v[u]);
    const bool ok = u * Cf::RPL + rg < nvalid;
#pragma unroll
    for (int e = 0; e < Cf::EPL; ++e) v[u][e] = ok ? v[u][e] : 0.f;
  }
  const float* base = pw + rg * (Cf::B / Cf::RPL);
#pragma unroll
  for (int h = 0; h < Cf::GM; ++h) {
#pragma unroll
    for (int k = 0; k < Cf::VL / 4; ++k) {
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(base + h * Cf::B + 4 * k);
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < Cf::EPL; ++e) acc[h][e] = fmaf(p4[m], v[4 * k + m][e], acc[h][e]);
    }
  }
}

// Sum the PV accumulator over the RPL row groups (lanes sharing a segment).
template <class Cf>
__device__ __forceinline__ void reduce_row_groups(float (&acc)[Cf::GM][Cf::EPL]) {
  if constexpr (Cf::RPL >= 2) {
#pragma unroll
    for (int h = 0; h < Cf::GM; ++h)
#pragma unroll
      for (int e = 0; e < Cf::EPL; ++e) acc[h][e] = xor32_sum(acc[h][e]);
  }
  if constexpr (Cf::RPL == 4) {
#pragma unroll
    for (int h = 0; h < Cf::GM; ++h)
#pragma unroll
      for (int e = 0; e < Cf::EPL; ++e) acc[h][e] = xor16_sum(acc[h][e]);
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
  __shared__ float part_a[C][GM][D];
  __shared__ float part_m[C][GM];
  __shared__ float part_l[C][GM];
  __shared__ __attribute__((aligned(16))) float p_lds[NWA][GM][B];
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
  const int rg = lane / Cf::LPR;
  const int sg = lane % Cf::LPR;
  const int slot = lane < C ? lane : C - 1;

  // Chunk entries, one per lane (slot = lane): logical block, page, fp8 scales.
  int ob_l = orow[min(slot, n - 1)];
  int pg_l = trow[ob_l];
  float ks_l = 1.f, vs_l = 1.f;

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

  int fetched = 0;
  for (int t0 = 0; t0 < n; t0 += C) {
    const int nt = min(C, n - t0);

    // ---- block phase: every load of the wave's blocks in flight, then reduce.
    // Slots past the chunk end re-read the last valid slot (an L2 hit), so the
    // loads are unconditional and the wait counts stay exact.
    BlockRegs<Cf> regs[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = min(w * BPW + i, nt - 1);
      const int pg = readlane(pg_l, b);
      const size_t off = ((size_t)pg * p.hkv + kvh) * tile;
      load_block<Cf>(regs[i], kbase + off, vbase + off, lane);
    }
    if constexpr (KV == KV_FP8) {
      ks_l = p.k_scale[(size_t)pg_l * p.hkv + kvh];
      vs_l = p.v_scale[(size_t)pg_l * p.hkv + kvh];
    }
    // next chunk's order entries (consumed after this chunk's scan)
    const int ob_n = orow[min(t0 + C + slot, n - 1)];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = w * BPW + i;
      if (b < nt) {
        const int ob = readlane(ob_l, b);
        const int nvalid = min(B, L - ob * B);
        float ksc = 1.f, vsc = 1.f;
        if constexpr (KV == KV_FP8) { ksc = readlanef(ks_l, b); vsc = readlanef(vs_l, b); }
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
        store_p<Cf>(&p_lds[w][0][0], lane, pq);
        const int c = lane & 15;
        if (c < GM && (lane >> 4) == 0) { part_m[b][c] = mb; part_l[b][c] = ls; }
        wave_lds_fence();
        float acc[GM][Cf::EPL];
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
          for (int e = 0; e < Cf::EPL; ++e) acc[h][e] = 0.f;
        pv_accumulate<Cf>(regs[i], nvalid, &p_lds[w][0][0], lane, acc);
        reduce_row_groups<Cf>(acc);
        if (rg == 0) {
#pragma unroll
          for (int h = 0; h < GM; ++h)
#pragma unroll
            for (int e = 0; e < Cf::EPL; ++e) part_a[b][h][sg * Cf::EPL + e] = acc[h][e];
        }
        wave_lds_fence();
      }
    }
    // next chunk's pages (the order entries have arrived by now)
    const int pg_n = trow[ob_n];
    fetched += nt;
    __syncthreads();

    // ---- scan phase: fold the chunk's partials in visit order, one wave per head
    const unsigned long long sinkbits = __ballot(lane < nt && ob_l == 0);
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      const int h = w + NWA * k;
      if (h < g && cAlive[k]) {
        float st[2 * C];
#pragma unroll
        for (int t = 0; t < C; ++t) {
          float nn = 0.f, ee = 0.f;
          if (t < nt) {
            const float mb = part_m[t][h];
            const float lb = part_l[t][h];
            const float Mn = fmaxf(cM[k], mb);
            const float al = __builtin_amdgcn_exp2f(cM[k] - Mn);
            const float be = __builtin_amdgcn_exp2f(mb - Mn);
            cL[k] = fmaf(al, cL[k], be * lb);
            cM[k] = Mn;
            const float rl = __builtin_amdgcn_rcpf(cL[k]);  // 1 ulp; statistics need ~1e-6
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
          }
          st[2 * t] = nn;
          st[2 * t + 1] = ee;
        }
        const float v0 = xreduce<2 * C>(st, lane);
        // lane (2t) << SH holds ‖O_t‖², lane (2t+1) << SH holds ‖O_t - O_{t-1}‖²
        const int idx = lane >> SH;
        const int tt = idx >> 1;
        const float e_t = __shfl(v0, (lane + (1 << SH)) & 63);
        float n_prev = __shfl(v0, (lane - (2 << SH)) & 63);
        if (tt == 0) n_prev = cNp[k];
        const bool lead = ((idx & 1) == 0) && ((lane & ((1 << SH) - 1)) == 0);
        bool ps = false;
        if (lead && tt < nt && (t0 + tt) >= 1) {
          const float a = sqrtf(v0);
          const float bn = sqrtf(n_prev);
          float dm, dd;
          if (a == 0.f && bn == 0.f) {
            dm = 0.f; dd = 0.f;
          } else if (bn == 0.f) {
            dm = __builtin_inff(); dd = 1.f;
          } else {
            const float df = a - bn;
            dm = fabsf(df) / bn;
            // 1 - cos = (‖O_t - O_{t-1}‖² - (‖O_t‖ - ‖O_{t-1}‖)²) / (2 ‖O_t‖ ‖O_{t-1}‖)
            dd = (a == 0.f) ? 1.f : fmaxf(0.f, (e_t - df * df) / (2.f * a * bn));
          }
          ps = (dm < p.eps_mag) && (dd < p.eps_dir);
        }
        const unsigned long long pm = __ballot(ps);
        const float n_last = __shfl(v0, ((2 * (nt - 1)) << SH) & 63);
        int cnt = cCnt[k];
        bool sink = cSink[k];
        int stop_t = -1;
        for (int t = 0; t < nt; ++t) {
          if (t0 + t >= 1) cnt = ((pm >> ((2 * t) << SH)) & 1ull) ? cnt + 1 : 0;
          sink = sink || ((sinkbits >> t) & 1ull);
          if (cnt >= p.patience && sink) { stop_t = t; break; }
        }
        if (stop_t >= 0) {
          float* o = p.out + (head0 + h) * D;
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[lane + 64 * j] = part_a[stop_t][h][lane + 64 * j];
          if (lane == 0) p.stop_block[head0 + h] = t0 + stop_t + 1;
          cAlive[k] = false;
        } else {
          cCnt[k] = cnt;
          cSink[k] = sink;
          cNp[k] = n_last;
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < HPW; ++k)
        if (w + NWA * k < g) alive_lds[w + NWA * k] = cAlive[k] ? 1 : 0;
    }
    ob_l = ob_n;
    pg_l = pg_n;
    __syncthreads();
    int any = 0;
    for (int h = 0; h < g; ++h) any |= alive_lds[h];
    if (!any) break;
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
}

// ---------------------------------------------------------------------------
// Full-attention split kernel
// ---------------------------------------------------------------------------
template <class Cf>
__device__ __forceinline__ void full_block(const BlockRegs<Cf>& r, int nvalid, float ksc, float vsc,
                                           const uint4 (&qf)[Cf::QF], float qk_log2, int lane, float& m_run,
                                           float& l_run, float (&acc)[Cf::GM][Cf::EPL], float* pw,
                                           float* alpha_w) {
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
  store_p<Cf>(pw, lane, pq);
  const int c = lane & 15;
  if (c < Cf::GM && (lane >> 4) == 0) alpha_w[c] = al;
  wave_lds_fence();
#pragma unroll
  for (int h = 0; h < Cf::GM; ++h) {
    const float a = alpha_w[h];
#pragma unroll
    for (int e = 0; e < Cf::EPL; ++e) acc[h][e] *= a;
  }
  pv_accumulate<Cf>(r, nvalid, pw, lane, acc);
  wave_lds_fence();
}

template <int KV, int D, int B, int GM>
__global__ __launch_bounds__(WG) void full_split_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int HPW = (GM + NW - 1) / NW, DPL = Cf::DPL, EPL = Cf::EPL;
  __shared__ __attribute__((aligned(16))) float p_lds[NW][GM][B];
  __shared__ float alpha_lds[NW][GM];
  __shared__ float mw_a[NW][GM][D];
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
  float acc[GM][EPL];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

  float* pw = &p_lds[w][0][0];
  float* aw = &alpha_lds[w][0];
  auto tile_of = [&](int k) { return ((size_t)readlane(tab, k) * p.hkv + kvh) * tile; };
  auto fold = [&](const BlockRegs<Cf>& r, int k) {
    const int b = b0 + w + NW * k;
    float ks = 1.f, vs = 1.f;
    if constexpr (KV == KV_FP8) { ks = readlanef(ks_t, k); vs = readlanef(vs_t, k); }
    full_block<Cf>(r, min(B, L - b * B), ks, vs, qf, p.qk_log2, lane, m_run, l_run, acc, pw, aw);
  };

  // Two register sets; block k+1 is in flight while block k is folded.  Each
  // fold site has a fixed number of younger loads outstanding.
  if (cnt > 0) {
    BlockRegs<Cf> ra, rb;
    load_block<Cf>(ra, kbase + tile_of(0), vbase + tile_of(0), lane);
    int k = 0;
    for (;;) {
      if (k + 1 < cnt) {
        const size_t o = tile_of(k + 1);
        load_block<Cf>(rb, kbase + o, vbase + o, lane);
        fold(ra, k);
      } else {
        fold(ra, k);
        break;
      }
      ++k;
      if (k + 1 < cnt) {
        const size_t o = tile_of(k + 1);
        load_block<Cf>(ra, kbase + o, vbase + o, lane);
        fold(rb, k);
      } else {
        fold(rb, k);
        break;
      }
      ++k;
    }
  }
  reduce_row_groups<Cf>(acc);

  // merge the four waves
  {
    const int c = lane & 15;
    if (c < g && (lane >> 4) == 0) { mw_m[w][c] = m_run; mw_l[w][c] = l_run; }
    if (lane / Cf::LPR == 0) {
      const int sg = lane % Cf::LPR;
#pragma unroll
      for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) mw_a[w][h][sg * EPL + e] = acc[h][e];
    }
  }
  __syncthreads();

  float* part = p.ws_part;
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
      float* dst = part + (((size_t)stream * p.splits + split) * GM + h) * (D + 2);
#pragma unroll
      for (int j = 0; j < DPL; ++j) dst[lane + 64 * j] = A[j];
      if (lane == 0) { dst[D] = M; dst[D + 1] = Ls; }
    }
  }
  if (p.splits == 1) {
    if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[stream] = n;
    return;
  }

}

// Merge of the full-attention splits: one workgroup per stream combines the
// per-split (M, L, A) of each query head (a separate launch, so stream order
// makes the partials visible without any device-scope fence).
template <int D, int GM>
__global__ __launch_bounds__(WG) void full_merge_kernel(Params p) {
  constexpr int HPW = (GM + NW - 1) / NW, DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stream = blockIdx.x;
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  const int g = p.g;
  const int n = (p.seq_lens[s] + p.block_size - 1) / p.block_size;
  const size_t head0 = (size_t)s * p.hq + (size_t)kvh * g;
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = w + NW * k;
    if (h >= g) continue;
    const float* src = p.ws_part + ((size_t)stream * p.splits * GM + h) * (D + 2);
    const size_t sstride = (size_t)GM * (D + 2);
    float M = NEG_INF;
    for (int sp = 0; sp < p.splits; ++sp) M = fmaxf(M, src[sp * sstride + D]);
    float Ls = 0.f;
    float A[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) A[j] = 0.f;
    for (int sp = 0; sp < p.splits; ++sp) {
      const float* q = src + sp * sstride;
      const float ms = q[D];
      const float f = (ms == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      Ls = fmaf(f, q[D + 1], Ls);
#pragma unroll
      for (int j = 0; j < DPL; ++j) A[j] = fmaf(f, q[lane + 64 * j], A[j]);
    }
    const float rl = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) p.out[(head0 + h) * D + lane + 64 * j] = A[j] * rl;
    if (lane == 0) p.stop_block[head0 + h] = n;
  }
  if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[stream] = n;
}

}  // namespace kern
}  // namespace art
