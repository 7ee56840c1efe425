// gfx950 kernels for ART paged decode attention.
//
// Method: "ART: Attention Run-time Termination for Efficient Large Language
// Model Decoding" (gist.science explainer), Technical Summary 2.1-2.4.
//
// Two kernels share one per-block datapath (QK on MFMA, block softmax, PV on
// the VALU in fp32):
//
//  * art_chunk_kernel -- the terminating path.  One workgroup (4 waves) owns
//    one stream = (sequence, kv-head) and walks its visit order in chunks of
//    C blocks.  All blocks of a chunk are fetched at once (speculatively) and
//    reduced to per-block partials (m_b, l_b, a_b) in LDS; then one wave per
//    query head folds the partials in visit order, forms O_t = A_t / L_t for
//    every t of the chunk, reduces ‖O_t‖² and ‖O_t - O_{t-1}‖² for all t at
//    once (transposed butterfly), evaluates both statistics for all t in
//    parallel (one lane per t) and runs the patience counter over the
//    resulting pass bitmask.  A head that stops writes O_t and is frozen; the
//    stream stops fetching when every head of its group stopped.
//
//  * full_split_kernel -- full attention (no detector).  Each workgroup owns
//    a contiguous slice of one stream's blocks; each wave keeps its own
//    online-softmax state; waves merge through LDS; slices merge through a
//    workspace, finished by the last-arriving workgroup of the stream.
//
// Data layout (HBM): k_pages/v_pages [page][kv_head][B][D], the (page, kvh)
// tile contiguous, so one block of one stream is B*D*es contiguous bytes.
//
// Lane layouts inside a wave (64 lanes):
//  * K, MFMA A operand: lane l loads 16 B of token row (l & 15) of each
//    16-row tile at byte (l >> 4) * 16 + 64 * i.  The d-index <-> k-slot map
//    is the same for the q operand (B operand, column = head l & 15), so the
//    dot product is exact in any order.
//  * Scores (16x16 MFMA result): lane l holds head (l & 15), tokens
//    4 * (l >> 4) + r, r = 0..3, of each 16-row tile.
//  * V and the PV accumulator: lane l owns VB contiguous bytes of a row:
//    segment (l % LPR) of rows j with j % RPL == l / LPR.
#pragma once
#include "art_internal.h"

#include <math.h>

namespace art {
namespace kern {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int NW = 4;         // waves per workgroup
constexpr int WG = 64 * NW;   // threads per workgroup
constexpr float NEG_INF = -__builtin_inff();

template <int KV> struct ElemSize;
template <> struct ElemSize<KV_F32> { static constexpr int v = 4; };
template <> struct ElemSize<KV_BF16> { static constexpr int v = 2; };
template <> struct ElemSize<KV_FP8> { static constexpr int v = 1; };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

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
  static constexpr int C0 = 256 / B;
  static constexpr int C1 = 8192 / (GM * D);
  static constexpr int C = C0 < C1 ? C0 : C1;         // ART chunk (blocks); partials fit 32 KiB
  static constexpr int BPW = C / NW;                  // blocks per wave per chunk
  static constexpr int HPW = (GM + NW - 1) / NW;      // query heads per wave in the scan
  static constexpr int DPL = D / 64;                  // d per lane in the scan
  static constexpr int LOG2C2 = ilog2(2 * C);
  static constexpr int SH = 6 - LOG2C2;               // stat reduction: lane >> SH = value index
  static_assert(BPW >= 1, "chunk must give every wave a block");
  static_assert(2 * C <= 64, "stat reduction holds at most 64 values");
  static_assert(LPR * EPL == D, "V lanes must tile a row");
};

template <int VB> struct VWordT;
template <> struct VWordT<4> { using type = uint32_t; };
template <> struct VWordT<8> { using type = uint2; };

template <class Cf>
struct BlockRegs {
  uint4 k[Cf::T][Cf::NKL];
  typename VWordT<Cf::VB>::type v[Cf::VL];
};

__device__ __forceinline__ float bits_f(uint32_t x) { return __uint_as_float(x); }

// 4 fp8 E4M3FN bytes -> 4 floats (exact).
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
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_f(kk.x), bits_f(qf[i].x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_f(kk.y), bits_f(qf[i].y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_f(kk.z), bits_f(qf[i].z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_f(kk.w), bits_f(qf[i].w), acc, 0, 0, 0);
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
  mb = fmaxf(mb, __shfl_xor(mb, 16));
  mb = fmaxf(mb, __shfl_xor(mb, 32));
  return mb;
}

__device__ __forceinline__ float sum_quads(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Decode one V word into EPL floats.
template <class Cf>
__device__ __forceinline__ void decode_v(typename VWordT<Cf::VB>::type w, float (&o)[Cf::EPL]) {
  if constexpr (Cf::KV == KV_BF16) {
    o[0] = bits_f(w << 16);
    o[1] = bits_f(w & 0xffff0000u);
  } else if constexpr (Cf::KV == KV_FP8) {
    float f[4];
    fp8x4_to_f32(w, f);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = f[e];
  } else if constexpr (Cf::VB == 4) {
    o[0] = bits_f(w);
  } else {
    o[0] = bits_f(w.x);
    o[1] = bits_f(w.y);
  }
}

// acc[h][e] += sum_j P[h][j] * V[j][d(e)] over the lane's rows of one block.
template <class Cf>
__device__ __forceinline__ void pv_accumulate(const BlockRegs<Cf>& r, int nvalid, const float* pw, int g, int lane,
                                              float (&acc)[Cf::GM][Cf::EPL]) {
  const int rg = lane / Cf::LPR;
#pragma unroll
  for (int u = 0; u < Cf::VL; ++u) {
    const int j = u * Cf::RPL + rg;
    float v[Cf::EPL];
    decode_v<Cf>(r.v[u], v);
    if (nvalid < Cf::B) {
      const bool ok = j < nvalid;
#pragma unroll
      for (int e = 0; e < Cf::EPL; ++e) v[e] = ok ? v[e] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < Cf::GM; ++h) {
      if (h < g) {
        const float pp = pw[h * Cf::B + j];
#pragma unroll
        for (int e = 0; e < Cf::EPL; ++e) acc[h][e] = fmaf(pp, v[e], acc[h][e]);
      }
    }
  }
}

// Sum the PV accumulator over the RPL row groups (lanes sharing a segment).
template <class Cf>
__device__ __forceinline__ void reduce_row_groups(float (&acc)[Cf::GM][Cf::EPL], int g) {
  if constexpr (Cf::RPL >= 2) {
#pragma unroll
    for (int h = 0; h < Cf::GM; ++h)
      if (h < g)
#pragma unroll
        for (int e = 0; e < Cf::EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], 32);
  }
  if constexpr (Cf::RPL == 4) {
#pragma unroll
    for (int h = 0; h < Cf::GM; ++h)
      if (h < g)
#pragma unroll
        for (int e = 0; e < Cf::EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], 16);
  }
}

// Transposed butterfly: returns, in every lane, the 64-lane sum of
// v[lane >> (6 - log2 K)].
template <int K>
__device__ __forceinline__ float xreduce(float (&v)[K], int lane) {
  constexpr int LOGK = ilog2(K);
#pragma unroll
  for (int st = 0; st < LOGK; ++st) {
    const int sft = 32 >> st;
    const int half = K >> (st + 1);
    const bool up = (lane & sft) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = up ? v[i] : v[i + half];
      const float keep = up ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, sft);
    }
  }
  float r = v[0];
#pragma unroll
  for (int sft = 32 >> LOGK; sft >= 1; sft >>= 1) r += __shfl_xor(r, sft);
  return r;
}

// ---------------------------------------------------------------------------
// Terminating kernel
// ---------------------------------------------------------------------------
template <int KV, int D, int B, int GM>
__global__ __launch_bounds__(WG) void art_chunk_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int C = Cf::C, BPW = Cf::BPW, HPW = Cf::HPW, DPL = Cf::DPL, SH = Cf::SH;
  __shared__ float part_a[C][GM][D];
  __shared__ float part_m[C][GM];
  __shared__ float part_l[C][GM];
  __shared__ __attribute__((aligned(16))) float p_lds[NW][GM][B];
  __shared__ int ord_lds[C];
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
    for (int i = threadIdx.x; i < g * D; i += WG) p.out[head0 * D + i] = 0.f;
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
  const int c = lane & 15;
  const int quad = lane >> 4;
  const int rg = lane / Cf::LPR;
  const int sg = lane % Cf::LPR;

  // Per-head streaming state, carried across chunks (head h = w + NW * k).
  float cM[HPW], cL[HPW], cNp[HPW];
  int cCnt[HPW];
  bool cAlive[HPW], cSink[HPW];
  float cA[HPW][DPL], cOp[HPW][DPL];
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    cM[k] = NEG_INF; cL[k] = 0.f; cNp[k] = 0.f; cCnt[k] = 0; cSink[k] = false;
    cAlive[k] = (w + NW * k) < g;
#pragma unroll
    for (int j = 0; j < DPL; ++j) { cA[k][j] = 0.f; cOp[k][j] = 0.f; }
  }

  int fetched = 0;
  for (int t0 = 0; t0 < n; t0 += C) {
    const int nt = min(C, n - t0);

    // ---- block phase: fetch the chunk (all of this wave's blocks in flight), then reduce
    BlockRegs<Cf> regs[BPW];
    int nval[BPW];
    float ksc[BPW], vsc[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = w * BPW + i;
      nval[i] = 0; ksc[i] = 1.f; vsc[i] = 1.f;
      if (b < nt) {
        const int ob = orow[t0 + b];
        const int pg = trow[ob];
        nval[i] = min(B, L - ob * B);
        const size_t off = ((size_t)pg * p.hkv + kvh) * tile;
        load_block<Cf>(regs[i], kbase + off, vbase + off, lane);
        if constexpr (KV == KV_FP8) {
          ksc[i] = p.k_scale[(size_t)pg * p.hkv + kvh];
          vsc[i] = p.v_scale[(size_t)pg * p.hkv + kvh];
        }
        if (lane == 0) ord_lds[b] = ob;
      }
    }
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = w * BPW + i;
      if (b < nt) {
        f32x4 S[Cf::T];
        qk_scores<Cf>(regs[i], qf, S);
        float x[Cf::T][4];
        const float mb = block_scores<Cf>(S, nval[i], p.qk_log2 * ksc[i], lane, x);
        float ls = 0.f;
        f32x4 pq[Cf::T];
#pragma unroll
        for (int t = 0; t < Cf::T; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(x[t][r] - mb);
            ls += e;
            pq[t][r] = e * vsc[i];
          }
        ls = sum_quads(ls);
        if (c < g) {
#pragma unroll
          for (int t = 0; t < Cf::T; ++t) *reinterpret_cast<f32x4*>(&p_lds[w][c][16 * t + 4 * quad]) = pq[t];
          if (quad == 0) { part_m[b][c] = mb; part_l[b][c] = ls; }
        }
        wave_lds_fence();
        float acc[GM][Cf::EPL];
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
          for (int e = 0; e < Cf::EPL; ++e) acc[h][e] = 0.f;
        pv_accumulate<Cf>(regs[i], nval[i], &p_lds[w][0][0], g, lane, acc);
        reduce_row_groups<Cf>(acc, g);
        if (rg == 0) {
#pragma unroll
          for (int h = 0; h < GM; ++h)
            if (h < g)
#pragma unroll
              for (int e = 0; e < Cf::EPL; ++e) part_a[b][h][sg * Cf::EPL + e] = acc[h][e];
        }
        wave_lds_fence();
      }
    }
    fetched += nt;
    __syncthreads();

    // ---- scan phase: fold the chunk's partials in visit order, one wave per head
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      const int h = w + NW * k;
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
            const float rl = 1.0f / cL[k];
#pragma unroll
            for (int j = 0; j < DPL; ++j) {
              float* slot = &part_a[t][h][lane + 64 * j];
              cA[k][j] = fmaf(al, cA[k][j], be * *slot);
              const float o = cA[k][j] * rl;
              const float df = o - cOp[k][j];
              nn = fmaf(o, o, nn);
              ee = fmaf(df, df, ee);
              cOp[k][j] = o;
              *slot = o;  // keep O_t for the epilogue
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
          sink = sink || (ord_lds[t] == 0);
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
        if (w + NW * k < g) alive_lds[w + NW * k] = cAlive[k] ? 1 : 0;
    }
    __syncthreads();
    int any = 0;
    for (int h = 0; h < g; ++h) any |= alive_lds[h];
    if (!any) break;
  }

  // heads that never stopped: output after all n blocks
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = w + NW * k;
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
template <int KV, int D, int B, int GM>
__device__ __forceinline__ void full_block(const BlockRegs<Cfg<KV, D, B, GM>>& r, int nvalid, float ksc, float vsc,
                                           const uint4 (&qf)[Cfg<KV, D, B, GM>::QF], const Params& p, int w,
                                           int lane, float& m_run, float& l_run,
                                           float (&acc)[GM][Cfg<KV, D, B, GM>::EPL], float (*p_lds)[GM][B],
                                           float (*alpha_lds)[GM]) {
  using Cf = Cfg<KV, D, B, GM>;
  const int c = lane & 15;
  const int quad = lane >> 4;
  f32x4 S[Cf::T];
  qk_scores<Cf>(r, qf, S);
  float x[Cf::T][4];
  const float mb = block_scores<Cf>(S, nvalid, p.qk_log2 * ksc, lane, x);
  const float mn = fmaxf(m_run, mb);
  const float al = __builtin_amdgcn_exp2f(m_run - mn);
  float ls = 0.f;
  f32x4 pq[Cf::T];
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float e = __builtin_amdgcn_exp2f(x[t][rr] - mn);
      ls += e;
      pq[t][rr] = e * vsc;
    }
  ls = sum_quads(ls);
  l_run = fmaf(al, l_run, ls);
  m_run = mn;
  const int g = p.g;
  if (c < g) {
#pragma unroll
    for (int t = 0; t < Cf::T; ++t) *reinterpret_cast<f32x4*>(&p_lds[w][c][16 * t + 4 * quad]) = pq[t];
    if (quad == 0) alpha_lds[w][c] = al;
  }
  wave_lds_fence();
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < g) {
      const float a = alpha_lds[w][h];
#pragma unroll
      for (int e = 0; e < Cf::EPL; ++e) acc[h][e] *= a;
    }
  }
  pv_accumulate<Cf>(r, nvalid, &p_lds[w][0][0], g, lane, acc);
  wave_lds_fence();
}

template <int KV, int D, int B, int GM>
__global__ __launch_bounds__(WG) void full_split_kernel(Params p) {
  using Cf = Cfg<KV, D, B, GM>;
  constexpr int HPW = Cf::HPW, DPL = Cf::DPL, EPL = Cf::EPL;
  __shared__ __attribute__((aligned(16))) float p_lds[NW][GM][B];
  __shared__ float alpha_lds[NW][GM];
  __shared__ float mw_a[NW][GM][D];
  __shared__ float mw_m[NW][GM];
  __shared__ float mw_l[NW][GM];
  __shared__ int last_flag;

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

  uint4 qf[Cf::QF];
  load_q<Cf>(p, s, kvh, lane, qf);

  const size_t tile = (size_t)B * Cf::R;
  const char* kbase = static_cast<const char*>(p.k_pages);
  const char* vbase = static_cast<const char*>(p.v_pages);
  const int32_t* trow = p.block_table + (size_t)s * p.max_blocks;

  float m_run = NEG_INF, l_run = 0.f;
  float acc[GM][EPL];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

  // Wave w folds blocks b0 + w, b0 + w + NW, ...; the next block is in flight
  // while the current one is computed (two register sets, unrolled by two).
  BlockRegs<Cf> ra, rb;
  int pa = 0, pb = 0;
  int b = b0 + w;
  if (b < b1) {
    pa = trow[b];
    load_block<Cf>(ra, kbase + ((size_t)pa * p.hkv + kvh) * tile, vbase + ((size_t)pa * p.hkv + kvh) * tile, lane);
  }
  for (; b < b1; b += 2 * NW) {
    const int bb = b + NW;
    if (bb < b1) {
      pb = trow[bb];
      load_block<Cf>(rb, kbase + ((size_t)pb * p.hkv + kvh) * tile, vbase + ((size_t)pb * p.hkv + kvh) * tile,
                     lane);
    }
    {
      float ks = 1.f, vs = 1.f;
      if constexpr (KV == KV_FP8) {
        ks = p.k_scale[(size_t)pa * p.hkv + kvh];
        vs = p.v_scale[(size_t)pa * p.hkv + kvh];
      }
      full_block<KV, D, B, GM>(ra, min(B, L - b * B), ks, vs, qf, p, w, lane, m_run, l_run, acc, p_lds, alpha_lds);
    }
    if (bb >= b1) break;
    const int bc = bb + NW;
    if (bc < b1) {
      pa = trow[bc];
      load_block<Cf>(ra, kbase + ((size_t)pa * p.hkv + kvh) * tile, vbase + ((size_t)pa * p.hkv + kvh) * tile,
                     lane);
    }
    {
      float ks = 1.f, vs = 1.f;
      if constexpr (KV == KV_FP8) {
        ks = p.k_scale[(size_t)pb * p.hkv + kvh];
        vs = p.v_scale[(size_t)pb * p.hkv + kvh];
      }
      full_block<KV, D, B, GM>(rb, min(B, L - bb * B), ks, vs, qf, p, w, lane, m_run, l_run, acc, p_lds,
                               alpha_lds);
    }
  }
  reduce_row_groups<Cf>(acc, g);

  // merge the four waves
  const int c = lane & 15;
  const int quad = lane >> 4;
  if (c < g && quad == 0) { mw_m[w][c] = m_run; mw_l[w][c] = l_run; }
  if (lane / Cf::LPR == 0) {
    const int sg = lane % Cf::LPR;
#pragma unroll
    for (int h = 0; h < GM; ++h)
      if (h < g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) mw_a[w][h][sg * EPL + e] = acc[h][e];
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

  // last-arriving workgroup of the stream merges the splits
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&p.ws_count[stream], 1);
    last_flag = (prev == p.splits - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = w + NW * k;
    if (h >= g) continue;
    const float* src = part + ((size_t)stream * p.splits * GM + h) * (D + 2);
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
  if (threadIdx.x == 0) {
    p.ws_count[stream] = 0;
    if (p.blocks_fetched) p.blocks_fetched[stream] = n;
  }
}

}  // namespace kern
}  // namespace art
