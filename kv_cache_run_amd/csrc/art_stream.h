// gfx950 kernel for ART paged decode attention: the stream kernel
// (art_stream_kernel), one workgroup per stream (sequence, kv-head).
//
// Method: "ART: Attention Run-time Termination for Efficient Large Language
// Model Decoding" (gist.science explainer), Technical Summary 2.1 (streaming,
// tile-wise accumulation), 2.2 (magnitude and direction statistics), 2.3
// (patience), 2.4 (visit order, block 0 folded before any stop).
//
// Two kinds of waves share one LDS ring of per-block results and run without
// a workgroup barrier between them:
//
//  * producer waves (NP): producer w takes visit positions w, w + NP, ...
//    For each block it loads the K and V tiles (a register ring PD blocks
//    deep, so that PD - 1 blocks' loads are in flight while one is folded),
//    computes the block's scores for the query group on MFMA, its maximum
//    m_b and sum l_b, and the block's own normalised output
//    o_b = (sum_j e^(s_j - m_b) v_j) / l_b for every head, and writes
//    (o_b, m_b, l_b) into ring slot t % RING followed by a ready word
//    (t + 1, plus a bit when the block is logical block 0).
//  * detector waves (NS, one query head each): fold the ring's blocks in
//    visit order, C positions at a time.  With the running maximum M_t and
//    sum L_t (lane-parallel prefix over the chunk), the block's weight in the
//    normalised output is w_t = e^(m_t - M_t) l_t / L_t and
//        O_t = O_{t-1} + w_t (o_t - O_{t-1}),
//    so O_t - O_{t-1} = w_t (o_t - O_{t-1}): the change of the output comes
//    straight from the difference vector, without cancellation.  Per lane and
//    position the wave accumulates ||O_t||^2 and ||o_t - O_{t-1}||^2 over its
//    D/64 coordinates; one transposed butterfly reduces the 2C sums; lane t
//    then evaluates both statistics of position t and the patience / block-0
//    rule (bit masks over the chunk).  A head that fires writes O at its stop
//    and leaves; the stream ends when every head of the group has fired.
//
// Flow control (LDS words): prog[w] = blocks detector wave w has consumed
// (a large value once it has no live head); a producer may overwrite the
// slot of block t only when every detector wave has consumed block
// t - RING, and issues the loads of a block only while it lies within the
// lookahead LA(f) = la0 + (f >> la_shift) blocks of the frontier f (the
// smallest prog), at most what the ring and the register ring hold: the KV
// read past a stop is bounded by that lookahead.  Every wait is bounded
// (p.spin_limit polls); a wait that runs out marks the stream failed (its
// unfinished heads get stop_block -1 and NaN output) instead of hanging.
#pragma once

#include <type_traits>

#include "art_kernels_impl.h"

namespace art {
namespace kern {

constexpr int stream_ring_depth(int kv, int d, int b, int gm) {
#ifdef ART_STREAM_PD_FP8
  if (kv == KV_FP8) return ART_STREAM_PD_FP8;
#endif
  return 2;
}

template <int KV_, int D_, int B_, int GM_>
struct StreamCfg : Cfg<KV_, D_, B_, GM_> {
  using Base = Cfg<KV_, D_, B_, GM_>;

  static constexpr int TILE_V = 2 * B_ * Base::R / 256;  // VGPRs of one block's K and V tiles
  static constexpr int NS2 = 4;                         // detector waves
  static constexpr int HP2 = GM_ / NS2 > 0 ? GM_ / NS2 : 1;  // heads per detector wave
#ifdef ART_STREAM_NP
  static constexpr int NP2 = ART_STREAM_NP;
#else
  // producer waves: ten for bf16/f32 16-token blocks of groups up to 4
  // heads (with the four detector waves, 14 waves at up to 128 VGPRs each;
  // measured faster than 8 and 12 on the Llama-3-8B and ragged shapes),
  // eight for the other small tiles (whose math needs more registers), four
  // for large ones
  static constexpr int NP2 = TILE_V >= 64 ? 4 : (GM_ <= 4 && KV_ != KV_FP8 && B_ == 16 ? 10 : 8);
#endif
  static constexpr int NW2 = NS2 + NP2;
  static constexpr int SLOTF = GM_ * D_ + 2 * GM_;     // floats per ring slot: o[GM][D], m[GM], l[GM]
  static constexpr int RING_RAW = 73728 / (SLOTF * 4);
  static constexpr int RING = RING_RAW >= 64 ? 64 : (RING_RAW >= 32 ? 32 : 16);
#ifdef ART_STREAM_C
  static constexpr int C2 = cmin(ART_STREAM_C, RING / 2);
#else
  static constexpr int C2 = 8;                          // positions per detector step
#endif
  // register ring depth of a producer (blocks whose loads are in flight or
  // in use): 2, measured fastest for the pipelined producer (depth 3 slowed
  // the Llama-3-8B and ragged shapes by 5-15 %)
#ifdef ART_STREAM_PD
  static constexpr int PD = ART_STREAM_PD;
#else
  static constexpr int PD = stream_ring_depth(KV_, D_, B_, GM_);
#endif
  // lookahead bounds: the producers' issue points can run at most this far
  // past the detectors' frontier; the smallest lookahead that lets every
  // block of the detectors' current chunk be produced is C + NP (PD - 1)
  static constexpr int LA_MAX = RING + PD * NP2;
  static constexpr int LA_MIN = 2 * C2;
  static constexpr int SH2 = 6 - ilog2(2 * C2);
  static_assert(RING >= 2 * C2 && RING % C2 == 0, "the ring holds whole chunks");
  static_assert(NS2 * HP2 >= GM_, "every head has a detector wave");
};

// LDS words of the stream kernel.
struct StreamShared {
  int rdy[64];   // per ring slot: visit position + 1 (bit 30: logical block 0)
  int prog[8];   // per detector wave: blocks consumed
  int done;      // every head fired (or a wait ran out)
  int nfired;    // heads that fired
  int fsum;      // blocks the producers loaded
  int pfin;      // producers finished
  int err;       // a bounded wait ran out
  int claim;     // next visit position for a producer to take
  int win[8];    // per entry-table window slot: 1 + index of the 256-position window it holds
  int pad[1];
};
constexpr int STREAM_ENT = 2048;  // entry table: (order entry, page) of visit positions t mod 2048
constexpr int STREAM_WIN = 256;   // refilled in windows of 256 positions
constexpr int STREAM_BIG = 0x3fffffff;

#ifdef ART_STREAM_TIMELINE
// Timestamps of one stream's events (a measurement build only): producers at
// [2 t] when the wait for block t ended and [2 t + 1] when it was published
// (t < 4096); detector wave w at [8192 + 8 c + 2 w] when chunk c was ready and
// [8192 + 8 c + 2 w + 1] when it had consumed it (c < 1023); the start at
// [16383].
static __device__ unsigned long long art_timeline[16384];
static __device__ int art_timeline_stream;
#define ART_TL(cond, idx)                                                                  \
  do {                                                                                     \
    if ((cond) && (int)blockIdx.x == art_timeline_stream && (idx) >= 0 && (idx) < 16384) \
      art_timeline[(idx)] = __builtin_amdgcn_s_memrealtime();                              \
  } while (0)
#define ART_TL_ADD(var, t0) var += __builtin_amdgcn_s_memrealtime() - (t0)
#define ART_TL_NOW() __builtin_amdgcn_s_memrealtime()
#else
#define ART_TL(cond, idx) \
  do {                    \
  } while (0)
#define ART_TL_ADD(var, t0) \
  do {                      \
  } while (0)
#define ART_TL_NOW() 0ull
#endif

__device__ __forceinline__ int lds_ld(const int* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
__device__ __forceinline__ void lds_st(int* a, int v) { __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
__device__ __forceinline__ int lds_add(int* a, int v) { return __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
// this wave's LDS operations have completed (loads and stores of the vector
// memory are not waited for)
__device__ __forceinline__ void lds_wait() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The group's query rows in LDS: ROWB bytes each (fp8 K: q stays bf16), rows
// STRIDE bytes apart; the 16 extra bytes put the rows on different banks, so
// that the lanes of different heads reading the same column do not collide.
template <class Cf>
struct QLds {
  static constexpr int ROWB = Cf::KV == KV_FP8 ? 2 * Cf::D : Cf::R;
  static constexpr int STRIDE = ROWB + 16;
};

// Copy the g query rows starting at src into the padded LDS rows (thread
// `tid` of `nthreads`).
template <class Cf>
__device__ __forceinline__ void q_to_lds(const char* src, char* dst, int g, int tid, int nthreads) {
  constexpr int W = QLds<Cf>::ROWB / 16;  // 16-byte words per row
  for (int i = tid; i < g * W; i += nthreads) {
    const int r = i / W, c = i - r * W;
    *reinterpret_cast<uint4*>(dst + r * QLds<Cf>::STRIDE + 16 * c) = reinterpret_cast<const uint4*>(src)[i];
  }
}

// q fragments of the group from its LDS copy (rows past the group repeat the
// last head: their columns are never read back).
template <class Cf>
__device__ __forceinline__ void q_from_lds(const char* qs, int g, int lane, uint4 (&qf)[Cf::QF]) {
  const char* row = qs + min(lane & 15, g - 1) * QLds<Cf>::STRIDE;
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

// Producer, first half of a block: scores of the group on MFMA, the block's
// maximum mb and sum ls per head (lane c < 16 holds head c), and its weights
// P = 2^(s - mb) (fp8: times the V scale) into the wave's LDS row buffer
// pb[GM][B] in the layout the PV product reads.
template <class Cf>
__device__ __forceinline__ void block_softmax(const BlockRegs<Cf>& r, const char* qs, int g, int nvalid, float ksc,
                                              float vsc, float qk_log2, int lane, float* pb, float& mb, float& ls) {
  f32x4 S[Cf::T];
  {
    uint4 qf[Cf::QF];
    q_from_lds<Cf>(qs, g, lane, qf);
    qk_scores<Cf>(r, qf, S);
  }
  float x[Cf::T][4];
  mb = block_scores<Cf>(S, nvalid, Cf::KV == KV_FP8 ? qk_log2 * ksc : qk_log2, lane, x);
  float sum = 0.f;
  float pq[Cf::T][4];
#pragma unroll
  for (int t = 0; t < Cf::T; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float e = __builtin_amdgcn_exp2f(x[t][rr] - mb);
      sum += e;
      pq[t][rr] = Cf::KV == KV_FP8 ? e * vsc : e;
    }
  ls = rows_sum(sum);
  const int c16 = lane & 15;
  const int q = lane >> 4;
  if (c16 < Cf::GM) {
    float* row = pb + c16 * Cf::B;
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
}

// Producer, second half of a block: P V on v_mfma_f32_4x4x1_16b_f32 with P from
// the row buffer, then the block's own normalised output o_b = (P V) / ls
// and (mb, ls) per head into its ring slot.
template <class Cf>
__device__ __forceinline__ void block_emit(const BlockRegs<Cf>& r, const float* pb, float mb, float ls, int lane,
                                           float* slot) {
  static_assert(Cf::PV4, "the stream kernel takes groups of up to 8 heads");
  f32x4 acc[Cf::NACC];
  pv_zero<Cf>(acc);
  const int rg = lane / Cf::LPR;
#pragma unroll
  for (int hg = 0; hg < Cf::HG; ++hg) {
    const float* src = pb + (4 * hg + (lane & 3)) * Cf::B + rg * Cf::NLD;
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
  pv_finish<Cf>(acc);
  // l >= 1 (the block maximum contributes 2^0) for every valid block
  const float rl = __builtin_amdgcn_rcpf(ls);
  if (lane < Cf::LPR) {
#pragma unroll
    for (int hg = 0; hg < Cf::HG; ++hg)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float sc = readlanef(rl, 4 * hg + rr);
        float* o = slot + (4 * hg + rr) * Cf::D + lane * Cf::EPL;
        float v[Cf::EPL];
#pragma unroll
        for (int e = 0; e < Cf::EPL; ++e) v[e] = acc[(hg * Cf::CH) * Cf::EPL + e][rr] * sc;
        if constexpr (Cf::EPL == 4) *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
        else if constexpr (Cf::EPL == 2) *reinterpret_cast<f32x2*>(o) = f32x2{v[0], v[1]};
        else o[0] = v[0];
      }
  }
  const int c16 = lane & 15;
  if (c16 < Cf::GM && (lane >> 4) == 0) {
    slot[Cf::GM * Cf::D + c16] = mb;
    slot[Cf::GM * Cf::D + Cf::GM + c16] = ls;
  }
}

// Detector state of one head, carried across chunks.
template <class Cf>
struct DetCarry {
  float M, L, Np;  // running maximum (log2 units), running sum, ||O_prev||^2
  int cnt;         // passes in a row
  bool sink;       // logical block 0 folded
  bool alive;
  float O[Cf::DPL];
};

// Fold chunk [t0, t0 + nt) of the ring into one head and evaluate the rule
// at every position.  Returns true if the head fired (it wrote out / stop).
template <class Cf>
__device__ __forceinline__ bool detect_chunk(DetCarry<Cf>& hc, const float* ring, int h, int t0, int nt,
                                             unsigned long long sinkbits, const Params& p, int lane, float* out_row,
                                             int32_t* stop_ptr) {
  constexpr int C = Cf::C2, DPL = Cf::DPL, SH = Cf::SH2, RING = Cf::RING, SLOTF = Cf::SLOTF;
  const int slot = lane < C ? lane : C - 1;
  const float* sl = ring + (size_t)((t0 + slot) & (RING - 1)) * SLOTF;
  const float m_in = lane < nt ? sl[Cf::GM * Cf::D + h] : NEG_INF;
  const float l_in = lane < nt ? sl[Cf::GM * Cf::D + Cf::GM + h] : 0.f;
  // this lane's coordinates of every block of the chunk
  float ob[C][DPL];
#pragma unroll
  for (int t = 0; t < C; ++t) {
    if (t < nt) {
      const float* src = ring + (size_t)((t0 + t) & (RING - 1)) * SLOTF + h * Cf::D + DPL * lane;
      if constexpr (DPL == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(src);
        ob[t][0] = v.x; ob[t][1] = v.y;
      } else {
        ob[t][0] = src[0];
      }
    } else {
#pragma unroll
      for (int j = 0; j < DPL; ++j) ob[t][j] = 0.f;
    }
  }
  // running maximum and sum at every position (lane t), from the carry
  float mx = m_in;
  if constexpr (C > 1) mx = fmaxf(mx, row_shr<1>(mx, NEG_INF));
  if constexpr (C > 2) mx = fmaxf(mx, row_shr<2>(mx, NEG_INF));
  if constexpr (C > 4) mx = fmaxf(mx, row_shr<4>(mx, NEG_INF));
  if constexpr (C > 8) mx = fmaxf(mx, row_shr<8>(mx, NEG_INF));
  mx = fmaxf(mx, hc.M);
  const float mprev = row_shr<1>(mx, hc.M);
  const float al = __builtin_amdgcn_exp2f(mprev - mx);
  const float be = __builtin_amdgcn_exp2f(m_in - mx) * l_in;
  float fa = al, fb = be;
  if constexpr (C > 1) { const float pa = row_shr<1>(fa, 1.f), pb = row_shr<1>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  if constexpr (C > 2) { const float pa = row_shr<2>(fa, 1.f), pb = row_shr<2>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  if constexpr (C > 4) { const float pa = row_shr<4>(fa, 1.f), pb = row_shr<4>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  if constexpr (C > 8) { const float pa = row_shr<8>(fa, 1.f), pb = row_shr<8>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  const float Lt = fmaf(fa, hc.L, fb);
  const float wt = lane < nt ? be * __builtin_amdgcn_rcpf(Lt) : 0.f;

  // the vector fold and the per-lane partial sums
  float st[2 * C];
  float oo[C][DPL];
#pragma unroll
  for (int t = 0; t < C; ++t) {
    const float w = readlanef(wt, t);
    float nn = 0.f, ee = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const float d = ob[t][j] - hc.O[j];
      hc.O[j] = fmaf(w, d, hc.O[j]);
      ee = fmaf(d, d, ee);
      nn = fmaf(hc.O[j], hc.O[j], nn);
      oo[t][j] = hc.O[j];
    }
    st[2 * t] = nn;
    st[2 * t + 1] = ee;
  }
  bool ps = false;
  float nn_t = 0.f;
  if (!p.skip_stats) {  // uniform: off only to measure what the statistics cost
    if (p.probe < Cf::D) {  // uniform: a probe counts only O's leading coordinates
      const bool in = DPL * lane < p.probe;
#pragma unroll
      for (int k = 0; k < 2 * C; ++k) st[k] = in ? st[k] : 0.f;
    }
    const float v0 = xreduce<2 * C>(st, lane);
    // lane (2t) << SH holds ||O_t||^2, lane (2t+1) << SH ||o_t - O_{t-1}||^2
    nn_t = __shfl(v0, (2 * slot) << SH);
    const float dd_t = __shfl(v0, (2 * slot + 1) << SH);
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
        // 1 - cos = (||O_t - O_{t-1}||^2 - (||O_t|| - ||O_{t-1}||)^2) / (2 ||O_t|| ||O_{t-1}||),
        // with O_t - O_{t-1} = w_t (o_t - O_{t-1})
        const float ee = wt * wt * dd_t;
        dd = (a == 0.f) ? 1.f : fmaxf(0.f, (ee - df * df) * __builtin_amdgcn_rcpf(2.f * a * bn));
      }
      ps = (dm < p.eps_mag) && (dd < p.eps_dir);
    }
  }
  // patience and block-0 rule at every position: passes in a row ending at t
  // (continuing the carried count when every test of the chunk up to t passed)
  const unsigned long long pass = __ballot(ps);
  const unsigned long long upto = (2ull << slot) - 1ull;
  const unsigned long long zeros = ~pass & upto;
  const int cnt_t = zeros == 0ull ? hc.cnt + slot + 1 : slot - (63 - __builtin_clzll(zeros));
  const bool sink_t = hc.sink || (sinkbits & upto) != 0ull;
  const unsigned long long fire = __ballot(lane < nt && cnt_t >= p.patience && sink_t);
  hc.M = readlanef(mx, nt - 1);
  hc.L = readlanef(Lt, nt - 1);
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
    if constexpr (DPL == 2) *reinterpret_cast<f32x2*>(out_row + 2 * lane) = f32x2{ov[0], ov[1]};
    else out_row[lane] = ov[0];
    if (lane == 0) *stop_ptr = t0 + stop_t + 1;
    hc.alive = false;
    return true;
  }
  hc.cnt = readlane(cnt_t, nt - 1);
  hc.sink = readlane(sink_t ? 1 : 0, nt - 1) != 0;
  hc.Np = readlanef(nn_t, nt - 1);
  return false;
}

template <int KV, int D, int B, int GM>
__global__ __launch_bounds__((64 * StreamCfg<KV, D, B, GM>::NW2)) void art_stream_kernel(Params p) {
  using Cf = StreamCfg<KV, D, B, GM>;
  constexpr int C = Cf::C2, NS = Cf::NS2, NP = Cf::NP2, HP = Cf::HP2, PD = Cf::PD, RING = Cf::RING;
  constexpr int SLOTF = Cf::SLOTF;
  __shared__ __attribute__((aligned(16))) float ring[RING * SLOTF];
  __shared__ __attribute__((aligned(16))) float pbuf_all[NP][PD][GM * B];
  __shared__ StreamShared sh;
  constexpr int QROWB = QLds<Cf>::ROWB;  // bytes of one query row (fp8 K: q stays bf16)
  __shared__ __attribute__((aligned(16))) char qs[GM * QLds<Cf>::STRIDE];
  __shared__ int2 ent[STREAM_ENT];

  const int stream = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = stream / p.hkv;
  const int kvh = stream - s * p.hkv;
  const int g = p.g;
  const int L = p.seq_lens[s];
  const int n = visit_count<B>(p, s, L);
  const size_t head0 = (size_t)s * p.hq + (size_t)kvh * g;

  if (n <= 0) {
    for (int i = threadIdx.x; i < g * D; i += 64 * Cf::NW2) p.out[head0 * D + i] = 0.f;
    if (threadIdx.x < g) p.stop_block[head0 + threadIdx.x] = 0;
    if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[stream] = 0;
    return;
  }
  if (threadIdx.x < 64) sh.rdy[threadIdx.x] = 0;
  // entries (order entry, page) of the first STREAM_ENT visit positions: a
  // thread's order entries are all loaded before its page lookups, so the
  // table costs two dependent loads whatever its length
  {
    const int32_t* trow = p.block_table + (size_t)s * p.max_blocks;
    const int32_t* orow = p.block_order + (size_t)s * p.max_blocks;
    constexpr int NT = 64 * Cf::NW2;
    constexpr int IT = (STREAM_ENT + NT - 1) / NT;
    const int nent = min(n, STREAM_ENT);
    int ob[IT], pg[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int t = (int)threadIdx.x + i * NT;
      ob[i] = t < nent ? orow[t] : 0;
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int t = (int)threadIdx.x + i * NT;
      pg[i] = t < nent ? trow[ob[i]] : 0;
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int t = (int)threadIdx.x + i * NT;
      if (t < nent) ent[t] = make_int2(ob[i], pg[i]);
    }
    if (threadIdx.x < 8) sh.win[threadIdx.x] = threadIdx.x + 1;
  }
  // the group's query rows, for the producers' MFMA operands
  q_to_lds<Cf>(static_cast<const char*>(p.q) + head0 * QROWB, qs, g, threadIdx.x, 64 * Cf::NW2);
  if (threadIdx.x < NS) sh.prog[threadIdx.x] = (int)threadIdx.x < g ? 0 : STREAM_BIG;
  if (threadIdx.x == 0) { sh.done = 0; sh.nfired = 0; sh.fsum = 0; sh.pfin = 0; sh.err = 0; sh.claim = 0; }
  lds_barrier();
  ART_TL(threadIdx.x == 0, 16383);

  if (w < NS) {
    // ============================ detector wave ============================
#ifndef ART_STREAM_NOPRIO
    __builtin_amdgcn_s_setprio(2);
#endif
    DetCarry<Cf> hc[HP];
    int live = 0;
#pragma unroll
    for (int k = 0; k < HP; ++k) {
      hc[k].M = NEG_INF; hc[k].L = 0.f; hc[k].Np = 0.f; hc[k].cnt = 0; hc[k].sink = false;
      hc[k].alive = w + NS * k < g;
      live += hc[k].alive ? 1 : 0;
#pragma unroll
      for (int j = 0; j < Cf::DPL; ++j) hc[k].O[j] = 0.f;
    }
    if (live == 0) return;
    bool failed = false;
    for (int t0 = 0; t0 < n; t0 += C) {
      const int nt = min(C, n - t0);
      // wait for the chunk's blocks
      int f = 0;
      bool ok;
      int spins = 0;
      for (;;) {
        f = lane < nt ? lds_ld(&sh.rdy[(t0 + lane) & (RING - 1)]) : 0;
        ok = lane >= nt || (f & 0x3fffffff) == t0 + lane + 1;
        if (__all(ok)) break;
        if (++spins > p.spin_limit || lds_ld(&sh.err)) { failed = true; break; }
        __builtin_amdgcn_s_sleep(1);
      }
      if (failed) break;
      ART_TL(lane == 0, 8192 + 8 * (t0 / C) + 2 * w);
      const unsigned long long sinkbits = __ballot(lane < nt && (f >> 30) != 0);
#pragma unroll
      for (int k = 0; k < HP; ++k) {
        const int h = w + NS * k;
        if (hc[k].alive) {
          if (detect_chunk<Cf>(hc[k], ring, h, t0, nt, sinkbits, p, lane, p.out + (head0 + h) * D,
                               p.stop_block + head0 + h)) {
            --live;
            if (lane == 0 && lds_add(&sh.nfired, 1) == g - 1) lds_st(&sh.done, 1);
          }
        }
      }
      lds_wait();  // this chunk's slots have been read
      if (lane == 0) lds_st(&sh.prog[w], live > 0 ? t0 + nt : STREAM_BIG);
      ART_TL(lane == 0, 8192 + 8 * (t0 / C) + 2 * w + 1);
      if (live == 0) break;
    }
    if (failed && lane == 0) {
      lds_st(&sh.err, 1);
      lds_st(&sh.done, 1);
      lds_st(&sh.prog[w], STREAM_BIG);
      if (p.sched_ctrl) st_dev32(p.sched_ctrl + 2, 1u);  // the workspace's sticky failure word
    }
    // heads that never fired: the output after every visited block
#pragma unroll
    for (int k = 0; k < HP; ++k) {
      const int h = w + NS * k;
      if (hc[k].alive) {
        float* o = p.out + (head0 + h) * D;
#pragma unroll
        for (int j = 0; j < Cf::DPL; ++j) o[Cf::DPL * lane + j] = failed ? __builtin_nanf("") : hc[k].O[j];
        if (lane == 0) p.stop_block[head0 + h] = failed ? -1 : n;
      }
    }
  } else {
    // ============================ producer wave ============================
    const int pw = w - NS;
    float (*pbuf)[GM * B] = pbuf_all[pw];
    const int32_t* trow = p.block_table + (size_t)s * p.max_blocks;
    const int32_t* orow = p.block_order + (size_t)s * p.max_blocks;
    const size_t tile = (size_t)B * Cf::R;
    const char* kbase = static_cast<const char*>(p.k_pages);
    const char* vbase = static_cast<const char*>(p.v_pages);
    auto frontier = [&]() __attribute__((always_inline)) {
      int f = STREAM_BIG;
#pragma unroll
      for (int k = 0; k < NS; ++k) f = min(f, lds_ld(&sh.prog[k]));
      return f;
    };
    bool failed = false;
    // Take the next visit position if it lies within the lookahead of the
    // detectors' frontier (-1 otherwise, or when every position is taken).
    // The taker of a multiple of STREAM_WIN refills the entry table's window
    // STREAM_ENT / STREAM_WIN - 2 windows ahead (its slot held positions
    // taken at least a window earlier).
    auto claim = [&]() __attribute__((always_inline)) -> int {
      // the words it decides on, read together (one LDS round trip)
      const int dn = lds_ld(&sh.done);
      const int nx = lds_ld(&sh.claim);
      const int f = frontier();
      if (dn) return -1;
      const int la = max(Cf::LA_MIN, min(Cf::LA_MAX, p.la0 + (f >> p.la_shift)));
      if (nx >= n || nx > f + la) return -1;
      int t = 0;
      if (lane == 0) t = lds_add(&sh.claim, 1);
      t = readlane(t, 0);
      if (t >= n) return -1;
      constexpr int NWIN = STREAM_ENT / STREAM_WIN;
      if (t % STREAM_WIN == 0 && t >= STREAM_WIN) {
        const int wi = t / STREAM_WIN + NWIN - 2;  // window to load
        const int lo = wi * STREAM_WIN;
        if (lo < n) {
#pragma unroll
          for (int k = 0; k < STREAM_WIN / 64; ++k) {
            const int tt = lo + 64 * k + lane;
            if (tt < n) {
              const int ob = orow[tt];
              ent[tt & (STREAM_ENT - 1)] = make_int2(ob, trow[ob]);
            }
          }
          lds_wait();
          if (lane == 0) lds_st(&sh.win[wi % NWIN], wi + 1);
        }
      }
      // this position's window must be in the table (the first windows were loaded up front)
      const int wt = t / STREAM_WIN;
      int spins = 0;
      while (t >= STREAM_ENT && lds_ld(&sh.win[wt % NWIN]) != wt + 1) {
        if (++spins > p.spin_limit) {
          failed = true;
          return -1;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      return t;
    };
    // the loads of visit position t (t < 0: a stand-in re-read of position
    // 0's tiles, so that the load instructions stay unconditional and the
    // compiler's waits on them exact)
    auto issue = [&](int t, BlockRegs<Cf>& rr, float& ks, float& vs, int& nv, int& sk) __attribute__((always_inline)) {
      const int2 e = ent[max(t, 0) & (STREAM_ENT - 1)];
      const int ob = __builtin_amdgcn_readfirstlane(e.x);
      const int pg = __builtin_amdgcn_readfirstlane(e.y);
      nv = min(B, L - ob * B);
      sk = ob == 0 ? (1 << 30) : 0;
      const size_t off = ((size_t)pg * p.hkv + kvh) * tile;
      load_block<Cf>(rr, kbase + off, vbase + off, lane, nv);
      if constexpr (KV == KV_FP8) {
        ks = p.k_scale[(size_t)pg * p.hkv + kvh];
        vs = p.v_scale[(size_t)pg * p.hkv + kvh];
      } else {
        ks = 1.f;
        vs = 1.f;
      }
    };
    int fetched = 0;  // blocks whose tiles were loaded
    unsigned long long tl_ring = 0, tl_empty = 0, tl_work = 0, tl_claim = 0, tl_iters = 0;
    BlockRegs<Cf> rg[PD];
    float ksr[PD], vsr[PD], mbs[PD], lss[PD];
    int nvr[PD], skr[PD], tr[PD];
    // prologue: a position for every register slot, then the first half of slot 0's block
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      tr[u] = claim();
      issue(tr[u], rg[u], ksr[u], vsr[u], nvr[u], skr[u]);
      fetched += tr[u] >= 0 ? 1 : 0;
      mbs[u] = 0.f;
      lss[u] = 1.f;
    }
    if (tr[0] >= 0) block_softmax<Cf>(rg[0], qs, g, nvr[0], ksr[0], vsr[0], p.qk_log2, lane, pbuf[0], mbs[0], lss[0]);
    // One iteration on register slot u (its block had its first half done)
    // and slot un (the next one), software-pipelined: wait until the ring
    // slot of u's block is free; the first half of un's block (scores,
    // softmax) and the second half of u's (PV, output) are independent and
    // share one basic block, so one's VALU work overlaps the other's MFMA
    // chain; u's block is published, and slot u takes the next position.
    // False when the producer is done.
    auto step = [&](auto uc, auto unc) __attribute__((always_inline)) -> bool {
      constexpr int u = decltype(uc)::value, un = decltype(unc)::value;
      const int t = tr[u];
      unsigned long long tl0 = ART_TL_NOW();
      (void)tl0;
      if (t >= 0) {
        int spins = 0;
        while (frontier() < t - RING + 1) {
          if (lds_ld(&sh.done)) return false;
          if (++spins > p.spin_limit) {
            failed = true;
            return false;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (lds_ld(&sh.done)) return false;
      ART_TL_ADD(tl_ring, tl0);
      tl0 = ART_TL_NOW();
      tl_iters += 1;
      ART_TL(lane == 0 && t >= 0 && t < 4096, 2 * t);
      float* sl = ring + (size_t)(max(t, 0) & (RING - 1)) * SLOTF;
      if (t >= 0 && tr[un] >= 0) {
        block_softmax<Cf>(rg[un], qs, g, nvr[un], ksr[un], vsr[un], p.qk_log2, lane, pbuf[un], mbs[un], lss[un]);
        block_emit<Cf>(rg[u], pbuf[u], mbs[u], lss[u], lane, sl);
      } else if (t >= 0) {
        block_emit<Cf>(rg[u], pbuf[u], mbs[u], lss[u], lane, sl);
      } else if (tr[un] >= 0) {
        block_softmax<Cf>(rg[un], qs, g, nvr[un], ksr[un], vsr[un], p.qk_log2, lane, pbuf[un], mbs[un], lss[un]);
      }
      if (t >= 0) {
        lds_wait();
        if (lane == 0) lds_st(&sh.rdy[t & (RING - 1)], (t + 1) | skr[u]);
        ART_TL(lane == 0 && t < 4096, 2 * t + 1);
      }
      ART_TL_ADD(tl_work, tl0);
      tl0 = ART_TL_NOW();
      tr[u] = claim();
      issue(tr[u], rg[u], ksr[u], vsr[u], nvr[u], skr[u]);
      fetched += tr[u] >= 0 ? 1 : 0;
      ART_TL_ADD(tl_claim, tl0);
      tl0 = ART_TL_NOW();
      if (failed) return false;
      bool any = false;
#pragma unroll
      for (int k = 0; k < PD; ++k) any = any || tr[k] >= 0;
      if (!any) {
        // nothing in hand: done once every position is taken, else wait for the frontier
        if (lds_ld(&sh.claim) >= n) return false;
        __builtin_amdgcn_s_sleep(2);
        ART_TL_ADD(tl_empty, tl0);
      }
      return true;
    };
    for (;;) {
      using std::integral_constant;
      if (!step(integral_constant<int, 0>{}, integral_constant<int, 1 % PD>{})) break;
      if (!step(integral_constant<int, 1 % PD>{}, integral_constant<int, 2 % PD>{})) break;
      if constexpr (PD >= 3)
        if (!step(integral_constant<int, 2 % PD>{}, integral_constant<int, 3 % PD>{})) break;
      if constexpr (PD >= 4)
        if (!step(integral_constant<int, 3 % PD>{}, integral_constant<int, 4 % PD>{})) break;
      if constexpr (PD >= 5)
        if (!step(integral_constant<int, 4 % PD>{}, integral_constant<int, 5 % PD>{})) break;
      if constexpr (PD >= 6)
        if (!step(integral_constant<int, 5 % PD>{}, integral_constant<int, 6 % PD>{})) break;
    }
    if (failed && lane == 0) {
      lds_st(&sh.err, 1);
      lds_st(&sh.done, 1);
      if (p.sched_ctrl) st_dev32(p.sched_ctrl + 2, 1u);  // the workspace's sticky failure word
    }
#ifdef ART_STREAM_TIMELINE
    if (lane == 0 && (int)blockIdx.x == art_timeline_stream) {
      art_timeline[12000 + 8 * pw + 0] = tl_ring;
      art_timeline[12000 + 8 * pw + 1] = tl_work;
      art_timeline[12000 + 8 * pw + 2] = tl_claim;
      art_timeline[12000 + 8 * pw + 3] = tl_empty;
      art_timeline[12000 + 8 * pw + 4] = tl_iters;
      art_timeline[12000 + 8 * pw + 5] = ART_TL_NOW();
    }
#endif
    // loads issued past a stop may still be in flight
    wait_all_memory();
    if (lane == 0) {
      lds_add(&sh.fsum, fetched);
      lds_wait();
      if (lds_add(&sh.pfin, 1) == NP - 1 && p.blocks_fetched) p.blocks_fetched[stream] = lds_ld(&sh.fsum);
    }
  }
}

}  // namespace kern
}  // namespace art

#ifdef ART_STREAM_TIMELINE
// measurement build only: choose the traced stream, read the timeline back
extern "C" int art_timeline_set_stream(int s) {
  return hipMemcpyToSymbol(HIP_SYMBOL(art::kern::art_timeline_stream), &s, sizeof(int)) == hipSuccess ? 0 : 1;
}
extern "C" int art_timeline_read(unsigned long long* host) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(art::kern::art_timeline), 16384 * 8) == hipSuccess ? 0 : 1;
}
#endif
