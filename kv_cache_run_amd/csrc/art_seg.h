// gfx950 kernel for ART paged decode attention: the segment kernel
// (art_seg_kernel).  A stream (sequence, kv-head) is cut into segments of S
// visit positions, and different workgroups work on different segments of
// one stream at once, so a long stream is not walked by one CU alone.
//
// Method: "ART: Attention Run-time Termination for Efficient Large Language
// Model Decoding" (gist.science explainer), Technical Summary 2.1 (streaming,
// tile-wise accumulation: the softmax state of a prefix is an associative
// combine of its blocks' states), 2.2 (magnitude and direction statistics),
// 2.3 (patience), 2.4 (visit order, block 0 folded before any stop).
//
// Persistent workgroups claim items (stream, segment j) in segment order per
// stream, at most `seg_win` + frontier / 2 segments past the stream's resolved
// frontier, so the KV read past a stop is bounded; a workgroup that would
// otherwise wait (every stream at its window) claims further ahead on the
// stream that has run longest without stopping (up to (seg_ext + 1) x
// frontier + 2 seg_win segments), so that idle CUs shorten the long streams.
// Every wait is on an item claimed earlier (a predecessor segment of the same
// stream, or an earlier item of the same workgroup), so no claim order can
// deadlock, and the results do not depend on the claim order.  Per item:
//  1. producer waves turn the segment's blocks into per-block results
//     (o_b = block-normalised output, m_b, l_b per head) in LDS, as the stream
//     kernel's producers do;
//  2. one detector wave per query head combines them into the segment's
//     aggregate G_j = (M, L, A) and publishes it; it takes the state entering
//     the segment, X_j = G_0 + ... + G_{j-1}, by decoupled look-back (the
//     nearest published inclusive state, then the aggregates after it), and
//     publishes X_j + G_j;
//  3. from X_j it folds the segment's blocks in visit order and evaluates both
//     statistics at every position (the stream kernel's detector arithmetic),
//     and publishes the pass bits and the block-0 bits of the segment;
//  4. the pass count, block-0 flag and running flag entering the segment are
//     replayed from the nearest resolved segment over the pass bits published
//     after it; with them the head's stop inside the segment, if any, is
//     found, its output (folded again from the chunk holding the stop) and
//     stop are written, and the segment's resolved state is published.
// A stream whose heads have all stopped takes no more claims.  Status words
// carry the call's epoch (words of earlier calls read as unset); per-stream
// counters are cleared by the last workgroup to finish.  Every wait is
// bounded (p.spin_limit polls); a wait that runs out marks the head with
// stop -1 and NaN output and sets the workspace's failure word.
#pragma once

#include "art_stream.h"

namespace art {
namespace kern {

template <int KV_, int D_, int B_, int GM_>
struct SegCfg : StreamCfg<KV_, D_, B_, GM_> {
  using SC = StreamCfg<KV_, D_, B_, GM_>;
  static constexpr int SLOTF = SC::SLOTF;
  // positions per segment: the segment's per-block results fit 66560 bytes
  // of LDS
  static constexpr int S_RAW = 66560 / (SLOTF * 4);
  static constexpr int S = S_RAW >= 32 ? 32 : (S_RAW >= 16 ? 16 : 8);
  static constexpr int NS3 = 4;                               // detector waves per set
  static constexpr int HP3 = GM_ / NS3 > 0 ? GM_ / NS3 : 1;   // query heads per detector wave
#ifdef ART_SEG_SETS
  static constexpr int SETS = ART_SEG_SETS;
#else
  static constexpr int SETS = 2;                              // detector sets (items alternate between them)
#endif
#ifdef ART_SEG_NP
  static constexpr int NP3 = ART_SEG_NP;
#else
  static constexpr int NP3 = 4;                               // producer waves
#endif
  static constexpr int NW3 = SETS * NS3 + NP3;
  // register ring of a producer: two blocks, one for 32-token blocks (bf16:
  // a block's tiles alone take 64 VGPRs of a lane; fp8: its conversions)
  static constexpr int PD = (SC::TILE_V >= 64 || (B_ >= 32 && KV_ != KV_F32)) ? 1 : SC::PD;
  static constexpr int C3 = 8;                                // positions per detector chunk
  static constexpr int NCH = S / C3;                          // detector chunks per segment
  static constexpr int SH3 = 6 - ilog2(2 * C3);
  static_assert(S % C3 == 0 && S <= 32, "a segment is whole chunks, at most 32 positions");
  static_assert(NS3 * HP3 >= GM_, "every head has a detector wave");
};

// Fields of a segment's resolved status (level LB_FIN): running flag,
// block-0-folded flag, pass count at the segment's end.
constexpr uint32_t SG_RUN = 1u << 3, SG_SINK = 1u << 4;
// A head known to have stopped in an earlier segment: resolved, not running,
// and nothing else published (no records).
constexpr uint32_t SG_DEAD = 5u;
constexpr int SG_CNT_SH = 5;
constexpr int SG_CNT_MAX = (1 << 26) - 1;
// Segments of at most 16 positions publish their pass bits inside the status
// word (level LB_PASS): bit 3 + t for position t, and at bit 19 one plus the
// position holding logical block 0 (0: none; block 0 occurs once in an
// order row).  One 64-bit store then carries the level and its bits, so the
// store needs no wait before it and the replay no load after its poll.
// Longer segments keep the bits in the record after the inclusive state.
constexpr int SG_PB_SH = 3, SG_PK_SH = 19;
__device__ __forceinline__ uint32_t sg_pass_word(uint32_t pass, uint32_t sinkb) {
  return LB_PASS | (pass << SG_PB_SH) | ((sinkb ? (uint32_t)__builtin_ctz(sinkb) + 1u : 0u) << SG_PK_SH);
}
__device__ __forceinline__ void sg_pass_bits(uint32_t w, uint32_t& pass, uint32_t& sinkb) {
  pass = (w >> SG_PB_SH) & 0xFFFFu;
  const uint32_t k = (w >> SG_PK_SH) & 31u;
  sinkb = k ? 1u << (k - 1u) : 0u;
}
constexpr int SEG_END = -1, SEG_BUBBLE = -2;

// LDS words of the segment kernel; [b]: item buffer b.  Item k of the
// workgroup goes to buffer k & 1 and to detector set k mod SETS.
struct SegShared {
  int info[2][5];   // stream (or SEG_END), segment, visit positions n, tokens L, group already stopped
  int claim[2];     // next segment position for a producer
  int claimed[2];   // k + 1 once item k's description is in the buffer
  int pdone[2];     // producer waves finished with the buffer's item
  int produced[2];  // k + 1 once item k's per-block results are complete
  int ddone[2];     // detector waves finished with the buffer's item
  int freed[2];     // k + 1 once item k's detectors are done with the buffer
  int end;          // index of the first item that does not exist
  int err;          // a bounded wait ran out
  int last_wg;
  int pad;
};

// Detector state of one head inside a segment.
template <class Cf>
struct SegCarry {
  float M, L, Np;  // running maximum (log2 units), running sum, ||O||^2 (probe coordinates)
  float O[Cf::DPL];
};

__device__ __forceinline__ float wave_max(float x) {
  x = rows_max(x);
  x = fmaxf(x, dpp<DPP_ROW_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_XOR2>(x));
  return fmaxf(x, dpp<DPP_XOR1>(x));
}

// Fold chunk [c0, c0 + nt) of the segment's LDS results into one head and
// evaluate both statistics at its positions (global visit positions tg0 ..);
// the same arithmetic as the stream kernel's detector.  Returns the pass bits
// (bit k: position c0 + k passed); KEEP: oo[k] = the output at position c0 + k.
template <class Cf, bool KEEP>
__device__ __forceinline__ unsigned long long seg_chunk(SegCarry<Cf>& hc, const float* slots, int h, int c0, int nt,
                                                        int tg0, const Params& p, int lane,
                                                        float (&oo)[Cf::C3][Cf::DPL]) {
  constexpr int C = Cf::C3, DPL = Cf::DPL, SH = Cf::SH3, SLOTF = Cf::SLOTF, GM = Cf::GM, D = Cf::D;
  const int slot = lane < C ? lane : C - 1;
  const float* sl = slots + (size_t)(c0 + slot) * SLOTF;
  const float m_in = lane < nt ? sl[GM * D + h] : NEG_INF;
  const float l_in = lane < nt ? sl[GM * D + GM + h] : 0.f;
  float ob[C][DPL];
#pragma unroll
  for (int t = 0; t < C; ++t) {
    if (t < nt) {
      const float* src = slots + (size_t)(c0 + t) * SLOTF + h * D + DPL * lane;
      if constexpr (DPL == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(src);
        ob[t][0] = v.x;
        ob[t][1] = v.y;
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
  mx = fmaxf(mx, row_shr<1>(mx, NEG_INF));
  mx = fmaxf(mx, row_shr<2>(mx, NEG_INF));
  mx = fmaxf(mx, row_shr<4>(mx, NEG_INF));
  mx = fmaxf(mx, hc.M);
  const float mprev = row_shr<1>(mx, hc.M);
  const float al = __builtin_amdgcn_exp2f(mprev - mx);
  const float be = __builtin_amdgcn_exp2f(m_in - mx) * l_in;
  float fa = al, fb = be;
  { const float pa = row_shr<1>(fa, 1.f), pb = row_shr<1>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  { const float pa = row_shr<2>(fa, 1.f), pb = row_shr<2>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  { const float pa = row_shr<4>(fa, 1.f), pb = row_shr<4>(fb, 0.f); fb = fmaf(fa, pb, fb); fa *= pa; }
  const float Lt = fmaf(fa, hc.L, fb);
  const float wt = lane < nt ? be * __builtin_amdgcn_rcpf(Lt) : 0.f;

  // the vector fold and the per-lane partial sums
  float st[2 * C];
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
      if constexpr (KEEP) oo[t][j] = hc.O[j];
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
    if (lane < nt && tg0 + lane >= 1) {
      const float a = __builtin_amdgcn_sqrtf(nn_t);
      const float bn = __builtin_amdgcn_sqrtf(np_t);
      float dm, dd;
      if (a == 0.f && bn == 0.f) {
        dm = 0.f;
        dd = 0.f;
      } else if (bn == 0.f) {
        dm = __builtin_inff();
        dd = 1.f;
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
  hc.M = readlanef(mx, nt - 1);
  hc.L = readlanef(Lt, nt - 1);
  hc.Np = readlanef(nn_t, nt - 1);
  return __ballot(ps);
}

// Patience and block-0 rule over one segment (lane t = position t < ns):
// from the state entering it (cnt, sink, run), the first position where the
// head fires (fire_at, or unchanged when none) and the state at its end.
__device__ __forceinline__ void seg_apply(int& cnt, bool& sink, bool& run, uint32_t pass, uint32_t sinkb, int ns,
                                          int cap, int patience, int lane, int& fire_at) {
  const int slot = lane < 32 ? lane : 31;
  const unsigned long long upto = (2ull << slot) - 1ull;
  const unsigned long long zeros = ~(unsigned long long)pass & upto;
  const int cnt_t = zeros == 0ull ? min(cnt + slot + 1, cap) : slot - (63 - __builtin_clzll(zeros));
  const bool sink_t = sink || ((unsigned long long)sinkb & upto) != 0ull;
  const unsigned long long fire = __ballot(run && lane < ns && cnt_t >= patience && sink_t);
  if (fire != 0ull) {
    fire_at = __builtin_ctzll(fire);
    run = false;
  }
  cnt = readlane(cnt_t, ns - 1);
  sink = readlane(sink_t ? 1 : 0, ns - 1) != 0;
}

// Status of segment j-1-lane of one head (all 64 lanes); before segment 0:
// resolved, running, nothing folded.
__device__ __forceinline__ uint32_t seg_probe(const u64* st0, int g, int j, uint32_t E, int lane) {
  const int jj = j - 1 - lane;
  return jj >= 0 ? tag_val(ld_dev(st0 + (size_t)jj * g), E, 0u) : (LB_FIN | SG_RUN);
}

// The query heads h0 + NS k (k < HP) of one item, in one detector wave:
// aggregate, look back, detect, resolve.  The heads go through every phase
// together, so their waits on other workgroups overlap: a poll reads the
// status words of both heads at once (lanes [k LPH, (k + 1) LPH) examine head
// k's segments j-1-(lane - k LPH)).  A wait that runs past the spin limit
// fails every head of the wave (stop -1, NaN output).
template <class Cf>
__device__ void seg_heads(const Params& p, uint32_t E, int s, int j, int n, int ns, int h0, const float* slots,
                          const int2* ent, int lane) {
  constexpr int S = Cf::S, C = Cf::C3, DPL = Cf::DPL, D = Cf::D, GM = Cf::GM, SLOTF = Cf::SLOTF, NCH = Cf::NCH;
  constexpr int HP = Cf::HP3, NS = Cf::NS3;
  constexpr int LPH = 64 / HP;  // lanes per head in a poll (segments examined per head)
  const int g = p.g;
  const int t0 = j * S;
  const bool last = t0 + ns >= n;
  const size_t rstride = (size_t)g * p.rec_floats;
  const int incl = D + 4;  // the inclusive state follows the aggregate
  const int cap = min(p.patience, SG_CNT_MAX);
  const int kh = lane / LPH;  // the head this lane examines in a poll
  const int li = lane - kh * LPH;
  auto head_of = [&](int k) { return h0 + NS * k; };
  auto stw_of = [&](int k) { return p.lb_st + ((size_t)s * p.max_chunks + j) * g + head_of(k); };
  auto rec_of = [&](int k) { return p.lb_rec + (((size_t)s * p.max_chunks + j) * g + head_of(k)) * p.rec_floats; };
  auto rec0_of = [&](int k) { return p.lb_rec + ((size_t)s * p.max_chunks * g + head_of(k)) * p.rec_floats; };
  auto part = [&](unsigned long long b, int k) -> unsigned long long {
    return HP == 1 ? b : (b >> (k * LPH)) & ((1ull << LPH) - 1ull);
  };
  // status of segment j-1-li of head kh (lanes of inactive heads read "resolved, running")
  auto probe = [&](const bool (&act)[HP]) {
    bool a = false;
#pragma unroll
    for (int k = 0; k < HP; ++k) a = (kh == k) ? act[k] : a;
    const int h = min(head_of(kh), g - 1);
    const int jj = j - 1 - li;
    if (!a || jj < 0) return (uint32_t)(LB_FIN | SG_RUN);
    return tag_val(ld_dev(p.lb_st + ((size_t)s * p.max_chunks + jj) * g + h), E, 0u);
  };

  bool act[HP];  // heads of the group, not yet dead
#pragma unroll
  for (int k = 0; k < HP; ++k) act[k] = head_of(k) < g;

  // ---- each head's own aggregate of the segment
  float gm[HP], gl[HP], ga[HP][DPL];
  {
    const int tl = min(lane, S - 1);
#pragma unroll
    for (int k = 0; k < HP; ++k) {
      const int h = min(head_of(k), GM - 1);
      const float mt = lane < ns ? slots[(size_t)tl * SLOTF + GM * D + h] : NEG_INF;
      const float lt = lane < ns ? slots[(size_t)tl * SLOTF + GM * D + GM + h] : 0.f;
      gm[k] = wave_max(mt);
      float e[1] = {lane < ns ? __builtin_amdgcn_exp2f(mt - gm[k]) * lt : 0.f};
      const float el = e[0];
      gl[k] = xreduce<1>(e, lane);
#pragma unroll
      for (int q = 0; q < DPL; ++q) ga[k][q] = 0.f;
      // eight positions' loads at a time, then their products in order
      for (int t0c = 0; t0c < ns; t0c += 8) {
        float v[8][DPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float* src = slots + (size_t)min(t0c + u, S - 1) * SLOTF + h * D + DPL * lane;
#pragma unroll
          for (int q = 0; q < DPL; ++q) v[u][q] = src[q];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float et = t0c + u < ns ? readlanef(el, t0c + u) : 0.f;
#pragma unroll
          for (int q = 0; q < DPL; ++q) ga[k][q] = fmaf(et, v[u][q], ga[k][q]);
        }
      }
    }
  }

  // A head whose stop lies in an earlier segment is dead here: its bit in
  // the stopped-head mask is set only once that segment has resolved, and a
  // segment resolves only after every segment before it published its pass
  // bits, so a bit seen before this segment's own pass bits are out means a
  // stop before this segment (once the pass bits are out, a bit may come
  // from a later stop, so the mask is not consulted after that).  Dead heads
  // publish SG_DEAD and nothing else.
  auto kill_dead = [&](uint32_t mword, unsigned long long dead_ballot) {
#pragma unroll
    for (int k = 0; k < HP; ++k)
      if (act[k] && ((((mword >> head_of(k)) & 1u) != 0u) || part(dead_ballot, k) != 0ull)) {
        if (lane == 0) st_dev(stw_of(k), tag_word(E, SG_DEAD));
        act[k] = false;
      }
  };
  kill_dead(ld_dev32(p.lb_heads + s), 0ull);

  // ---- state entering the segment: nearest published inclusive state, then
  // the aggregates after it in segment order; a head publishes its aggregate
  // first unless that state can be had at once
  LbState<Cf> x[HP];
#pragma unroll
  for (int k = 0; k < HP; ++k) {
    x[k].M = NEG_INF;
    x[k].L = 0.f;
#pragma unroll
    for (int q = 0; q < DPL; ++q) x[k].A[q] = 0.f;
  }
  bool ok = true;
  if (j > 0) {
    bool found[HP], pub[HP];
    int f[HP];
#pragma unroll
    for (int k = 0; k < HP; ++k) { found[k] = !act[k]; pub[k] = false; f[k] = 0; }
    for (int spin = 0;; ++spin) {
      const uint32_t v = probe(act);
      const uint32_t lvl = v & LB_LEVEL;
      const uint32_t mword = ld_dev32(p.lb_heads + s);
      kill_dead(mword, __ballot(lvl == SG_DEAD));
      const unsigned long long inc = __ballot(lvl >= LB_INCL && lvl <= LB_FIN);
      const unsigned long long agg = __ballot(lvl >= LB_AGG && lvl <= LB_FIN);
      bool all = true;
#pragma unroll
      for (int k = 0; k < HP; ++k) {
        if (!act[k]) { found[k] = true; continue; }
        if (!found[k]) {
          const unsigned long long ik = part(inc, k);
          if (ik != 0ull) {
            const int fk = __builtin_ctzll(ik);
            const unsigned long long need = (1ull << fk) - 1ull;
            if ((part(agg, k) & need) == need) { found[k] = true; f[k] = fk; }
          }
        }
        all = all && found[k];
      }
      if (all) break;
      bool stored = false;
#pragma unroll
      for (int k = 0; k < HP; ++k)
        if (!found[k] && !pub[k]) {
          lb_store<Cf>(rec_of(k), lane, gm[k], gl[k], ga[k]);
          pub[k] = true;
          stored = true;
        }
      if (stored) {
        wait_all_memory();
#pragma unroll
        for (int k = 0; k < HP; ++k)
          if (pub[k] && !found[k] && lane == 0) st_dev(stw_of(k), tag_word(E, LB_AGG));
      }
      if (lb_give_up(p, E, spin)) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (ok) {
#pragma unroll
      for (int k = 0; k < HP; ++k) {
        if (!act[k]) continue;
        const float* rec0 = rec0_of(k);
        const int jb = j - 1 - f[k];
        if (jb >= 0) lb_load<Cf>(rec0 + (size_t)jb * rstride + incl, lane, x[k].M, x[k].L, x[k].A);
        // the aggregates after it, folded in segment order; their loads go
        // out LB at a time (the fold order, and so the bits, is unchanged)
#ifdef ART_SEG_LB
        constexpr int LB = ART_SEG_LB;
#else
        constexpr int LB = 8;
#endif
        for (int i0 = f[k] - 1; i0 >= 0; i0 -= LB) {
          float mb[LB], lb[LB], ab[LB][DPL];
#pragma unroll
          for (int u = 0; u < LB; ++u)
            if (i0 - u >= 0) lb_load<Cf>(rec0 + (size_t)(j - 1 - (i0 - u)) * rstride, lane, mb[u], lb[u], ab[u]);
#pragma unroll
          for (int u = 0; u < LB; ++u)
            if (i0 - u >= 0) lb_combine<Cf>(x[k], mb[u], lb[u], ab[u]);
        }
      }
    }
  }
  if (ok) {
#pragma unroll
    for (int k = 0; k < HP; ++k) {
      if (!act[k]) continue;
      LbState<Cf> xi = x[k];
      lb_combine<Cf>(xi, gm[k], gl[k], ga[k]);
      lb_store<Cf>(rec_of(k) + incl, lane, xi.M, xi.L, xi.A);
    }
    wait_all_memory();
#pragma unroll
    for (int k = 0; k < HP; ++k)
      if (act[k] && lane == 0) st_dev(stw_of(k), tag_word(E, LB_INCL));
  }

  // ---- statistics of every position, from X_j (a head found dead here is
  // resolved as stopped; the mask is read before the statistics and looked at
  // after them, so its latency hides behind them)
  const uint32_t mword2 = ld_dev32(p.lb_heads + s);
  // the carry entering the segment, from X_j
  auto enter = [&](SegCarry<Cf>& e, const LbState<Cf>& xs) {
    const float rl = xs.L > 0.f ? __builtin_amdgcn_rcpf(xs.L) : 0.f;
    float sq[1] = {0.f};
#pragma unroll
    for (int q = 0; q < DPL; ++q) {
      e.O[q] = xs.L > 0.f ? xs.A[q] * rl : 0.f;
      const float op = DPL * lane + q < p.probe ? e.O[q] : 0.f;
      sq[0] = fmaf(op, op, sq[0]);
    }
    e.M = xs.M;
    e.L = xs.L;
    e.Np = xreduce<1>(sq, lane);
  };
  SegCarry<Cf> hc[HP];
  uint32_t passb[HP];
#pragma unroll
  for (int k = 0; k < HP; ++k) {
    enter(hc[k], x[k]);
    passb[k] = 0u;
  }
  if (ok) {
    float oo_unused[C][DPL];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c * C < ns) {
#pragma unroll
        for (int k = 0; k < HP; ++k)
          if (act[k]) {
            const u64 pb = seg_chunk<Cf, false>(hc[k], slots, head_of(k), c * C, min(C, ns - c * C), t0 + c * C, p,
                                                lane, oo_unused);
            passb[k] |= (uint32_t)pb << (c * C);
          }
      }
    }
  }
  bool dead[HP];
#pragma unroll
  for (int k = 0; k < HP; ++k) {
    dead[k] = act[k] && ((mword2 >> head_of(k)) & 1u) != 0u;
    if (dead[k]) passb[k] = 0u;
  }
  const uint32_t sinkb = (uint32_t)__ballot(lane < ns && ent[min(lane, S - 1)].x == 0);
  constexpr bool BITS_IN_STATUS = S <= 16;
  if (ok) {
    if constexpr (BITS_IN_STATUS) {
#pragma unroll
      for (int k = 0; k < HP; ++k)
        if (act[k] && lane == 0) st_dev(stw_of(k), tag_word(E, sg_pass_word(passb[k], sinkb)));
    } else {
#pragma unroll
      for (int k = 0; k < HP; ++k)
        if (act[k] && lane == 0) st_dev(reinterpret_cast<u64*>(rec_of(k) + D + 2), ((u64)sinkb << 32) | passb[k]);
      wait_all_memory();
#pragma unroll
      for (int k = 0; k < HP; ++k)
        if (act[k] && lane == 0) st_dev(stw_of(k), tag_word(E, LB_PASS));
    }
  }

  // ---- pass count, block-0 flag and running flag entering the segment
  int cnt[HP];
  bool sink[HP], run[HP];
#pragma unroll
  for (int k = 0; k < HP; ++k) { cnt[k] = 0; sink[k] = false; run[k] = act[k]; }
  if (ok && j > 0) {
    uint32_t v = 0u;
    int f[HP];
#pragma unroll
    for (int k = 0; k < HP; ++k) f[k] = 0;
    for (int spin = 0;; ++spin) {
      v = probe(act);
      const uint32_t lvl = v & LB_LEVEL;
      const unsigned long long fin = __ballot(lvl == LB_FIN || lvl == SG_DEAD);
      const unsigned long long pas = __ballot(lvl == LB_PASS);
      bool all = true;
#pragma unroll
      for (int k = 0; k < HP; ++k) {
        if (!act[k]) continue;
        const unsigned long long fk = part(fin, k);
        bool got = false;
        if (fk != 0ull) {
          f[k] = __builtin_ctzll(fk);
          const unsigned long long need = (1ull << f[k]) - 1ull;
          got = (part(pas, k) & need) == need;
        }
        all = all && got;
      }
      if (all) break;
      if (lb_give_up(p, E, spin)) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (ok) {
#pragma unroll
      for (int k = 0; k < HP; ++k) {
        if (!act[k]) continue;
        const uint32_t wf = (uint32_t)readlane((int)v, k * LPH + f[k]);
        cnt[k] = (int)(wf >> SG_CNT_SH);
        sink[k] = (wf & SG_SINK) != 0u;
        run[k] = (wf & LB_LEVEL) == LB_FIN && (wf & SG_RUN) != 0u;
        // bits of segments j-f .. j-1 (lane i: segment j-1-i): in the
        // status words of the last poll, or read together from the records
        u64 bits = 0ull;
        if constexpr (!BITS_IN_STATUS)
          if (lane < f[k]) bits = ld_dev(reinterpret_cast<const u64*>(rec0_of(k) + (size_t)(j - 1 - lane) * rstride + D + 2));
        for (int i = f[k] - 1; i >= 0 && run[k]; --i) {
          uint32_t pw, kw;
          if constexpr (BITS_IN_STATUS) {
            sg_pass_bits((uint32_t)readlane((int)v, k * LPH + i), pw, kw);
          } else {
            pw = (uint32_t)readlane((int)(uint32_t)bits, i);
            kw = (uint32_t)readlane((int)(uint32_t)(bits >> 32), i);
          }
          int unused = -1;
          seg_apply(cnt[k], sink[k], run[k], pw, kw, S, cap, p.patience, lane, unused);
        }
      }
    }
  }

  // ---- the segment's own positions, the resolved states, the outputs
  bool stopped[HP];
#pragma unroll
  for (int k = 0; k < HP; ++k) {
    stopped[k] = false;
    if (!act[k]) continue;
    const int h = head_of(k);
    const size_t head = (size_t)(s / p.hkv) * p.hq + (size_t)(s % p.hkv) * g + h;
    float* out_row = p.out + head * D;
    int fire_at = -1;
    if (ok && run[k] && !dead[k]) seg_apply(cnt[k], sink[k], run[k], passb[k], sinkb, ns, cap, p.patience, lane, fire_at);
    if (ok && dead[k]) run[k] = false;
    if (ok && lane == 0)
      st_dev(stw_of(k), tag_word(E, LB_FIN | (run[k] ? SG_RUN : 0u) | (sink[k] ? SG_SINK : 0u) |
                                        ((uint32_t)min(cnt[k], cap) << SG_CNT_SH)));
    if (ok && fire_at >= 0) {
      // fold the segment again up to the chunk holding the stop (the same
      // arithmetic, so the same output as the statistics saw)
      const int c = fire_at / C;
      SegCarry<Cf> h2;
      enter(h2, x[k]);
      float oo[C][DPL];
      for (int cc = 0; cc < c; ++cc)
        (void)seg_chunk<Cf, false>(h2, slots, h, cc * C, C, t0 + cc * C, p, lane, oo);
      (void)seg_chunk<Cf, true>(h2, slots, h, c * C, min(C, ns - c * C), t0 + c * C, p, lane, oo);
      const int kk = fire_at - c * C;
      float ov[DPL];
#pragma unroll
      for (int q = 0; q < DPL; ++q) ov[q] = oo[0][q];
#pragma unroll
      for (int t = 1; t < C; ++t)
        if (kk == t)
#pragma unroll
          for (int q = 0; q < DPL; ++q) ov[q] = oo[t][q];
#pragma unroll
      for (int q = 0; q < DPL; ++q) out_row[DPL * lane + q] = ov[q];
      if (lane == 0) p.stop_block[head] = t0 + fire_at + 1;
      stopped[k] = true;
    } else if (ok && run[k] && last) {
      // never stopped: the output after all n blocks
#pragma unroll
      for (int q = 0; q < DPL; ++q) out_row[DPL * lane + q] = hc[k].O[q];
      if (lane == 0) p.stop_block[head] = n;
      stopped[k] = true;  // its result is written
    }
    if (!ok) {
#pragma unroll
      for (int q = 0; q < DPL; ++q) out_row[DPL * lane + q] = __builtin_nanf("");
      if (lane == 0) {
        p.stop_block[head] = -1;
        lb_fail(p, E);
      }
      stopped[k] = true;
    }
  }
  bool any = false;
#pragma unroll
  for (int k = 0; k < HP; ++k) any = any || stopped[k];
  if (any) wait_all_memory();  // the resolved statuses are out before the mask bits
  if (any && lane == 0) {
    // mark the heads finished; close the stream when the whole group is
    uint32_t bits = 0u;
#pragma unroll
    for (int k = 0; k < HP; ++k)
      if (stopped[k]) bits |= 1u << head_of(k);
    const uint32_t was = __hip_atomic_fetch_or(p.lb_heads + s, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((was | bits) == (1u << g) - 1u && was != (was | bits))
      __hip_atomic_fetch_or(p.lb_claim + s, CLAIM_FIN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Claim the next item (whole wave 0): a segment of the current stream while
// its window has room, else of the stream with the most unclaimed segments
// (counted up to 16; ties spread over the workgroups), else (every stream at
// its window) past the window of the longest-running stream, within
// p.seg_ext's bound.  Loads the segment's
// (order entry, page) pairs and the group's query rows into LDS.
template <class Cf>
__device__ void seg_claim(const Params& p, uint32_t E, int* info, int* pclaim, int2* ent, char* qdst, int& cur,
                          bool& ended, int lane) {
  constexpr int S = Cf::S;
  constexpr int QROWB = Cf::KV == KV_FP8 ? 2 * Cf::D : Cf::R;
  const int NSTR = p.batch * p.hkv;
  int got_s = -1, got_j = 0;
  auto nseg_of = [&](int st) { return (visit_count<Cf::B>(p, st / p.hkv, p.seq_lens[st / p.hkv]) + S - 1) / S; };
  auto take = [&](int st) {  // lane 0 adds, the wave gets the segment index (or -1)
    uint32_t k = 0;
    if (lane == 0) k = __hip_atomic_fetch_add(p.lb_claim + st, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    k = (uint32_t)readlane((int)k, 0);
    return ((k & CLAIM_FIN) || (int)k >= nseg_of(st)) ? -1 : (int)k;
  };
  // the words the current stream's claim decides on are loaded together:
  // the call's failure word, the stream's claim count and frontier, its length
  const uint32_t failw = ld_dev32(p.sched_ctrl + 3);
  uint32_t cv0 = CLAIM_FIN, prog0 = 0u;
  int n0 = 0;
  if (cur >= 0) {
    cv0 = ld_dev32(p.lb_claim + cur);
    prog0 = ld_dev32(p.lb_prog + cur);
    n0 = visit_count<Cf::B>(p, cur / p.hkv, p.seq_lens[cur / p.hkv]);
  }
  // the order entries of the segment this claim most likely takes (the one
  // the claim count names) are loaded with the claim itself
  int pred_s = -1, pred_j = -1, ob_pred = 0;
  if (!ended && failw == E) ended = true;  // a bounded wait of this call gave up
  if (!ended) {
    // segments claimable past the resolved frontier: seg_win + frontier / 2
    auto window = [&](uint32_t prog) { return prog + (uint32_t)p.seg_win + (prog >> 1); };
    if (cur >= 0) {
      if (!(cv0 & CLAIM_FIN) && (int)cv0 < (n0 + S - 1) / S && cv0 < window(prog0)) {
        pred_s = cur;
        pred_j = (int)cv0;
        const int tp = pred_j * S + lane;
        if (lane < S && tp < n0) ob_pred = p.block_order[(size_t)(cur / p.hkv) * p.max_blocks + tp];
        const int k = take(cur);
        if (k >= 0) {
          got_s = cur;
          got_j = k;
        }
      }
    }
    if (got_s < 0) {
      uint32_t best = 0u;  // (min(remaining, 16) << 24) | (hash << 16) | stream, 0 = none
      // idle speculation: every live stream is at its window, so this
      // workgroup would wait; claim past the window of the stream that has
      // run longest without stopping, up to (seg_ext + 1) x frontier +
      // 2 seg_win segments.  Key (min(frontier, 255) << 24) | (hash << 16) |
      // stream.
      uint32_t best2 = 0u;
      bool live_any = false;
      const uint32_t hw = (blockIdx.x * 2654435761u) >> 24;
      auto ext_window = [&](uint32_t prog) {
        return p.seg_ext <= 0 ? 0u
               : p.seg_ext >= 4096 ? 0xFFFFFFFFu
                                   : (uint32_t)(p.seg_ext + 1) * prog + 2u * (uint32_t)p.seg_win;
      };
      for (int base = 0; base < NSTR; base += 64) {
        const int st = base + lane;
        uint32_t key = 0u, key2 = 0u;
        if (st < NSTR) {
          const uint32_t cv = ld_dev32(p.lb_claim + st);
          const uint32_t prog = ld_dev32(p.lb_prog + st);
          const int ns = nseg_of(st);
          const bool live = !(cv & CLAIM_FIN) && (int)cv < ns;
          live_any |= live;
          const uint32_t hash = ((((uint32_t)st * 40503u) ^ hw) & 0xFFu) << 16;
          if (live && cv < window(prog))
            key = ((uint32_t)min(ns - (int)cv, 16) << 24) | hash | (uint32_t)st;
          else if (live && cv < ext_window(prog))
            key2 = (min(prog, 255u) << 24) | hash | (uint32_t)st;
        }
        uint32_t mk = key, mk2 = key2;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          mk = max(mk, (uint32_t)__shfl_xor((int)mk, o));
          mk2 = max(mk2, (uint32_t)__shfl_xor((int)mk2, o));
        }
        best = max(best, mk);
        best2 = max(best2, mk2);
      }
      live_any = __ballot(live_any) != 0ull;
      if (best == 0u) best = best2;
      if (best != 0u) {
        const int st = (int)(best & 0xFFFFu);
        const int k = take(st);
        if (k >= 0) {
          got_s = st;
          got_j = k;
        }
        cur = st;
      } else if (!live_any) {
        ended = true;
      }
    }
  }
  if (got_s < 0) {
    if (lane == 0) info[0] = ended ? SEG_END : SEG_BUBBLE;
    return;
  }
  cur = got_s;
  const int sq = got_s / p.hkv;
  const int kvh = got_s - sq * p.hkv;
  const int L = p.seq_lens[sq];
  const int n = visit_count<Cf::B>(p, sq, L);
  const int t0 = got_j * S;
  const int ns = min(S, n - t0);
  const int32_t* orow = p.block_order + (size_t)sq * p.max_blocks;
  const int32_t* trow = p.block_table + (size_t)sq * p.max_blocks;
  if (lane < ns) {
    const int ob = got_s == pred_s && got_j == pred_j ? ob_pred : orow[t0 + lane];
    ent[lane] = make_int2(ob, trow[ob]);
  }
  q_to_lds<Cf>(static_cast<const char*>(p.q) + ((size_t)sq * p.hq + (size_t)kvh * p.g) * QROWB, qdst, p.g, lane, 64);
  // a group whose heads have all stopped needs nothing more (the stops lie
  // in earlier segments: a segment resolves only after this one's pass bits)
  const bool done = ld_dev32(p.lb_heads + got_s) == (1u << p.g) - 1u;
  if (lane == 0) {
    info[0] = got_s;
    info[1] = got_j;
    info[2] = n;
    info[3] = L;
    info[4] = done ? 1 : 0;
    *pclaim = 0;
    if (!done)
      __hip_atomic_fetch_add(p.lb_fetch + got_s, (uint32_t)ns, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int KV, int D, int B, int GM>
__global__ __launch_bounds__((64 * SegCfg<KV, D, B, GM>::NW3)) void art_seg_kernel(Params p) {
  using Cf = SegCfg<KV, D, B, GM>;
  constexpr int S = Cf::S, NS = Cf::NS3, NP = Cf::NP3, HP = Cf::HP3, PD = Cf::PD, SLOTF = Cf::SLOTF;
  constexpr int QROWB = KV == KV_FP8 ? 2 * D : Cf::R;
  __shared__ __attribute__((aligned(16))) float slots[2][S * SLOTF];
  __shared__ __attribute__((aligned(16))) float pbuf_all[NP][PD][GM * B];
  __shared__ __attribute__((aligned(16))) char qs[2][GM * QLds<Cf>::STRIDE];
  __shared__ int2 ent[2][S];
  __shared__ SegShared sh;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NSTR = p.batch * p.hkv;
  const int g = p.g;
  const uint32_t E = epoch_of(ld_dev32(p.sched_ctrl));

  // streams without visits: out = 0, stop = 0
  for (int st = blockIdx.x; st < NSTR; st += gridDim.x) {
    const int sq = st / p.hkv;
    if (visit_count<B>(p, sq, p.seq_lens[sq]) <= 0) {
      const size_t head0 = (size_t)sq * p.hq + (size_t)(st - sq * p.hkv) * g;
      for (int i = threadIdx.x; i < g * D; i += blockDim.x) p.out[head0 * D + i] = 0.f;
      if ((int)threadIdx.x < g) p.stop_block[head0 + threadIdx.x] = 0;
    }
  }
  if (threadIdx.x < 2) {
    sh.claimed[threadIdx.x] = 0;
    sh.pdone[threadIdx.x] = 0;
    sh.produced[threadIdx.x] = 0;
    sh.ddone[threadIdx.x] = 0;
    sh.freed[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) {
    sh.end = STREAM_BIG;
    sh.err = 0;
  }
  lds_barrier();

  // a bounded LDS wait: false (and every wave told to stop) if it ran out
  auto wait_for = [&](auto cond) __attribute__((always_inline)) -> bool {
    for (int spin = 0;; ++spin) {
      if (cond()) return true;
      if (lds_ld(&sh.err)) return false;
      if (spin > p.spin_limit) {
        if (lane == 0) {
          lds_st(&sh.err, 1);
          lds_st(&sh.end, 0);
          lb_fail(p, E);
        }
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };

  if (w >= Cf::SETS * NS) {
    // ============================ producer waves ============================
    const int pw = w - Cf::SETS * NS;
    float (*pbuf)[GM * B] = pbuf_all[pw];
    const size_t tile = (size_t)B * Cf::R;
    const char* kbase = static_cast<const char*>(p.k_pages);
    const char* vbase = static_cast<const char*>(p.v_pages);
    int cur = (int)(blockIdx.x % (unsigned)NSTR);
    bool ended = false;
    for (int k = 0;; ++k) {
      const int b = k & 1;
      // the buffer's previous item (k - 2) is done
      if (!wait_for([&]() { return lds_ld(&sh.freed[b]) >= k - 1; })) break;
      if (pw == 0) {
        for (int bub = 0;; ++bub) {
          seg_claim<Cf>(p, E, sh.info[b], &sh.claim[b], ent[b], qs[b], cur, ended, lane);
          lds_wait();
          if (sh.info[b][0] != SEG_BUBBLE) break;
          // every stream with segments left is at its window: wait for progress
          if (bub > p.spin_limit) {
            if (lane == 0) {
              lb_fail(p, E);
              sh.info[b][0] = SEG_END;
            }
            lds_wait();
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        if (lane == 0) {
          if (sh.info[b][0] == SEG_END) lds_st(&sh.end, k);
          lds_wait();
          lds_st(&sh.claimed[b], k + 1);
        }
      } else if (!wait_for([&]() { return lds_ld(&sh.claimed[b]) == k + 1; })) {
        break;
      }
      const int s = sh.info[b][0];
      if (s == SEG_END) break;
      const int j = sh.info[b][1], n = sh.info[b][2], L = sh.info[b][3];
      const bool done = sh.info[b][4] != 0;
      const int ns = min(S, n - j * S);
      const int kvh = s % p.hkv;
      if (!done) {
        const int2* en = ent[b];
        const char* qb = qs[b];
        float* sb = slots[b];
        auto claim = [&]() __attribute__((always_inline)) -> int {
          int t = 0;
          if (lane == 0) t = lds_add(&sh.claim[b], 1);
          t = readlane(t, 0);
          return t < ns ? t : -1;
        };
        // the loads of segment position t (t < 0: a stand-in re-read of
        // position 0's tiles, so the loads stay unconditional)
        auto issue = [&](int t, BlockRegs<Cf>& rr, float& ks, float& vs, int& nv) __attribute__((always_inline)) {
          const int2 e = en[max(t, 0)];
          const int ob = __builtin_amdgcn_readfirstlane(e.x);
          const int pg = __builtin_amdgcn_readfirstlane(e.y);
          nv = min(B, L - ob * B);
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
        BlockRegs<Cf> rg[PD];
        float ksr[PD], vsr[PD], mbs[PD], lss[PD];
        int nvr[PD], tr[PD];
#pragma unroll
        for (int u = 0; u < PD; ++u) {
          tr[u] = claim();
          issue(tr[u], rg[u], ksr[u], vsr[u], nvr[u]);
          mbs[u] = 0.f;
          lss[u] = 1.f;
        }
        if (tr[0] >= 0) block_softmax<Cf>(rg[0], qb, g, nvr[0], ksr[0], vsr[0], p.qk_log2, lane, pbuf[0], mbs[0], lss[0]);
        // one step on register slot u (its block had its first half done) and
        // slot un (the next one): the first half of un's block and the second
        // half of u's share one basic block; then slot u takes a new position
        auto step = [&](auto uc, auto unc) __attribute__((always_inline)) -> bool {
          constexpr int u = decltype(uc)::value, un = decltype(unc)::value;
          const int t = tr[u];
          float* sl = sb + (size_t)max(t, 0) * SLOTF;
          if (t >= 0 && tr[un] >= 0) {
            block_softmax<Cf>(rg[un], qb, g, nvr[un], ksr[un], vsr[un], p.qk_log2, lane, pbuf[un], mbs[un], lss[un]);
            block_emit<Cf>(rg[u], pbuf[u], mbs[u], lss[u], lane, sl);
          } else if (t >= 0) {
            block_emit<Cf>(rg[u], pbuf[u], mbs[u], lss[u], lane, sl);
          } else if (tr[un] >= 0) {
            block_softmax<Cf>(rg[un], qb, g, nvr[un], ksr[un], vsr[un], p.qk_log2, lane, pbuf[un], mbs[un], lss[un]);
          }
          tr[u] = claim();
          issue(tr[u], rg[u], ksr[u], vsr[u], nvr[u]);
          bool any = false;
#pragma unroll
          for (int q = 0; q < PD; ++q) any = any || tr[q] >= 0;
          return any;
        };
        for (;;) {
          using std::integral_constant;
          if (!step(integral_constant<int, 0>{}, integral_constant<int, 1 % PD>{})) break;
          if (!step(integral_constant<int, 1 % PD>{}, integral_constant<int, 2 % PD>{})) break;
          if constexpr (PD >= 3)
            if (!step(integral_constant<int, 2 % PD>{}, integral_constant<int, 3 % PD>{})) break;
          if constexpr (PD >= 4)
            if (!step(integral_constant<int, 3 % PD>{}, integral_constant<int, 4 % PD>{})) break;
        }
        // stand-in loads may still be in flight
        wait_all_memory();
      }
      lds_wait();  // this wave's results are in the buffer
      if (lane == 0 && lds_add(&sh.pdone[b], 1) == NP - 1) {
        lds_st(&sh.pdone[b], 0);
        lds_wait();
        lds_st(&sh.produced[b], k + 1);
      }
    }
  } else {
    // ==================== detector waves: set w / NS takes items k = set mod SETS
#ifndef ART_SEG_NOPRIO
    __builtin_amdgcn_s_setprio(2);
#endif
    const int set = w / NS;
    const int dw = w - set * NS;
    for (int k = set;; k += Cf::SETS) {
      const int b = k & 1;
      if (!wait_for([&]() { return lds_ld(&sh.produced[b]) == k + 1 || lds_ld(&sh.end) <= k; })) break;
      if (lds_ld(&sh.produced[b]) != k + 1) break;  // no item k
      const int s = sh.info[b][0], j = sh.info[b][1], n = sh.info[b][2];
      const bool done = sh.info[b][4] != 0;
      const int ns = min(S, n - j * S);
      if (done) {
        // every head stopped in an earlier segment
        if (dw == 0 && lane < g) st_dev(p.lb_st + ((size_t)s * p.max_chunks + j) * g + lane, tag_word(E, SG_DEAD));
      } else {
        if (dw < g) seg_heads<Cf>(p, E, s, j, n, ns, dw, slots[b], ent[b], lane);
      }
      lds_wait();  // this wave's reads of the buffer are complete
      if (lane == 0 && lds_add(&sh.ddone[b], 1) == NS - 1) {
        lds_st(&sh.ddone[b], 0);
        __hip_atomic_fetch_max(p.lb_prog + s, (uint32_t)j + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_wait();
        lds_st(&sh.freed[b], k + 1);
      }
    }
  }

  // count this workgroup out; the last one publishes the fetched counts,
  // clears the per-stream words and advances the epoch
  wait_all_memory();
  lds_barrier();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(p.sched_ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last_wg = prev == gridDim.x - 1 ? 1 : 0;
  }
  lds_barrier();
  if (sh.last_wg) {
    // a call in which a bounded wait gave up: heads whose result was never
    // written get stop -1 and NaN output
    const bool failed = ld_dev32(p.sched_ctrl + 3) == E;
    for (int st = threadIdx.x; st < NSTR; st += blockDim.x) {
      const uint32_t f = ld_dev32(p.lb_fetch + st);
      if (p.blocks_fetched) p.blocks_fetched[st] = (int32_t)f;
      const int sq = st / p.hkv;
      if (failed && visit_count<B>(p, sq, p.seq_lens[sq]) > 0) {
        const uint32_t fin = ld_dev32(p.lb_heads + st);
        const size_t head0 = (size_t)sq * p.hq + (size_t)(st - sq * p.hkv) * g;
        for (int h = 0; h < g; ++h)
          if (!((fin >> h) & 1u)) {
            for (int i = 0; i < D; ++i) p.out[(head0 + h) * D + i] = __builtin_nanf("");
            p.stop_block[head0 + h] = -1;
          }
      }
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

}  // namespace kern
}  // namespace art
