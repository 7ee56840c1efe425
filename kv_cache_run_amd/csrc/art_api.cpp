// C-ABI front end: argument validation (host only, before any HIP call),
// kernel selection, workspace plan and launch.
#include "../../include/art_decode.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "art_internal.h"

namespace art {

}  // namespace art

namespace {

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Shape/type checks that need no data.  Returns ART_OK or the error.
art_status check_desc(const art_decode_desc* d) {
  if (!d) return ART_ERR_INVALID_ARG;
  if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->max_blocks_per_seq < 1 ||
      d->num_pages < 1)
    return ART_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return ART_ERR_INVALID_ARG;
  if (d->flags & ~(uint32_t)(ART_FLAG_FULL | ART_FLAG_KEEP_DETECTOR | ART_FLAG_SKIP_STATS | ART_FLAG_PROBE_MASK))
    return ART_ERR_INVALID_ARG;
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g > 16) return ART_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return ART_ERR_UNSUPPORTED;
  if (((d->flags & ART_FLAG_PROBE_MASK) >> ART_FLAG_PROBE_SHIFT) * 8 > (uint32_t)d->head_dim) return ART_ERR_INVALID_ARG;
  if (d->block_size != 16 && d->block_size != 32) return ART_ERR_UNSUPPORTED;
  const bool ok_types = (d->q_dtype == ART_DTYPE_F32 && d->kv_dtype == ART_DTYPE_F32) ||
                        (d->q_dtype == ART_DTYPE_BF16 && d->kv_dtype == ART_DTYPE_BF16) ||
                        (d->q_dtype == ART_DTYPE_BF16 && d->kv_dtype == ART_DTYPE_FP8_E4M3FN);
  if (!ok_types) {
    const bool known = d->q_dtype >= 0 && d->q_dtype <= 2 && d->kv_dtype >= 0 && d->kv_dtype <= 2;
    return known ? ART_ERR_UNSUPPORTED : ART_ERR_INVALID_ARG;
  }
  // 32-bit limits used inside the kernels
  if ((long long)d->batch * d->num_kv_heads * 64 > 0x7fffffffLL) return ART_ERR_UNSUPPORTED;
  if ((long long)d->max_blocks_per_seq * d->block_size > 0x7fffffffLL) return ART_ERR_UNSUPPORTED;
  return ART_OK;
}

// Scheduler tuning knobs, read from the environment once (at the first call
// that needs them, and again whenever art_decode_reload_environment is
// called; defaults when unset).  ART_SCHED selects the terminating kernel:
// "stream" (one workgroup per stream: producer waves and detector waves
// sharing an LDS ring), "seg" (segments of a stream on many workgroups,
// joined by decoupled look-back), "scan" (one scanner workgroup per stream
// that folds chunks in lock step, optional helpers), "lb" (the look-back
// scheduler), "win" (the windowed scheduler) or "auto" (default): for groups
// of up to 8 query heads, segments when the streams are few (at most half
// the CUs) and long (at least 256 chunks), where one workgroup per stream
// would leave most CUs idle for a long walk, and for groups of 5 to 8 heads
// with long streams (at least 32 chunks); the stream kernel otherwise.  For
// larger groups: windows for few, long streams, the look-back scheduler for
// long streams, scanners otherwise.
// Segment kernel: ART_SEG_WIN (default 2) segments claimable past a stream's
// resolved frontier, plus half the frontier; ART_SEG_EXT (default 8): a
// workgroup that finds every stream at its window claims on the
// longest-running stream up to (ART_SEG_EXT + 1) x frontier + 2 ART_SEG_WIN
// segments (0: never; 4096: without bound); ART_SEG_WGS persistent
// workgroups (0: one per CU).
// Stream kernel: ART_LA0 and ART_LA_SHIFT set its lookahead, la0 +
// (frontier >> la_shift) blocks (defaults 32 and 1).  Windowed:
// ART_WIN_SPLIT fold workgroups per (stream, head) (1 .. 4; 0, the default:
// 2 when there are few heads, else 1), ART_WIN_FIRST chunks in the first
// window (0, the default: 1/8 of the longest stream's chunks, 2 .. 64) and
// ART_WIN_GROWTH the factor from one window to the next (default 2, windows
// at most 64 chunks); results depend on none of them.  Look-back: ART_WINDOW
// chunks claimable past a stream's resolved frontier (0: 1/16 of the longest
// stream's chunks, clamped to 8 .. 32), ART_WORKERS workgroups (0: one per
// resident slot); results do not depend on either.  Scanners: ART_RING slots
// per stream, ART_LOOKAHEAD initial helper window, ART_HELPERS helper
// workgroups (default 0; -1: enough to reach ART_TARGET_WGS workgroups in
// total).  ART_SPIN_LIMIT bounds every wait loop.  The workspace size depends
// on ART_RING only.
int env_int(const char* name, int def, int lo, int hi) {
  const char* v = getenv(name);
  int x = v ? atoi(v) : def;
  return x < lo ? lo : (x > hi ? hi : x);
}
struct Knobs {
  int ring, lookahead, helpers, target, lb, window, workers, win_split, win_first, win_growth;
  int la0, la_shift, spin_limit, full_wgs, seg_win, seg_wgs, seg_ext;
};
enum { SCHED_SCAN = 0, SCHED_LB = 1, SCHED_AUTO = 2, SCHED_WIN = 3, SCHED_STREAM = 4, SCHED_SEG = 5 };
Knobs read_knobs() {
  const char* sched = getenv("ART_SCHED");
  int mode = SCHED_SCAN;
  if (!sched || strcmp(sched, "auto") == 0) mode = SCHED_AUTO;
  else if (strcmp(sched, "lb") == 0) mode = SCHED_LB;
  else if (strcmp(sched, "win") == 0) mode = SCHED_WIN;
  else if (strcmp(sched, "stream") == 0) mode = SCHED_STREAM;
  else if (strcmp(sched, "seg") == 0) mode = SCHED_SEG;
  const Knobs k = {env_int("ART_RING", 8, 1, 64),          env_int("ART_LOOKAHEAD", 3, 1, 64),
                   env_int("ART_HELPERS", 0, -1, 1 << 16), env_int("ART_TARGET_WGS", 512, 1, 1 << 16),
                   mode,                                    env_int("ART_WINDOW", 0, 0, 32),
                   env_int("ART_WORKERS", 0, 0, 1 << 20),       env_int("ART_WIN_SPLIT", 0, 0, art::art_win_split),
                   env_int("ART_WIN_FIRST", 0, 0, 64),          env_int("ART_WIN_GROWTH", 2, 2, 8),
                   env_int("ART_LA0", 32, 1, 1 << 20),          env_int("ART_LA_SHIFT", 1, 0, 30),
                   env_int("ART_SPIN_LIMIT", 1 << 20, 1, 1 << 30), env_int("ART_FULL_WGS", 0, 0, 1 << 20),
                   env_int("ART_SEG_WIN", 2, 1, 1 << 20),      env_int("ART_SEG_WGS", 0, 0, 1 << 20),
                   env_int("ART_SEG_EXT", 8, 0, 4096)};
  return k;
}
// The knobs in effect; guarded by a flag so that the environment is read once.
Knobs g_knobs;
bool g_knobs_read = false;
const Knobs& knobs() {
  if (!g_knobs_read) {
    g_knobs = read_knobs();
    g_knobs_read = true;
  }
  return g_knobs;
}
// CUs of a device, queried once per device.
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workgroups of the full-attention kernel: ART_FULL_WGS, else 256 (one per
// CU: measured fastest for bf16 on the Llama-3-8B, ragged and 128k shapes)
// and 512 for fp8 KV (two per CU: its block math needs the second wave per
// SIMD to keep the loads flowing).  Fixed per descriptor, so that the
// workspace size needs no device query.
int full_wgs(const art_decode_desc* d) {
  const int k = knobs().full_wgs;
  return k > 0 ? k : (d->kv_dtype == ART_DTYPE_FP8_E4M3FN ? 512 : 256);
}

art::WorkspacePlan plan_workspace(const art_decode_desc* d) {
  art::WorkspacePlan w;
  memset(&w, 0, sizeof(w));
  if (d->batch == 0) return w;
  const Knobs& k = knobs();
  const int g = d->num_q_heads / d->num_kv_heads;
  const int gm = art::group_capacity(g);
  const size_t streams = (size_t)d->batch * d->num_kv_heads;
  const int chunk = art::art_chunk_blocks(gm, d->head_dim);
  w.ring = k.ring;
  w.lookahead = k.lookahead < k.ring ? k.lookahead : k.ring;
  w.slot_floats = (art::art_slot_floats(gm, d->head_dim) + 63) / 64 * 64;
  const long max_chunks = (d->max_blocks_per_seq + chunk - 1) / chunk;
  long h = k.helpers >= 0 ? k.helpers : (long)k.target - (long)streams;
  const long useful = (long)streams * (max_chunks - 1);  // chunks a helper could ever take
  if (h > useful) h = useful;
  if (h < 0) h = 0;
  w.helpers = (int)h;
  w.max_chunks = (int)max_chunks;
  w.rec_floats = 2 * (d->head_dim + 4);
  // default window: 1/16 of the longest stream's chunks, 8 .. 32
  w.window = k.window > 0 ? k.window : (int)(max_chunks / 16 < 8 ? 8 : (max_chunks / 16 > 32 ? 32 : max_chunks / 16));
  // Control words and counters never share memory with another mode's data:
  // [0] stored epoch, [1] finished workgroups, [2] error flag; look-back
  // counters and epoch-tagged words; scanner words; then one data region
  // (helper ring, look-back records or full-mode partials).
  size_t off = 256;
  w.lb_fetch = off;
  off += round256(streams * 4);
  w.lb_claim = off;
  off += round256(streams * 8);
  w.lb_prog = off;
  off += round256(streams * 8);
  w.lb_heads = off;
  off += round256(streams * 8);
  w.lb_st = off;
  off += round256(streams * (size_t)max_chunks * g * 8);
  w.win_dead = off;
  off += round256(streams * 4);
  w.win_dwin = off;
  off += round256(streams * 4);
  w.win_state = off;
  off += round256(streams * (size_t)g * (d->head_dim + 8) * sizeof(float));
  w.win_cnt = off;
  off += round256(streams * (size_t)g * 4);
  // windowed path: slots for the largest window, at most 64 chunks and about
  // 256 MB over all streams
  {
    w.win_slot = (art::art_slot_floats(gm, d->head_dim) + gm * (d->head_dim + 4) + 63) / 64 * 64;
    const size_t slot_bytes = (size_t)w.win_slot * sizeof(float);
    long wm = (long)((256ull << 20) / (streams * slot_bytes));
    if (wm > 64) wm = 64;
    if (wm < 2) wm = 2;
    w.win_max = (int)wm;
  }
  w.win_pass = off;
  off += round256(streams * (size_t)g * w.win_max * 4);
  w.full_cnt = off;
  off += round256(streams * 4);
  w.claim = off;
  off += round256(streams * 8);
  w.done = off;
  off += round256(streams * 8);
  w.ready = off;
  off += round256(streams * (size_t)w.ring * 8);
  w.data = off;
  const size_t ring_bytes = streams * (size_t)w.ring * w.slot_floats * sizeof(float);
  const size_t rec_bytes = streams * (size_t)max_chunks * g * w.rec_floats * sizeof(float);
  const size_t part = art::full_part_floats((long)streams, full_wgs(d), gm, d->head_dim) * sizeof(float);
  size_t data = ring_bytes > part ? ring_bytes : part;
  if (rec_bytes > data) data = rec_bytes;
  const size_t win_bytes = streams * (size_t)w.win_max * w.win_slot * sizeof(float);
  if (win_bytes > data) data = win_bytes;
  off += round256(data);
  w.total = off;
  return w;
}

// Terminating kernel for a valid call.  The look-back records hold pass
// counts up to 2047 and its claim sweep packs a stream index in 16 bits; the
// windowed path carries the pass count as a float (exact to 2^24).  Either
// falls back to the scanners outside those limits.
enum Sched { SCHED_RUN_SCAN = 0, SCHED_RUN_LB = 1, SCHED_RUN_WIN = 2, SCHED_RUN_STREAM = 3, SCHED_RUN_SEG = 4 };
Sched terminating_kernel(const art_decode_desc* d, const art::WorkspacePlan& wp, int32_t patience) {
  const Knobs& k = knobs();
  const long streams = (long)d->batch * d->num_kv_heads;
  const int g = d->num_q_heads / d->num_kv_heads;
  int want = k.lb == SCHED_LB ? SCHED_RUN_LB
             : k.lb == SCHED_WIN ? SCHED_RUN_WIN
             : k.lb == SCHED_STREAM ? SCHED_RUN_STREAM
             : k.lb == SCHED_SEG ? SCHED_RUN_SEG
                                    : SCHED_RUN_SCAN;
  if (k.lb == SCHED_AUTO) {
    // groups of up to 8 heads: segments for few, long streams (at most half
    // the CUs, at least 256 chunks) and for groups of more than 4 heads with
    // long streams (at least 32 chunks), else the stream kernel; larger
    // groups: windows for few, long streams, look-back for long streams,
    // else scanners
    const bool few_long = 2 * streams <= cu_count() && wp.max_chunks >= 256;
    if (g <= 8 && (few_long || (g > 4 && wp.max_chunks >= 32)))
      want = SCHED_RUN_SEG;
    else if (g <= 8)
      want = SCHED_RUN_STREAM;
    else if (few_long)
      want = SCHED_RUN_WIN;
    else if (wp.max_chunks >= 32)
      want = SCHED_RUN_LB;
  }
  if (want == SCHED_RUN_STREAM && g > 8) want = SCHED_RUN_SCAN;
  if (want == SCHED_RUN_SEG && (g > 8 || patience > (1 << 26) - 1 || streams > 65535)) want = SCHED_RUN_SCAN;
  if (want == SCHED_RUN_LB && (patience > 2047 || streams > 65535)) want = SCHED_RUN_SCAN;
  if (want == SCHED_RUN_WIN && patience > (1 << 24)) want = SCHED_RUN_SCAN;
  return static_cast<Sched>(want);
}

bool full_mode(const art_decode_desc* d, float eps_mag, float eps_dir) {
  return (d->flags & ART_FLAG_FULL) ||
         ((eps_mag == 0.f || eps_dir == 0.f) && !(d->flags & (ART_FLAG_KEEP_DETECTOR | ART_FLAG_SKIP_STATS)));
}

}  // namespace

extern "C" {

size_t art_decode_workspace_bytes(const art_decode_desc* desc) {
  if (check_desc(desc) != ART_OK) return 0;
  return plan_workspace(desc).total;
}

art_status art_decode_workspace_status(const void* workspace, size_t workspace_bytes, int32_t* failed, void* stream) {
  if (!failed) return ART_ERR_INVALID_ARG;
  *failed = 0;
  if (!workspace || workspace_bytes < 16 || !aligned(workspace, 256)) return ART_ERR_INVALID_ARG;
  uint32_t word = 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&word, static_cast<const char*>(workspace) + 8, sizeof(word), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return ART_ERR_HIP;
  *failed = word != 0 ? 1 : 0;
  return ART_OK;
}

art_status art_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return ART_OK;
  if (!workspace || !aligned(workspace, 256)) return ART_ERR_INVALID_ARG;
  if (art::launch_zero_fill(workspace, workspace_bytes, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ART_ERR_HIP;
  return ART_OK;
}

art_status art_decode(const art_decode_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      const int32_t* block_order, const int32_t* seq_lens, float eps_mag, float eps_dir,
                      int32_t patience, float* out, int32_t* stop_block, int32_t* blocks_fetched,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return art_decode_visits(desc, q, k_pages, v_pages, k_scale, v_scale, block_table, block_order, seq_lens, nullptr,
                           eps_mag, eps_dir, patience, out, stop_block, blocks_fetched, workspace, workspace_bytes,
                           stream);
}

}  // extern "C"

namespace {

// One decode call.  noalloc: no caller workspace; full attention's split
// partials go to the static scratch (rejected when they would not fit) and
// ART mode runs the kernels that need no scratch (the stream kernel for
// groups of up to 8 heads, the scanners without helpers otherwise).
art_status decode_impl(const art_decode_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                       const float* k_scale, const float* v_scale, const int32_t* block_table,
                       const int32_t* block_order, const int32_t* seq_lens, const int32_t* visit_lens,
                       float eps_mag, float eps_dir, int32_t patience, float* out, int32_t* stop_block,
                       int32_t* blocks_fetched, void* workspace, size_t workspace_bytes, void* stream,
                       bool noalloc) {
  const art_status ds = check_desc(desc);
  if (ds != ART_OK) return ds;
  if (!(eps_mag >= 0.f) || !(eps_dir >= 0.f) || patience < 1) return ART_ERR_INVALID_ARG;
  const bool fp8 = desc->kv_dtype == ART_DTYPE_FP8_E4M3FN;
  if (!q || !k_pages || !v_pages || !block_table || !block_order || !seq_lens || !out || !stop_block)
    return ART_ERR_INVALID_ARG;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return ART_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(block_order, 4) || !aligned(seq_lens, 4) || !aligned(stop_block, 4) ||
      (blocks_fetched && !aligned(blocks_fetched, 4)) || (k_scale && !aligned(k_scale, 4)) ||
      (v_scale && !aligned(v_scale, 4)) || (visit_lens && !aligned(visit_lens, 4)))
    return ART_ERR_INVALID_ARG;
  const art::WorkspacePlan wp = plan_workspace(desc);
  const bool full = full_mode(desc, eps_mag, eps_dir);
  const int g = desc->num_q_heads / desc->num_kv_heads;
  if (noalloc) {
    // full attention's piece partials and counters are the only scratch this call uses
    workspace = nullptr;
    if (full && desc->batch > 0) {
      const size_t streams = (size_t)desc->batch * desc->num_kv_heads;
      const size_t need = art::noalloc_part_offset() +
                          art::full_part_floats((long)streams, full_wgs(desc), art::group_capacity(g), desc->head_dim) *
                              sizeof(float);
      if (streams > art::noalloc_max_streams() || need > art::noalloc_scratch_bytes()) return ART_ERR_WORKSPACE;
      if (art::noalloc_scratch(&workspace) != hipSuccess) return ART_ERR_HIP;
    }
  } else if (wp.total > 0) {
    if (!workspace || workspace_bytes < wp.total) return ART_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return ART_ERR_INVALID_ARG;
  }
  if (desc->batch == 0) return ART_OK;

  art::Variant v;
  v.kv = desc->kv_dtype == ART_DTYPE_F32 ? art::KV_F32 : (fp8 ? art::KV_FP8 : art::KV_BF16);
  v.d = desc->head_dim;
  v.b = desc->block_size;
  v.gm = art::group_capacity(g);

  art::Params p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.k_pages = k_pages;
  p.v_pages = v_pages;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.block_order = block_order;
  p.visit_lens = visit_lens;
  {
    const int probe8 = (int)((desc->flags & ART_FLAG_PROBE_MASK) >> ART_FLAG_PROBE_SHIFT);
    p.probe = probe8 ? 8 * probe8 : desc->head_dim;
  }
  if (desc->flags & ART_FLAG_SKIP_STATS) {
    // no test may pass in any kernel; the scanners also skip computing them
    eps_mag = 0.f;
    eps_dir = 0.f;
    p.skip_stats = 1;
  }
  p.seq_lens = seq_lens;
  p.out = out;
  p.stop_block = stop_block;
  p.blocks_fetched = blocks_fetched;
  p.batch = desc->batch;
  p.hq = desc->num_q_heads;
  p.hkv = desc->num_kv_heads;
  p.g = g;
  p.block_size = desc->block_size;
  p.max_blocks = desc->max_blocks_per_seq;
  p.eps_mag = eps_mag;
  p.eps_dir = eps_dir;
  p.patience = patience;
  p.qk_log2 = (float)(1.4426950408889634 / sqrt((double)desc->head_dim));

  hipError_t e;
  if (full) {
    p.splits = full_wgs(desc);
    char* ws = static_cast<char*>(workspace);
    p.ws_part = reinterpret_cast<float*>(ws + (noalloc ? art::noalloc_part_offset() : wp.data));
    p.full_cnt = reinterpret_cast<uint32_t*>(ws + (noalloc ? 0 : wp.full_cnt));
    e = v.kv == art::KV_F32 ? art::launch_full_f32(v, p, static_cast<hipStream_t>(stream))
        : v.kv == art::KV_BF16 ? art::launch_full_bf16(v, p, static_cast<hipStream_t>(stream))
                               : art::launch_full_fp8(v, p, static_cast<hipStream_t>(stream));
  } else {
    p.splits = 1;
    // no-alloc calls (no workspace) run kernels that touch none of its regions: null views
    char* ws = static_cast<char*>(workspace);
    auto at = [&](size_t off) { return ws ? ws + off : nullptr; };
    p.sched_ctrl = reinterpret_cast<uint32_t*>(ws);
    p.sched_claim = reinterpret_cast<unsigned long long*>(at(wp.claim));
    p.sched_done = reinterpret_cast<unsigned long long*>(at(wp.done));
    p.sched_ready = reinterpret_cast<unsigned long long*>(at(wp.ready));
    p.sched_ring = reinterpret_cast<float*>(at(wp.data));
    p.ring = wp.ring;
    p.slot_floats = wp.slot_floats;
    p.helpers = wp.helpers;
    p.lookahead = wp.lookahead;
    p.spin_limit = knobs().spin_limit;
    p.lb_fetch = reinterpret_cast<uint32_t*>(at(wp.lb_fetch));
    p.lb_claim = reinterpret_cast<uint32_t*>(at(wp.lb_claim));
    p.lb_prog = reinterpret_cast<uint32_t*>(at(wp.lb_prog));
    p.lb_heads = reinterpret_cast<uint32_t*>(at(wp.lb_heads));
    p.lb_st = reinterpret_cast<unsigned long long*>(at(wp.lb_st));
    p.lb_rec = reinterpret_cast<float*>(at(wp.data));
    p.max_chunks = wp.max_chunks;
    p.rec_floats = wp.rec_floats;
    p.window = wp.window;
    const Sched sched = noalloc ? (g <= 8 ? SCHED_RUN_STREAM : SCHED_RUN_SCAN) : terminating_kernel(desc, wp, patience);
    if (noalloc) p.helpers = 0;
    p.lb = sched == SCHED_RUN_LB ? 1 : 0;
    p.stream2 = sched == SCHED_RUN_STREAM ? 1 : 0;
    p.seg = sched == SCHED_RUN_SEG ? 1 : 0;
    p.seg_win = knobs().seg_win;  // segments past the frontier: seg_win + frontier / 2
    p.seg_wgs = knobs().seg_wgs > 0 ? knobs().seg_wgs : cu_count();
    p.seg_ext = knobs().seg_ext;
    p.la0 = knobs().la0;
    p.la_shift = knobs().la_shift;
    p.workers = knobs().workers;
    auto launch = [&](const art::Params& pp) {
      return v.kv == art::KV_F32 ? art::launch_art_f32(v, pp, static_cast<hipStream_t>(stream))
             : v.kv == art::KV_BF16 ? art::launch_art_bf16(v, pp, static_cast<hipStream_t>(stream))
                                    : art::launch_art_fp8(v, pp, static_cast<hipStream_t>(stream));
    };
    if (sched == SCHED_RUN_WIN) {
      // growing windows of chunks (at most win_max), two launches each: the
      // window's partials, then its fold
      p.lb = 0;
      p.win_max = wp.win_max;
      p.win_slot = wp.win_slot;
      p.win_slots = reinterpret_cast<float*>(at(wp.data));
      p.win_state = reinterpret_cast<float*>(at(wp.win_state));
      p.win_dead = reinterpret_cast<uint32_t*>(at(wp.win_dead));
      p.win_dwin = reinterpret_cast<uint32_t*>(at(wp.win_dwin));
      p.win_pass = reinterpret_cast<uint32_t*>(at(wp.win_pass));
      p.win_cnt = reinterpret_cast<uint32_t*>(at(wp.win_cnt));
      const Knobs& kn = knobs();
      // fold workgroups per (stream, head): ART_WIN_SPLIT, else 2 while the
      // doubled fold grid still fits two workgroups per CU (few heads: the
      // split shortens each window's fold), 1 otherwise (many heads: the
      // chip is full and the split only repeats the prefix work)
      int split = kn.win_split;
      if (split == 0) {
        const long folds = (long)desc->batch * desc->num_q_heads;
        split = 2 * folds <= 2L * cu_count() ? 2 : 1;
      }
      e = hipSuccess;
      // first window: ART_WIN_FIRST, else 1/8 of the longest stream's chunks
      // (2 .. win_max): the windowed path serves long streams, whose fixed
      // cost per window outweighs reading a few chunks past early stops
      int first = kn.win_first > 0 ? kn.win_first : wp.max_chunks / 8;
      first = first < 2 ? 2 : (first > wp.win_max ? wp.win_max : first);
      for (int c0 = 0, size = first, idx = 0; c0 < wp.max_chunks && e == hipSuccess; ++idx) {
        const int nw = size < wp.max_chunks - c0 ? size : wp.max_chunks - c0;
        p.win_c0 = c0;
        p.win_n = nw;
        p.win_idx = idx;
        const int k = (nw + art::art_win_waves - 1) / art::art_win_waves;
        p.win_k = k < split ? k : split;
        p.win = 1;
        e = launch(p);
        if (e != hipSuccess) break;
        p.win = 2;
        e = launch(p);
        c0 += nw;
        size = kn.win_growth * size < wp.win_max ? kn.win_growth * size : wp.win_max;
      }
    } else {
      e = launch(p);
    }
  }
  return e == hipSuccess ? ART_OK : ART_ERR_HIP;
}

}  // namespace

extern "C" {

art_status art_decode_visits(const art_decode_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             const int32_t* block_order, const int32_t* seq_lens, const int32_t* visit_lens,
                             float eps_mag, float eps_dir, int32_t patience, float* out, int32_t* stop_block,
                             int32_t* blocks_fetched, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(desc, q, k_pages, v_pages, k_scale, v_scale, block_table, block_order, seq_lens, visit_lens,
                     eps_mag, eps_dir, patience, out, stop_block, blocks_fetched, workspace, workspace_bytes, stream,
                     false);
}

art_status art_decode_noalloc(const art_decode_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                              const float* k_scale, const float* v_scale, const int32_t* block_table,
                              const int32_t* block_order, const int32_t* seq_lens, float eps_mag, float eps_dir,
                              int32_t patience, float* out, int32_t* stop_block, int32_t* blocks_fetched,
                              void* stream) {
  return decode_impl(desc, q, k_pages, v_pages, k_scale, v_scale, block_table, block_order, seq_lens, nullptr,
                     eps_mag, eps_dir, patience, out, stop_block, blocks_fetched, nullptr, 0, stream, true);
}

art_status art_block_key_summary(const art_decode_desc* desc, const void* k_pages, const float* k_scale,
                                 const int32_t* block_table, const int32_t* seq_lens, float* summary, void* stream) {
  const art_status ds = check_desc(desc);
  if (ds != ART_OK) return ds;
  const bool fp8 = desc->kv_dtype == ART_DTYPE_FP8_E4M3FN;
  if (!k_pages || !block_table || !seq_lens || !summary || fp8 != (k_scale != nullptr)) return ART_ERR_INVALID_ARG;
  if (!aligned(k_pages, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(summary, 16) ||
      (k_scale && !aligned(k_scale, 4)))
    return ART_ERR_INVALID_ARG;
  if (desc->batch == 0) return ART_OK;
  const int kv = desc->kv_dtype == ART_DTYPE_F32 ? art::KV_F32 : (fp8 ? art::KV_FP8 : art::KV_BF16);
  const hipError_t e = art::launch_order_summary(k_pages, k_scale, block_table, seq_lens, summary, desc->batch,
                                                 desc->max_blocks_per_seq, desc->num_kv_heads, desc->head_dim,
                                                 desc->block_size, kv, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ART_OK : ART_ERR_HIP;
}

size_t art_importance_order_workspace_bytes(const art_decode_desc* desc) {
  if (check_desc(desc) != ART_OK || desc->batch == 0) return 0;
  return round256((size_t)desc->batch * desc->max_blocks_per_seq * sizeof(float));
}

art_status art_importance_order(const art_decode_desc* desc, const void* q, const float* summary,
                                const int32_t* block_table, const int32_t* seq_lens, int32_t* block_order,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const art_status ds = check_desc(desc);
  if (ds != ART_OK) return ds;
  if (!q || !summary || !block_table || !seq_lens || !block_order) return ART_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(summary, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      !aligned(block_order, 4))
    return ART_ERR_INVALID_ARG;
  if (desc->max_blocks_per_seq > art::order_max_blocks()) return ART_ERR_UNSUPPORTED;
  const size_t need = art_importance_order_workspace_bytes(desc);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return ART_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return ART_ERR_INVALID_ARG;
  }
  if (desc->batch == 0) return ART_OK;
  const int qd = desc->q_dtype == ART_DTYPE_F32 ? art::KV_F32 : art::KV_BF16;
  const hipError_t e = art::launch_order(q, summary, block_table, seq_lens, block_order, static_cast<float*>(workspace),
                                         desc->batch, desc->max_blocks_per_seq, desc->num_q_heads, desc->num_kv_heads,
                                         desc->head_dim, desc->block_size, qd, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ART_OK : ART_ERR_HIP;
}

art_status art_check_inputs(const art_decode_desc* desc, const int32_t* block_table, const int32_t* block_order,
                            const int32_t* seq_lens, const int32_t* visit_lens, int32_t* result, void* stream) {
  const art_status ds = check_desc(desc);
  if (ds != ART_OK) return ds;
  if (!block_table || !block_order || !seq_lens || !result) return ART_ERR_INVALID_ARG;
  if (!aligned(block_table, 4) || !aligned(block_order, 4) || !aligned(seq_lens, 4) || !aligned(result, 8) ||
      (visit_lens && !aligned(visit_lens, 4)))
    return ART_ERR_INVALID_ARG;
  if (desc->max_blocks_per_seq > art::check_max_blocks()) return ART_ERR_UNSUPPORTED;
  const hipError_t e =
      art::launch_check(block_table, block_order, seq_lens, visit_lens, result, desc->batch, desc->max_blocks_per_seq,
                        desc->block_size, desc->num_pages, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ART_OK : ART_ERR_HIP;
}

const char* art_status_string(art_status s) {
  switch (s) {
    case ART_OK: return "ART_OK";
    case ART_ERR_INVALID_ARG: return "ART_ERR_INVALID_ARG: invalid argument";
    case ART_ERR_UNSUPPORTED: return "ART_ERR_UNSUPPORTED: shape or type outside the supported matrix";
    case ART_ERR_WORKSPACE: return "ART_ERR_WORKSPACE: workspace missing or too small";
    case ART_ERR_HIP: return "ART_ERR_HIP: HIP runtime error";
  }
  return "ART: unknown status";
}

int32_t art_decode_version(void) { return 300; }

void art_decode_reload_environment(void) {
  g_knobs = read_knobs();
  g_knobs_read = true;
}

int32_t art_decode_kernel_choice(const art_decode_desc* desc, float eps_mag, float eps_dir, int32_t patience) {
  const art_status ds = check_desc(desc);
  if (ds != ART_OK) return -(int32_t)ds;
  if (!(eps_mag >= 0.f) || !(eps_dir >= 0.f) || patience < 1) return -(int32_t)ART_ERR_INVALID_ARG;
  if (full_mode(desc, eps_mag, eps_dir)) return ART_KERNEL_FULL;
  switch (terminating_kernel(desc, plan_workspace(desc), patience)) {
    case SCHED_RUN_LB: return ART_KERNEL_LOOKBACK;
    case SCHED_RUN_WIN: return ART_KERNEL_WINDOWED;
    case SCHED_RUN_STREAM: return ART_KERNEL_STREAM;
    case SCHED_RUN_SEG: return ART_KERNEL_SEGMENTS;
    default: return ART_KERNEL_SCANNERS;
  }
}

}  // extern "C"
