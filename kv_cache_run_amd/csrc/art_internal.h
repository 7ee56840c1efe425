// Internal interface between the C-ABI front end (art_api.cpp) and the
// gfx950 kernels (art_kernels*.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace art {

enum KvType { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

// Blocks per ART chunk: 8, fewer when a chunk's partials [C][GM][D] fp32
// would pass 32 KiB.
constexpr int art_chunk_blocks(int gm, int d) { return 8192 / (gm * d) < 8 ? 8192 / (gm * d) : 8; }
// Floats of one chunk's partials: a[C][GM][D], m[C][GM], l[C][GM].
constexpr int art_slot_floats(int gm, int d) {
  return art_chunk_blocks(gm, d) * gm * d + 2 * art_chunk_blocks(gm, d) * gm;
}

// Windowed path: waves of a workgroup, and at most this many fold
// workgroups per (stream, head).
constexpr int art_win_waves = 16;
constexpr int art_win_split = 4;

// Everything a kernel needs, passed by value as the kernel argument.
struct Params {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* block_order;
  const int32_t* seq_lens;
  const int32_t* visit_lens;  // [batch] visited leading entries of block_order (null: all n_s)
  float* out;
  int32_t* stop_block;
  int32_t* blocks_fetched;  // may be null
  float* ws_part;           // full mode: piece partials [streams + workgroups][GM][D + 2]
  uint32_t* full_cnt;       // full mode: [streams] pieces finished (0 between calls)
  // ART scheduler (workspace): epoch-tagged control words and the ring of
  // partial-result slots helpers hand to scanners
  uint32_t* sched_ctrl;                // [0] stored epoch, [1] finished workgroups, [2] error flag, [3] epoch of a failed call
  unsigned long long* sched_claim;     // [streams]
  unsigned long long* sched_done;      // [streams]
  unsigned long long* sched_ready;     // [streams][ring]
  float* sched_ring;                   // [streams][ring][slot_floats]
  int32_t ring;                        // slots per stream
  int32_t slot_floats;                 // stride of one slot (>= art_slot_floats, multiple of 64)
  int32_t helpers;                     // helper workgroups launched after the scanners
  int32_t lookahead;                   // helper window: chunk c is claimable while c < done + min(ring, lookahead + done)
  int32_t spin_limit;                  // bound of every wait loop
  // look-back scheduler (art_lb_kernel): plain per-stream words (zero at the
  // start of a call, reset by its last workgroup), an epoch-tagged status
  // word and a record per (stream, chunk, head)
  uint32_t* lb_claim;                  // [streams] chunks claimed | CLAIM_FIN
  uint32_t* lb_prog;                   // [streams] resolved frontier (atomic max)
  uint32_t* lb_heads;                  // [streams] bit mask of stopped heads
  uint32_t* lb_fetch;                  // [streams] blocks loaded
  unsigned long long* lb_st;           // [streams][max_chunks][g]
  float* lb_rec;                       // [streams][max_chunks][g][rec_floats]
  int32_t max_chunks;                  // ceil(max_blocks / chunk)
  int32_t rec_floats;                  // 2 * (D + 4)
  int32_t window;                      // chunks claimable past the resolved frontier (1..32)
  int32_t lb;                          // 1: launch art_lb_kernel, 0: scanners (+ helpers)
  int32_t stream2;                     // 1: launch art_stream_kernel (one workgroup per stream)
  int32_t seg;                         // 1: launch art_seg_kernel (segments of a stream on many workgroups)
  int32_t seg_win;                     // segment kernel: segments claimable past a stream's resolved frontier
  int32_t seg_wgs;                     // segment kernel: persistent workgroups
  int32_t seg_ext;                     // segment kernel: idle claims up to (seg_ext + 1) x frontier + 2 seg_win (0: none)
  int32_t la0, la_shift;               // stream kernel: lookahead la0 + (frontier >> la_shift) blocks
  int32_t workers;                     // art_lb_kernel workgroups (0: one per resident slot)
  // windowed path (art_win_kernel): per window, a launch in the partials
  // role, then one in the fold role
  int32_t win;                         // 0: not windowed; 1: partials role; 2: fold role
  int32_t win_c0, win_n, win_idx;      // the window's first chunk, chunk count and index
  int32_t win_k;                       // fold role: workgroups per (stream, head)
  int32_t win_max;                     // chunk slots per stream (largest window)
  int32_t win_slot;                    // floats per slot: partials, then [GM][D + 4] chunk aggregates
  float* win_slots;                    // [streams][win_max][win_slot]
  float* win_state;                    // [streams][g][D + 8]: A, M, L, pass count, block-0 flag, running
  uint32_t* win_dead;                  // [streams] bit mask of stopped heads
  uint32_t* win_dwin;                  // [streams] 1 + index of the window in which the stream stopped (0: running)
  uint32_t* win_pass;                  // [streams][g][win_max] pass bits | block-0 bits << 8, per chunk
  uint32_t* win_cnt;                   // [streams][g] fold workgroups arrived (zero between launches)
  int32_t batch, hq, hkv, g;
  int32_t block_size;
  int32_t max_blocks;
  int32_t splits;           // full mode: workgroups over the flattened blocks
  float eps_mag, eps_dir;
  int32_t patience;
  int32_t probe;            // the detector's statistics use coordinates [0, probe) of O (D: all)
  int32_t skip_stats;       // 1: scanners skip the statistics (thresholds are then 0: no test passes)
  float qk_log2;            // log2(e) / sqrt(D)
};

// Kernel variant key.
struct Variant {
  int kv;   // KvType
  int d;    // 64 | 128
  int b;    // 16 | 32
  int gm;   // 4 | 8 | 16 (register capacity for the query group)
};

inline int group_capacity(int g) { return g <= 4 ? 4 : (g <= 8 ? 8 : 16); }

// Full-attention split plan (depends only on the descriptor).
// Full attention's partials: one slot per (stream, workgroup) piece, at most
// streams + workgroups of them.
inline size_t full_part_floats(long streams, int wgs, int gm, int d) { return (size_t)(streams + wgs) * gm * (d + 2); }

// Workspace layout (bytes from the workspace base, each region 256-B aligned).
struct WorkspacePlan {
  size_t lb_fetch, lb_claim, lb_prog, lb_heads, lb_st;  // look-back scheduler
  size_t win_dead, win_dwin, win_state, win_pass, win_cnt;  // windowed path (its slots are in data)
  size_t claim, done, ready, data, total;               // scanner + helpers; data: ring | records | full partials
  size_t full_cnt;                                      // full mode: per-stream count of finished slices
  int ring, slot_floats, helpers, lookahead, max_chunks, rec_floats, window, win_max, win_slot;
};

// Launchers; return hipSuccess or the launch error.  One translation unit per
// (kernel, KV storage type): kern_<kernel>_<type>.hip.
hipError_t launch_art_f32(const Variant& v, const Params& p, hipStream_t stream);
hipError_t launch_art_bf16(const Variant& v, const Params& p, hipStream_t stream);
hipError_t launch_art_fp8(const Variant& v, const Params& p, hipStream_t stream);
hipError_t launch_full_f32(const Variant& v, const Params& p, hipStream_t stream);
hipError_t launch_full_bf16(const Variant& v, const Params& p, hipStream_t stream);
hipError_t launch_full_fp8(const Variant& v, const Params& p, hipStream_t stream);

// Static scratch of art_decode_noalloc (kern_noalloc.hip): its size, and its
// device address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
// Its layout: the full-mode slice counters [streams] at offset 0 (at most
// noalloc_max_streams()), the split partials from noalloc_part_offset().
constexpr size_t noalloc_part_offset() { return 64 << 10; }
constexpr size_t noalloc_max_streams() { return noalloc_part_offset() / 4; }
hipError_t noalloc_scratch(void** ptr);

// Input-contract check (kern_check.hip).
int check_max_blocks();
hipError_t launch_check(const int32_t* block_table, const int32_t* block_order, const int32_t* seq_lens,
                        const int32_t* visit_lens, int32_t* result, int batch, int max_blocks, int bs, int num_pages,
                        hipStream_t stream);
// Zero a device range with a fill kernel (also valid under stream capture).
hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t stream);

// Importance-first order pre-pass (kern_order.hip).
int order_max_blocks();
hipError_t launch_order_summary(const void* k_pages, const float* k_scale, const int32_t* block_table,
                                const int32_t* seq_lens, float* summary, int batch, int max_blocks, int hkv, int d,
                                int bs, int kv_dtype, hipStream_t st);
hipError_t launch_order(const void* q, const float* summary, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t* block_order, float* scores, int batch, int max_blocks, int hq, int hkv, int d, int bs,
                        int q_dtype, hipStream_t st);

}  // namespace art
