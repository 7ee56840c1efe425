/*
 * art_decode.h -- C ABI of the ART paged decode-attention library (gfx950).
 *
 * One call computes single-token decode attention for a batch of sequences
 * over a paged KV cache, with ART run-time termination: for every
 * (sequence, query head) the KV blocks are folded in a caller-given visit
 * order into an online-softmax accumulator, and the head stops once its
 * normalized partial output is stable -- relative change of its L2 norm
 * below eps_mag AND cosine deviation (1 - cos) below eps_dir -- on
 * `patience` consecutive blocks, with logical block 0 folded first.
 * A kv-head stops fetching KV once every query head of its group stopped.
 *
 * Method: "ART: Attention Run-time Termination for Efficient Large Language
 * Model Decoding" (gist.science explainer), Technical Summary 2.1 (streaming
 * tile-wise accumulation), 2.2 (magnitude and direction statistics, both
 * under their thresholds on the same block), 2.3 (patience), 2.4 (visit
 * order, attention sink, RoPE/mask applied before accumulation).
 *
 * Conventions shared by every entry point:
 *  - All pointers except `desc` and `stream` are DEVICE pointers unless
 *    stated otherwise; the caller owns every buffer.  The library never
 *    allocates or frees memory and never synchronizes the stream.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *    and runs asynchronously.  Argument errors are detected on the host,
 *    before anything is enqueued, and returned synchronously.
 *  - Content errors (a block_order row that is not a permutation of
 *    [0, n_s), a block_table entry outside [0, num_pages), seq_lens[s] >
 *    max_blocks_per_seq * block_size) are undefined behaviour in the decode;
 *    art_check_inputs finds them.
 *  - Two calls that share a workspace must not overlap in time.
 */
#ifndef ART_DECODE_H
#define ART_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ART_OK = 0,
  ART_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or scalar   */
  ART_ERR_UNSUPPORTED = 2, /* valid but outside the supported shape matrix  */
  ART_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  ART_ERR_HIP = 4          /* the HIP runtime refused a launch              */
} art_status;

typedef enum {
  ART_DTYPE_F32 = 0,        /* IEEE binary32                                  */
  ART_DTYPE_BF16 = 1,       /* bfloat16 (upper half of binary32)              */
  ART_DTYPE_FP8_E4M3FN = 2  /* OCP FP8 E4M3 (bias 7, no inf, S.1111.111 NaN)  */
} art_dtype;

enum {
  ART_FLAG_NONE = 0,
  /* Full attention: every block is folded, stop_block = n.  Selected
   * automatically when eps_mag == 0 or eps_dir == 0 (a strict "<" test can
   * then never pass), unless ART_FLAG_KEEP_DETECTOR or ART_FLAG_SKIP_STATS
   * is set. */
  ART_FLAG_FULL = 1u,
  /* Run the terminating kernel (statistics and patience counters) even when
   * the thresholds make a stop impossible; used to measure detector cost. */
  ART_FLAG_KEEP_DETECTOR = 2u,
  /* Measurement only: run the terminating kernel over every block with no
   * test able to pass (both thresholds taken as 0, like KEEP_DETECTOR with
   * zero thresholds) and the scanners not computing the statistics at all.
   * The result is full attention; against ART_FLAG_KEEP_DETECTOR with zero
   * thresholds it isolates what the detector costs (the ART explainer,
   * section 4, reports about 1.3 %). */
  ART_FLAG_SKIP_STATS = 4u
};

/* Probe-vector detector: bits 8..15 of flags hold P / 8, where the two
 * statistics are computed over the leading P coordinates of the output only
 * (O[0 .. P-1] of O_t and O_{t-1}; the explainer's Technical Summary 2.2
 * mentions monitoring a subset of coordinates).  0 = all D coordinates.  P
 * must not exceed D (else ART_ERR_INVALID_ARG).  The output written at the
 * stop is still the whole D-vector. */
#define ART_FLAG_PROBE_SHIFT 8
#define ART_FLAG_PROBE_MASK (0xFFu << ART_FLAG_PROBE_SHIFT)
#define ART_FLAG_PROBE(P) (((uint32_t)(P) / 8u) << ART_FLAG_PROBE_SHIFT)

/* Shapes and storage types of one call (host memory). */
typedef struct {
  int32_t batch;               /* number of sequences, >= 0                    */
  int32_t num_q_heads;         /* Hq                                           */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0, g = Hq / Hkv in [1, 16]  */
  int32_t head_dim;            /* D in {64, 128}                               */
  int32_t block_size;          /* B (tokens per KV page) in {16, 32}           */
  int32_t max_blocks_per_seq;  /* row stride of block_table and block_order   */
  int32_t num_pages;           /* number of physical pages in k_pages/v_pages */
  int32_t q_dtype;             /* art_dtype of q                               */
  int32_t kv_dtype;            /* art_dtype of k_pages / v_pages               */
  uint32_t flags;              /* ART_FLAG_* bits                              */
} art_decode_desc;

/*
 * Bytes of device workspace art_decode needs for `desc` (0 = none).  Depends
 * on the descriptor and on the tuning variable ART_RING (slots per stream of
 * the scanners' helper ring), read once per process (see
 * art_decode_reload_environment).  Returns 0 also for an invalid descriptor.
 */
size_t art_decode_workspace_bytes(const art_decode_desc* desc);

/*
 * Put a workspace into its initial state (all bytes zero) on `stream`.
 * Must be called once on a new workspace before its first art_decode call.
 * The workspace holds the terminating kernel's scheduler state -- words
 * tagged with a per-call epoch that the kernel itself advances, and per-stream
 * counters that the kernel's last workgroup clears, so later calls need no
 * clearing and may be captured in a HIP graph -- and the data handed between
 * workgroups: per-chunk records of the look-back scheduler, the partial
 * results helper workgroups hand to the per-stream scanners, or the
 * full-attention slices before their merge.  Calls that share a workspace
 * must not overlap.  The clearing is a small fill kernel, not a memset, so
 * this call may be captured in a HIP graph as well.
 * Errors: ART_ERR_INVALID_ARG for NULL with bytes > 0 or a pointer that is
 * not 256-byte aligned, ART_ERR_HIP.
 */
art_status art_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Whether a bounded wait gave up in any terminating-kernel call that used
 * this workspace since art_decode_workspace_init: *failed = 1, else 0.  The
 * waits between workgroups (look-back records, helper hand-offs) and between
 * the waves of one workgroup (the stream kernel's ring) are bounded by
 * ART_SPIN_LIMIT polls so that a fault in the hand-off can never hang the
 * device; a call in which one gave up wrote stop_block = -1 or NaN output for
 * the heads it had not finished, and art_decode still returned ART_OK (it
 * returns before the kernels run).  The word is sticky until
 * art_decode_workspace_init.  Reads the workspace back to the host and
 * synchronizes `stream`: for diagnostics, not for the decode loop.
 * Errors: ART_ERR_INVALID_ARG (NULL failed; NULL, misaligned or shorter than
 * 16-byte workspace), ART_ERR_HIP.
 */
art_status art_decode_workspace_status(const void* workspace, size_t workspace_bytes, int32_t* failed, void* stream);

/*
 * ART decode attention, one decode step of one layer.
 *
 * q            [batch][Hq][D] in q_dtype (post-RoPE).  16-byte aligned.
 * k_pages,
 * v_pages      [num_pages][Hkv][B][D] in kv_dtype; the (page, kv-head) tile
 *              [B][D] is contiguous.  Row r of logical block b of sequence s
 *              is token b*B + r.  16-byte aligned.
 * k_scale,
 * v_scale      [num_pages][Hkv] float32 per-tile dequantization scales
 *              (value = scale * decoded byte); required for FP8 KV, must be
 *              NULL otherwise.
 * block_table  [batch][max_blocks_per_seq] int32: logical block -> page.
 * block_order  [batch][max_blocks_per_seq] int32: visit position t ->
 *              logical block; the first n_s = ceil(seq_lens[s] / B) entries
 *              of row s are a permutation of [0, n_s).
 * seq_lens     [batch] int32, 0 <= seq_lens[s] <= max_blocks_per_seq * B.
 * eps_mag      threshold on |‖O_t‖ - ‖O_{t-1}‖| / ‖O_{t-1}‖ (>= 0, not NaN).
 * eps_dir      threshold on max(0, 1 - cos(O_t, O_{t-1})) (>= 0, not NaN).
 * patience     consecutive passing blocks needed to stop (>= 1).
 * out          [batch][Hq][D] float32: the head's normalized attention output
 *              over the blocks it folded (0 for an empty sequence).
 * stop_block   [batch][Hq] int32: number of folded blocks = visit positions
 *              0 .. stop-1 (n_s when the head never stopped, 0 when empty;
 *              -1 or NaN output, either of which marks the head, when a
 *              bounded wait between the kernel's workgroups or waves gave
 *              up: art_decode_workspace_status).
 * blocks_fetched  optional [batch][Hkv] int32 (NULL to skip): KV blocks the
 *              kernels actually read for each (sequence, kv-head), speculative
 *              reads (chunks fetched ahead of the stop) included.
 *
 * The terminating kernel has three schedulers (environment ART_SCHED:
 * "auto", the default, "scan", "lb" or "win"): one scanner workgroup per
 * stream that folds the stream's blocks in order; persistent workgroups that
 * take chunks of any stream and obtain the state entering a chunk from the
 * records of the chunks before it (look-back); or growing windows of chunks
 * (the first 1/8 of the longest stream, doubling, at most 64), two launches
 * per window (partials, then fold).  Each is
 * deterministic; the look-back and windowed schedulers give the same bits,
 * the scanners differ from them only in floating-point rounding order
 * (within the same tolerance of the method).  "auto" takes the windowed
 * scheduler for few, long streams (at most half as many streams as CUs, at
 * least 256 chunks of up to 8 blocks), the look-back scheduler for groups of
 * more than 4 query heads, the scanners otherwise.
 * workspace    device scratch of at least art_decode_workspace_bytes(desc)
 *              bytes, initialized once with art_decode_workspace_init; may be
 *              NULL when that size is 0.  256-byte aligned.
 * stream       hipStream_t to enqueue on.
 *
 * Supported: D in {64, 128}; B in {16, 32}; g = Hq/Hkv in 1..16;
 * (q_dtype, kv_dtype) in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3FN)}.
 * Softmax scale is 1/sqrt(D); tokens at positions >= seq_lens[s] are masked
 * and never read into the result (their rows may hold any bits).
 */
art_status art_decode(const art_decode_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      const int32_t* block_order, const int32_t* seq_lens, float eps_mag, float eps_dir,
                      int32_t patience, float* out, int32_t* stop_block, int32_t* blocks_fetched,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * ART over a pruned cache: art_decode with every sequence visiting only the
 * first visit_lens[s] entries of its block_order row -- a caller-chosen
 * subset of its blocks, e.g. block 0 plus a recent window, or a selected set
 * (the ART explainer, Technical Summary 2.4, layers ART over cache-pruning
 * methods through the traversal order; section 4 evaluates it combined with
 * them).  The detector, the patience rule and the block-0 condition run over
 * the visited blocks only, so a head whose subset lacks block 0 never stops
 * early.
 *
 * visit_lens   [batch] int32 device array, or NULL (= art_decode: n_s each).
 *              Entry s is clamped to [0, n_s]; the first visit_lens[s]
 *              entries of block_order row s must be distinct logical blocks
 *              in [0, n_s) (they need not be a permutation of all of them).
 * stop_block   then counts visited blocks: 0 .. visit_lens[s] (visit_lens[s]
 *              when the head never stopped; 0 for an empty subset, with out 0).
 * Full attention (ART_FLAG_FULL or a zero threshold) attends over the
 * visited blocks.  Every other argument, error and the workspace are as for
 * art_decode, which equals art_decode_visits with visit_lens = NULL.
 */
art_status art_decode_visits(const art_decode_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             const int32_t* block_order, const int32_t* seq_lens, const int32_t* visit_lens,
                             float eps_mag, float eps_dir, int32_t patience, float* out, int32_t* stop_block,
                             int32_t* blocks_fetched, void* workspace, size_t workspace_bytes, void* stream);

/*
 * art_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The library itself allocates nothing either: full
 * attention's per-piece partial results and per-stream piece counters (the
 * only scratch this entry point uses) go to a static 8 MiB device array that
 * every device holds until the process ends; its device address is looked up
 * once per device, with that device current, at the first call there.  ART mode runs the kernels that
 * need no scratch: the stream kernel for groups of up to 8 query heads, the
 * per-stream scanners (without helper workgroups) for larger groups, whatever
 * ART_SCHED says.  Results are those art_decode gives with ART_SCHED=stream
 * (respectively scan with ART_HELPERS=0), bit for bit; full attention gives
 * art_decode's full-attention bits.
 * The static array is shared by every call on a device and keeps the last
 * call's contents: the piece counters start at zero when the library is
 * loaded and every full-attention call leaves them at zero; the partials need
 * no clearing.  Calls that overlap in time on one device race, whatever their
 * streams.
 * Errors: as art_decode; ART_ERR_WORKSPACE in full-attention mode when the
 * streams (batch x Hkv) pass 16384 or 64 KiB of counters plus the partials
 * ((streams + workgroups) x GM x (D + 2) floats, GM = g rounded up to 4, 8
 * or 16, workgroups = ART_FULL_WGS, default 256, 512 for fp8 KV) pass 8 MiB -- use
 * art_decode then; ART_ERR_HIP when the array's address cannot be looked up
 * or a launch fails.
 */
art_status art_decode_noalloc(const art_decode_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                              const float* k_scale, const float* v_scale, const int32_t* block_table,
                              const int32_t* block_order, const int32_t* seq_lens, float eps_mag, float eps_dir,
                              int32_t patience, float* out, int32_t* stop_block, int32_t* blocks_fetched,
                              void* stream);

/*
 * Importance-first traversal (the ART explainer, Technical Summary 2.4,
 * names it beside recency-first as an order ART can take): a pre-pass that
 * writes block_order from a cheap per-block summary of the keys, after which
 * art_decode runs unchanged.
 *
 * art_block_key_summary: summary[page][kv-head][d] (float32, device,
 * [num_pages][Hkv][D]) = the mean of the block's valid key rows (fp8: times
 * the tile's k_scale), for every page that some (s, b < n_s) references;
 * other pages are not written.  A cache would store this when it writes a
 * block.  Arguments as for art_decode.
 *
 * art_importance_order: block_order[s] (device, [batch][max_blocks_per_seq],
 * written for positions < n_s only) = block 0 first, then the other blocks
 * by descending score(s, b) = max over query heads h of
 * q_h . summary[page(s, b)][kv-head(h)] / sqrt(D) (float32 dot products),
 * ties to the higher (newer) block.  Needs max_blocks_per_seq <= 4096 (else
 * ART_ERR_UNSUPPORTED) and a device workspace of
 * art_importance_order_workspace_bytes(desc) bytes (the scores between the
 * pre-pass's two launches; 256-byte aligned; no initialisation needed; calls
 * that share one must not overlap).
 *
 * Both enqueue on `stream` and never synchronize.  Errors: ART_ERR_INVALID_ARG
 * (NULL or misaligned pointers: 16 bytes for q, k_pages and summary, 4 for
 * the rest; fp8 without k_scale), ART_ERR_WORKSPACE, the descriptor's errors,
 * ART_ERR_HIP.
 */
art_status art_block_key_summary(const art_decode_desc* desc, const void* k_pages, const float* k_scale,
                                 const int32_t* block_table, const int32_t* seq_lens, float* summary, void* stream);
size_t art_importance_order_workspace_bytes(const art_decode_desc* desc);
art_status art_importance_order(const art_decode_desc* desc, const void* q, const float* summary,
                                const int32_t* block_table, const int32_t* seq_lens, int32_t* block_order,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Input-contract check: finds, on the device, the content errors the decode
 * takes as absent (its inputs walk a sequence's blocks in a traversal order
 * through a paged cache: the ART explainer, Technical Summary 2.4).  Meant
 * for debugging and for callers that take tables from elsewhere; the decode
 * itself never checks.  For each sequence s in turn:
 *   code 1  seq_lens[s] < 0 or > max_blocks_per_seq * block_size
 *           (position 0, value = seq_lens[s]);
 * and with n_s = ceil(seq_lens[s] / block_size) and v_s = n_s, or
 * visit_lens[s] clamped to [0, n_s] when visit_lens is not NULL (as for
 * art_decode_visits), at each visit position t < v_s, b = block_order[s][t]:
 *   code 2  b outside [0, n_s)                              (value = b),
 *   code 3  b also at another visit position t' < v_s       (value = b),
 *   code 4  block_table[s][b] outside [0, desc->num_pages)  (value = page).
 * result (device int32[4], 8-byte aligned, caller-owned; also used as
 * scratch while the check runs) receives {code, s, t, value} of the first
 * violation in (s, t, code) order, or {0, 0, 0, 0}.  Only cells of
 * block_order and block_table at visited positions and their blocks are
 * read (all within [batch][max_blocks_per_seq]), so any contents are safe.
 * Enqueued on `stream` (three small launches, no synchronization; calls
 * that share `result` must not overlap).  Needs max_blocks_per_seq <= 2^18
 * (else ART_ERR_UNSUPPORTED).  Errors: ART_ERR_INVALID_ARG (NULL or
 * misaligned pointers: 8 bytes for result, 4 for the rest), the
 * descriptor's errors, ART_ERR_HIP.
 */
enum { ART_CHECK_OK = 0, ART_CHECK_SEQ_LEN = 1, ART_CHECK_ORDER_RANGE = 2, ART_CHECK_ORDER_REPEAT = 3,
       ART_CHECK_PAGE_RANGE = 4 };
art_status art_check_inputs(const art_decode_desc* desc, const int32_t* block_table, const int32_t* block_order,
                            const int32_t* seq_lens, const int32_t* visit_lens, int32_t* result, void* stream);

/* Static, human-readable name of a status code (host memory, never NULL). */
const char* art_status_string(art_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t art_decode_version(void);

/* Which kernel art_decode would run for these arguments (host only; the
 * environment knob ART_SCHED and the current device's CU count are taken as
 * art_decode takes them):
 *   ART_KERNEL_FULL      full attention (ART_FLAG_FULL, or a zero threshold
 *                        without ART_FLAG_KEEP_DETECTOR),
 *   ART_KERNEL_SCANNERS  one scanner workgroup per stream, lock-step chunks,
 *   ART_KERNEL_LOOKBACK  the look-back scheduler,
 *   ART_KERNEL_WINDOWED  the windowed scheduler,
 *   ART_KERNEL_STREAM    the stream kernel (one workgroup per stream,
 *                        producer and detector waves sharing an LDS ring),
 *   ART_KERNEL_SEGMENTS  the segment kernel (segments of one stream on many
 *                        workgroups, joined by decoupled look-back),
 * or minus the art_status art_decode would return for rejected arguments. */
enum { ART_KERNEL_FULL = 0, ART_KERNEL_SCANNERS = 1, ART_KERNEL_LOOKBACK = 2, ART_KERNEL_WINDOWED = 3,
       ART_KERNEL_STREAM = 4, ART_KERNEL_SEGMENTS = 5 };
int32_t art_decode_kernel_choice(const art_decode_desc* desc, float eps_mag, float eps_dir, int32_t patience);

/* Re-read the tuning environment variables (ART_SCHED and the scheduler
 * knobs listed with art_decode).  The library reads them once, at the first
 * call that needs them; a process that changes them afterwards calls this
 * for the change to take effect.  Host only; not thread-safe against
 * concurrent art_decode calls. */
void art_decode_reload_environment(void);

#ifdef __cplusplus
}
#endif

#endif /* ART_DECODE_H */
