// Importance-first traversal: a pre-pass that writes block_order from
// per-block key summaries, so that ART visits the blocks most likely to
// carry a head's attention first (the ART explainer, Technical Summary 2.4,
// lists "importance-first" beside "recency-first" as a traversal order).
//
//   * order_summary_kernel: the mean of each block's valid keys per kv-head
//     (what a cache would store at write time): one workgroup per
//     (sequence, logical block), a thread per (kv-head, eight coordinates),
//     16-byte row loads.
//   * order_score_kernel: score(s, b) = max over query heads h of
//     q_h . summary(page(s, b), kv-head of h) / sqrt(D); 16 blocks per
//     workgroup, q staged in LDS transposed, one lane per query head forming
//     its dot products, one max over the lanes per block, into a workspace.
//   * order_rank_kernel: the visit position of each block is the number of
//     the sequence's (score, block) keys that sort before its own -- block 0
//     first, then descending score, ties to the newer block; each workgroup
//     holds all of the sequence's keys in LDS and ranks 256 of them, four
//     threads per candidate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "art_internal.h"

namespace art {
namespace {

constexpr int ORDER_MAX_BLOCKS = 4096;  // keys of one sequence in LDS (32 KiB)

__device__ __forceinline__ float load_elem(const void* base, size_t idx, int dtype) {
  if (dtype == KV_F32) return static_cast<const float*>(base)[idx];
  if (dtype == KV_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(base)[idx] << 16);
  return __builtin_amdgcn_cvt_f32_fp8((int) static_cast<const uint8_t*>(base)[idx], 0);  // OCP E4M3FN
}

// Eight consecutive elements of a row (16-byte aligned for bf16, 8 for fp8,
// two 16-byte loads for f32) as floats.
// Every key is read once: the loads are non-temporal (streamed past the caches).
typedef unsigned int ou32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int ou32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void load8(const void* base, size_t idx, int dtype, float (&v)[8]) {
  if (dtype == KV_F32) {
    const ou32x4* p = reinterpret_cast<const ou32x4*>(static_cast<const float*>(base) + idx);
    const ou32x4 a = __builtin_nontemporal_load(p), c = __builtin_nontemporal_load(p + 1);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z);
    v[3] = __uint_as_float(a.w); v[4] = __uint_as_float(c.x); v[5] = __uint_as_float(c.y);
    v[6] = __uint_as_float(c.z); v[7] = __uint_as_float(c.w);
  } else if (dtype == KV_BF16) {
    const ou32x4 w =
        __builtin_nontemporal_load(reinterpret_cast<const ou32x4*>(static_cast<const uint16_t*>(base) + idx));
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const ou32x2 w =
        __builtin_nontemporal_load(reinterpret_cast<const ou32x2*>(static_cast<const uint8_t*>(base) + idx));
    const uint32_t u[2] = {w.x, w.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // OCP E4M3FN; the byte selector must be a literal
      v[4 * i + 0] = __builtin_amdgcn_cvt_f32_fp8((int)u[i], 0);
      v[4 * i + 1] = __builtin_amdgcn_cvt_f32_fp8((int)u[i], 1);
      v[4 * i + 2] = __builtin_amdgcn_cvt_f32_fp8((int)u[i], 2);
      v[4 * i + 3] = __builtin_amdgcn_cvt_f32_fp8((int)u[i], 3);
    }
  }
}

__global__ __launch_bounds__(256) void order_summary_kernel(const void* k_pages, const float* k_scale,
                                                            const int32_t* block_table, const int32_t* seq_lens,
                                                            float* summary, int max_blocks, int hkv, int d, int bs,
                                                            int kv_dtype) {
  const int s = blockIdx.x / max_blocks;
  const int b = blockIdx.x - s * max_blocks;
  const int L = seq_lens[s];
  const int n = (L + bs - 1) / bs;
  if (b >= n) return;
  const int page = block_table[(size_t)s * max_blocks + b];
  const int rows = min(bs, L - b * bs);
  const float inv = 1.f / (float)rows;
  // a thread sums eight consecutive coordinates of one kv-head over the rows
  const int d8 = d / 8;
  for (int e = threadIdx.x; e < hkv * d8; e += blockDim.x) {
    const int kvh = e / d8, c = (e - kvh * d8) * 8;
    const size_t tile = ((size_t)page * hkv + kvh) * bs * d;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < rows; ++r) {
      float v[8];
      load8(k_pages, tile + (size_t)r * d + c, kv_dtype, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    const float f = inv * (kv_dtype == KV_FP8 ? k_scale[(size_t)page * hkv + kvh] : 1.f);
    float4* dst = reinterpret_cast<float4*>(summary + ((size_t)page * hkv + kvh) * d + c);
    dst[0] = make_float4(acc[0] * f, acc[1] * f, acc[2] * f, acc[3] * f);
    dst[1] = make_float4(acc[4] * f, acc[5] * f, acc[6] * f, acc[7] * f);
  }
}

constexpr int SCORE_BLOCKS = 16;  // blocks per score workgroup (4 per wave)

__global__ __launch_bounds__(256) void order_score_kernel(const void* q, const float* summary,
                                                          const int32_t* block_table, const int32_t* seq_lens,
                                                          float* scores, int max_blocks, int hq, int hkv, int d,
                                                          int bs, int q_dtype) {
  __shared__ float qt[128 * 64];  // q of 64 heads, transposed: [coordinate][head]
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int per = (max_blocks + SCORE_BLOCKS - 1) / SCORE_BLOCKS;
  const int s = blockIdx.x / per;
  const int b0 = (blockIdx.x - s * per) * SCORE_BLOCKS;
  const int L = seq_lens[s];
  const int n = (L + bs - 1) / bs;
  if (b0 >= n) return;
  const int g = hq / hkv;
  const float scale = 1.f / sqrtf((float)d);
  float best[SCORE_BLOCKS / 4];
#pragma unroll
  for (int i = 0; i < SCORE_BLOCKS / 4; ++i) best[i] = -__builtin_inff();
  // lane = query head (64 at a time); each lane forms its own dot products
  for (int hg = 0; hg < hq; hg += 64) {
    __syncthreads();
    for (int e = threadIdx.x; e < d * 64; e += blockDim.x) {
      const int c = e >> 6, hl = e & 63;
      const int h = hg + hl;
      qt[e] = h < hq ? load_elem(q, ((size_t)s * hq + h) * d + c, q_dtype) : 0.f;
    }
    __syncthreads();
    const int h = hg + lane;
    const int kvh = min(h, hq - 1) / g;
#pragma unroll
    for (int i = 0; i < SCORE_BLOCKS / 4; ++i) {
      const int b = b0 + wv + 4 * i;
      if (b >= n) break;
      const int page = block_table[(size_t)s * max_blocks + b];
      const float4* sm = reinterpret_cast<const float4*>(summary + ((size_t)page * hkv + kvh) * d);
      float acc = 0.f;
#pragma unroll 4
      for (int c4 = 0; c4 < d / 4; ++c4) {
        const float4 v = sm[c4];
        const float* qc = qt + 4 * c4 * 64 + lane;
        acc = fmaf(qc[0], v.x, acc);
        acc = fmaf(qc[64], v.y, acc);
        acc = fmaf(qc[128], v.z, acc);
        acc = fmaf(qc[192], v.w, acc);
      }
      if (h < hq) best[i] = fmaxf(best[i], acc * scale);
    }
  }
#pragma unroll
  for (int i = 0; i < SCORE_BLOCKS / 4; ++i) {
    const int b = b0 + wv + 4 * i;
    if (b >= n) break;
    float m = best[i];
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) scores[(size_t)s * max_blocks + b] = m;
  }
}

// Sort key (ascending = visit order): block 0 is 0; any other block
// (~ordered(score), ~b), so a higher score and then a newer block come first.
__device__ __forceinline__ unsigned long long order_key(int b, uint32_t score_bits) {
  if (b == 0) return 0ull;
  const uint32_t ord = (score_bits & 0x80000000u) ? ~score_bits : (score_bits | 0x80000000u);
  return ((unsigned long long)(~ord) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)b);
}

// Rank of every block: the number of the sequence's keys below its own
// (keys are distinct: the block index is part of them), which is its visit
// position.  A workgroup holds all of the sequence's keys in LDS and ranks
// RANK_CANDS of them; each candidate's comparisons are split over
// RANK_SPLIT threads whose counts meet in LDS.
constexpr int RANK_CANDS = 256;
constexpr int RANK_SPLIT = 4;
constexpr int RANK_THREADS = RANK_CANDS * RANK_SPLIT;

__global__ __launch_bounds__(RANK_THREADS) void order_rank_kernel(const float* scores, const int32_t* seq_lens,
                                                                  int32_t* block_order, int max_blocks, int bs) {
  __shared__ unsigned long long keys[ORDER_MAX_BLOCKS];
  __shared__ int rk[RANK_CANDS];
  const int per = (max_blocks + RANK_CANDS - 1) / RANK_CANDS;
  const int s = blockIdx.x / per;
  const int c0 = (blockIdx.x - s * per) * RANK_CANDS;
  const int L = seq_lens[s];
  const int n = (L + bs - 1) / bs;
  if (c0 >= n) return;
  const float* row = scores + (size_t)s * max_blocks;
  for (int i = threadIdx.x; i < n; i += blockDim.x) keys[i] = order_key(i, __float_as_uint(row[i]));
  if (threadIdx.x < RANK_CANDS) rk[threadIdx.x] = 0;
  __syncthreads();
  const int cand = threadIdx.x % RANK_CANDS, part = threadIdx.x / RANK_CANDS;
  const int b = c0 + cand;
  if (b < n) {
    const unsigned long long mine = keys[b];
    const int len = (n + RANK_SPLIT - 1) / RANK_SPLIT;
    const int i0 = part * len, i1 = min(n, i0 + len);
    int cnt = 0;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) cnt += keys[i] < mine ? 1 : 0;
    atomicAdd(&rk[cand], cnt);
  }
  __syncthreads();
  if (threadIdx.x < RANK_CANDS && b < n) block_order[(size_t)s * max_blocks + rk[cand]] = b;
}

}  // namespace

int order_max_blocks() { return ORDER_MAX_BLOCKS; }

hipError_t launch_order_summary(const void* k_pages, const float* k_scale, const int32_t* block_table,
                                const int32_t* seq_lens, float* summary, int batch, int max_blocks, int hkv, int d,
                                int bs, int kv_dtype, hipStream_t st) {
  hipLaunchKernelGGL(order_summary_kernel, dim3((unsigned)(batch * max_blocks)), dim3(256), 0, st, k_pages, k_scale,
                     block_table, seq_lens, summary, max_blocks, hkv, d, bs, kv_dtype);
  return hipGetLastError();
}

hipError_t launch_order(const void* q, const float* summary, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t* block_order, float* scores, int batch, int max_blocks, int hq, int hkv, int d, int bs,
                        int q_dtype, hipStream_t st) {
  const int per = (max_blocks + SCORE_BLOCKS - 1) / SCORE_BLOCKS;
  hipLaunchKernelGGL(order_score_kernel, dim3((unsigned)(batch * per)), dim3(256), 0, st, q, summary, block_table,
                     seq_lens, scores, max_blocks, hq, hkv, d, bs, q_dtype);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rper = (max_blocks + RANK_CANDS - 1) / RANK_CANDS;
  hipLaunchKernelGGL(order_rank_kernel, dim3((unsigned)(batch * rper)), dim3(RANK_THREADS), 0, st, scores, seq_lens,
                     block_order, max_blocks, bs);
  return hipGetLastError();
}

}  // namespace art
