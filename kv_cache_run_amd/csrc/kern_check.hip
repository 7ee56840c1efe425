// Input-contract check for the decode (art_check_inputs): the integer inputs
// the decode takes as given -- sequence lengths within capacity, visited
// order entries distinct logical blocks of the sequence (the ART explainer,
// Technical Summary 2.4: a traversal order over the sequence's blocks), the
// pages they map to inside the cache -- checked on the device, reporting the
// first violation by (sequence, visit position, code).
//
//   * check_init_kernel: the 64-bit report key (held in the result buffer
//     while the check runs) = none.
//   * check_kernel: one workgroup per sequence.  Pass 1 marks every visited
//     in-range entry in an LDS bitmap of the sequence's blocks and, in a
//     second bitmap, those marked twice; pass 2 tests each visited position
//     (entry out of range, entry repeated, page out of range) and takes the
//     lowest failing position of each thread into one atomic minimum over
//     the key (sequence << 32 | position << 2 | code - 1).
//   * check_final_kernel: the key -> (code, sequence, position, value).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "art_internal.h"

namespace art {
namespace {

constexpr int CHECK_THREADS = 256;
constexpr int CHECK_MAX_BLOCKS = 1 << 18;  // two bitmaps of 2^18 bits: 64 KiB of LDS
constexpr unsigned long long CHECK_NONE = ~0ull;

__global__ void check_init_kernel(unsigned long long* key) {
  if (threadIdx.x == 0) *key = CHECK_NONE;
}

__global__ __launch_bounds__(CHECK_THREADS) void check_kernel(const int32_t* table, const int32_t* order,
                                                              const int32_t* lens, const int32_t* visit,
                                                              int max_blocks, int bs, int num_pages,
                                                              unsigned long long* key) {
  extern __shared__ uint32_t bits[];  // [W] entries seen, then [W] entries seen more than once
  const int s = blockIdx.x;
  const int W = (max_blocks + 31) >> 5;
  const int L = lens[s];
  if (L < 0 || (long long)L > (long long)max_blocks * bs) {
    if (threadIdx.x == 0) atomicMin(key, (unsigned long long)s << 32);  // code 1 at position 0
    return;
  }
  const int n = (L + bs - 1) / bs;
  int v = n;
  if (visit) {
    const int x = visit[s];
    v = x < 0 ? 0 : (x > n ? n : x);
  }
  for (int i = threadIdx.x; i < 2 * W; i += CHECK_THREADS) bits[i] = 0u;
  __syncthreads();
  const int32_t* orow = order + (size_t)s * max_blocks;
  const int32_t* trow = table + (size_t)s * max_blocks;
  for (int t = threadIdx.x; t < v; t += CHECK_THREADS) {
    const int b = orow[t];
    if (b >= 0 && b < n) {
      const uint32_t bit = 1u << (b & 31);
      if (atomicOr(&bits[b >> 5], bit) & bit) atomicOr(&bits[W + (b >> 5)], bit);
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < v; t += CHECK_THREADS) {
    const int b = orow[t];
    int code = 0;
    if (b < 0 || b >= n) {
      code = 2;
    } else if (bits[W + (b >> 5)] & (1u << (b & 31))) {
      code = 3;
    } else {
      const int pg = trow[b];
      if (pg < 0 || pg >= num_pages) code = 4;
    }
    if (code != 0) {  // this thread's positions rise: the first failure is its lowest
      atomicMin(key, ((unsigned long long)s << 32) | ((unsigned long long)t << 2) | (unsigned long long)(code - 1));
      break;
    }
  }
}

__global__ void check_final_kernel(const int32_t* table, const int32_t* order, const int32_t* lens, int max_blocks,
                                   int32_t* result) {
  if (threadIdx.x != 0) return;
  const unsigned long long k = *reinterpret_cast<const unsigned long long*>(result);
  int32_t code = 0, s = 0, t = 0, val = 0;
  if (k != CHECK_NONE) {
    s = (int32_t)(k >> 32);
    t = (int32_t)((k >> 2) & 0x3FFFFFFFull);
    code = (int32_t)(k & 3ull) + 1;
    if (code == 1) {
      val = lens[s];
    } else {
      const int b = order[(size_t)s * max_blocks + t];
      val = code == 4 ? table[(size_t)s * max_blocks + b] : b;  // code 4: b was inside [0, n_s)
    }
  }
  result[0] = code;
  result[1] = s;
  result[2] = t;
  result[3] = val;
}

// Zero `bytes` bytes at a 16-byte aligned address: 16-byte stores over a
// grid-stride loop, the remaining bytes one at a time.
__global__ __launch_bounds__(256) void zero_fill_kernel(unsigned char* ptr, size_t bytes) {
  const size_t words = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride)
    reinterpret_cast<uint4*>(ptr)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < bytes - 16 * words) ptr[16 * words + threadIdx.x] = 0;
}

}  // namespace

int check_max_blocks() { return CHECK_MAX_BLOCKS; }

hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const size_t words = (bytes + 15) / 16;
  const size_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, stream,
                     static_cast<unsigned char*>(ptr), bytes);
  return hipGetLastError();
}

hipError_t launch_check(const int32_t* block_table, const int32_t* block_order, const int32_t* seq_lens,
                        const int32_t* visit_lens, int32_t* result, int batch, int max_blocks, int bs, int num_pages,
                        hipStream_t stream) {
  unsigned long long* key = reinterpret_cast<unsigned long long*>(result);
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, key);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (batch > 0) {
    const size_t lds = 2 * (size_t)((max_blocks + 31) >> 5) * sizeof(uint32_t);
    hipLaunchKernelGGL(check_kernel, dim3(batch), dim3(CHECK_THREADS), lds, stream, block_table, block_order,
                       seq_lens, visit_lens, max_blocks, bs, num_pages, key);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(check_final_kernel, dim3(1), dim3(64), 0, stream, block_table, block_order, seq_lens, max_blocks,
                     result);
  return hipGetLastError();
}

}  // namespace art
