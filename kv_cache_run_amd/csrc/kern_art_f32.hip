// Instantiations of the terminating kernels (scanners, look-back, windowed) for KV storage F32 (one translation unit per
// storage type and kernel so that the build runs in parallel).
#include "art_kernels_impl.h"
#include "art_stream.h"
#include "art_seg.h"

namespace art {
namespace {

// Workgroups of the look-back kernel: one per resident slot (occupancy x
// CUs of the current device, computed once per device), unless given.
template <class K>
int resident_slots(K kernel, int threads) {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

template <int D, int B, int GM>
hipError_t go(const Params& p, hipStream_t st) {
  constexpr int threads = 64 * kern::Cfg<KV_F32, D, B, GM>::NWA;
  if (p.seg) {
    if constexpr (GM <= 8) {
      hipLaunchKernelGGL((kern::art_seg_kernel<KV_F32, D, B, GM>), dim3((unsigned)p.seg_wgs),
                         dim3(64 * kern::SegCfg<KV_F32, D, B, GM>::NW3), 0, st, p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (p.stream2) {
    if constexpr (GM <= 8) {
      hipLaunchKernelGGL((kern::art_stream_kernel<KV_F32, D, B, GM>), dim3(p.batch * p.hkv),
                         dim3(64 * kern::StreamCfg<KV_F32, D, B, GM>::NW2), 0, st, p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (p.win == 1) {
    // windowed, partials: one workgroup per (stream, chunk of the window)
    hipLaunchKernelGGL((kern::art_win_part_kernel<KV_F32, D, B, GM>), dim3(p.batch * p.hkv * p.win_n),
                       dim3(64 * kern::Cfg<KV_F32, D, B, GM>::C), 0, st, p);
  } else if (p.win == 2) {
    // windowed, fold: win_k workgroups per (stream, query head)
    hipLaunchKernelGGL((kern::art_win_scan_kernel<KV_F32, D, B, GM, 64>), dim3(p.batch * p.hkv * p.g * p.win_k),
                       dim3(64 * kern::WNW), 0, st, p);
  } else if (p.lb) {
    auto kernel = kern::art_lb_kernel<KV_F32, D, B, GM>;
    long wgs = p.workers > 0 ? p.workers : resident_slots(kernel, threads);
    const long items = (long)p.batch * p.hkv * p.max_chunks;
    if (wgs > items) wgs = items;
    if (wgs < 1) wgs = 1;
    hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(threads), 0, st, p);
  } else {
    hipLaunchKernelGGL((kern::art_sched_kernel<KV_F32, D, B, GM>), dim3(p.batch * p.hkv + p.helpers), dim3(threads), 0, st, p);
  }
  return hipGetLastError();
}

template <int D, int B>
hipError_t by_gm(int gm, const Params& p, hipStream_t st) {
  switch (gm) {
    case 4: return go<D, B, 4>(p, st);
    case 8: return go<D, B, 8>(p, st);
    case 16: return go<D, B, 16>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_art_f32(const Variant& v, const Params& p, hipStream_t st) {
  if (v.d == 64 && v.b == 16) return by_gm<64, 16>(v.gm, p, st);
  if (v.d == 64 && v.b == 32) return by_gm<64, 32>(v.gm, p, st);
  if (v.d == 128 && v.b == 16) return by_gm<128, 16>(v.gm, p, st);
  if (v.d == 128 && v.b == 32) return by_gm<128, 32>(v.gm, p, st);
  return hipErrorInvalidValue;
}

}  // namespace art
