// Instantiations of full_split_kernel for KV storage BF16 (one translation unit per
// storage type and kernel so that the build runs in parallel).
#include "art_kernels_impl.h"

namespace art {
namespace {

template <int D, int B, int GM>
hipError_t go(const Params& p, hipStream_t st) {
  hipLaunchKernelGGL((kern::full_split_kernel<KV_BF16, D, B, GM>), dim3(p.splits), dim3(kern::WG), 0, st, p);
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

hipError_t launch_full_bf16(const Variant& v, const Params& p, hipStream_t st) {
  if (v.d == 64 && v.b == 16) return by_gm<64, 16>(v.gm, p, st);
  if (v.d == 64 && v.b == 32) return by_gm<64, 32>(v.gm, p, st);
  if (v.d == 128 && v.b == 16) return by_gm<128, 16>(v.gm, p, st);
  if (v.d == 128 && v.b == 32) return by_gm<128, 32>(v.gm, p, st);
  return hipErrorInvalidValue;
}

}  // namespace art
