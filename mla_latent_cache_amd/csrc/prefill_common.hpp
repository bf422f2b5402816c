// Definitions shared by the two naive-form prefill kernels (decompression
// GEMM and causal attention), for gfx950.
#pragma once

#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace prefill {

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time.
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Per-request data-error bits (the decode path's codes).
constexpr uint32_t kNegLen = 0x1u, kLenOverTable = 0x2u, kLenBelowTq = 0x4u, kBadBlock = 0x8u;

template <int DR>
struct PGeom {
  static constexpr int KR = 512;       // latent rank
  static constexpr int DN = 256 - DR;  // query-key width without rope
  static constexpr int DV = 256;       // value width
  static constexpr int D = KR + DR;    // cache row width
};

__device__ __forceinline__ uint32_t prefill_flags(int64_t L, int t_q, int max_blocks) {
  if (L < 0) return kNegLen;
  if (L > (int64_t)max_blocks * 16) return kLenOverTable;
  if (L > 0 && L < t_q) return kLenBelowTq;
  return 0u;
}

}  // namespace prefill

// Causal attention of the naive form over the decompressed rows.
hipError_t launch_prefill_attend(const PrefillArgs& a, int d_rope, hipStream_t stream);

}  // namespace mla
