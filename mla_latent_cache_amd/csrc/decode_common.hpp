// Pieces shared by the decode kernels: data-error bits, request validity and
// the context-parallel row count.
#pragma once

#include "device_common.hpp"

namespace mla {

// Device data-error bits (the MLA_DATA_* values of the C header).
constexpr uint32_t kNegLen = 0x1u, kLenOverTable = 0x2u, kLenBelowTq = 0x4u, kBadBlock = 0x8u;

// log2 headroom before the online-softmax reference moves.
constexpr float kSlack = 8.f;

// Rows j < x that this rank holds when the rows of a request are dealt to
// `world` ranks in runs of `il` (row j on rank (j / il) % world, the context-
// parallel layout whose settings the vLLM CPU MLA backend page names); x
// itself on a single rank.  A rank keeps its rows in order, so the rows below
// any global position form a prefix of its own rows.
__device__ __forceinline__ int64_t held_rows(int64_t x, int world, int rank, int il) {
  if (world == 1) return x;
  if (x <= 0) return 0;
  const int64_t full = x / il, rem = x - full * il;
  return ((full + world - 1 - rank) / world) * il + (full % world == rank ? rem : 0);
}

// Data errors of a request of global length Lg holding L rows here.
__device__ __forceinline__ uint32_t request_flags(int64_t Lg, int64_t L, int t_q, int max_blocks) {
  if (Lg < 0) return kNegLen;
  if (L > (int64_t)max_blocks * 16) return kLenOverTable;
  if (Lg > 0 && Lg < t_q) return kLenBelowTq;
  return 0u;
}

}  // namespace mla
