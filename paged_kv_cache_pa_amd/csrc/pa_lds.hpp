// LDS shared by the two kinds of work item of the fused attention kernel.
//
// A work-group runs its prefill items and its decode items in two phases
// that never overlap: the prefill phase starts and ends with work-group
// barriers (its item fetches), so once any wave is in its decode phase
// every wave is done with prefill tiles, and no wave starts a prefill tile
// before every wave has finished decoding.  Prefill keeps its K/V tile ring
// in an array of its own; decode waves turn K chunks into the matrix-core
// layout in per-wave slices of the staging buffer here, whose first word
// also holds the prefill phase's item slot (written by thread 0 only after
// its own wave has left the decode phase).
#pragma once

#include <hip/hip_runtime.h>

namespace pa {

// Bytes of the decode staging buffer: 8 waves x 16 key rows of D elements
// of `es` bytes.
template <int D, int es>
constexpr int decode_stage_bytes() { return 8 * 16 * D * es; }

// The staging buffer of one kernel instantiation (template arguments of the
// kernel plus the cache element size): used by that kernel alone, so its
// LDS address is a compile-time constant.
template <typename T, int D, bool CAP, bool WIN, int es>
__device__ __forceinline__ unsigned char* decode_stage() {
  __shared__ __attribute__((aligned(1024))) unsigned char buf[decode_stage_bytes<D, es>()];
  return buf;
}

}  // namespace pa
