// select.hip -- per-unit eviction choice ("mark" of mark-then-compact).
//
// Policies (KV cache compression guide, sections 2 and 16 "the 4 methods";
// eviction-in-practice blog, "scorers are overrated" and "reference
// implementation"):
//   StreamingLLM  keep pos < n_sink and the n_recent most recent positions;
//   H2O           keep the n_recent most recent, plus the n_heavy others with
//                 the largest accumulated attention score;
//   random        keep pos < prompt_len, plus n_keep others per head drawn
//                 uniformly: every candidate gets a Philox4x32-10 key and the
//                 n_keep smallest keys stay.
// Ties go to the lower original position.  Ranking uses one 64-bit key per
// candidate, (primary << 32) | (0xFFFFFFFF - pos), which is unique inside a
// unit, and an MSB-first 8-bit radix select in LDS: the kept set is exactly
// the n_best largest keys, whatever the slot order.
#include "generic.h"

namespace kvc {

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
    __shared__ SelLds<kSelLdsSlots> S;
    select_unit<kSelLdsSlots>(a, blockIdx.x, S);
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
    const int units = a.c.B * a.c.Hkv;
    hipLaunchKernelGGL(select_kernel, dim3(units), dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvc
