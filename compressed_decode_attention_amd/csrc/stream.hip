// stream.hip -- read-only streaming of a device buffer (measurement helper).
//
// Every 16-byte word is loaded exactly once: a grid-stride loop over the
// buffer in which one wave instruction covers 1 KB of consecutive bytes.  The
// loaded words are folded into one value that is stored only when it equals
// a marker, so the loads cannot be dropped and nothing else is written.
#include "kvc_internal.h"

namespace kvc {

// non-temporal loads: the policy the step kernels read K and V with, and
// the faster one for a read-once stream
constexpr int kStreamThreads = 256;
constexpr int kStreamBlocks = 4096;   // 16 workgroups per compute unit
constexpr uint32_t kStreamMarker = 0x9E3779B9u;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4 *__restrict__ p,
                                                                      size_t n16, uint32_t *sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * kStreamThreads;
    for (size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n16; i += stride) {
        typedef uint32_t v4u __attribute__((ext_vector_type(4)));
        const uint4 v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p + i)));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kStreamMarker) *sink = acc;
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s) {
    const size_t n16 = bytes / 16;
    const size_t need = (n16 + kStreamThreads - 1) / kStreamThreads;
    const int blocks = need < (size_t)kStreamBlocks ? (int)need : kStreamBlocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kStreamThreads), 0, s,
                       static_cast<const uint4 *>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace kvc
