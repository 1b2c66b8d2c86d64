// compact.hip -- "compact" of mark-then-compact (online KV compaction study,
// section 4.2): survivors are copied so that every unit is again a dense run
// of slots 0..n_out-1, with pos[] as the slot -> original position map.
//
// In place ("hole fill"): with n_out kept of n slots, the kept slots at index
// >= n_out move, in ascending order, into the evicted slots below n_out, in
// ascending order.  Sources lie at or above n_out, destinations below it, so
// no row is both read and written and the copies need no ordering.
//
// Ordered gather: the kept entries are written to a second cache in ascending
// position -- the regular [kv_heads, prompt_len + n_keep, head_dim] layout of
// the eviction-in-practice blog's reference hook (per-head gather, ascending
// order kept for paged kernels and prefix caching).
#include "generic.h"

namespace kvc {

template <typename T, int D>
__global__ __launch_bounds__(kCompThreads) void compact_kernel(CompactArgs a) {
    __shared__ CompLds CL;
    compact_unit<T, D, kCompThreads, true>(a, blockIdx.x, CL);
}

template <typename T, int D>
__global__ __launch_bounds__(kCompThreads) void ordered_kernel(CompactArgs a) {
    const CacheDev &c = a.c;
    const CacheDev &d = a.dst;
    const int u = blockIdx.x, b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x;
    __shared__ uint64_t key[kOrderedMax];

    const int n = load_count(c, u, tid == 0);
    int m = a.n_out[u];
    if (m < 0 || m > n || m > kOrderedMax || m > d.cap) {
        if (tid == 0) raise_flag(c, KVC_FLAG_BAD_COUNT);
        m = max(0, min(min(m, n), min(kOrderedMax, d.cap)));
    }
    int len = 1;
    while (len < m) len <<= 1;
    const int32_t *ks = a.keep_slots + (size_t)u * c.cap;
    const int32_t *P = c.pos + (size_t)u * c.cap;
    for (int i = tid; i < len; i += kCompThreads) {
        uint64_t kk = ~0ull;
        if (i < m) {
            int j = ks[i];
            j = (j < 0 || j >= n) ? 0 : j;
            kk = ((uint64_t)(uint32_t)P[j] << 32) | (uint32_t)j;
        }
        key[i] = kk;
    }
    __syncthreads();
    bitonic_sort(key, len);

    const T *K = (const T *)c.k;
    const T *V = (const T *)c.v;
    T *Kd = (T *)d.k;
    T *Vd = (T *)d.v;
    int32_t *Pd = d.pos + (size_t)u * d.cap;
    for (int i = tid; i < m; i += kCompThreads) {
        const int src = (int)(key[i] & 0xFFFFFFFFu);
        copy_row<T, D>(Kd + row_of(d, b, h, i) * D, K + row_of(c, b, h, src) * D);
        copy_row<T, D>(Vd + row_of(d, b, h, i) * D, V + row_of(c, b, h, src) * D);
        Pd[i] = (int32_t)(key[i] >> 32);
    }
    if (tid == 0) d.n_slots[u] = m;
}

template <typename T, int D>
static hipError_t launch_compact_typed(const CompactArgs &a, hipStream_t s) {
    const int units = a.c.B * a.c.Hkv;
    if (a.ordered)
        hipLaunchKernelGGL((ordered_kernel<T, D>), dim3(units), dim3(kCompThreads), 0, s, a);
    else
        hipLaunchKernelGGL((compact_kernel<T, D>), dim3(units), dim3(kCompThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, int dtype, hipStream_t s) {
    if (dtype == KVC_FP8_E5M2) {
        if (a.c.D == 128) return launch_compact_typed<e5m2_t, 128>(a, s);
        if (a.c.D == 64) return launch_compact_typed<e5m2_t, 64>(a, s);
    }
    if (dtype == KVC_BF16) {
        if (a.c.D == 128) return launch_compact_typed<uint16_t, 128>(a, s);
        if (a.c.D == 64) return launch_compact_typed<uint16_t, 64>(a, s);
    } else {
        if (a.c.D == 128) return launch_compact_typed<float, 128>(a, s);
        if (a.c.D == 64) return launch_compact_typed<float, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvc
