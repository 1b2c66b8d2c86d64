// attn.hip -- decode attention over a per-head KV cache, split over
// workgroups, with the H2O accumulated-attention update folded in.
//
// Per unit (sequence b, kv head h) the G query heads of the group attend the
// n cached slots plus the new token: z = scale * q.k, p = softmax(z),
// o = sum p v (KV cache compression guide, section 16, "prefill, decode, TP":
// a decode step reads all kept history).  With H2O scores requested, every
// slot's score grows by the group-summed probability (same guide, sections 2
// and 16, "the 4 methods"; section 16 "limits" notes that fused attention
// normally hides these probabilities -- here they are computed exactly, with
// the final softmax normaliser).
//
// This file holds the generic VALU path: one workgroup per (unit, split),
// logits kept in a global scratch row per (unit, query head), a combine pass
// when a unit is split across workgroups.
#include "generic.h"

namespace kvc {

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_valu_kernel(AttnArgs a) {
    __shared__ AttnLds<D> L;
    attn_unit_generic<T, D>(a, blockIdx.x / a.nsplit, blockIdx.x % a.nsplit, L);
}

struct CombLds {
    float fac[kMaxSplit][kMaxGroup];   // exp(m_s - M) / L
    float ms[kMaxSplit][kMaxGroup], ls[kMaxSplit][kMaxGroup];   // the splits' m, l
    float Mg[kMaxGroup], Lg[kMaxGroup];
};

// Combine the splits of one unit: rescale partial sums to the global max,
// normalise, update scores and the slot count.
template <int D>
__device__ inline void combine_unit(const AttnArgs &a, int u, CombLds &CB) {
    const CacheDev &c = a.c;
    const int G = c.G, ns = a.nsplit;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x;
    auto &fac = CB.fac;
    float *Mg = CB.Mg, *Lg = CB.Lg;

    const int n = load_count(c, u, false);
    const bool can_store = n < c.cap;
    const int T_len = n + 1;
    const int chunk = split_chunk(T_len, ns);
    const float *pp = a.part + (size_t)u * ns * G * (D + 2);

    // the splits' (m, l), one load per thread, then the global max and sum
    for (int i = tid; i < ns * G; i += kAttnThreads) {
        const int s = i / G, g = i % G;
        CB.ms[s][g] = pp[(s * G + g) * (D + 2) + D];
        CB.ls[s][g] = pp[(s * G + g) * (D + 2) + D + 1];
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, CB.ms[s][tid]);
        float L = 0.f;
        for (int s = 0; s < ns; ++s) {
            const float ms = CB.ms[s][tid];
            L += (ms == -INFINITY) ? 0.f : CB.ls[s][tid] * __expf(ms - M);
        }
        Mg[tid] = M;
        Lg[tid] = L;
        for (int s = 0; s < ns; ++s) {
            const float ms = CB.ms[s][tid];
            fac[s][tid] = (ms == -INFINITY) ? 0.f : __expf(ms - M) / L;
        }
    }
    __syncthreads();
    for (int e = tid; e < G * D; e += kAttnThreads) {
        const int g = e / D, d = e % D;
        float o = 0.f;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) o += pp[(s * G + g) * (D + 2) + d] * fac[s][g];
        a.out[((size_t)b * c.Hq + (size_t)h * G + g) * D + d] = o;
    }
    if (a.scores) {
        const size_t ld = (size_t)c.cap + 1;
        const float *lg = a.logits + (size_t)u * G * ld;
        float *sc = a.scores + (size_t)u * c.cap;
#pragma unroll 2
        for (int j = tid; j < T_len; j += kAttnThreads) {
            const int s = j / chunk;
            float ps = 0.f;
            for (int g = 0; g < G; ++g) ps += lg[g * ld + j] * fac[s][g];
            if (j < n) sc[j] = score_update(sc[j], ps, a.decay);
            else if (can_store) sc[n] = score_update(0.f, ps, a.decay);
        }
    }
    if (tid == 0 && can_store) c.n_slots[u] = n + 1;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_combine_kernel(AttnArgs a) {
    __shared__ CombLds CB;
    combine_unit<D>(a, blockIdx.x, CB);
}

// The rest of a decode step after the split kernels, one workgroup per unit:
// combine (output, scores, the appended slot), then selection, then
// compaction, each phase reading what the previous one wrote.
union FinishLds {
    CombLds comb;
    SelLds<kSelLdsSlots> sel;
    CompLds comp;
};

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void finish_kernel(AttnArgs a, SelectArgs sa,
                                                            CompactArgs ca) {
    __shared__ FinishLds F;
    const int u = blockIdx.x;
    if (a.nsplit > 1) {
        combine_unit<D>(a, u, F.comb);
        __syncthreads();
    }
    const int e = select_unit<kSelLdsSlots>(sa, u, F.sel);
    __syncthreads();
    if (e >= -1) compact_one<T, D>(ca, u, e);
    else compact_unit<T, D>(ca, u, F.comp);
}

template <typename T, int D>
static hipError_t launch_typed(const AttnArgs &a, bool combine, hipStream_t s) {
    const int units = a.c.B * a.c.Hkv;
    hipLaunchKernelGGL((attn_valu_kernel<T, D>), dim3(units * a.nsplit), dim3(kAttnThreads), 0, s,
                       a);
    if (a.nsplit > 1 && combine)
        hipLaunchKernelGGL((attn_combine_kernel<D>), dim3(units), dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

// combine = false leaves the split partials for finish_kernel
static hipError_t launch_attn_impl(const AttnArgs &a, int dtype, bool combine, hipStream_t s) {
    if (a.nsplit > 1 && mfma_tiles_ok(dtype, a.c.D, a.c.bs)) {
        const hipError_t e = launch_split(a, dtype == KVC_FP8_E5M2, a.max_len, s);
        if (e != hipSuccess || !combine) return e;
        hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(a.c.B * a.c.Hkv), dim3(kAttnThreads), 0,
                           s, a);
        return hipGetLastError();
    }
    if (dtype == KVC_BF16) {
        if (a.c.D == 128) return launch_typed<uint16_t, 128>(a, combine, s);
        if (a.c.D == 64) return launch_typed<uint16_t, 64>(a, combine, s);
    } else if (dtype == KVC_FP8_E5M2) {
        if (a.c.D == 128) return launch_typed<e5m2_t, 128>(a, combine, s);
        if (a.c.D == 64) return launch_typed<e5m2_t, 64>(a, combine, s);
    } else {
        if (a.c.D == 128) return launch_typed<float, 128>(a, combine, s);
        if (a.c.D == 64) return launch_typed<float, 64>(a, combine, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnArgs &a, int dtype, hipStream_t s) {
    return launch_attn_impl(a, dtype, true, s);
}

template <typename T, int D>
static void launch_finish_typed(const AttnArgs &a, const SelectArgs &sa, const CompactArgs &ca,
                                hipStream_t s) {
    hipLaunchKernelGGL((finish_kernel<T, D>), dim3(a.c.B * a.c.Hkv), dim3(kAttnThreads), 0, s, a,
                       sa, ca);
}

hipError_t launch_step_split(const AttnArgs &a, const SelectArgs &sa, const CompactArgs &ca,
                             int dtype, hipStream_t s) {
    hipError_t e = launch_attn_impl(a, dtype, false, s);
    if (e != hipSuccess) return e;
    if (dtype == KVC_BF16) {
        if (a.c.D == 128) launch_finish_typed<uint16_t, 128>(a, sa, ca, s);
        else launch_finish_typed<uint16_t, 64>(a, sa, ca, s);
    } else if (dtype == KVC_FP8_E5M2) {
        if (a.c.D == 128) launch_finish_typed<e5m2_t, 128>(a, sa, ca, s);
        else launch_finish_typed<e5m2_t, 64>(a, sa, ca, s);
    } else {
        if (a.c.D == 128) launch_finish_typed<float, 128>(a, sa, ca, s);
        else launch_finish_typed<float, 64>(a, sa, ca, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Unfused H2O score pass over m_rows query rows per sequence: each row's
// group-summed probabilities are added to the scores (no append).  Two
// traversals of K per row: one for the softmax statistics, one to add the
// normalised probabilities.  The thread that owns a slot is the only writer of
// its score, so the accumulation order is fixed.
// ---------------------------------------------------------------------------
template <typename TK, int D>
__global__ __launch_bounds__(kAttnThreads) void accumulate_kernel(AccumArgs a) {
    using TA = typename ActOf<TK>::type;
    const CacheDev &c = a.c;
    const int G = c.G;
    const int u = blockIdx.x, b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    __shared__ float q_s[kMaxGroup * D];
    __shared__ float st_m[kMaxGroup], st_l[kMaxGroup];
    __shared__ float red[kAttnThreads / 64][kMaxGroup];

    const int n = load_count(c, u, tid == 0);
    const TK *K = (const TK *)c.k;
    const int32_t *P = c.pos + (size_t)u * c.cap;
    float *sc = a.scores + (size_t)u * c.cap;

    for (int r = 0; r < a.m_rows; ++r) {
        const TA *qp = (const TA *)a.q_rows +
                      (((size_t)b * a.m_rows + r) * c.Hq + (size_t)h * G) * D;
        const int limit = a.q_pos ? a.q_pos[(size_t)b * a.m_rows + r] : 0x7FFFFFFF;
        __syncthreads();
        for (int e = tid; e < G * D; e += kAttnThreads) q_s[e] = Elem<TA>::get(qp, e);
        __syncthreads();
        float mloc[kMaxGroup], lloc[kMaxGroup];
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) {
            mloc[g] = -INFINITY;
            lloc[g] = 0.f;
        }
        // online max / sum over the thread's keys
        for (int j = tid; j < n; j += kAttnThreads) {
            if (P[j] > limit) continue;
            const TK *row = K + row_of(c, b, h, j) * D;
            float acc[kMaxGroup];
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g) acc[g] = 0.f;
            for (int d = 0; d < D; ++d) {
                const float kv = Elem<TK>::get(row, d);
#pragma unroll
                for (int g = 0; g < kMaxGroup; ++g)
                    if (g < G) acc[g] = fmaf(q_s[g * D + d], kv, acc[g]);
            }
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g)
                if (g < G) {
                    const float z = acc[g] * a.scale;
                    const float mn = fmaxf(mloc[g], z);
                    lloc[g] = lloc[g] * __expf(mloc[g] - mn) + __expf(z - mn);
                    mloc[g] = mn;
                }
        }
        // merge (m, l) over the block
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) {
            const float mw = wave_max(mloc[g]);
            const float lw = wave_sum(mloc[g] == -INFINITY ? 0.f : lloc[g] * __expf(mloc[g] - mw));
            if (lane == 0) {
                red[wv][g] = mw;
            }
            lloc[g] = lw;
            mloc[g] = mw;
        }
        __syncthreads();
        if (tid < G) {
            float M = red[0][tid];
            for (int w = 1; w < kAttnThreads / 64; ++w) M = fmaxf(M, red[w][tid]);
            st_m[tid] = M;
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g)
            if (lane == 0) red[wv][g] = (mloc[g] == -INFINITY || g >= G) ? 0.f : lloc[g] * __expf(mloc[g] - st_m[g]);
        __syncthreads();
        if (tid < G) {
            float L = 0.f;
            for (int w = 0; w < kAttnThreads / 64; ++w) L += red[w][tid];
            st_l[tid] = L;
        }
        __syncthreads();
        // add normalised probabilities
        for (int j = tid; j < n; j += kAttnThreads) {
            if (P[j] > limit) continue;
            const TK *row = K + row_of(c, b, h, j) * D;
            float acc[kMaxGroup];
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g) acc[g] = 0.f;
            for (int d = 0; d < D; ++d) {
                const float kv = Elem<TK>::get(row, d);
#pragma unroll
                for (int g = 0; g < kMaxGroup; ++g)
                    if (g < G) acc[g] = fmaf(q_s[g * D + d], kv, acc[g]);
            }
            float ps = 0.f;
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g)
                if (g < G) ps += __expf(acc[g] * a.scale - st_m[g]) / st_l[g];
            sc[j] += ps;
        }
    }
}

hipError_t launch_accumulate(const AccumArgs &a, int dtype, hipStream_t s) {
    const int units = a.c.B * a.c.Hkv;
    if (a.m_rows <= 0) return hipSuccess;
    if (dtype == KVC_BF16) {
        if (a.c.D == 128)
            hipLaunchKernelGGL((accumulate_kernel<uint16_t, 128>), dim3(units), dim3(kAttnThreads), 0, s, a);
        else
            hipLaunchKernelGGL((accumulate_kernel<uint16_t, 64>), dim3(units), dim3(kAttnThreads), 0, s, a);
    } else if (dtype == KVC_FP8_E5M2) {
        if (a.c.D == 128)
            hipLaunchKernelGGL((accumulate_kernel<e5m2_t, 128>), dim3(units), dim3(kAttnThreads), 0, s, a);
        else
            hipLaunchKernelGGL((accumulate_kernel<e5m2_t, 64>), dim3(units), dim3(kAttnThreads), 0, s, a);
    } else {
        if (a.c.D == 128)
            hipLaunchKernelGGL((accumulate_kernel<float, 128>), dim3(units), dim3(kAttnThreads), 0, s, a);
        else
            hipLaunchKernelGGL((accumulate_kernel<float, 64>), dim3(units), dim3(kAttnThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kvc
