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

// Partials staged per pass of the output combine: 48 float per thread where
// the kernel's LDS holds a larger union anyway (the finish pass), 16 in the
// attention-only combine kernel (which then keeps four workgroups per CU).
constexpr int kCombStage = 48 * kAttnThreads;
constexpr int kCombStageSmall = 16 * kAttnThreads;

template <int STAGE>
struct CombLdsT {
    float fac[kMaxSplit][kMaxGroup];   // exp(m_s - M), then exp(m_s - M) / L
    float ms[kMaxSplit][kMaxGroup], ls[kMaxSplit][kMaxGroup];   // the splits' m, l
    float Mg[kMaxGroup], Lg[kMaxGroup];
    float stage[STAGE + kMaxGroup * 128];   // raw partials of a block of splits (+ pad)
};
using CombLds = CombLdsT<kCombStage>;

// The splits' (m, l) of one unit into LDS (the caller syncs).
template <int D, int NT = kAttnThreads, typename CL>
__device__ inline void combine_load_ml(const float *pp, int ns, int G, CL &CB) {
    for (int i = threadIdx.x; i < ns * G; i += NT) {
        const int s = i / G, g = i % G;
        CB.ms[s][g] = pp[(s * G + g) * (D + 2) + D];
        CB.ls[s][g] = pp[(s * G + g) * (D + 2) + D + 1];
    }
}

// Global max M and normaliser L per head, then the factor of each split,
// exp(m_s - M) / L (0 for an empty split); L sums the splits in order.
template <int NT = kAttnThreads, typename CL>
__device__ inline void combine_factors(int ns, int G, CL &CB) {
    const int tid = threadIdx.x;
    if (tid < G) {
        float M = -INFINITY;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) M = fmaxf(M, CB.ms[s][tid]);
        CB.Mg[tid] = M;
    }
    __syncthreads();
    for (int i = tid; i < ns * G; i += NT) {
        const int s = i / G, g = i % G;
        const float ms = CB.ms[s][g];
        CB.fac[s][g] = (ms == -INFINITY) ? 0.f : __expf(ms - CB.Mg[g]);
    }
    __syncthreads();
    if (tid < G) {
        float L = 0.f;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) L += CB.ls[s][tid] * CB.fac[s][tid];
        CB.Lg[tid] = L;
    }
    __syncthreads();
    for (int i = tid; i < ns * G; i += NT) {
        const int s = i / G, g = i % G;
        CB.fac[s][g] = CB.fac[s][g] / CB.Lg[g];
    }
    __syncthreads();
}

// o[g][d] = sum over splits, in split order, of part[s][g][d] * fac[s][g],
// written to out_row[g * D + d].  Each pass stages the raw partials of as
// many splits as fit in LDS; the loads are branch-free (a buffer resource over
// the unit's partials returns zeros past its end), so all of a thread's loads
// of a pass are in flight at once.  Lanes past the live elements compute on
// padding and store nothing.
template <int D, int STAGE, int NT = kAttnThreads>
__device__ inline void combine_output(const float *pp, int ns, int G, CombLdsT<STAGE> &CB,
                                      float *out_row) {
    const int tid = threadIdx.x;
    const int GD = G * D, GD2 = GD / 2;
    const int sb_max = STAGE / GD;
    const uint32_t bytes = (uint32_t)(ns * G * (D + 2)) * 4u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(pp, bytes);
    constexpr int kE = (kMaxGroup * D + NT - 1) / NT;
    constexpr int kL = STAGE / 2 / NT;   // float2 loads per thread and pass
    float o[kE];
#pragma unroll
    for (int k = 0; k < kE; ++k) o[k] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += sb_max) {
        const int sb = min(sb_max, ns - s0);
        const int n2 = sb * GD2;
        u32x2_t r[kL];
#pragma unroll
        for (int k = 0; k < kL; ++k) {
            const int i = tid + k * NT;   // float2 index within the block
            const int s = s0 + i / GD2, e2 = 2 * (i % GD2);
            const uint32_t off = (i < n2) ? (uint32_t)((s * G + e2 / D) * (D + 2) + e2 % D) * 4u : bytes;
            r[k] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
        }
#pragma unroll
        for (int k = 0; k < kL; ++k)
            reinterpret_cast<u32x2_t *>(CB.stage)[tid + k * NT] = r[k];
        __syncthreads();
        for (int s = 0; s < sb; ++s) {
            const float *st = CB.stage + s * GD;
#pragma unroll
            for (int k = 0; k < kE; ++k) {
                const int el = tid + k * NT;
                o[k] += st[el] * CB.fac[s0 + s][el / D];
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < kE; ++k) {
        const int el = tid + k * NT;
        if (el < GD) out_row[el] = o[k];
    }
}

// Combine the splits of one unit: rescale partial sums to the global max,
// normalise, update scores and the slot count.
template <int D, int STAGE, int NT = kAttnThreads>
__device__ inline void combine_unit(const AttnArgs &a, int u, CombLdsT<STAGE> &CB) {
    const CacheDev &c = a.c;
    const int G = c.G, ns = a.nsplit;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x;
    auto &fac = CB.fac;

    const int n = load_count(c, u, false);
    const bool can_store = n < c.cap;
    const int T_len = n + 1;
    const int chunk = split_chunk(T_len, ns, a.max_len);
    const int nse = split_count(T_len, ns, a.max_len);   // the splits that hold entries
    const float *pp = a.part + (size_t)u * ns * G * (D + 2);

    combine_load_ml<D, NT>(pp, nse, G, CB);
    __syncthreads();
    combine_factors<NT>(nse, G, CB);
    combine_output<D, STAGE, NT>(pp, nse, G, CB, a.out + ((size_t)b * c.Hq + (size_t)h * G) * D);
    if (a.scores) {
        // p summed over the group for every attended slot (heads in order),
        // kJ slots per thread at a time; every logit load of a batch goes out
        // before the sums (a buffer resource over the unit's logits returns
        // zeros for heads past G, which the sums skip)
        const size_t ld = (size_t)c.cap + 1;
        const float *lg = a.logits + (size_t)u * G * ld;
        const uint32_t lbytes = (uint32_t)((size_t)G * ld * 4);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(lg, lbytes);
        float *sc = a.scores + (size_t)u * c.cap;
        constexpr int kJ = (STAGE == kCombStage) ? 4 : 2;
        for (int j0 = tid; j0 < T_len; j0 += kJ * NT) {
            int jj[kJ], sj[kJ];
            float ps[kJ], old[kJ], lv[kMaxGroup][kJ];
#pragma unroll
            for (int q = 0; q < kJ; ++q) {
                const int j = j0 + q * NT;
                jj[q] = j < T_len ? j : T_len - 1;
                sj[q] = jj[q] / chunk;
                ps[q] = 0.f;
                old[q] = jj[q] < n ? sc[jj[q]] : 0.f;
            }
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g)
#pragma unroll
                for (int q = 0; q < kJ; ++q) {
                    const uint32_t off = g < G ? (uint32_t)((g * ld + jj[q]) * 4) : lbytes;
                    lv[g][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
                }
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g)
                if (g < G)
#pragma unroll
                    for (int q = 0; q < kJ; ++q) ps[q] += lv[g][q] * fac[sj[q]][g];
#pragma unroll
            for (int q = 0; q < kJ; ++q) {
                const int j = j0 + q * NT;
                if (j < n) sc[j] = score_update(old[q], ps[q], a.decay);
                else if (j == n && can_store) sc[n] = score_update(0.f, ps[q], a.decay);
            }
        }
    }
    if (tid == 0 && can_store) c.n_slots[u] = n + 1;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_combine_kernel(AttnArgs a) {
    __shared__ CombLdsT<kCombStageSmall> CB;
    combine_unit<D>(a, blockIdx.x, CB);
}

// The rest of a decode step after the split kernels, one workgroup per unit:
// combine (output, scores, the appended slot), then selection, then
// compaction, each phase reading what the previous one wrote.  Two LDS
// sizes: units of up to kSelLdsSmall attended slots (over-budget first steps
// of prompts of a few thousand tokens) keep four workgroups per CU; longer
// ones keep up to kSelLdsSlots selection keys in LDS, two per CU.
constexpr int kSelLdsSmall = 3072;
template <int SEL, int STAGE>
union FinishLdsT {
    CombLdsT<STAGE> comb;
    SelLds<SEL> sel;
    CompLds comp;
};

// Random eviction after split kernels that ranked their own chunks: the
// unit's candidate count and worst candidate from the splits' records
// (wave 0).  Returns the slot that leaves, -1 when none does, or -2 when
// more than one does (the full selection runs then).
__device__ inline int presel_finish(const AttnArgs &a, const SelectArgs &sa, int u, int nse) {
    const int lane = threadIdx.x & 63;
    const int nrec = nse * kPreselWaves;   // the records of the splits that hold entries
    const PreselRecord *R = reinterpret_cast<const PreselRecord *>(a.presel) +
                            (size_t)u * a.nsplit * kPreselWaves;
    uint32_t cnt = 0;
    uint64_t best = ~0ull;
    int arg = -1;
    for (int i = lane; i < nrec; i += 64) {
        const PreselRecord r = R[i];
        cnt += r.ncand;
        const uint64_t key = ((uint64_t)r.key_hi << 32) | r.key_lo;
        if (r.slot >= 0 && (arg < 0 || key < best || (key == best && r.slot < arg))) {
            best = key;
            arg = r.slot;
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        cnt += __shfl_xor(cnt, o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
        const uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
        const int oa = __shfl_xor(arg, o, 64);
        const uint64_t ok = ((uint64_t)hi << 32) | lo;
        if (ok < best || (ok == best && (unsigned)oa < (unsigned)arg)) {
            best = ok;
            arg = oa;
        }
    }
    // the selection's rule: keep n_keep candidates (none when n_keep <= 0)
    const int ncand = (int)cnt, want = sa.n_keep;
    const int extra = (ncand > want) ? (want <= 0 ? ncand : ncand - want) : 0;
    return extra == 0 ? -1 : (extra == 1 ? arg : -2);
}

// The rest of a random-eviction step whose split kernels ranked their own
// chunks, when at most one slot leaves: the same results as combine_unit,
// then the selection's one-eviction case, then compact_one, with fewer
// dependent memory round trips (the first loads go out together, and the
// moved row is copied while the output is combined).  Returns false, having
// written nothing, when more than one slot leaves.
template <typename T, int D, int NT, int STAGE>
__device__ inline bool finish_presel(const AttnArgs &a, const SelectArgs &sa, int u, CombLdsT<STAGE> &CB,
                                     int &sh_e) {
    const CacheDev &c = a.c;
    const int G = c.G, ns = a.nsplit;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x;
    const float *pp = a.part + (size_t)u * ns * G * (D + 2);

    int n = c.n_slots[u];
    n = (n < 0) ? 0 : (n > c.cap ? c.cap : n);
    const int nse = split_count(n + 1, ns, a.max_len);   // the splits that hold entries
    combine_load_ml<D, NT>(pp, nse, G, CB);
    if (tid < 64) {
        const int e = presel_finish(a, sa, u, nse);
        if (tid == 0) sh_e = e;
    }
    __syncthreads();
    const int e = sh_e;
    if (e == -2) return false;

    // the slot count after the append (the selection ran over these slots);
    // one eviction e fills its hole from the last slot, whose row is read
    // now and written after the output pass
    const int cnt = (n < c.cap) ? n + 1 : n;
    const int src = cnt - 1;
    const bool move = e >= 0 && e < src;
    constexpr int kParts = (int)(D * sizeof(T) / 16);
    T *X = (tid < kParts) ? (T *)c.k : (T *)c.v;
    uint4 row;
    int32_t psrc = 0;
    int32_t *P = c.pos + (size_t)u * c.cap;
    if (move && tid < 2 * kParts)
        row = reinterpret_cast<const uint4 *>(X + row_of(c, b, h, src) * D)[tid % kParts];
    if (move && tid == 0) psrc = P[src];

    combine_factors<NT>(nse, G, CB);
    combine_output<D, STAGE, NT>(pp, nse, G, CB, a.out + ((size_t)b * c.Hq + (size_t)h * G) * D);
    if (move && tid < 2 * kParts)
        reinterpret_cast<uint4 *>(X + row_of(c, b, h, e) * D)[tid % kParts] = row;
    if (move && tid == 0) P[e] = psrc;
    if (tid == 0) c.n_slots[u] = (e >= 0 && e < cnt) ? cnt - 1 : cnt;
    return true;
}

// Three instances: SMALL (up to kSelLdsSmall attended slots, 256 threads,
// four workgroups per CU), MID (up to kSelLdsSlots, 256 threads, two per CU)
// and LONG (longer units: 512 threads, still two per CU, so that the score
// update and the selection passes over tens of thousands of slots, one unit's
// critical path, have twice the threads and loads in flight; 1,024 threads
// would leave one workgroup per CU for the batch's many shorter units).
enum FinishSize { kFinishSmall, kFinishMid, kFinishLong };
template <int SZ>
struct FinishCfg {
    static constexpr int SEL = SZ == kFinishSmall ? kSelLdsSmall : kSelLdsSlots;
    static constexpr int STAGE = SZ == kFinishSmall ? kCombStageSmall : kCombStage;
    static constexpr int NT = SZ == kFinishLong ? 512 : kAttnThreads;
    static constexpr int WPE = SZ == kFinishMid ? 1 : 4;
};

// The order in which the long-unit finish pass takes the units: longest
// first (ties: lower unit), so that the longest units, each one workgroup's
// critical path, start in the first round of workgroup slots and the shorter
// ones fill in around them.  One workgroup sorts the units' slot counts in
// LDS (bitonic); every unit appears once, so the pass computes exactly what
// it computes in unit order.
constexpr int kOrderMax = 4096;   // units a launch can order
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void unit_order_kernel(CacheDev c, int32_t *order) {
    __shared__ uint64_t key[kOrderMax];
    const int units = c.B * c.Hkv;
    int len = 1;
    while (len < units) len <<= 1;
    for (int i = threadIdx.x; i < len; i += kOrderThreads) {
        uint64_t k = ~0ull;
        if (i < units) {
            int n = c.n_slots[i];
            n = n < 0 ? 0 : (n > c.cap ? c.cap : n);
            k = ((uint64_t)(uint32_t)(c.cap - n) << 32) | (uint32_t)i;
        }
        key[i] = k;
    }
    __syncthreads();
    bitonic_sort(key, len);
    for (int i = threadIdx.x; i < units; i += kOrderThreads) order[i] = (int32_t)(uint32_t)key[i];
}

template <typename T, int D, int SZ>
__global__ __launch_bounds__(FinishCfg<SZ>::NT) __attribute__((amdgpu_waves_per_eu(FinishCfg<SZ>::WPE)))
void finish_kernel(AttnArgs a, SelectArgs sa, CompactArgs ca) {
    using Cfg = FinishCfg<SZ>;
    __shared__ FinishLdsT<Cfg::SEL, Cfg::STAGE> F;
    __shared__ int sh_e;
    const int u = a.order ? a.order[blockIdx.x] : (int)blockIdx.x;
    if (a.presel && !a.scores && a.nsplit > 1) {
        if (finish_presel<T, D, Cfg::NT, Cfg::STAGE>(a, sa, u, F.comb, sh_e)) return;
        __syncthreads();
    }
    if (a.nsplit > 1) {
        combine_unit<D, Cfg::STAGE, Cfg::NT>(a, u, F.comb);
        __syncthreads();
    }
    const int e = select_unit<Cfg::SEL, Cfg::NT>(sa, u, F.sel);
    __syncthreads();
    if (e >= -1) compact_one<T, D>(ca, u, e);
    else compact_unit<T, D, Cfg::NT, true>(ca, u, F.comp);
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
    const dim3 grid(a.c.B * a.c.Hkv);
    AttnArgs au = a;   // the shorter instances take the units in order
    au.order = nullptr;
    if (a.max_len <= kSelLdsSmall)
        hipLaunchKernelGGL((finish_kernel<T, D, kFinishSmall>), grid, dim3(FinishCfg<kFinishSmall>::NT), 0,
                           s, au, sa, ca);
    else if (a.max_len <= kSelLdsSlots)
        hipLaunchKernelGGL((finish_kernel<T, D, kFinishMid>), grid, dim3(FinishCfg<kFinishMid>::NT), 0, s,
                           au, sa, ca);
    else {
        // longest units first, when the launch has few enough units to sort
        AttnArgs ao = a;
        const int units = a.c.B * a.c.Hkv;
        if (a.order && units <= kOrderMax)
            hipLaunchKernelGGL(unit_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, a.c, a.order);
        else
            ao.order = nullptr;
        hipLaunchKernelGGL((finish_kernel<T, D, kFinishLong>), grid, dim3(FinishCfg<kFinishLong>::NT), 0,
                           s, ao, sa, ca);
    }
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
