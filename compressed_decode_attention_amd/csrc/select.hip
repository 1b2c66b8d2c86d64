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
#include "kvc_internal.h"

namespace kvc {

constexpr int kSelThreads = 256;
constexpr int kSelLds = 8192;   // units up to this many slots keep keys in LDS

enum : uint8_t { kDrop = 0, kKeep = 1, kCand = 2 };

struct SelView {
    int kind, n_sink, n_recent, prompt_len;
    uint32_t step, seed_lo, seed_hi;
    int u, b, h, n, L;
    const int32_t *P;
    const float *S;
};

// class and 64-bit ranking key of slot j
__device__ inline uint8_t sel_class(const SelView &v, int j, int32_t p) {
    switch (v.kind) {
        case KVC_POLICY_STREAMING:
            return (p < v.n_sink || (int64_t)p >= (int64_t)v.L - v.n_recent) ? kKeep : kDrop;
        case KVC_POLICY_H2O:
            return ((int64_t)p >= (int64_t)v.L - v.n_recent) ? kKeep : kCand;
        case KVC_POLICY_RANDOM:
            return (p < v.prompt_len) ? kKeep : kCand;
        default:
            return kKeep;
    }
}

__device__ inline uint32_t sel_primary(const SelView &v, int j, int32_t p) {
    if (v.kind == KVC_POLICY_H2O) return float_order_bits(v.S[j]);
    // random: smaller Philox word = better -> invert
    const uint32_t w = philox_word0((uint32_t)p, v.step, (uint32_t)v.h, (uint32_t)v.b,
                                    v.seed_lo, v.seed_hi);
    return ~w;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
    const CacheDev &c = a.c;
    const int u = blockIdx.x;
    const int tid = threadIdx.x;

    __shared__ uint32_t prim_s[kSelLds];
    __shared__ int32_t pos_s[kSelLds];
    __shared__ uint8_t cls_s[kSelLds];
    __shared__ int hist[256];
    __shared__ int red[kSelThreads / 64];
    __shared__ int sh_digit, sh_krem, sh_done;

    SelView v;
    v.kind = a.kind;
    v.n_sink = a.n_sink;
    v.n_recent = a.n_recent;
    v.prompt_len = a.prompt_len;
    v.step = a.step;
    v.seed_lo = (uint32_t)(a.seed & 0xFFFFFFFFu);
    v.seed_hi = (uint32_t)(a.seed >> 32);
    v.u = u;
    v.b = u / c.Hkv;
    v.h = u % c.Hkv;
    v.n = load_count(c, u, tid == 0);
    v.P = c.pos + (size_t)u * c.cap;
    v.S = a.scores ? a.scores + (size_t)u * c.cap : nullptr;
    const int n = v.n;
    const bool in_lds = n <= kSelLds;

    int mx = -1;
    for (int j = tid; j < n; j += kSelThreads) mx = max(mx, v.P[j]);
    v.L = block_max_i(mx, red) + 1;

    // classify, count candidates, cache keys
    int ncand = 0;
    for (int j = tid; j < n; j += kSelThreads) {
        const int32_t p = v.P[j];
        const uint8_t k = sel_class(v, j, p);
        if (in_lds) {
            cls_s[j] = k;
            pos_s[j] = p;
            if (k == kCand) prim_s[j] = sel_primary(v, j, p);
        }
        ncand += (k == kCand);
    }
    int tot;
    (void)block_excl_scan(ncand, red, &tot);
    ncand = tot;
    const int want = (a.kind == KVC_POLICY_H2O) ? a.n_heavy : a.n_keep;

    // radix select of the 'want' largest composite keys among candidates
    uint64_t prefix = 0, mask = 0;
    const bool rank = ncand > want;          // otherwise every candidate stays
    const bool keep_none = rank && want <= 0;
    if (rank && want > 0) {
        int krem = want;
        for (int shift = 56; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
            __syncthreads();
            for (int j = tid; j < n; j += kSelThreads) {
                int32_t p;
                uint8_t k;
                if (in_lds) {
                    k = cls_s[j];
                    p = pos_s[j];
                } else {
                    p = v.P[j];
                    k = sel_class(v, j, p);
                }
                if (k != kCand) continue;
                const uint32_t pr = in_lds ? prim_s[j] : sel_primary(v, j, p);
                const uint64_t key = ((uint64_t)pr << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
            }
            __syncthreads();
            if (tid == 0) {
                // digit holding the krem-th largest matching key
                int cum = 0, dsel = 0;
                for (int d = 255; d >= 0; --d) {
                    if (cum + hist[d] >= krem) {
                        dsel = d;
                        break;
                    }
                    cum += hist[d];
                }
                sh_digit = dsel;
                sh_krem = krem - cum;
                sh_done = (hist[dsel] == krem - cum);
            }
            __syncthreads();
            krem = sh_krem;
            prefix |= (uint64_t)sh_digit << shift;
            mask |= (uint64_t)255 << shift;
            const int done = sh_done;
            __syncthreads();
            if (done) break;   // every key of the selected bin is kept
        }
    }

    // keep flags -> ascending slot list
    int32_t *ks = a.keep_slots + (size_t)u * c.cap;
    int base = 0;
    for (int j0 = 0; j0 < n; j0 += kSelThreads) {
        const int j = j0 + tid;
        int keep = 0;
        if (j < n) {
            int32_t p;
            uint8_t k;
            if (in_lds) {
                k = cls_s[j];
                p = pos_s[j];
            } else {
                p = v.P[j];
                k = sel_class(v, j, p);
            }
            if (k == kKeep) keep = 1;
            else if (k == kCand) {
                if (!rank) keep = 1;
                else if (!keep_none) {
                    const uint32_t pr = in_lds ? prim_s[j] : sel_primary(v, j, p);
                    const uint64_t key = ((uint64_t)pr << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
                    keep = (key & mask) >= prefix;
                }
            }
        }
        int t;
        const int off = block_excl_scan(keep, red, &t);
        if (keep) ks[base + off] = j;
        base += t;
    }
    if (tid == 0) a.n_out[u] = base;
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
    const int units = a.c.B * a.c.Hkv;
    hipLaunchKernelGGL(select_kernel, dim3(units), dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvc
