// generic.h -- per-unit device routines of libkvc that work for any unit
// length, dtype and head_dim: attention with logits in a global scratch row,
// radix selection, hole-fill and ordered compaction.  The standalone kernels
// wrap them one unit per workgroup; the fused step kernel falls back to them
// for units that do not fit its LDS-resident fast path.
#pragma once

#include "kvc_internal.h"

namespace kvc {

constexpr int kAttnThreads = 256;
constexpr int kMaxSplit = 64;

template <int D>
struct AttnLds {
    float q_s[kMaxGroup * D];
    float st_m[kMaxGroup], st_l[kMaxGroup];
    float red[kAttnThreads / 64][kMaxGroup];
    float pv[kAttnThreads / D][kMaxGroup][D];
};

// ===========================================================================
// decode attention (see attn.hip for the method and citations)
// ===========================================================================
// TK: cache element; its activations (q, k_new, v_new) are ActOf<TK>.
template <typename TK, int D>
__device__ inline void attn_unit_generic(const AttnArgs &a, int u, int s, AttnLds<D> &L) {
    using TA = typename ActOf<TK>::type;
    const CacheDev &c = a.c;
    const int G = c.G;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int kParts = kAttnThreads / D;

    float *q_s = L.q_s;
    float *st_m = L.st_m, *st_l = L.st_l;
    auto &red = L.red;
    auto &pv = L.pv;

    const int n = load_count(c, u, s == 0 && tid == 0);
    const bool can_store = a.append && n < c.cap;
    if (a.append && !can_store && s == 0 && tid == 0) raise_flag(c, KVC_FLAG_FULL);
    const int T_len = n + 1;
    const int chunk = split_chunk(T_len, a.nsplit, a.max_len);
    const int j0 = min(s * chunk, T_len), j1 = min(T_len, j0 + chunk);

    const TA *qp = (const TA *)a.q + ((size_t)b * c.Hq + (size_t)h * G) * D;
    for (int e = tid; e < G * D; e += kAttnThreads) q_s[e] = Elem<TA>::get(qp, e);
    __syncthreads();

    const TK *K = (const TK *)c.k;
    const TK *V = (const TK *)c.v;
    const TA *kn = (const TA *)a.k_new + ((size_t)b * c.Hkv + h) * D;
    const TA *vn = (const TA *)a.v_new + ((size_t)b * c.Hkv + h) * D;
    // the new token as the cache holds it (an E5M2 cache rounds it)
    auto knew = [&](int d) {
        const float x = Elem<TA>::get(kn, d);
        if constexpr (kIsE5M2<TK>) return e5m2_round(x);
        else return x;
    };
    auto vnew = [&](int d) {
        const float x = Elem<TA>::get(vn, d);
        if constexpr (kIsE5M2<TK>) return e5m2_round(x);
        else return x;
    };
    const size_t ld = (size_t)c.cap + 1;
    float *lg = a.logits + (size_t)u * G * ld;

    // ---- logits and running max (thread owns keys j = j0 + tid + k*256)
    float mloc[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) mloc[g] = -INFINITY;
    for (int j = j0 + tid; j < j1; j += kAttnThreads) {
        const TK *row = (j < n) ? K + row_of(c, b, h, j) * D : nullptr;
        float acc[kMaxGroup];
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) acc[g] = 0.f;
        for (int d = 0; d < D; ++d) {
            const float kv = (j < n) ? Elem<TK>::get(row, d) : knew(d);
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g)
                if (g < G) acc[g] = fmaf(q_s[g * D + d], kv, acc[g]);
        }
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g)
            if (g < G) {
                const float z = acc[g] * a.scale;
                lg[g * ld + j] = z;
                mloc[g] = fmaxf(mloc[g], z);
            }
    }
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
        const float w = wave_max(mloc[g]);
        if (lane == 0) red[wv][g] = w;
    }
    __syncthreads();
    if (tid < G) {
        float m = red[0][tid];
        for (int w = 1; w < kAttnThreads / 64; ++w) m = fmaxf(m, red[w][tid]);
        st_m[tid] = m;
    }
    __syncthreads();

    // ---- unnormalised weights w = exp(z - m), row sums
    float lloc[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) lloc[g] = 0.f;
    for (int j = j0 + tid; j < j1; j += kAttnThreads) {
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g)
            if (g < G) {
                const float w = __expf(lg[g * ld + j] - st_m[g]);
                lg[g * ld + j] = w;
                lloc[g] += w;
            }
    }
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
        const float w = wave_sum(lloc[g]);
        if (lane == 0) red[wv][g] = w;
    }
    __syncthreads();
    if (tid < G) {
        float l = 0.f;
        for (int w = 0; w < kAttnThreads / 64; ++w) l += red[w][tid];
        st_l[tid] = l;
    }
    __syncthreads();

    // ---- P.V: thread owns one dimension d and every kParts-th key
    {
        const int d = tid % D, part = tid / D;
        float acc[kMaxGroup];
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) acc[g] = 0.f;
        for (int j = j0 + part; j < j1; j += kParts) {
            const float vv = (j < n) ? Elem<TK>::get(V + row_of(c, b, h, j) * D, d) : vnew(d);
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g)
                if (g < G) acc[g] = fmaf(lg[g * ld + j], vv, acc[g]);
        }
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) pv[part][g][d] = acc[g];
    }
    __syncthreads();

    if (a.nsplit == 1) {
        if (tid < D) {
            for (int g = 0; g < G; ++g) {
                float o = 0.f;
                for (int p = 0; p < kParts; ++p) o += pv[p][g][tid];
                a.out[((size_t)b * c.Hq + (size_t)h * G + g) * D + tid] = o / st_l[g];
            }
        }
        if (a.scores) {
            float *sc = a.scores + (size_t)u * c.cap;
            for (int j = j0 + tid; j < j1; j += kAttnThreads) {
                float ps = 0.f;
                for (int g = 0; g < G; ++g) ps += lg[g * ld + j] / st_l[g];
                if (j < n) sc[j] = score_update(sc[j], ps, a.decay);
                else if (can_store) sc[n] = score_update(0.f, ps, a.decay);
            }
        }
    } else {
        float *pp = a.part + ((size_t)u * a.nsplit + s) * G * (D + 2);
        if (tid < D) {
            for (int g = 0; g < G; ++g) {
                float o = 0.f;
                for (int p = 0; p < kParts; ++p) o += pv[p][g][tid];
                pp[g * (D + 2) + tid] = o;
            }
        }
        if (tid < G) {
            pp[tid * (D + 2) + D] = st_m[tid];
            pp[tid * (D + 2) + D + 1] = st_l[tid];
        }
    }

    // ---- append the new token (the workgroup whose range holds index n)
    if (can_store && j0 <= n && n < j1) {
        TK *Kw = (TK *)c.k;
        TK *Vw = (TK *)c.v;
        const size_t r = row_of(c, b, h, n) * D;
        for (int e = tid; e < D; e += kAttnThreads) {
            if constexpr (kIsE5M2<TK>) {
                Kw[r + e].v = e5m2_encode(Elem<TA>::get(kn, e));
                Vw[r + e].v = e5m2_encode(Elem<TA>::get(vn, e));
            } else {
                Kw[r + e] = kn[e];
                Vw[r + e] = vn[e];
            }
        }
        if (tid == 0) c.pos[(size_t)u * c.cap + n] = a.new_pos[b];
    }
    if (a.nsplit == 1 && tid == 0 && can_store) c.n_slots[u] = n + 1;
}

// ===========================================================================
// selection (see select.hip for the policies and citations)
// ===========================================================================
enum : uint8_t { kDrop = 0, kKeep = 1, kCand = 2 };

constexpr int kSelThreads = 256;
constexpr int kMaxBlockWaves = 16;   // the block helpers' scratch: up to 1,024 threads

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

constexpr int kSelLdsSlots = 8192;   // units up to this many slots keep keys in LDS

template <int kSelLds>
struct SelLds {
    uint32_t prim_s[kSelLds];
    int32_t pos_s[kSelLds];
    uint8_t cls_s[kSelLds];
    int hist[256];
    int red[kMaxBlockWaves];
    uint32_t red3[3 * kMaxBlockWaves];
    int sh_digit, sh_krem, sh_done;
};

// Units of up to kSelLds slots keep their ranking keys in LDS; longer units
// recompute them from global memory on every pass.  Returns the evicted slot
// when at most one slot leaves (-1: none leaves), else -2.
template <int kSelLds, int NT = kSelThreads>
__device__ inline int select_unit(const SelectArgs &a, int u, SelLds<kSelLds> &S) {
    const CacheDev &c = a.c;
    const int tid = threadIdx.x;
    uint32_t *prim_s = S.prim_s;
    int32_t *pos_s = S.pos_s;
    uint8_t *cls_s = S.cls_s;
    int *hist = S.hist;
    int *red = S.red;
    int &sh_digit = S.sh_digit, &sh_krem = S.sh_krem, &sh_done = S.sh_done;

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

    // one pass over global memory: positions (and H2O score keys) go to LDS
    // when they fit, and the newest position gives L; the loads of a thread
    // are independent, so the unrolled loop keeps several in flight
    const bool h2o_keys = in_lds && a.kind == KVC_POLICY_H2O;
    int mx = -1;
    if (in_lds) {
#pragma unroll 4
        for (int j = tid; j < n; j += NT) {
            const int32_t p = v.P[j];
            pos_s[j] = p;
            if (h2o_keys) prim_s[j] = float_order_bits(v.S[j]);
            mx = max(mx, p);
        }
    } else {
#pragma unroll 4
        for (int j = tid; j < n; j += NT) mx = max(mx, v.P[j]);
    }
    v.L = block_max_i(mx, red) + 1;   // (its barriers publish the LDS copies)

    // Units longer than the LDS copy are read from global memory kU slots per
    // thread at a time (slots j0 + q * NT, the same order as one at
    // a time), every load of a group issued before any is used; scores are
    // fetched for every policy (positions stand in when there are none).  A
    // caller with no LDS copy (a fallback inside another kernel) takes one
    // slot at a time and keeps its registers for its own work.
    constexpr int kU = kSelLds > 1 ? 8 : 1;
    const float *Sg = v.S ? v.S : reinterpret_cast<const float *>(v.P);
    auto fetch = [&](int j0, int32_t (&pg)[kU], uint32_t (&sg)[kU]) {
#pragma unroll
        for (int q = 0; q < kU; ++q) {
            const int j = min(j0 + q * NT, n - 1);
            pg[q] = v.P[j];
            sg[q] = __float_as_uint(Sg[j]);
        }
    };
    // a candidate's primary key from its fetched position and score bits
    auto primary = [&](int j, int32_t p, uint32_t sbits) -> uint32_t {
        return a.kind == KVC_POLICY_H2O ? float_order_bits(__uint_as_float(sbits))
                                        : sel_primary(v, j, p);
    };

    // classify, count candidates and drops, cache keys; the smallest
    // candidate key and the last dropped slot serve the one-eviction case
    int ncand = 0, ndrop = 0, dslot = -1, barg = -1;
    uint64_t best = ~0ull;
    auto classify = [&](int j, int32_t p, uint8_t k, uint32_t pr) {
        if (k == kCand) {
            const uint64_t key = ((uint64_t)pr << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
            if (barg < 0 || key < best) {
                best = key;
                barg = j;
            }
            ++ncand;
        } else if (k == kDrop) {
            ++ndrop;
            dslot = j;
        }
    };
    if (in_lds) {
        for (int j = tid; j < n; j += NT) {
            const int32_t p = pos_s[j];
            const uint8_t k = sel_class(v, j, p);
            cls_s[j] = k;
            uint32_t pr = 0;
            if (k == kCand) {
                pr = h2o_keys ? prim_s[j] : sel_primary(v, j, p);
                prim_s[j] = pr;
            }
            classify(j, p, k, pr);
        }
    } else {
        for (int j0 = tid; j0 < n; j0 += kU * NT) {
            int32_t pg[kU];
            uint32_t sg[kU];
            fetch(j0, pg, sg);
#pragma unroll
            for (int q = 0; q < kU; ++q) {
                const int j = j0 + q * NT;
                if (j >= n) break;
                const uint8_t k = sel_class(v, j, pg[q]);
                classify(j, pg[q], k, k == kCand ? primary(j, pg[q], sg[q]) : 0u);
            }
        }
    }
    int tot;
    (void)block_excl_scan(ncand, red, &tot);
    ncand = tot;
    (void)block_excl_scan(ndrop, red, &tot);
    ndrop = tot;
    const int want = (a.kind == KVC_POLICY_H2O) ? a.n_heavy : a.n_keep;
    const int extra = (ncand > want) ? (want <= 0 ? ncand : ncand - want) : 0;
    if (ndrop + extra <= 1) {
        // at most one slot leaves (the steady state): it is the smallest
        // candidate key or the one dropped slot, and the keep list is every
        // other slot in order, with no ranking passes
        block_min_u64(best, barg, S.red3);
        dslot = block_max_i(dslot, red);
        const int e = (extra == 1) ? barg : (ndrop == 1 ? dslot : -1);
        int32_t *ks = a.keep_slots + (size_t)u * c.cap;
        for (int j = tid; j < n; j += NT)
            if (j != e) ks[(e >= 0 && j > e) ? j - 1 : j] = j;
        if (tid == 0) a.n_out[u] = (e >= 0) ? n - 1 : n;
        return e;
    }

    // radix select of the 'want' largest composite keys among candidates
    uint64_t prefix = 0, mask = 0;
    const bool rank = ncand > want;          // otherwise every candidate stays
    const bool keep_none = rank && want <= 0;
    if (rank && want > 0) {
        int krem = want;
        for (int shift = 56; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += NT) hist[i] = 0;
            __syncthreads();
            auto count = [&](int32_t p, uint32_t pr) {
                const uint64_t key = ((uint64_t)pr << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
                if ((key & mask) == prefix) hist_add_wave(hist, (int)((key >> shift) & 255));
            };
            if (in_lds) {
                for (int j = tid; j < n; j += NT)
                    if (cls_s[j] == kCand) count(pos_s[j], prim_s[j]);
            } else {
                for (int j0 = tid; j0 < n; j0 += kU * NT) {
                    int32_t pg[kU];
                    uint32_t sg[kU];
                    fetch(j0, pg, sg);
#pragma unroll
                    for (int q = 0; q < kU; ++q) {
                        const int j = j0 + q * NT;
                        if (j >= n) break;
                        if (sel_class(v, j, pg[q]) == kCand) count(pg[q], primary(j, pg[q], sg[q]));
                    }
                }
            }
            __syncthreads();
            if (tid < 64) radix_pick_bin(hist, krem, sh_digit, sh_krem, sh_done);
            __syncthreads();
            krem = sh_krem;
            prefix |= (uint64_t)sh_digit << shift;
            mask |= (uint64_t)255 << shift;
            const int done = sh_done;
            __syncthreads();
            if (done) break;   // every key of the selected bin is kept
        }
    }

    // keep flags -> ascending slot list: each thread owns a run of
    // consecutive slots, so one scan orders a whole run of the block
    int32_t *ks = a.keep_slots + (size_t)u * c.cap;
    auto kept = [&](int j, int32_t p, uint8_t k, uint32_t pr) -> bool {
        if (k == kKeep) return true;
        if (k != kCand) return false;
        if (!rank) return true;
        if (keep_none) return false;
        const uint64_t key = ((uint64_t)pr << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
        return (key & mask) >= prefix;
    };
    int base = 0;
    if (in_lds) {
        const int per = (n + NT - 1) / NT;
        const int r0 = min(n, tid * per), r1 = min(n, r0 + per);
        int mine = 0;
        for (int j = r0; j < r1; ++j) mine += kept(j, pos_s[j], cls_s[j], prim_s[j]) ? 1 : 0;
        int off = block_excl_scan(mine, red, &base);
        for (int j = r0; j < r1; ++j)
            if (kept(j, pos_s[j], cls_s[j], prim_s[j])) ks[off++] = j;
    } else {
        // blocks of kU * NT slots, a run of kU per thread
        for (int c0 = 0; c0 < n; c0 += kU * NT) {
            const int r0 = c0 + tid * kU;
            int32_t pg[kU];
            uint32_t sg[kU];
#pragma unroll
            for (int q = 0; q < kU; ++q) {
                const int j = min(r0 + q, n - 1);
                pg[q] = v.P[j];
                sg[q] = __float_as_uint(Sg[j]);
            }
            uint32_t flags = 0;
#pragma unroll
            for (int q = 0; q < kU; ++q) {
                const int j = r0 + q;
                if (j < n) {
                    const uint8_t k = sel_class(v, j, pg[q]);
                    if (kept(j, pg[q], k, k == kCand ? primary(j, pg[q], sg[q]) : 0u))
                        flags |= 1u << q;
                }
            }
            int t;
            int off = block_excl_scan(__popc(flags), red, &t);
#pragma unroll
            for (int q = 0; q < kU; ++q)
                if ((flags >> q) & 1u) ks[base + off++] = r0 + q;
            base += t;
        }
    }
    if (tid == 0) a.n_out[u] = base;
    return -2;
}

// ===========================================================================
// compaction (see compact.hip)
// ===========================================================================
constexpr int kCompThreads = 256;
constexpr int kOrderedMax = 8192;

template <typename T, int D>
__device__ inline void copy_row(T *dst, const T *src) {
    static_assert((D * sizeof(T)) % 16 == 0, "row must be a multiple of 16 bytes");
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
    uint4 *d = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int i = 0; i < (int)(D * sizeof(T) / 16); ++i) d[i] = s[i];
}

struct CompLds {
    uint32_t kept_bits[kMaxCapacity / 32];
    int red[kMaxBlockWaves];
};

// Compaction when slot e alone leaves a unit of n slots (e < 0: none): the
// last slot fills the hole, the hole-fill pairing of one hole with one source.
template <typename T, int D>
__device__ inline void compact_one(const CompactArgs &a, int u, int e) {
    const CacheDev &c = a.c;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x;
    const int n = load_count(c, u, false);
    if (e < 0 || e >= n) return;
    const int src = n - 1;
    constexpr int kParts = (int)(D * sizeof(T) / 16);
    if (e < src) {
        if (tid < 2 * kParts) {
            T *X = (tid < kParts) ? (T *)c.k : (T *)c.v;
            const int part = tid % kParts;
            reinterpret_cast<uint4 *>(X + row_of(c, b, h, e) * D)[part] =
                reinterpret_cast<const uint4 *>(X + row_of(c, b, h, src) * D)[part];
        }
        if (tid == 0) {
            int32_t *P = c.pos + (size_t)u * c.cap;
            P[e] = P[src];
            if (a.scores) a.scores[(size_t)u * c.cap + e] = a.scores[(size_t)u * c.cap + src];
        }
    }
    if (tid == 0) c.n_slots[u] = src;
}

// WAVE_COPY: the waves copy the rows together with batched loads (the
// compaction and finish kernels); without it each lane with a move copies its
// row alone (kept for callers whose registers are at their limit).
template <typename T, int D, int NT = kCompThreads, bool WAVE_COPY = false>
__device__ inline void compact_unit(const CompactArgs &a, int u, CompLds &CL) {
    const CacheDev &c = a.c;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x;
    uint32_t *kept_bits = CL.kept_bits;
    int *red = CL.red;

    const int n = load_count(c, u, tid == 0);
    int m = a.n_out[u];
    if (m < 0 || m > n) {
        if (tid == 0) raise_flag(c, KVC_FLAG_BAD_COUNT);
        m = m < 0 ? 0 : n;
    }
    const int32_t *ks = a.keep_slots + (size_t)u * c.cap;
    const int words = (m + 31) / 32;
    // kept slots below m form a prefix of the ascending list; mark them
    for (int w = tid; w < words; w += NT) kept_bits[w] = 0;
    __syncthreads();
    int below = 0;
    for (int i = tid; i < m; i += NT) {
        const int j = ks[i];
        if (j >= 0 && j < m) {
            atomicOr(&kept_bits[j >> 5], 1u << (j & 31));
            ++below;
        }
    }
    int cnt;
    (void)block_excl_scan(below, red, &cnt);
    below = cnt;   // sources are ks[below .. m)
    __syncthreads();

    int32_t *P = c.pos + (size_t)u * c.cap;
    float *S = a.scores ? a.scores + (size_t)u * c.cap : nullptr;
    // WAVE_COPY: each wave copies its lanes' moves together: kParts lanes per row, one
    // 16-byte part each of K and V, the row addresses taken from the lane that
    // owns the move; a lane's loads of kBatch such steps go out before its
    // stores (a move's source is a kept slot >= m and its destination a hole
    // below m, so no row is both read and written), instead of one lane
    // copying a row with a round trip per part.
    constexpr int kParts = (int)(D * sizeof(T) / 16);
    static_assert(64 % kParts == 0, "a row's 16-byte parts must tile a wave");
    constexpr int kPerStep = 64 / kParts;   // moves per wave step
    constexpr int kBatch = 4;               // wave steps whose loads go out together
    static_assert(kParts % kBatch == 0, "steps per wave must be a multiple of the batch");
    const int lane = tid & 63, part = lane % kParts, which = lane / kParts;
    uint4 *Kq = reinterpret_cast<uint4 *>(c.k), *Vq = reinterpret_cast<uint4 *>(c.v);
    int base = 0;
    for (int j0 = 0; j0 < m; j0 += NT) {
        const int j = j0 + tid;
        const int hole = (j < m) && !((kept_bits[j >> 5] >> (j & 31)) & 1u);
        int t;
        const int r = block_excl_scan(hole, red, &t);
        const int idx = below + base + r;
        if constexpr (!WAVE_COPY) {
            if (hole && idx < m) {
                const int src = ks[idx];
                if (src >= m && src < n) {
                    copy_row<T, D>((T *)c.k + row_of(c, b, h, j) * D, (T *)c.k + row_of(c, b, h, src) * D);
                    copy_row<T, D>((T *)c.v + row_of(c, b, h, j) * D, (T *)c.v + row_of(c, b, h, src) * D);
                    P[j] = P[src];
                    if (S) S[j] = S[src];
                }
            }
            base += t;
            continue;
        }
        // this lane's move: destination and source rows in 16-byte units
        long long dq = -1, sq = 0;
        if (hole && idx < m) {
            const int src = ks[idx];
            if (src >= m && src < n) {
                dq = (long long)row_of(c, b, h, j) * kParts;
                sq = (long long)row_of(c, b, h, src) * kParts;
                P[j] = P[src];
                if (S) S[j] = S[src];
            }
        }
        // (the batch is written out: arrays indexed in loops here were kept on
        // the stack)
        for (int s0 = 0; s0 < kParts; s0 += kBatch) {   // kParts steps cover the wave's 64 lanes
            const int o0 = s0 * kPerStep + which;
            const long long d0 = __shfl(dq, o0, 64), d1 = __shfl(dq, o0 + kPerStep, 64);
            const long long d2 = __shfl(dq, o0 + 2 * kPerStep, 64), d3 = __shfl(dq, o0 + 3 * kPerStep, 64);
            const long long r0 = __shfl(sq, o0, 64) + part, r1 = __shfl(sq, o0 + kPerStep, 64) + part;
            const long long r2 = __shfl(sq, o0 + 2 * kPerStep, 64) + part;
            const long long r3 = __shfl(sq, o0 + 3 * kPerStep, 64) + part;
            uint4 k0{}, k1{}, k2{}, k3{}, v0{}, v1{}, v2{}, v3{};
            if (d0 >= 0) { k0 = Kq[r0]; v0 = Vq[r0]; }
            if (d1 >= 0) { k1 = Kq[r1]; v1 = Vq[r1]; }
            if (d2 >= 0) { k2 = Kq[r2]; v2 = Vq[r2]; }
            if (d3 >= 0) { k3 = Kq[r3]; v3 = Vq[r3]; }
            if (d0 >= 0) { Kq[d0 + part] = k0; Vq[d0 + part] = v0; }
            if (d1 >= 0) { Kq[d1 + part] = k1; Vq[d1 + part] = v1; }
            if (d2 >= 0) { Kq[d2 + part] = k2; Vq[d2 + part] = v2; }
            if (d3 >= 0) { Kq[d3 + part] = k3; Vq[d3 + part] = v3; }
        }
        base += t;
    }
    if (tid == 0) c.n_slots[u] = m;
}

// bitonic sort of 64-bit keys in LDS, ascending (len a power of two)
__device__ inline void bitonic_sort(uint64_t *x, int len) {
    for (int k = 2; k <= len; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < len; i += blockDim.x) {
                const int p = i ^ j;
                if (p > i) {
                    const bool up = (i & k) == 0;
                    const uint64_t xi = x[i], xp = x[p];
                    if ((xi > xp) == up) {
                        x[i] = xp;
                        x[p] = xi;
                    }
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace kvc
