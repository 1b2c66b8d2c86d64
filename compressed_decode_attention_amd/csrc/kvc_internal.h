// kvc_internal.h -- device-side view of the cache and small helpers shared by
// the libkvc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kMaxGroup = 16;       // q heads per kv head handled by one workgroup
constexpr int kMaxCapacity = 65536; // slots per unit
constexpr int kWave = 64;

// Device copy of kvc_cache, passed by value to kernels.
struct CacheDev {
    int32_t B, Hq, Hkv, D, cap, G;
    int32_t bs, max_blocks, num_blocks;
    void *k, *v;
    const int32_t *bt;
    int32_t *pos, *n_slots, *flags;
};

inline CacheDev make_dev(const kvc_cache &c) {
    CacheDev d;
    d.B = c.batch;
    d.Hq = c.q_heads;
    d.Hkv = c.kv_heads;
    d.D = c.head_dim;
    d.cap = c.capacity;
    d.G = c.q_heads / c.kv_heads;
    d.bs = c.block_size;
    d.max_blocks = c.max_blocks;
    d.num_blocks = c.num_blocks;
    d.k = c.k;
    d.v = c.v;
    d.bt = c.block_table;
    d.pos = c.pos;
    d.n_slots = c.n_slots;
    d.flags = c.flags;
    return d;
}

__device__ inline void raise_flag(const CacheDev &c, int32_t bit) {
    if (c.flags) atomicOr(c.flags, bit);
}

// Row index (in units of head_dim elements) of slot j of unit (b, h).
// Paged caches look the block up in the block table; an id outside the pool
// is reported and redirected to block 0 so that no access leaves the pool.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// A buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros (no fault), so a load needs no branch to stay in bounds.
constexpr int kRsrcWord3 = 0x00020000;   // buffer resource dword 3 on gfx9-family parts
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ inline size_t row_of(const CacheDev &c, int b, int h, int j) {
    if (c.bs == 0) return ((size_t)(b * c.Hkv + h)) * (size_t)c.cap + (size_t)j;
    int blk = c.bt[(size_t)b * c.max_blocks + j / c.bs];
    if (blk < 0 || blk >= c.num_blocks) {
        raise_flag(c, KVC_FLAG_BAD_BLOCK);
        blk = 0;
    }
    return ((size_t)blk * c.Hkv + h) * (size_t)c.bs + (size_t)(j % c.bs);
}

// Filled slots of unit u, clamped into [0, cap] (reported when clamped).
__device__ inline int load_count(const CacheDev &c, int u, bool report) {
    int n = c.n_slots[u];
    if (n < 0 || n > c.cap) {
        if (report) raise_flag(c, KVC_FLAG_BAD_COUNT);
        n = n < 0 ? 0 : c.cap;
    }
    return n;
}

// ---------------------------------------------------------------------------
// element access: bf16 is kept as raw 16-bit patterns; widening is exact
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
    __device__ static inline float get(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
};
template <> struct Elem<float> {
    __device__ static inline float get(const float *p, size_t i) { return p[i]; }
};

// E5M2 (OCP 8-bit float: sign, 5 exponent bits with bias 15, 2 mantissa
// bits) cache element.  Decoding uses the hardware conversion (exact); the
// activations of an E5M2 cache are bf16.
struct e5m2_t {
    uint8_t v;
};
template <> struct Elem<e5m2_t> {
    __device__ static inline float get(const e5m2_t *p, size_t i) {
        return __builtin_amdgcn_cvt_f32_bf8((int)p[i].v, 0);
    }
};
template <typename T> struct ActOf { using type = T; };
template <> struct ActOf<e5m2_t> { using type = uint16_t; };
template <typename T> struct IsE5M2 { static constexpr bool value = false; };
template <> struct IsE5M2<e5m2_t> { static constexpr bool value = true; };
template <typename T> inline constexpr bool kIsE5M2 = IsE5M2<T>::value;

// Nearest E5M2 code of x: round to nearest, ties to the even code;
// magnitudes at or beyond the largest finite value 57344 saturate to it; NaN
// stays NaN.  Integer arithmetic on the binary32 pattern.
__device__ inline uint8_t e5m2_encode(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return (uint8_t)(sign | 0x7Fu);            // NaN
    if (a >= 0x47600000u) return (uint8_t)(sign | 0x7Bu);           // >= 57344: saturate
    if (a < 0x38800000u) {                                           // < 2^-14: m * 2^-16
        const float m = rintf(__uint_as_float(a) * 65536.0f);        // exact scaling; ties to even
        return (uint8_t)(sign | (uint32_t)m);                        // m == 4 is the code of 2^-14
    }
    // keep 2 of the 23 mantissa bits, ties to even, then re-bias 127 -> 15
    const uint32_t r = (a + 0x000FFFFFu + ((a >> 21) & 1u)) >> 21;
    uint32_t code = r - (112u << 2);
    if (code > 0x7Bu) code = 0x7Bu;
    return (uint8_t)(sign | code);
}
__device__ inline float e5m2_round(float x) {   // the value an E5M2 cache stores for x
    return __builtin_amdgcn_cvt_f32_bf8((int)e5m2_encode(x), 0);
}

// ---------------------------------------------------------------------------
// wave / block reductions
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
    return x;
}
__device__ inline float wave_sum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}
__device__ inline int wave_sum_i(int x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}
__device__ inline int wave_max_i(int x) {
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, kWave));
    return x;
}
__device__ inline int wave_min_i(int x) {
    for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, kWave));
    return x;
}

// The value of lane (lane ^ M) without a trip through the LDS unit: DPP
// quad permutes for M = 1, 2; for M = 4 and 8 a row mirror (lane ^ 7, lane ^ 15)
// composed with a quad permute or the half-row mirror; for M = 16 and 32 the
// CDNA4 swaps of rows and of wave halves (v_permlane16/32_swap).  Every lane of
// the wave must be active.  A butterfly step x op lane_xor<M>(x) gives every
// lane the result the LDS shuffle gives (op commutative).
template <int M>
__device__ inline uint32_t lane_xor(uint32_t x) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane_xor mask");
    const int v = (int)x;
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
    } else if constexpr (M == 4) {
        const int h = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);     // lane ^ 7
        return (uint32_t)__builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, false);   // then ^ 3
    } else if constexpr (M == 8) {
        const int h = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);     // lane ^ 15
        return (uint32_t)__builtin_amdgcn_mov_dpp(h, 0x141, 0xF, 0xF, false);  // then ^ 7
    } else if constexpr (M == 16) {
        // .x: the even row of each row pair, .y: the odd row
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (__lane_id() & 16) ? r[0] : r[1];
    } else {
        // .x: the lower half of the wave, .y: the upper half
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (__lane_id() & 32) ? r[0] : r[1];
    }
}
template <int M>
__device__ inline float lane_xor_f(float x) {
    return __builtin_bit_cast(float, lane_xor<M>(__builtin_bit_cast(uint32_t, x)));
}
// x + (x of lane ^ 32) and x + (x of lane ^ 16), summed lower half (row) first
// in every lane: the same value as the butterfly sum, without the lane select.
// The two words are copied out of the result vector before the bit casts: a
// bit cast applied to an element of it reads element 0 (hipcc 7.2).
__device__ inline float pair_sum32(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t lo = r[0], hi = r[1];
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}
__device__ inline float pair_sum16(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t ev = r[0], od = r[1];
    return __builtin_bit_cast(float, ev) + __builtin_bit_cast(float, od);
}
// whole-wave reductions through lane_xor (every lane active)
__device__ inline int wave_sum_iv(int x) {
    x += (int)lane_xor<32>((uint32_t)x);
    x += (int)lane_xor<16>((uint32_t)x);
    x += (int)lane_xor<8>((uint32_t)x);
    x += (int)lane_xor<4>((uint32_t)x);
    x += (int)lane_xor<2>((uint32_t)x);
    x += (int)lane_xor<1>((uint32_t)x);
    return x;
}
__device__ inline int wave_max_iv(int x) {
    x = max(x, (int)lane_xor<32>((uint32_t)x));
    x = max(x, (int)lane_xor<16>((uint32_t)x));
    x = max(x, (int)lane_xor<8>((uint32_t)x));
    x = max(x, (int)lane_xor<4>((uint32_t)x));
    x = max(x, (int)lane_xor<2>((uint32_t)x));
    x = max(x, (int)lane_xor<1>((uint32_t)x));
    return x;
}

// Block-wide max of an int (blockDim.x a multiple of 64, <= 1024).
__device__ inline int block_max_i(int x, int *red) {
    x = wave_max_i(x);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) red[w] = x;
    __syncthreads();
    int r = red[0];
    for (int i = 1; i < nw; ++i) r = max(r, red[i]);
    __syncthreads();
    return r;
}

// Block-wide minimum of 64-bit keys with the argument that holds it (equal
// keys: the lower argument, compared unsigned so that -1, "none", loses);
// red needs 3 words per wave.
__device__ inline void block_min_u64(uint64_t &key, int &arg, uint32_t *red) {
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t hi = __shfl_xor((uint32_t)(key >> 32), o, kWave);
        const uint32_t lo = __shfl_xor((uint32_t)key, o, kWave);
        const int oa = __shfl_xor(arg, o, kWave);
        const uint64_t ok = ((uint64_t)hi << 32) | lo;
        if (ok < key || (ok == key && (unsigned)oa < (unsigned)arg)) {
            key = ok;
            arg = oa;
        }
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) {
        red[3 * w] = (uint32_t)(key >> 32);
        red[3 * w + 1] = (uint32_t)key;
        red[3 * w + 2] = (uint32_t)arg;
    }
    __syncthreads();
    for (int i = 0; i < nw; ++i) {
        const uint64_t ok = ((uint64_t)red[3 * i] << 32) | red[3 * i + 1];
        if (ok < key || (ok == key && red[3 * i + 2] < (uint32_t)arg)) {
            key = ok;
            arg = (int)red[3 * i + 2];
        }
    }
    __syncthreads();
}

// One pass of an MSB-first radix select, run by the 64 lanes of one wave:
// among 256 digit bins (hist[d] = matching keys whose current digit is d),
// the bin holding the krem-th largest key is the d with (matches in bins
// above d) < krem <= (that + hist[d]).  Writes that digit, the rank left
// inside the bin (krem minus the matches above it) and whether the bin is
// kept whole.  Lane l reads bins 4l..4l+3 and a suffix scan over the lanes
// gives each lane the count above its bins.
__device__ inline void radix_pick_bin(const int *hist, int krem, int &digit, int &krem_out,
                                      int &done) {
    const int l = threadIdx.x & 63;
    const int h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
    const int mine = h0 + h1 + h2 + h3;
    int suf = mine;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(suf, o, kWave);
        if (l + o < 64) suf += y;
    }
    int cum = suf - mine, dsel = -1, dcum = 0;
    const int hb[4] = {h3, h2, h1, h0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (dsel < 0 && cum < krem && cum + hb[i] >= krem) {
            dsel = 4 * l + 3 - i;
            dcum = cum;
        }
        cum += hb[i];
    }
    if (__ballot(dsel >= 0) == 0) {
        // fewer matches than krem (not reached for valid counts): what a
        // scan from the top that never stops leaves, bin 0 and the count of
        // every bin (lane 0's suffix is the total)
        if (l == 0) {
            digit = 0;
            krem_out = krem - suf;
            done = (h0 == krem - suf);
        }
    } else if (dsel >= 0) {
        digit = dsel;
        krem_out = krem - dcum;
        done = (hist[dsel] == krem - dcum);
    }
}

// hist[digit] += 1 for every calling lane, lanes of a wave that share a
// digit adding together: up to four rounds take the first lane's digit and
// its whole group (the few crowded bins of a radix pass's early digits),
// then each remaining lane adds alone.  Integer counts: the totals are those
// of one atomic add per lane.
__device__ inline void hist_add_wave(int *hist, int digit) {
    const int lane = threadIdx.x & 63;
    bool active = true;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const unsigned long long act = __ballot(active);
        if (act == 0) return;
        const int leader = __ffsll(act) - 1;
        const int d0 = __shfl(digit, leader, kWave);
        const bool mine = active && digit == d0;
        const unsigned long long same = __ballot(mine);
        if (lane == leader) atomicAdd(&hist[d0], (int)__popcll(same));
        if (mine) active = false;
    }
    if (active) atomicAdd(&hist[digit], 1);
}

// Block-wide exclusive prefix sum of small ints; returns the exclusive prefix
// of the calling thread and writes the block total to *total.
__device__ inline int block_excl_scan(int x, int *red, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int incl = x;
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) red[w] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int i = 0; i < nw; ++i) {
        if (i < w) base += red[i];
        tot += red[i];
    }
    __syncthreads();
    *total = tot;
    return base + incl - x;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11): returns word 0 for counter (c0..c3) and key (k0, k1).
// ---------------------------------------------------------------------------
__device__ inline uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t a = c0, cc = c2;
        const uint32_t lo_a = a * 0xD2511F53u, hi_a = __umulhi(a, 0xD2511F53u);
        const uint32_t lo_c = cc * 0xCD9E8D57u, hi_c = __umulhi(cc, 0xCD9E8D57u);
        c0 = hi_c ^ c1 ^ k0;
        c1 = lo_c;
        c2 = hi_a ^ c3 ^ k1;
        c3 = lo_a;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

// order-preserving map float -> uint32 (larger float -> larger uint)
__device__ inline uint32_t float_order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace kvc

// ---------------------------------------------------------------------------
// host-side launchers (defined in the kernel files, called by kvc_api.hip)
// ---------------------------------------------------------------------------
namespace kvc {

struct AttnArgs {
    CacheDev c;
    const int32_t *new_pos;
    const void *q, *k_new, *v_new;
    float *out;
    float *scores;        // may be null
    float scale;
    float decay;          // 0: scores += p; in (0, 1): scores = decay*scores + (1-decay)*p
    int nsplit;
    int max_len;          // attended length bound of every unit (n_slots + 1)
    bool append;          // store the new token at slot n (false: attend it only)
    float *part;          // [units][nsplit][G][D+2] when nsplit > 1
    float *logits;        // [units][G][cap+1] scratch (scores and/or nsplit > 1)
    // Whole steps under random eviction over long units: each split also
    // ranks its own chunk's candidates (slots past the pinned prompt) and
    // writes one PreselRecord per wave, so that the step's finish pass needs no
    // second look at positions when at most one slot leaves.  Null otherwise.
    uint32_t *presel = nullptr;   // [units][nsplit][kPreselWaves] PreselRecord
    int32_t presel_prompt_len = 0;
    uint32_t presel_step = 0;
    uint64_t presel_seed = 0;
    // Finish pass over long units: scratch for the order in which its
    // workgroups take the units ([units] int32, longest first).
    int32_t *order = nullptr;
};

// One wave's share of a split's random-eviction ranking: the number of
// candidate slots among those it ranked and the smallest composite key among them (the key the
// selection ranks by: inverted Philox word, then inverted position) with its
// slot; an empty share has ncand 0, key ~0 and slot -1.
struct PreselRecord {
    uint32_t ncand, key_hi, key_lo;
    int32_t slot;
};
constexpr int kPreselWaves = 4;   // records per split: one per wave of the split kernel

hipError_t launch_attn(const AttnArgs &a, int dtype, hipStream_t s);

// Slots per split of a launch over ns splits whose units attend at most
// max_len entries: equal shares of max_len rounded up to whole 16-slot tiles,
// at least kMinChunk.  Every unit of the launch uses the same chunk, so a unit
// shorter than max_len fills only its first split_count splits (split s
// covers [s*chunk, (s+1)*chunk) of the unit's T attended entries, clipped to
// T; the later splits hold nothing, and the matrix-core split kernel and
// every combine skip them).  A unit longer than the bound takes shares of its
// own length, so ns splits still cover it.
constexpr int kMinChunk = 128;
__host__ __device__ inline int split_chunk(int T, int ns, int max_len) {
    const int L = T > max_len ? T : max_len;
    const int c = ((L + ns - 1) / ns + 15) & ~15;
    return c > kMinChunk ? c : kMinChunk;
}
__host__ __device__ inline int split_count(int T, int ns, int max_len) {
    const int c = split_chunk(T, ns, max_len);
    const int k = (T + c - 1) / c;
    return k < 1 ? 1 : (k > ns ? ns : k);
}

// Matrix-core split kernels (split.hip): bf16 or E5M2, head_dim 128, block
// sizes 0 or a power of two >= 16; ns >= 2 splits of at most kFusedMaxT slots.
inline bool mfma_tiles_ok(int dtype, int head_dim, int block_size) {
    return (dtype == KVC_BF16 || dtype == KVC_FP8_E5M2) && head_dim == 128 &&
           (block_size == 0 || (block_size >= 16 && (block_size & (block_size - 1)) == 0));
}
hipError_t launch_split(const AttnArgs &a, bool e5m2, int max_len, hipStream_t s);

// New H2O score of a slot from its old score s and the group-summed
// probability w of this step: a plain sum, or a decayed attention activity
// d*s + (1-d)*w (online compaction study, sections 3.1 and 4.1).
__device__ inline float score_update(float s, float w, float d) {
    return d == 0.f ? s + w : d * s + (1.f - d) * w;
}

struct AccumArgs {
    CacheDev c;
    const void *q_rows;
    int m_rows;
    const int32_t *q_pos;
    float *scores;
    float scale;
};
hipError_t launch_accumulate(const AccumArgs &a, int dtype, hipStream_t s);

// Scores from a block of causal query rows on the matrix cores (bf16, head
// dim 128): pass 1 writes every row's log-sum-exp to lse, pass 2 adds the
// probabilities to the scores.
struct PromptArgs {
    CacheDev c;
    const void *q_rows;   // [batch, m_rows, q_heads, head_dim] bf16
    int m_rows;
    const int32_t *q_pos; // [batch, m_rows] or null (every slot visible)
    float *scores;
    float scale;
    float *lse;           // workspace [units][m_rows * G]
    int row_tiles_lds;    // pass 2: row tiles tracked in LDS (0: none, every tile visited)
};
size_t prompt_workspace_bytes(int units, int m_rows, int G);
hipError_t launch_prompt_scores(const PromptArgs &a, hipStream_t s);

struct SelectArgs {
    CacheDev c;
    int kind;             // kvc_policy_kind
    int n_sink, n_heavy, n_recent, prompt_len, n_keep;
    uint64_t seed;
    uint32_t step;
    const float *scores;
    int32_t *keep_slots, *n_out;
};
hipError_t launch_select(const SelectArgs &a, hipStream_t s);

struct CompactArgs {
    CacheDev c;
    const int32_t *keep_slots, *n_out;
    float *scores;        // may be null
    bool ordered;
    CacheDev dst;         // ordered destination
};
hipError_t launch_compact(const CompactArgs &a, int dtype, hipStream_t s);

// KIVI-style quantized cache (kivi.hip); the layout is the one kvc.h states.
struct KiviArgs {
    int B, Hq, Hkv, G, max_quant;
    uint8_t *k_codes, *v_codes;
    float *k_scale, *k_lo, *v_scale, *v_lo;
    uint16_t *k_res, *v_res;
    int32_t *n_quant, *n_res, *flags;
    // decode
    const uint16_t *q, *k_new, *v_new;
    float *out;
    float scale;
    int nsq;              // shares of the quantized tokens per unit (>= 1; the last one
                          // also attends the residual and the new token)
    float *part_q;        // [units][nsq][G][D+2] when nsq > 1
    // prefill
    const uint16_t *pk, *pv;
    const int32_t *lengths;
    int max_len;
};
constexpr int kKivGroup = 32;      // quantized tokens per group
constexpr int kKivResidual = 128;  // residual tokens at most
hipError_t launch_kivi_prefill(const KiviArgs &a, hipStream_t s);
hipError_t launch_kivi_decode(const KiviArgs &a, hipStream_t s);

// A whole decode step through the split kernels (attended lengths above the
// one-workgroup kernel's): attention partials, then one workgroup per unit
// for combine + selection + compaction.
hipError_t launch_step_split(const AttnArgs &a, const SelectArgs &sa, const CompactArgs &ca,
                             int dtype, hipStream_t s);

// one-workgroup-per-unit fast path (bf16 or E5M2, head_dim 128): attention only
// (decode_attn) or the whole step (decode_step)
enum { kModeAttn = 0, kModeStep = 1 };
constexpr int kFusedMaxT = 1024;   // largest attended length of the LDS fast path
constexpr int kFusedSmallT = 528;  // LDS capacity used up to a 512 budget + 1

struct FusedArgs {
    AttnArgs attn;      // nsplit must be 1; logits = global scratch of the fallback
    SelectArgs sel;     // step mode: policy, keep_slots / n_out scratch
    CompactArgs comp;   // step mode: in-place compaction of the fallback
    int tcap;           // attended entries held in LDS: kFusedSmallT or kFusedMaxT
    bool e5m2;          // K / V held as E5M2 codes (else bf16)
};
size_t fused_smem_bytes(int G, int tcap);
hipError_t launch_fused(const FusedArgs &fa, int mode, hipStream_t s);

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s);

}  // namespace kvc
