// mfma_tiles.h -- device pieces shared by the matrix-core attention kernels
// (fused.hip: one workgroup per unit; split.hip: one workgroup per chunk of a
// unit): operand types, the logit column permutation, bf16 / E5M2 row
// conversions, and bounded buffer-resource loads of 16-key K / V tiles.
#pragma once
#include "generic.h"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kFThreads = 256;
constexpr int kFWaves = kFThreads / 64;
constexpr int kHD = 128;   // head_dim of the fast path
constexpr int kDK = 3;    // K tiles (16 keys x 256 B) in flight per wave
constexpr int kDV = 2;    // V tiles (16 keys x 256 B) in flight per wave
constexpr int kDK8 = 4;   // the same for E5M2 rows (16 keys x 128 B)
constexpr int kDV8 = 3;
constexpr int kWavesPerEU = 4;   // 4 workgroups of 4 waves per CU

__device__ inline bf16x8_t as_bf16x8(u16x8_t x) { return __builtin_bit_cast(bf16x8_t, x); }

// LDS column of key j in a logit row. Inside each 16-key tile, key 4e + r sits
// at column 4r + e, so that the four probabilities one lane feeds to the P.V
// MFMA (keys r, r+4, r+8, r+12 of the tile) are contiguous.
__device__ inline int lg_col(int j) { return (j & ~15) | ((j & 3) << 2) | ((j >> 2) & 3); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ inline short bf16_bits(float x) { return __builtin_bit_cast(short, (__bf16)x); }
__device__ inline float bf16_value(short b) { return __uint_as_float((uint32_t)(uint16_t)b << 16); }

// E5M2 codes of one lane's 8 dims -> bf16 (v_cvt_scalef32_pk_bf16_bf8 with
// scale 1 widens two codes; exact for all 256 codes incl. inf / NaN)
__device__ inline u16x8_t e5m2x8_to_bf16(u32x2_t x) {
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x[0], 1.f, false));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x[0], 1.f, true));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x[1], 1.f, false));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x[1], 1.f, true));
    return __builtin_bit_cast(u16x8_t, o);
}
__device__ inline u16x8_t as_bf16_row(u16x8_t x) { return x; }
__device__ inline u16x8_t as_bf16_row(u32x2_t x) { return e5m2x8_to_bf16(x); }

// 8 bf16 values -> their nearest E5M2 codes (the cache's rounding of a new token)
__device__ inline u32x2_t e5m2x8_encode(u16x8_t x) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo |= (uint32_t)e5m2_encode(__uint_as_float((uint32_t)x[e] << 16)) << (8 * e);
        hi |= (uint32_t)e5m2_encode(__uint_as_float((uint32_t)x[4 + e] << 16)) << (8 * e);
    }
    return u32x2_t{lo, hi};
}

// one lane's 8 dims of a K or V row as loaded: 8 bf16 (16 B) or 8 E5M2 codes (8 B)
template <bool F8> struct KvRow { using type = u16x8_t; static constexpr int kBytes = 16; };
template <> struct KvRow<true> { using type = u32x2_t; static constexpr int kBytes = 8; };

__device__ inline void load_q(u16x8_t (&qa)[4], const uint16_t *qp, bool valid, int r) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
        if (valid) qa[c4] = *reinterpret_cast<const u16x8_t *>(qp + 32 * c4 + 8 * r);
        else qa[c4] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
}

// Where the matrix-core kernels read K and V: buffer resources whose range
// ends at the last row the workgroup attends from the cache (the unit's n-th
// row, or the end of its chunk), so that rows past it (the new token's slot,
// the padding of the last tile, the next chunk) read as zeros, with no branch
// and no clamp, and every load address is one per-lane offset plus an
// immediate.  Contiguous caches take one resource per workgroup; paged caches
// one per 16-slot tile (block sizes are powers of two of at least 16, so a
// tile never straddles a block).
// K and V rows are read once per step.  From a contiguous cache,
// non-temporal loads (the "nt" cache policy bit) keep them from displacing
// what the caches hold for others: about 10% faster for the whole step than
// the default policy.  From a block-paged pool the one-workgroup step is
// faster with the default policy (1-2% at the mixed-length batch), while the
// split kernel, which streams long units chunk by chunk, is about 5% faster
// with non-temporal loads (PAGED_NT).
constexpr int kLoadPolicy = 2;        // cache policy bits of the buffer loads: non-temporal
constexpr int kLoadPolicyPaged = 0;   // the default policy
template <bool F8, bool PAGED, bool PAGED_NT = false>
__device__ inline typename KvRow<F8>::type buffer_row(__amdgpu_buffer_rsrc_t rs, int voff) {
    constexpr int pol = (PAGED && !PAGED_NT) ? kLoadPolicyPaged : kLoadPolicy;
    if constexpr (F8)
        return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, 0, pol));
    else
        return __builtin_bit_cast(u16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, pol));
}

// Cached rows [start, end) of one unit, tile t = slots start + 16t ..
// start + 16t + 15 (start is a multiple of 16).  RB = bytes of one K or V row
// (256 for bf16, 128 for E5M2).  Paged: blk holds the block ids of the slots
// from block blk0 on, staged in LDS.
template <bool PAGED, int RB>
struct TileSrc {
    const unsigned char *k0, *v0;   // contiguous: slot 'start'; paged: pool + head offset
    const int *blk_s;
    uint32_t nbytes;                // contiguous: the rows [start, end)
    uint32_t blk_bytes;             // paged: bytes of one block (all kv heads)
    int start, end, blk0, shift, mask;

    __device__ inline TileSrc(const CacheDev &c, int b, int h, int start_, int end_,
                              const int *blk, int blk0_) {
        start = start_;
        end = end_;
        blk_s = blk;
        blk0 = blk0_;
        shift = PAGED ? __ffs(c.bs) - 1 : 0;
        mask = PAGED ? c.bs - 1 : 0;
        const size_t first = PAGED ? (size_t)h * c.bs
                                   : ((size_t)b * c.Hkv + h) * (size_t)c.cap + (size_t)start;
        k0 = static_cast<const unsigned char *>(c.k) + first * RB;
        v0 = static_cast<const unsigned char *>(c.v) + first * RB;
        nbytes = (uint32_t)max(end - start, 0) * RB;
        blk_bytes = PAGED ? (uint32_t)(c.Hkv * c.bs * RB) : 0u;
    }
    // the whole unit: rows [0, n)
    __device__ inline TileSrc(const CacheDev &c, int b, int h, int n, const int *blk)
        : TileSrc(c, b, h, 0, n, blk, 0) {}
    // resource holding tile t (K or V) and the tile's byte offset inside it
    __device__ inline void tile(int t, bool v, __amdgpu_buffer_rsrc_t &rs, int &toff) const {
        if constexpr (!PAGED) {
            rs = make_rsrc(v ? v0 : k0, nbytes);
            toff = 16 * RB * t;
        } else {
            const int j0 = start + 16 * t;
            const int rows = min(max(end - j0, 0), 16);
            const int last = end > start ? end - 1 : start;
            int blk = __builtin_amdgcn_readfirstlane(blk_s[((j0 < last ? j0 : last) >> shift) - blk0]);
            blk = rows > 0 ? blk : 0;
            const size_t off = (size_t)blk * blk_bytes + (size_t)(j0 & mask) * RB;
            rs = make_rsrc((v ? v0 : k0) + off, (uint32_t)rows * RB);
            toff = 0;
        }
    }
};

// one wave's K staging tile: 16 rows of 256 B (bf16 after any widening)
constexpr size_t kStageBytes = 16 * 256;   // 16 rows x 256 B per wave

}  // namespace kvc
