// kivi.hip -- a KIVI-style quantized KV cache on the matrix cores of gfx950:
// every token kept, the old ones as 4-bit codes on per-channel K grids and
// per-token V grids, the newest in a bf16 residual (KV cache compression
// guide, section 2: group 32 and residual 128; section 16, "KV capacity
// formula", "the four methods" and "limits").  The grids, the layout and the
// step are the ones kvc.h states.
//
// Attention over the quantized tokens (kivi_qattn_kernel), one workgroup per
// (unit, share of its groups); each of its four waves walks its own groups
// with its own running maximum, sums and accumulators (online softmax), and
// the waves merge once at the end, so the loop has no workgroup barrier:
//  * K of group g, channel d: k = c * s_gd + lo_gd, so
//        q . k_j = sum_d (q_d s_gd) c_jd + sum_d q_d lo_gd.
//    The scale folds into the query: A = 128 q_d s_gd as a bf16 high part
//    and the bf16 rounding of the rest, the two halves of one 256-long
//    contraction; a code enters B exactly as the bf16 value 1 + c/128 (bits
//    0x3F80 | c).  The product is then sum_d A_d + sum_d (A_d / 128) c_jd,
//    and the first sum with the lo term is one constant per (group, head)
//    that starts the group's accumulators.  The operand is built once per
//    (wave, group): each lane scales 16 of the group's (head, dim) pairs into
//    the wave's LDS tile and reads its own operand back.
//  * V of token j, channel group c (32 channels): v = code * s_jc + lo_jc.  In
//    the P.V tile MFMA m covers dims 16m .. 16m + 15, inside one channel
//    group, so the token scale folds into P: A = 128 p_j s_jc (high / low
//    rows), B the codes as above (one 16-byte load per lane and tile from
//    the tiled V layout), and sum_j (p_j lo_jc - A_j) is added per
//    (head, channel group) at the end; those two sums come from one more MFMA
//    per tile, P against a B of the tile's lo and 128 s values (high / low
//    columns), whose error is that of the bf16 pairs, 2^-17 relative.
//  * the weights of a group's 32 keys go from the product layout to the P.V
//    operand layout through the wave's LDS; the group's grids are staged
//    there too.
// The unit's last share also attends the bf16 residual and the new token on
// the same running softmax.  With one share per unit the workgroup then
// writes the output, turns a full residual's 32 oldest tokens into a group
// and appends the new token: the whole step is one launch.  With several,
// kivi_update_kernel merges the shares' partials and does the same update.
// kivi_prefill_kernel quantizes a prompt.  The quantizer takes every decision
// in binary32.
#include "mfma_tiles.h"

namespace kvc {

constexpr int kKivRow = kHD / 2;                     // bytes of one token's 4-bit codes
constexpr int kKivWavesPerEU = 3;                    // waves per SIMD of the quantized kernel
constexpr int kKivVG = kHD / 32;                     // V grids per token

// codes and grids are read once per step: non-temporal loads
template <typename T>
__device__ inline T kiv_load(const T *p) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    if constexpr (sizeof(T) == 16)
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p)));
    else return __builtin_nontemporal_load(p);
}

// Two codes of one dword -> two bf16 values 1 + c/128 (the code in the low
// mantissa bits: bits 0x3F80 | c).  A K dword holds eight codes of one key,
// slots 0..3 (bits 0..15) the even elements and slots 4..7 the odd ones; a V
// word holds four codes of each of two keys, one key per half.  Either way
// pair J sits at bits 4J and 16 + 4J: one shift and one bit-field select.
// The mask and the bits of 1.0 are passed in registers (KivMagic) so that
// each pair is one v_and_or_b32 (VOP3 takes no literal constants here).
struct KivMagic {
    uint32_t mask, one;
    __device__ inline KivMagic() : mask(0x000F000Fu), one(0x3F803F80u) {
        asm volatile("" : "+s"(mask));
        asm volatile("" : "+v"(one));
    }
};
template <int J>
__device__ inline uint32_t kiv_pair(uint32_t x, const KivMagic &km) {
    return ((J == 0 ? x : x >> (4 * J)) & km.mask) | km.one;
}
__device__ inline u16x8_t kiv_widen8(uint32_t x, const KivMagic &km) {
    return __builtin_bit_cast(u16x8_t, uint4{kiv_pair<0>(x, km), kiv_pair<1>(x, km),
                                             kiv_pair<2>(x, km), kiv_pair<3>(x, km)});
}

// Residual V rows keep dim d at element 8 (d % 16) + d / 16: the 16 bytes
// at 16 c of a row are dims c, 16 + c, .., 112 + c, one lane's B operand of
// the P.V products (the dims of lane column c in the quantized tiles too).
__device__ inline int kiv_vres_elem(int d) { return 8 * (d % 16) + d / 16; }
// the 16 bytes at 16 c of a residual V row, from a row in dim order
__device__ inline uint4 kiv_vres_chunk(const uint16_t *row, int c) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)row[32 * i + c] | ((uint32_t)row[32 * i + 16 + c] << 16);
    return uint4{w[0], w[1], w[2], w[3]};
}

// Quantize one group of kKivGroup tokens, K rows Kr and V rows Vr (bf16,
// consecutive rows of kHD; V in dim order, or in the residual's element
// order when VRES), into group slot g of unit u.  256 threads: the first 128
// take one K channel each, the others one (token, channel group) of V; codes
// go through LDS to be packed into the layout.
struct KivQuantLds {
    uint8_t kc[kKivGroup][kHD], vc[kKivGroup][kHD];
};

template <bool VRES>
__device__ inline void kivi_quantize_group(const KiviArgs &a, int u, int g, const uint16_t *Kr,
                                           const uint16_t *Vr, KivQuantLds &L) {
    const int tid = threadIdx.x;
    constexpr float kTop = 15.f;
    const size_t gslot = (size_t)u * (a.max_quant / kKivGroup) + g;
    const size_t tok0 = (size_t)u * a.max_quant + (size_t)g * kKivGroup;
    if (tid < kHD) {
        const int d = tid;
        float x[kKivGroup];
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < kKivGroup; ++i) {
            x[i] = __uint_as_float((uint32_t)Kr[(size_t)i * kHD + d] << 16);
            mn = fminf(mn, x[i]);
            mx = fmaxf(mx, x[i]);
        }
        const float sc = (mx - mn) / kTop;
#pragma unroll
        for (int i = 0; i < kKivGroup; ++i) {
            float cq = 0.f;
            if (sc > 0.f) cq = fminf(fmaxf(rintf((x[i] - mn) / sc), 0.f), kTop);
            L.kc[i][d] = (uint8_t)cq;
        }
        a.k_scale[gslot * kHD + d] = sc;
        a.k_lo[gslot * kHD + d] = mn;
    } else {
        const int i = (tid - kHD) / kKivVG, c = (tid - kHD) % kKivVG;
        float x[32];
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int d = 32 * c + j;
            x[j] = __uint_as_float((uint32_t)Vr[(size_t)i * kHD + (VRES ? kiv_vres_elem(d) : d)] << 16);
            mn = fminf(mn, x[j]);
            mx = fmaxf(mx, x[j]);
        }
        const float sc = (mx - mn) / kTop;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            float cq = 0.f;
            if (sc > 0.f) cq = fminf(fmaxf(rintf((x[j] - mn) / sc), 0.f), kTop);
            L.vc[i][32 * c + j] = (uint8_t)cq;
        }
        a.v_scale[(tok0 + i) * kKivVG + c] = sc;
        a.v_lo[(tok0 + i) * kKivVG + c] = mn;
    }
    __syncthreads();
    // pack: 512 words of K codes (token rows), then 512 of V codes (tiles)
    for (int idx = tid; idx < 2 * kKivGroup * 16; idx += blockDim.x) {
        const bool isv = idx >= kKivGroup * 16;
        const int rem = idx % (kKivGroup * 16);
        uint32_t word = 0;
        uint8_t *dst;
        if (!isv) {
            // token i, dword wd: dim 32 * (wd % 4) + 8 * (wd / 4) + e at slot k,
            // e = 2k (k < 4) or 2 (k - 4) + 1
            const int i = rem / 16, wd = rem % 16;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = (k < 4) ? 2 * k : 2 * (k - 4) + 1;
                word |= (uint32_t)L.kc[i][32 * (wd % 4) + 8 * (wd / 4) + e] << (4 * k);
            }
            dst = a.k_codes + (tok0 + i) * kKivRow + 4 * wd;
        } else {
            // tile t, lane (r, c), word w: tokens 16 t + r + 8 (w / 2) (low
            // half) and 4 more (high half), dims c + 16 (2 k + (w & 1)) at
            // bits 4 k of each half
            const int t = rem / 256, lr = (rem / 4) % 64, w = rem % 4;
            const int r = lr / 16, c = lr % 16;
            const int i0 = 16 * t + r + 8 * (w / 2);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int d = c + 16 * (2 * k + (w & 1));
                word |= (uint32_t)L.vc[i0][d] << (4 * k);
                word |= (uint32_t)L.vc[i0 + 4][d] << (16 + 4 * k);
            }
            dst = a.v_codes + (tok0 + 16 * t) * kKivRow + 16 * lr + 4 * w;
        }
        *reinterpret_cast<uint32_t *>(dst) = word;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// prefill: block (u, y): y < groups of the unit quantizes group y; the last
// y copies the residual and sets the counts
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kivi_prefill_kernel(KiviArgs a) {
    __shared__ KivQuantLds L;
    const int u = blockIdx.x, y = blockIdx.y;
    const int b = u / a.Hkv;
    const int ny = gridDim.y - 1;
    int len = a.lengths[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int over = len > kKivResidual ? len - kKivResidual : 0;
    const int nq = (over + kKivGroup - 1) / kKivGroup * kKivGroup;
    const uint16_t *K = a.pk + (size_t)u * a.max_len * kHD;
    const uint16_t *V = a.pv + (size_t)u * a.max_len * kHD;
    if (y < ny) {
        if (y * kKivGroup >= nq) return;
        kivi_quantize_group<false>(a, u, y, K + (size_t)y * kKivGroup * kHD,
                                   V + (size_t)y * kKivGroup * kHD, L);
        return;
    }
    const int nr = len - nq;
    const uint4 *ks = reinterpret_cast<const uint4 *>(K + (size_t)nq * kHD);
    uint4 *kd = reinterpret_cast<uint4 *>(a.k_res + (size_t)u * kKivResidual * kHD);
    uint4 *vd = reinterpret_cast<uint4 *>(a.v_res + (size_t)u * kKivResidual * kHD);
    for (int i = threadIdx.x; i < nr * (kHD / 8); i += blockDim.x) {
        kd[i] = ks[i];
        vd[i] = kiv_vres_chunk(V + (size_t)(nq + i / (kHD / 8)) * kHD, i % (kHD / 8));
    }
    if (threadIdx.x == 0) {
        a.n_quant[u] = nq;
        a.n_res[u] = nr;
    }
}

// ---------------------------------------------------------------------------
// cache update after a step's attention: if the residual is full, its 32
// oldest tokens become the next group and the rest move down; then the new
// token joins the residual.  All threads of a 256-thread block.
// ---------------------------------------------------------------------------
__device__ inline void kivi_cache_update(const KiviArgs &a, int u, KivQuantLds &L) {
    const int tid = threadIdx.x;
    const int b = u / a.Hkv, h = u % a.Hkv;
    int nq = a.n_quant[u], nr = a.n_res[u];
    const bool bad = nq < 0 || nq > a.max_quant || (nq % kKivGroup) != 0 || nr < 0 ||
                     nr > kKivResidual;
    if (bad) {
        if (tid == 0 && a.flags) atomicOr(a.flags, KVC_FLAG_BAD_COUNT);
        return;
    }
    uint16_t *Kr = a.k_res + (size_t)u * kKivResidual * kHD;
    uint16_t *Vr = a.v_res + (size_t)u * kKivResidual * kHD;
    if (nr == kKivResidual) {
        if (nq + kKivGroup > a.max_quant) {
            if (tid == 0 && a.flags) atomicOr(a.flags, KVC_FLAG_FULL);
            return;
        }
        kivi_quantize_group<true>(a, u, nq / kKivGroup, Kr, Vr, L);
        // rows 32..127 move down to 0..95: all reads before any write
        constexpr int kMove = (kKivResidual - kKivGroup) * (kHD / 8);   // uint4 per tensor
        static_assert(kMove % 256 == 0, "the row move takes whole passes of 256 threads");
        constexpr int kPer = kMove / 256;
        // (plain vectors, so that the copies stay in registers)
        typedef uint32_t row16_t __attribute__((ext_vector_type(4)));
        row16_t tk[kPer], tv[kPer];
        const row16_t *ks = reinterpret_cast<const row16_t *>(Kr + kKivGroup * kHD);
        const row16_t *vs = reinterpret_cast<const row16_t *>(Vr + kKivGroup * kHD);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            tk[k] = ks[tid + 256 * k];
            tv[k] = vs[tid + 256 * k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            reinterpret_cast<row16_t *>(Kr)[tid + 256 * k] = tk[k];
            reinterpret_cast<row16_t *>(Vr)[tid + 256 * k] = tv[k];
        }
        nq += kKivGroup;
        nr -= kKivGroup;
    }
    if (tid < kHD / 8) {
        const size_t src = ((size_t)b * a.Hkv + h) * kHD;
        reinterpret_cast<uint4 *>(Kr + (size_t)nr * kHD)[tid] =
            reinterpret_cast<const uint4 *>(a.k_new + src)[tid];
        reinterpret_cast<uint4 *>(Vr + (size_t)nr * kHD)[tid] = kiv_vres_chunk(a.v_new + src, tid);
    }
    if (tid == 0) {
        a.n_quant[u] = nq;
        a.n_res[u] = nr + 1;
    }
}

// ---------------------------------------------------------------------------
// attention over the quantized tokens
// ---------------------------------------------------------------------------
struct KivSmall {
    float m[kFWaves][8];             // each wave's reference maximum per head (base-2 logits)
    float l[kFWaves][8];             // each wave's running sum per head
    float corr[kFWaves][8][kKivVG];
    float M[8], il[8];               // the share's maximum per head, 1 / its sum
};
// A tile: one row per head, the high parts of its 128 (scaled) query values in
// columns 0..127 and their low parts in 128..255 (padded against bank clashes)
constexpr int kKivAS = 2 * kHD + 8;
constexpr int kKivPL = 2 * 16 + 4;   // fp32 row stride of a wave's P tile (32 keys)
// one wave's LDS: A tile [8][kKivAS] bf16, K grids [128 s | lo][128], V grids
// [32 tokens][4 x 128 s, 4 x lo], P tile [8][kKivPL], alpha [8], logit constants [8]
constexpr size_t kKivWaveLds = 8 * kKivAS * 2 + 2 * kHD * 4 + kKivGroup * 2 * kKivVG * 4 +
                               8 * kKivPL * 4 + 8 * 4 + 8 * 4;
// A wave keeps a reference maximum per head and rescales its sums only when a
// group's logit exceeds it by more than this (base-2 units): the weights stay
// at most 2^8, far inside fp32 and the bf16 pairs' exponent range.
constexpr float kKivLazy = 8.f;
constexpr float kKivNoMax = -1e30f;   // reference maximum before the first group

__host__ __device__ constexpr size_t kivi_qattn_smem(int G) {
    (void)G;
    return (size_t)kFWaves * kKivWaveLds + sizeof(KivSmall);
}

// bf16 high part of a pair of floats, packed, and the value of each half
__device__ inline uint32_t bf16_pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)x, (__bf16)y});
}
__device__ inline float bf16_lo_half(uint32_t p) { return __uint_as_float(p << 16); }
__device__ inline float bf16_hi_half(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// x.lo * y.lo + x.hi * y.hi + c on a pair of bf16 values (v_dot2_f32_bf16)
__device__ inline float dot2_bf16(uint32_t x, uint32_t y, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                           __builtin_bit_cast(bf16x2_t, y), c, false);
}
constexpr uint32_t kBfNegLo = 0x0000BF80u;     // (-1, 0)
constexpr uint32_t kBfNegHi = 0xBF800000u;     // (0, -1)
constexpr uint32_t kBfNegBoth = 0xBF80BF80u;   // (-1, -1)
// The pair operands of dot2_bf16 reach it in registers, never as constants:
// this toolchain encodes the pair (-1, 0) as the inline constant -1.0, which
// the instruction reads as the 32-bit pattern of -1.0, i.e. the pair (0, -1)
// (measured on every residue of 4M random values).
__device__ inline uint32_t bf16_pair_reg(uint32_t x) {
    asm volatile("" : "+s"(x));
    return x;
}

// One bf16 pair of (a0, a1) for an operand whose rows 0..7 carry the values'
// bf16 roundings and rows 8..15 the roundings of what is left over: with
// sel0 = sel1 = 0 the pair is bf16(a0), bf16(a1); with sel0 = (-1, 0) and
// sel1 = (0, -1) it is bf16(a0 - bf16(a0)), bf16(a1 - bf16(a1)), the
// differences taken exactly by the dot product with the rounded pair.
__device__ inline uint32_t bf16_part2(float a0, float a1, uint32_t sel0, uint32_t sel1) {
    const uint32_t hp = bf16_pack2(a0, a1);
    return bf16_pack2(dot2_bf16(hp, sel0, a0), dot2_bf16(hp, sel1, a1));
}

// Every wave walks its own groups (w, w + 4, ...) with its own reference
// maxima, sums and P.V accumulators; the waves merge once at the end.  Per
// group the wave stages the group's grids in its own LDS, builds the scaled
// query operand there, runs the K products, the softmax weights and the P.V
// products; LDS traffic of one wave needs no workgroup barrier.
//  * The K products take the query operand's high and low parts as two halves
//    of a 256-long contraction (rows of the A tile are heads; rows 8..15 of
//    the MFMA operand repeat rows 0..7), so each head's logit is whole in one
//    accumulator and the lanes of rows 8..15 hold the same logits as rows
//    0..7: the weights' rescaling below needs no exchange between the wave's
//    halves.  The per-head constant starts the accumulator.
//  * Logits are in base-2 units (scale * log2 e, folded into the query for
//    the quantized groups); rows of heads past G get -inf (the quantized
//    groups' constant, the residual's bias after its scaling).  A head's
//    reference maximum moves only when a logit exceeds it by more than
//    kKivLazy; then the whole wave takes the exact maxima and rescales (a
//    wave-uniform branch).
//  * After its groups, the unit's last share takes the residual and the new
//    token in 16-key bf16 tiles on the same running softmax (below).
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(kKivWavesPerEU)))
void kivi_qattn_kernel(KiviArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int ns = a.nsq;
    const int u = blockIdx.x / ns, s = blockIdx.x % ns;
    const int b = u / a.Hkv, h = u % a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane >> 4, col = lane & 15;
    const int G = a.G;
    const int ga = col & 7;          // A row: query head (rows 8..15 carry low parts)
    const bool hi_lane = col < 8;
    const float sc2 = a.scale * 1.44269504088896340736f;   // logits in base-2 units

    unsigned char *wl = smem + (size_t)w * kKivWaveLds;
    uint16_t *ast = reinterpret_cast<uint16_t *>(wl);                      // [8][kKivAS]
    float *kg = reinterpret_cast<float *>(wl + 8 * kKivAS * 2);            // [2][kHD]
    float *vg = kg + 2 * kHD;                                              // [32][8]
    float *pt = vg + kKivGroup * 2 * kKivVG;                               // [8][kKivPL]
    float *al = pt + 8 * kKivPL;                                           // [8]
    float *csb = al + 8;                                                   // [8]
    KivSmall &sm = *reinterpret_cast<KivSmall *>(smem + (size_t)kFWaves * kKivWaveLds);

    // the query slice this lane scales for the K products: head gh, dims
    // d0 .. d0 + 15, times the logit scale in base-2 units (so the products
    // are the base-2 logits themselves)
    const int gh = lane >> 3, d0 = 16 * (lane & 7);
    float qf[16];
    {
        const bool ok = gh < G;
        const uint16_t *qp = a.q + ((size_t)b * a.Hq + (size_t)h * G + (ok ? gh : 0)) * kHD + d0;
        const uint4 z4 = {0, 0, 0, 0};
        const uint4 q0 = ok ? *reinterpret_cast<const uint4 *>(qp) : z4;
        const uint4 q1 = ok ? *reinterpret_cast<const uint4 *>(qp + 8) : z4;
        const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qf[2 * i] = bf16_lo_half(qw[i]) * sc2;
            qf[2 * i + 1] = bf16_hi_half(qw[i]) * sc2;
        }
    }

    int nq = __builtin_amdgcn_readfirstlane(a.n_quant[u]);
    if (nq < 0 || nq > a.max_quant || (nq % kKivGroup) != 0) {
        if (s == 0 && tid == 0 && a.flags) atomicOr(a.flags, KVC_FLAG_BAD_COUNT);
        nq = nq < 0 ? 0 : (nq > a.max_quant ? a.max_quant : nq) / kKivGroup * kKivGroup;
    }
    const int ngr = nq / kKivGroup;
    const int cg = (ngr + ns - 1) / ns;
    const int g0 = min(s * cg, ngr), g1 = min(ngr, g0 + cg);
    const size_t ubase = (size_t)u * a.max_quant;
    const size_t gbase = (size_t)u * (a.max_quant / kKivGroup);
    const KivMagic km;
    const uint32_t neg_lo = bf16_pair_reg(kBfNegLo), neg_hi = bf16_pair_reg(kBfNegHi);
    const uint32_t neg_both = bf16_pair_reg(kBfNegBoth);

    f32x4_t oacc[8];
#pragma unroll
    for (int m8 = 0; m8 < 8; ++m8) oacc[m8] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t cacc = {0.f, 0.f, 0.f, 0.f};   // sum_j p_j x_j for the columns of the V grids
    float lsum = 0.f;                        // A-layout lanes: head ga
    // C-layout rows' heads 4 (r & 1) + ii: reference maxima and their thresholds
    float mref[4] = {kKivNoMax, kKivNoMax, kKivNoMax, kKivNoMax};
    float thr[4] = {kKivNoMax, kKivNoMax, kKivNoMax, kKivNoMax};
    // this lane's column of the V-grid product: n < 8 the lo of grid n & 3,
    // n >= 8 the 128x scale; n & 4 selects the low bf16 part
    const int vcol = (col & 8) ? (col & 3) : kKivVG + (col & 3);
    const bool vlow = (col & 4) != 0;
    // selectors of bf16_part2: P rows 8..15 and the low columns of the V-grid B
    const uint32_t pa0 = hi_lane ? 0u : kBfNegLo, pa1 = hi_lane ? 0u : kBfNegHi;
    const uint32_t pb0 = vlow ? kBfNegLo : 0u, pb1 = vlow ? kBfNegHi : 0u;

    // the group's data for this lane: K codes of both tiles (16 B of key
    // 16 tt + col), V codes (the lane's 16 B of each tile: dims col + 16 m of
    // keys 16 tt + 4 e + r), 16 B of the K grids and of the V grids
    struct GroupData {
        uint4 kc[2];
        uint4 vz[2];
        float4 kgr, vgr;
    };
    auto gload = [&](int g, GroupData &d) {
        const size_t tok = ubase + (size_t)g * kKivGroup;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            d.kc[tt] = kiv_load(reinterpret_cast<const uint4 *>(a.k_codes + (tok + 16 * tt + col) * kKivRow + 16 * r));
            d.vz[tt] = kiv_load(reinterpret_cast<const uint4 *>(a.v_codes + (tok + 16 * tt) * kKivRow +
                                                                 16 * (16 * r + col)));
        }
        // K grids: lanes 0..31 the scales (4 each), 32..63 the lo
        const float *kgsrc = (lane < 32 ? a.k_scale : a.k_lo) + (gbase + g) * kHD + 4 * (lane & 31);
        d.kgr = kiv_load(reinterpret_cast<const float4 *>(kgsrc));
        // V grids: lanes 0..31 token lane's scales, 32..63 its lo
        const float *vgsrc = (lane < 32 ? a.v_scale : a.v_lo) + (tok + (lane & 31)) * kKivVG;
        d.vgr = kiv_load(reinterpret_cast<const float4 *>(vgsrc));
    };

    // Reference maxima: lm[ii] is the lane's largest logit of row ii in the
    // current keys.  When one passes its threshold anywhere in the wave, every
    // row takes its exact maximum so far and the sums are rescaled.
    auto update_max = [&](const float (&lm)[4]) {
        bool over = false;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) over |= lm[ii] > thr[ii];
        if (__builtin_amdgcn_ballot_w64(over) == 0) return;
        float alpha[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            float m = lm[ii];
            m = fmaxf(m, lane_xor_f<8>(m));
            m = fmaxf(m, lane_xor_f<4>(m));
            m = fmaxf(m, lane_xor_f<2>(m));
            m = fmaxf(m, lane_xor_f<1>(m));
            const float mnew = fmaxf(mref[ii], m);
            alpha[ii] = __builtin_amdgcn_exp2f(mref[ii] - mnew);
            mref[ii] = mnew;
            thr[ii] = mnew + kKivLazy;
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
            for (int m8 = 0; m8 < 8; ++m8) oacc[m8][ii] *= alpha[ii];
            cacc[ii] *= alpha[ii];
        }
        if (r < 2 && col == 0)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) al[4 * r + ii] = alpha[ii];
        __builtin_amdgcn_wave_barrier();
        lsum *= al[ga];
    };

#pragma unroll 1
    for (int gi = g0 + w; gi < g1; gi += kFWaves) {
        GroupData cur;
        gload(gi, cur);
        // ---- the group's grids into the wave's LDS (scales x 128)
        {
            const float m = lane < 32 ? 128.f : 1.f;
            const float4 kv = {cur.kgr.x * m, cur.kgr.y * m, cur.kgr.z * m, cur.kgr.w * m};
            *reinterpret_cast<float4 *>(kg + (lane < 32 ? 0 : kHD) + 4 * (lane & 31)) = kv;
            const float4 vv = {cur.vgr.x * m, cur.vgr.y * m, cur.vgr.z * m, cur.vgr.w * m};
            *reinterpret_cast<float4 *>(vg + (lane & 31) * 2 * kKivVG + (lane < 32 ? 0 : kKivVG)) = vv;
        }
        __builtin_amdgcn_wave_barrier();
        // ---- A = 128 q_d s_gd of this lane's 16 (head, dim), high and low
        // parts into the A tile; the head's constant sum_d q_d lo_gd - sum_d A_d
        float cst = 0.f;
        {
            uint32_t hw[8], lw[8];
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const float2 s2 = *reinterpret_cast<const float2 *>(kg + d0 + j);
                const float2 l2 = *reinterpret_cast<const float2 *>(kg + kHD + d0 + j);
                const float a0 = qf[j] * s2.x, a1 = qf[j + 1] * s2.y;
                const uint32_t hp = bf16_pack2(a0, a1);
                const uint32_t lp = bf16_pack2(dot2_bf16(hp, neg_lo, a0), dot2_bf16(hp, neg_hi, a1));
                hw[j / 2] = hp;
                lw[j / 2] = lp;
                cst = fmaf(qf[j], l2.x, cst);
                cst = fmaf(qf[j + 1], l2.y, cst);
                cst = dot2_bf16(hp, neg_both, cst);
                cst = dot2_bf16(lp, neg_both, cst);
            }
            uint4 *ah = reinterpret_cast<uint4 *>(ast + gh * kKivAS + d0);
            uint4 *alo = reinterpret_cast<uint4 *>(ast + gh * kKivAS + kHD + d0);
            ah[0] = uint4{hw[0], hw[1], hw[2], hw[3]};
            ah[1] = uint4{hw[4], hw[5], hw[6], hw[7]};
            alo[0] = uint4{lw[0], lw[1], lw[2], lw[3]};
            alo[1] = uint4{lw[4], lw[5], lw[6], lw[7]};
        }
        cst += lane_xor_f<1>(cst);
        cst += lane_xor_f<2>(cst);
        cst += lane_xor_f<4>(cst);   // lanes 8 gh .. 8 gh + 7: head gh's constant
        if ((lane & 7) == 0) csb[gh] = gh < G ? cst : -INFINITY;
        __builtin_amdgcn_wave_barrier();
        // ---- base-2 logits of the group's 32 keys (C layout: rows 4 (r & 1) + ii)
        float z[2][4];
        {
            const f32x4_t c0 = *reinterpret_cast<const f32x4_t *>(csb + 4 * (r & 1));
            f32x4_t acc[2] = {c0, c0};
            const uint16_t *arow = ast + ga * kKivAS + 8 * r;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const u16x8_t ahi = *reinterpret_cast<const u16x8_t *>(arow + 32 * c4);
                const u16x8_t alo = *reinterpret_cast<const u16x8_t *>(arow + kHD + 32 * c4);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const uint4 kc = cur.kc[tt];
                    const u16x8_t kop = kiv_widen8(c4 == 0 ? kc.x : c4 == 1 ? kc.y : c4 == 2 ? kc.z : kc.w, km);
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ahi), as_bf16x8(kop),
                                                                      acc[tt], 0, 0, 0);
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(alo), as_bf16x8(kop),
                                                                      acc[tt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) z[tt][ii] = acc[tt][ii];
        }
        {
            float lm[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) lm[ii] = fmaxf(z[0][ii], z[1][ii]);
            update_max(lm);
        }
        // ---- the weights 2^(z - reference) into the P tile (heads past G: 0)
        if (r < 2) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int g = 4 * r + ii;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    // key col of tile tt at column lg_col(16 tt + col)
                    const int jc = 16 * tt + (((col & 3) << 2) | (col >> 2));
                    pt[g * kKivPL + jc] = __builtin_amdgcn_exp2f(z[tt][ii] - mref[ii]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        // ---- P.V of the two tiles
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const f32x4_t p = *reinterpret_cast<const f32x4_t *>(pt + ga * kKivPL + 16 * tt + 4 * r);
            lsum += (p[0] + p[1]) + (p[2] + p[3]);   // read from the rows 0..7 lanes
            const s16x4_t ap = __builtin_bit_cast(
                s16x4_t, uint2{bf16_part2(p[0], p[1], pa0, pa1), bf16_part2(p[2], p[3], pa0, pa1)});
            const uint32_t za = cur.vz[tt].x, zb = cur.vz[tt].y, zc = cur.vz[tt].z, zd = cur.vz[tt].w;
            const uint2 bw[8] = {{kiv_pair<0>(za, km), kiv_pair<0>(zc, km)}, {kiv_pair<0>(zb, km), kiv_pair<0>(zd, km)},
                                 {kiv_pair<1>(za, km), kiv_pair<1>(zc, km)}, {kiv_pair<1>(zb, km), kiv_pair<1>(zd, km)},
                                 {kiv_pair<2>(za, km), kiv_pair<2>(zc, km)}, {kiv_pair<2>(zb, km), kiv_pair<2>(zd, km)},
                                 {kiv_pair<3>(za, km), kiv_pair<3>(zc, km)}, {kiv_pair<3>(zb, km), kiv_pair<3>(zd, km)}};
            float4 sv[4];
            float bx[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float *vgk = vg + (16 * tt + 4 * e + r) * 2 * kKivVG;
                sv[e] = *reinterpret_cast<const float4 *>(vgk);
                bx[e] = vgk[vcol];
            }
            uint32_t avw[kKivVG][2];
#pragma unroll
            for (int c = 0; c < kKivVG; ++c) {
#pragma unroll
                for (int hpair = 0; hpair < 2; ++hpair) {
                    const int e0 = 2 * hpair;
                    avw[c][hpair] = bf16_part2(p[e0] * sv[e0][c], p[e0 + 1] * sv[e0 + 1][c], pa0, pa1);
                }
            }
            const s16x4_t bc = __builtin_bit_cast(
                s16x4_t, uint2{bf16_part2(bx[0], bx[1], pb0, pb1), bf16_part2(bx[2], bx[3], pb0, pb1)});
            cacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ap, bc, cacc, 0, 0, 0);
#pragma unroll
            for (int m8 = 0; m8 < 8; ++m8)
                oacc[m8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(s16x4_t, uint2{avw[m8 >> 1][0], avw[m8 >> 1][1]}),
                    __builtin_bit_cast(s16x4_t, bw[m8]), oacc[m8], 0, 0, 0);
        }
    }

    // ---------------- the residual and the new token (the unit's last share):
    // bf16 rows in 16-key tiles, tile t to wave t % 4, on the same running
    // softmax.  Keys 0 .. nr-1 are the residual rows, key nr the new token,
    // later keys of the last tile weigh nothing.  K products: A = the query
    // rows as given (bf16 x bf16 products are exact), B = the K rows (lane:
    // dims 32 c4 + 8 r .. of key 16 t + col).  P.V: B of MFMA m8 is element
    // m8 of the four V rows the lane holds (keys 16 t + 4 e + r); the
    // residual's element order puts dim 16 m8 + col there, the column of the
    // quantized products.
    if (s == ns - 1) {
        int nr = __builtin_amdgcn_readfirstlane(a.n_res[u]);
        if (nr < 0 || nr > kKivResidual) {
            if (tid == 0 && a.flags) atomicOr(a.flags, KVC_FLAG_BAD_COUNT);
            nr = nr < 0 ? 0 : kKivResidual;
        }
        const int ntile = (nr + 16) / 16;   // nr + 1 keys
        if (w < ntile) {
            u16x8_t qa[4];
            {
                const bool ok = ga < G;
                const uint16_t *qp = a.q + ((size_t)b * a.Hq + (size_t)h * G + (ok ? ga : 0)) * kHD + 8 * r;
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    qa[c4] = ok ? *reinterpret_cast<const u16x8_t *>(qp + 32 * c4)
                                : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
            }
            // rows past nr read as zeros
            const uint32_t rbytes = (uint32_t)nr * kHD * 2;
            const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k_res + (size_t)u * kKivResidual * kHD, rbytes);
            const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v_res + (size_t)u * kKivResidual * kHD, rbytes);
            const uint16_t *kn = a.k_new + ((size_t)b * a.Hkv + h) * kHD;
            const uint16_t *vn = a.v_new + ((size_t)b * a.Hkv + h) * kHD;
#pragma unroll 1
            for (int t = w; t < ntile; t += kFWaves) {
                const int key = 16 * t + col;
                u16x8_t kr[4], vr[4];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    kr[c4] = buffer_row<false, false>(krs, key * (2 * kHD) + 64 * c4 + 16 * r);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vr[e] = buffer_row<false, false>(vrs, (16 * t + 4 * e + r) * (2 * kHD) + 16 * col);
                if (key == nr)
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4)
                        kr[c4] = *reinterpret_cast<const u16x8_t *>(kn + 32 * c4 + 8 * r);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * t + 4 * e + r == nr) vr[e] = __builtin_bit_cast(u16x8_t, kiv_vres_chunk(vn, col));
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[c4]), as_bf16x8(kr[c4]),
                                                                  acc, 0, 0, 0);
                const float kb = key <= nr ? 0.f : -INFINITY;
                float zt[4];   // rows of heads past G and keys past nr: -inf
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    zt[ii] = fmaf(acc[ii], sc2, 4 * (r & 1) + ii < G ? kb : -INFINITY);
                update_max(zt);
                if (r < 2)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        pt[(4 * r + ii) * kKivPL + (((col & 3) << 2) | (col >> 2))] =
                            __builtin_amdgcn_exp2f(zt[ii] - mref[ii]);
                __builtin_amdgcn_wave_barrier();
                const f32x4_t p = *reinterpret_cast<const f32x4_t *>(pt + ga * kKivPL + 4 * r);
                lsum += (p[0] + p[1]) + (p[2] + p[3]);
                const s16x4_t ap = __builtin_bit_cast(
                    s16x4_t, uint2{bf16_part2(p[0], p[1], pa0, pa1), bf16_part2(p[2], p[3], pa0, pa1)});
#pragma unroll
                for (int m8 = 0; m8 < 8; ++m8)
                    oacc[m8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        ap, s16x4_t{(short)vr[0][m8], (short)vr[1][m8], (short)vr[2][m8], (short)vr[3][m8]},
                        oacc[m8], 0, 0, 0);
            }
        }
    }

    // ---------------- merge the four waves: the output (one share per unit)
    // or the share's partial (o, m, l)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
        for (int m8 = 0; m8 < 8; ++m8) oacc[m8][ii] += __shfl_xor(oacc[m8][ii], 32, 64);
        cacc[ii] += __shfl_xor(cacc[ii], 32, 64);
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    float cv[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        float v = (col & 8) ? -cacc[ii] : cacc[ii];
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 8, 64);
        cv[ii] = v;
    }
    if (r < 2 && col == 0)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            if (4 * r + ii < G) sm.m[w][4 * r + ii] = mref[ii];
    if (lane < G) sm.l[w][lane] = lsum;
    __syncthreads();   // every wave is done with its LDS: partial P.V of the waves go there
    float *opart = reinterpret_cast<float *>(smem);   // [waves][G][kHD] (G <= 8: 16 KB)
    if (r < 2) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int g = 4 * r + ii;
            if (g < G) {
#pragma unroll
                for (int m8 = 0; m8 < 8; ++m8)
                    opart[((size_t)w * G + g) * kHD + 16 * m8 + col] = oacc[m8][ii];
                if (col < kKivVG) sm.corr[w][g][col] = cv[ii];
            }
        }
    }
    __syncthreads();
    const bool direct = ns == 1;
    if (tid < G) {
        float M = kKivNoMax;
        for (int v = 0; v < kFWaves; ++v) M = fmaxf(M, sm.m[v][tid]);
        float l = 0.f;
        for (int v = 0; v < kFWaves; ++v) l += __builtin_amdgcn_exp2f(sm.m[v][tid] - M) * sm.l[v][tid];
        sm.M[tid] = M;
        sm.il[tid] = 1.f / l;
        if (!direct) {
            // the partial's maximum goes out in natural-log units
            float *pp = a.part_q + ((size_t)u * ns + s) * G * (kHD + 2);
            pp[tid * (kHD + 2) + kHD] = M * 0.69314718055994530942f;
            pp[tid * (kHD + 2) + kHD + 1] = l;
        }
    }
    __syncthreads();
    for (int e = tid; e < G * kHD; e += kFThreads) {
        const int g = e / kHD, d = e % kHD;
        const float M = sm.M[g];
        float o = 0.f;
        for (int v = 0; v < kFWaves; ++v) {
            const float f = __builtin_amdgcn_exp2f(sm.m[v][g] - M);
            o += f * (opart[((size_t)v * G + g) * kHD + d] + sm.corr[v][g][d / 32]);
        }
        if (direct) a.out[((size_t)b * a.Hq + (size_t)h * G + g) * kHD + d] = o * sm.il[g];
        else a.part_q[(((size_t)u * ns + s) * G + g) * (kHD + 2) + d] = o;
    }
    if (direct) {
        __syncthreads();   // the wave partials are read: the LDS serves the conversion
        kivi_cache_update(a, u, *reinterpret_cast<KivQuantLds *>(smem));
    }
}

// ---------------------------------------------------------------------------
// several shares per unit: combine their partials, then the cache update;
// one workgroup per unit
// ---------------------------------------------------------------------------
struct KivUpdLds {
    float fac[kMaxSplit][kMaxGroup];
    float ms[kMaxSplit][kMaxGroup], ls[kMaxSplit][kMaxGroup];
    KivQuantLds q;
};

__global__ __launch_bounds__(256) void kivi_update_kernel(KiviArgs a) {
    __shared__ KivUpdLds L;
    const int u = blockIdx.x, b = u / a.Hkv, h = u % a.Hkv;
    const int tid = threadIdx.x;
    const int G = a.G, ns = a.nsq;
    auto part = [&](int s) -> const float * { return a.part_q + ((size_t)u * ns + s) * G * (kHD + 2); };
    for (int i = tid; i < ns * G; i += blockDim.x) {
        const int s = i / G, g = i % G;
        L.ms[s][g] = part(s)[g * (kHD + 2) + kHD];
        L.ls[s][g] = part(s)[g * (kHD + 2) + kHD + 1];
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, L.ms[s][tid]);
        float S = 0.f;
        for (int s = 0; s < ns; ++s) S += L.ls[s][tid] * __expf(L.ms[s][tid] - M);
        for (int s = 0; s < ns; ++s) L.fac[s][tid] = __expf(L.ms[s][tid] - M) / S;
    }
    __syncthreads();
    for (int e = tid; e < G * kHD; e += blockDim.x) {
        const int g = e / kHD, d = e % kHD;
        float o = 0.f;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) o += part(s)[g * (kHD + 2) + d] * L.fac[s][g];
        a.out[((size_t)b * a.Hq + (size_t)h * G + g) * kHD + d] = o;
    }
    kivi_cache_update(a, u, L.q);
}

// ---------------------------------------------------------------------------
hipError_t launch_kivi_prefill(const KiviArgs &a, hipStream_t s) {
    const int over = a.max_len > kKivResidual ? a.max_len - kKivResidual : 0;
    const int ngr = (over + kKivGroup - 1) / kKivGroup;
    hipLaunchKernelGGL(kivi_prefill_kernel, dim3(a.B * a.Hkv, ngr + 1), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kivi_decode(const KiviArgs &a, hipStream_t s) {
    const int units = a.B * a.Hkv;
    if (a.nsq < 1 || a.nsq > kMaxSplit) return hipErrorInvalidValue;
    static hipError_t attr = hipFuncSetAttribute((const void *)kivi_qattn_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)kivi_qattn_smem(kMaxGroup));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kivi_qattn_kernel, dim3(units * a.nsq), dim3(kFThreads),
                       kivi_qattn_smem(a.G), s, a);
    if (a.nsq > 1) hipLaunchKernelGGL(kivi_update_kernel, dim3(units), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvc
