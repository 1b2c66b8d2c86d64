// kivi.hip -- a KIVI-style quantized KV cache on the matrix cores of gfx950:
// every token kept, the old ones as 4-bit codes on per-channel K grids and
// per-token V grids, the newest in a bf16 residual (KV cache compression
// guide, section 2: group 32 and residual 128; section 16, "KV capacity
// formula", "the four methods" and "limits").  The grids, the layout and the
// step are the ones kvc.h states.
//
// Attention over the quantized tokens (kivi_qattn_kernel), one workgroup per
// (unit, share of its groups):
//  * K of group g, channel d: k = c * s_gd + lo_gd, so
//        q . k_j = sum_d (q_d s_gd) c_jd + sum_d q_d lo_gd.
//    The scale folds into the query: A = 16 q_d s_gd as a bf16 high part in
//    rows 0..7 and the bf16 rounding of the rest in rows 8..15; a code enters
//    B exactly as the bf16 value 1 + c/16 (bits 0x3F80 | c << 3).  The
//    product is then sum_d A_d + sum_d (A_d / 16) c_jd, and the first sum with
//    the lo term is one constant per (group, head) added to the group's logits.
//  * V of token j, channel group c (32 channels): v = code * s_jc + lo_jc.  In
//    the P.V tile MFMA m covers dims 16m .. 16m + 15, inside one channel
//    group, so the token scale folds into P: A = 16 p_j s_jc (high / low
//    rows), B the codes as above, and sum_j (p_j lo_jc - A_j) is added per
//    (head, channel group) at the end.
//  * the logits of up to 512 tokens stay in LDS; a longer share runs in pieces
//    of 512 with the running maximum rescaling the partial sums.
// The residual and the new token go through split_kernel (bf16, attend
// only).  kivi_update_kernel merges the partials, turns a full residual's 32
// oldest tokens into a group, and appends the new token; kivi_prefill_kernel
// quantizes a prompt.  The quantizer takes every decision in binary32.
#include "mfma_tiles.h"

namespace kvc {

constexpr int kKivRow = kHD / 2;                     // bytes of one token's 4-bit codes
constexpr int kKivSub = 16;                          // groups per LDS piece
constexpr int kKivSubT = kKivSub * kKivGroup;        // 512 tokens
constexpr int kKivLD = kKivSubT + 4;
constexpr int kKivVG = kHD / 32;                     // V grids per token

// Two codes of one dword -> two bf16 values 1 + c/16.  A dword holds eight
// codes, slots 0..3 (bits 0..15) the even elements and slots 4..7 the odd
// ones, so pair J (elements 2J and 2J + 1) sits at bits 4J and 16 + 4J.
template <int J>
__device__ inline uint32_t kiv_pair(uint32_t x) {
    if constexpr (J == 0) return ((x << 3) & 0x00780078u) | 0x3F803F80u;
    else return ((x >> (4 * J - 3)) & 0x00780078u) | 0x3F803F80u;
}
__device__ inline u16x8_t kiv_widen8(uint32_t x) {
    return __builtin_bit_cast(u16x8_t, uint4{kiv_pair<0>(x), kiv_pair<1>(x), kiv_pair<2>(x),
                                             kiv_pair<3>(x)});
}

// Quantize one group of kKivGroup tokens, K rows Kr and V rows Vr (bf16,
// consecutive rows of kHD), into group slot g of unit u.  256 threads: the
// first 128 take one K channel each, the others one (token, channel group)
// of V; codes go through LDS to be packed into the layout.
struct KivQuantLds {
    uint8_t kc[kKivGroup][kHD], vc[kKivGroup][kHD];
};

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
            x[j] = __uint_as_float((uint32_t)Vr[(size_t)i * kHD + 32 * c + j] << 16);
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
    // pack: 32 tokens x 16 dwords for K, then for V
    for (int idx = tid; idx < 2 * kKivGroup * 16; idx += blockDim.x) {
        const bool isv = idx >= kKivGroup * 16;
        const int rem = idx % (kKivGroup * 16);
        const int i = rem / 16, wd = rem % 16;
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = (k < 4) ? 2 * k : 2 * (k - 4) + 1;
            // K: dword wd = 4 * ((d % 32) / 8) + d / 32, element d % 8;
            // V: dword d % 16, element d / 16
            const int d = isv ? 16 * e + wd : 32 * (wd % 4) + 8 * (wd / 4) + e;
            const uint32_t cq = isv ? L.vc[i][d] : L.kc[i][d];
            word |= cq << (4 * k);
        }
        uint8_t *dst = (isv ? a.v_codes : a.k_codes) + (tok0 + i) * kKivRow + 4 * wd;
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
        kivi_quantize_group(a, u, y, K + (size_t)y * kKivGroup * kHD,
                            V + (size_t)y * kKivGroup * kHD, L);
        return;
    }
    const int nr = len - nq;
    const uint4 *ks = reinterpret_cast<const uint4 *>(K + (size_t)nq * kHD);
    const uint4 *vs = reinterpret_cast<const uint4 *>(V + (size_t)nq * kHD);
    uint4 *kd = reinterpret_cast<uint4 *>(a.k_res + (size_t)u * kKivResidual * kHD);
    uint4 *vd = reinterpret_cast<uint4 *>(a.v_res + (size_t)u * kKivResidual * kHD);
    for (int i = threadIdx.x; i < nr * (kHD / 8); i += blockDim.x) {
        kd[i] = ks[i];
        vd[i] = vs[i];
    }
    if (threadIdx.x == 0) {
        a.n_quant[u] = nq;
        a.n_res[u] = nr;
    }
}

// ---------------------------------------------------------------------------
// attention over the quantized tokens
// ---------------------------------------------------------------------------
struct KivSmall {
    float mrun[kMaxGroup];                   // running max per head
    float alpha[kMaxGroup];                  // rescale of the running sums at a new piece
    float wred[kFWaves][kMaxGroup];
    float corr[kFWaves][kMaxGroup][kKivVG];
};

__host__ __device__ constexpr size_t kivi_qattn_smem(int G) {
    return (size_t)G * kKivLD * 4 + (size_t)kKivSub * 2 * kHD * 4 +
           (size_t)kKivSubT * 2 * kKivVG * 4 + sizeof(KivSmall);
}

__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(3)))
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
    const bool arow = ga < G;
    const bool hi_lane = col < 8;

    float *lg = reinterpret_cast<float *>(smem);             // [G][kKivLD] logits of a piece
    float *kgr = lg + G * kKivLD;                             // [group][scale | lo][kHD]
    float *vgr = kgr + kKivSub * 2 * kHD;                     // [token][4 scales, 4 lo]
    KivSmall &sm = *reinterpret_cast<KivSmall *>(vgr + kKivSubT * 2 * kKivVG);

    // this lane's query: dims 32 c4 + 8 r + e of head ga (16x16x32 A layout)
    u16x8_t qa[4];
    load_q(qa, a.q + ((size_t)b * a.Hq + (size_t)h * G + (arow ? ga : 0)) * kHD, arow, r);

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

    if (tid < G) sm.mrun[tid] = -INFINITY;
    f32x4_t oacc[8];
#pragma unroll
    for (int m8 = 0; m8 < 8; ++m8) oacc[m8] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    float corr[kKivVG] = {0.f, 0.f, 0.f, 0.f};

    for (int gs = g0; gs < g1; gs += kKivSub) {
        const int ng = min(kKivSub, g1 - gs);
        __syncthreads();   // the previous piece is done with the LDS
        for (int i = tid; i < ng * kHD; i += kFThreads) {
            const int gi = i / kHD, d = i % kHD;
            kgr[gi * 2 * kHD + d] = a.k_scale[(gbase + gs + gi) * kHD + d];
            kgr[gi * 2 * kHD + kHD + d] = a.k_lo[(gbase + gs + gi) * kHD + d];
        }
        for (int i = tid; i < ng * kKivGroup * kKivVG; i += kFThreads) {
            const int t = i / kKivVG, c = i % kKivVG;
            const size_t src = (ubase + (size_t)gs * kKivGroup + t) * kKivVG + c;
            vgr[t * 2 * kKivVG + c] = a.v_scale[src];
            vgr[t * 2 * kKivVG + kKivVG + c] = a.v_lo[src];
        }
        __syncthreads();

        // ---------------- logits: wave w takes groups w, w + 4, w + 8, w + 12
        float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll 1
        for (int i = 0; i < kKivSub / kFWaves; ++i) {
            const int gi = w + kFWaves * i;
            if (gi >= ng) break;   // wave-uniform
            u16x8_t aop[4];
            float cst = 0.f;
            const float *sg = kgr + gi * 2 * kHD;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const int d0 = 32 * c4 + 8 * r;
                const float4 s0 = *reinterpret_cast<const float4 *>(sg + d0);
                const float4 s1 = *reinterpret_cast<const float4 *>(sg + d0 + 4);
                const float4 l0 = *reinterpret_cast<const float4 *>(sg + kHD + d0);
                const float4 l1 = *reinterpret_cast<const float4 *>(sg + kHD + d0 + 4);
                const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float qd = bf16_value((short)qa[c4][e]);
                    const float av = 16.f * (qd * sv[e]);
                    const short hb = bf16_bits(av);
                    const short lb = bf16_bits(av - bf16_value(hb));
                    aop[c4][e] = (uint16_t)(hi_lane ? hb : lb);
                    cst += qd * lv[e] - (bf16_value(hb) + bf16_value(lb));
                }
            }
            cst += __shfl_xor(cst, 16, 64);
            cst += __shfl_xor(cst, 32, 64);   // the head's constant, in every lane of its row
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const size_t tok = ubase + (size_t)(gs + gi) * kKivGroup + 16 * tt + col;
                const uint4 kc = *reinterpret_cast<const uint4 *>(a.k_codes + tok * kKivRow + 16 * r);
                const u16x8_t kop[4] = {kiv_widen8(kc.x), kiv_widen8(kc.y), kiv_widen8(kc.z),
                                        kiv_widen8(kc.w)};
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aop[c4]),
                                                                  as_bf16x8(kop[c4]), acc, 0, 0, 0);
                const int jc = 32 * gi + 16 * tt + (((col & 3) << 2) | (col >> 2));
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int g = 4 * (r & 1) + ii;   // rows g and g + 8 hold its two parts
                    const float tot = acc[ii] + __shfl_xor(acc[ii], 32, 64);
                    const float z = (tot + __shfl(cst, g, 64)) * a.scale;
                    if (r < 2 && g < G) lg[g * kKivLD + jc] = z;
                    mx[ii] = fmaxf(mx[ii], g < G ? z : -INFINITY);
                }
            }
        }
        // new running maximum of each head and the rescale of the old sums
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            float m = mx[ii];
            m = fmaxf(m, __shfl_xor(m, 8, 64));
            m = fmaxf(m, __shfl_xor(m, 4, 64));
            m = fmaxf(m, __shfl_xor(m, 2, 64));
            m = fmaxf(m, __shfl_xor(m, 1, 64));
            if (col == 0 && r < 2 && 4 * r + ii < G) sm.wred[w][4 * r + ii] = m;
        }
        __syncthreads();
        if (tid < G) {
            float m = sm.wred[0][tid];
            for (int v = 1; v < kFWaves; ++v) m = fmaxf(m, sm.wred[v][tid]);
            // a wave without groups in this piece left -inf
            const float mold = sm.mrun[tid];
            const float mnew = fmaxf(mold, m);
            sm.alpha[tid] = (mold == -INFINITY) ? 0.f : __expf(mold - mnew);
            sm.mrun[tid] = mnew;
        }
        __syncthreads();
#pragma unroll
        for (int m8 = 0; m8 < 8; ++m8)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int g = (4 * r + ii) & 7;
                oacc[m8][ii] *= (g < G) ? sm.alpha[g] : 0.f;
            }
        const float al = arow ? sm.alpha[ga] : 0.f;
        lsum *= al;
#pragma unroll
        for (int c = 0; c < kKivVG; ++c) corr[c] *= al;
        const float mrow = arow ? sm.mrun[ga] : 0.f;
        const float *lrow = lg + (arow ? ga : 0) * kKivLD;

        // ---------------- P.V over the same groups' tiles
#pragma unroll 1
        for (int i = 0; i < kKivSub / kFWaves; ++i) {
            const int gi = w + kFWaves * i;
            if (gi >= ng) break;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int t = 2 * gi + tt;                       // tile of the piece
                const f32x4_t z = *reinterpret_cast<const f32x4_t *>(lrow + 16 * t + 4 * r);
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) p[e] = arow ? __expf(z[e] - mrow) : 0.f;
                if (hi_lane) lsum += (p[0] + p[1]) + (p[2] + p[3]);
                // codes: dword col of keys 16t + 4e + r
                const size_t tok0 = ubase + (size_t)gs * kKivGroup + 16 * t + r;
                uint32_t x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[e] = *reinterpret_cast<const uint32_t *>(a.v_codes + (tok0 + 4 * e) * kKivRow +
                                                               4 * col);
                const uint32_t za = (x[0] & 0xFFFFu) | (x[1] << 16), zb = (x[0] >> 16) | (x[1] & 0xFFFF0000u);
                const uint32_t zc = (x[2] & 0xFFFFu) | (x[3] << 16), zd = (x[2] >> 16) | (x[3] & 0xFFFF0000u);
                const uint2 bw[8] = {{kiv_pair<0>(za), kiv_pair<0>(zc)}, {kiv_pair<0>(zb), kiv_pair<0>(zd)},
                                     {kiv_pair<1>(za), kiv_pair<1>(zc)}, {kiv_pair<1>(zb), kiv_pair<1>(zd)},
                                     {kiv_pair<2>(za), kiv_pair<2>(zc)}, {kiv_pair<2>(zb), kiv_pair<2>(zd)},
                                     {kiv_pair<3>(za), kiv_pair<3>(zc)}, {kiv_pair<3>(zb), kiv_pair<3>(zd)}};
                // A per channel group c: 16 p_e s_{key e, c}, high / low part
                s16x4_t av[kKivVG];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float *vg = vgr + (16 * t + 4 * e + r) * 2 * kKivVG;
                    const float4 sv = *reinterpret_cast<const float4 *>(vg);
                    const float4 lv = *reinterpret_cast<const float4 *>(vg + kKivVG);
                    const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
                    const float lvv[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
                    for (int c = 0; c < kKivVG; ++c) {
                        const float aa = 16.f * (p[e] * svv[c]);
                        const short hb = bf16_bits(aa);
                        const short lb = bf16_bits(aa - bf16_value(hb));
                        av[c][e] = hi_lane ? hb : lb;
                        corr[c] += p[e] * lvv[c] - (bf16_value(hb) + bf16_value(lb));
                    }
                }
#pragma unroll
                for (int m8 = 0; m8 < 8; ++m8)
                    oacc[m8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        av[m8 >> 1], __builtin_bit_cast(s16x4_t, bw[m8]), oacc[m8], 0, 0, 0);
            }
        }
    }

    // ---------------- the split's partial (o, m, l)
#pragma unroll
    for (int m8 = 0; m8 < 8; ++m8)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) oacc[m8][ii] += __shfl_xor(oacc[m8][ii], 32, 64);
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
    for (int c = 0; c < kKivVG; ++c) {
        corr[c] += __shfl_xor(corr[c], 16, 64);
        corr[c] += __shfl_xor(corr[c], 32, 64);
    }
    __syncthreads();   // the LDS grids are free: partial P.V of the waves go there
    float *opart = kgr;   // [waves][G][kHD] (G <= 8: 16 KB)
    if (r < 2)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int g = 4 * r + ii;
            if (g < G)
#pragma unroll
                for (int m8 = 0; m8 < 8; ++m8) opart[((size_t)w * G + g) * kHD + 16 * m8 + col] = oacc[m8][ii];
        }
    if (lane < G) {
        sm.wred[w][lane] = lsum;
#pragma unroll
        for (int c = 0; c < kKivVG; ++c) sm.corr[w][lane][c] = corr[c];
    }
    __syncthreads();
    float *pp = a.part_q + ((size_t)u * ns + s) * G * (kHD + 2);
    for (int e = tid; e < G * kHD; e += kFThreads) {
        const int g = e / kHD, d = e % kHD;
        float o = 0.f;
        for (int v = 0; v < kFWaves; ++v) o += opart[((size_t)v * G + g) * kHD + d] + sm.corr[v][g][d / 32];
        pp[g * (kHD + 2) + d] = o;
    }
    if (tid < G) {
        float l = 0.f;
        for (int v = 0; v < kFWaves; ++v) l += sm.wred[v][tid];
        pp[tid * (kHD + 2) + kHD] = sm.mrun[tid];
        pp[tid * (kHD + 2) + kHD + 1] = l;
    }
}

// ---------------------------------------------------------------------------
// combine, residual conversion, append: one workgroup per unit
// ---------------------------------------------------------------------------
struct KivUpdLds {
    float fac[kMaxSplit + 1][kMaxGroup];
    float ms[kMaxSplit + 1][kMaxGroup], ls[kMaxSplit + 1][kMaxGroup];
    float lsum[kMaxGroup];
    KivQuantLds q;
};

__global__ __launch_bounds__(256) void kivi_update_kernel(KiviArgs a) {
    __shared__ KivUpdLds L;
    const int u = blockIdx.x, b = u / a.Hkv, h = u % a.Hkv;
    const int tid = threadIdx.x;
    const int G = a.G, ns = a.nsq, nt = ns + 1;   // split ns: residual + new token
    auto part = [&](int s) -> const float * {
        return s < ns ? a.part_q + ((size_t)u * ns + s) * G * (kHD + 2)
                      : a.part_r + (size_t)u * G * (kHD + 2);
    };
    for (int i = tid; i < nt * G; i += blockDim.x) {
        const int s = i / G, g = i % G;
        L.ms[s][g] = part(s)[g * (kHD + 2) + kHD];
        L.ls[s][g] = part(s)[g * (kHD + 2) + kHD + 1];
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int s = 0; s < nt; ++s) M = fmaxf(M, L.ms[s][tid]);
        float S = 0.f;
        for (int s = 0; s < nt; ++s)
            S += (L.ms[s][tid] == -INFINITY) ? 0.f : L.ls[s][tid] * __expf(L.ms[s][tid] - M);
        for (int s = 0; s < nt; ++s)
            L.fac[s][tid] = (L.ms[s][tid] == -INFINITY) ? 0.f : __expf(L.ms[s][tid] - M) / S;
    }
    __syncthreads();
    for (int e = tid; e < G * kHD; e += blockDim.x) {
        const int g = e / kHD, d = e % kHD;
        float o = 0.f;
#pragma unroll 8
        for (int s = 0; s < nt; ++s) o += part(s)[g * (kHD + 2) + d] * L.fac[s][g];
        a.out[((size_t)b * a.Hq + (size_t)h * G + g) * kHD + d] = o;
    }

    // ---- the cache update
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
        kivi_quantize_group(a, u, nq / kKivGroup, Kr, Vr, L.q);
        // rows 32..127 move down to 0..95: all reads before any write
        constexpr int kMove = (kKivResidual - kKivGroup) * (kHD / 8);   // uint4 per tensor
        constexpr int kPer = (kMove + 255) / 256;
        uint4 tk[kPer], tv[kPer];
        const uint4 *ks = reinterpret_cast<const uint4 *>(Kr + kKivGroup * kHD);
        const uint4 *vs = reinterpret_cast<const uint4 *>(Vr + kKivGroup * kHD);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = tid + 256 * k;
            if (i < kMove) {
                tk[k] = ks[i];
                tv[k] = vs[i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = tid + 256 * k;
            if (i < kMove) {
                reinterpret_cast<uint4 *>(Kr)[i] = tk[k];
                reinterpret_cast<uint4 *>(Vr)[i] = tv[k];
            }
        }
        nq += kKivGroup;
        nr -= kKivGroup;
    }
    if (tid < kHD / 8) {
        const size_t src = ((size_t)b * a.Hkv + h) * kHD;
        reinterpret_cast<uint4 *>(Kr + (size_t)nr * kHD)[tid] =
            reinterpret_cast<const uint4 *>(a.k_new + src)[tid];
        reinterpret_cast<uint4 *>(Vr + (size_t)nr * kHD)[tid] =
            reinterpret_cast<const uint4 *>(a.v_new + src)[tid];
    }
    if (tid == 0) {
        a.n_quant[u] = nq;
        a.n_res[u] = nr + 1;
    }
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
    if (a.nsq > 0) {
        static hipError_t attr = hipFuncSetAttribute((const void *)kivi_qattn_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)kivi_qattn_smem(kMaxGroup));
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(kivi_qattn_kernel, dim3(units * a.nsq), dim3(kFThreads),
                           kivi_qattn_smem(a.G), s, a);
    }
    // the residual and the new token: bf16 rows, attended only
    AttnArgs r;
    r.c.B = a.B;
    r.c.Hq = a.Hq;
    r.c.Hkv = a.Hkv;
    r.c.D = kHD;
    r.c.cap = kKivResidual;
    r.c.G = a.G;
    r.c.bs = 0;
    r.c.max_blocks = 0;
    r.c.num_blocks = 0;
    r.c.k = a.k_res;
    r.c.v = a.v_res;
    r.c.bt = nullptr;
    r.c.pos = nullptr;
    r.c.n_slots = a.n_res;
    r.c.flags = a.flags;
    r.new_pos = nullptr;
    r.q = a.q;
    r.k_new = a.k_new;
    r.v_new = a.v_new;
    r.out = nullptr;
    r.scores = nullptr;
    r.scale = a.scale;
    r.decay = 0.f;
    r.nsplit = 1;
    r.max_len = kKivResidual + 1;
    r.append = false;
    r.part = a.part_r;
    r.logits = nullptr;
    hipError_t e = launch_split(r, false, r.max_len, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kivi_update_kernel, dim3(units), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvc
