// fused.hip -- one whole decode step per unit (sequence b, kv head h) in one
// workgroup, on the matrix cores of gfx950.
//
// What a step computes (KV cache compression guide, section 16, "prefill,
// decode, TP" and "the 4 methods"; eviction-in-practice blog, "reference
// implementation"; online compaction study, section 4.2):
//   z_gj = scale * q_g . k_j over the n cached slots and the new token,
//   p = softmax_j(z), o_g = sum_j p_gj v_j,
//   H2O: s_j += sum_g p_gj (exact probabilities, final normaliser),
//   then the policy's kept set, then hole-fill compaction.
//
// Layout of the work (bf16 K/V, head_dim 128, G <= 16 query heads):
//  * QK^T runs as v_mfma_f32_16x16x32_bf16 with the group's queries as the A
//    operand (rows = query heads, padded to 16) and 16 keys as the B operand:
//    every lane loads 16 contiguous bytes of one key row straight from HBM
//    into its operand registers; bf16 x bf16 products are exact in fp32.
//  * the logits of the whole unit stay in LDS ([G][n+1] fp32), so the softmax
//    is exact (no online rescaling) and the H2O update uses the final
//    normaliser without a second pass over K.
//  * P.V runs as v_mfma_f32_16x16x4_f32 with fp32 probabilities (no bf16
//    rounding of P): each lane loads 16 contiguous bytes of a V row (4 rows x
//    256 B per wave instruction, fully coalesced) and feeds its 8 values to 8
//    MFMAs whose output columns are dims 8c+t.
//  * selection runs on the LDS copies of pos / scores / random keys; the
//    common steady-state case (exactly one eviction) is an arg-min, the
//    general case an 8-bit radix select over 64-bit (key, position) words.
//  * compaction pairs evicted slots below n_out with kept slots at or above
//    n_out; the new token is written straight into its final slot.
// Units longer than the launch's LDS capacity (or a full cache) take the
// generic per-unit routines inside the same workgroup, so results never
// depend on the length hint.
#include "generic.h"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

constexpr int kFThreads = 256;
constexpr int kFWaves = kFThreads / 64;
constexpr int kHD = 128;   // head_dim of the fast path
#ifndef KVC_DK
#define KVC_DK 3
#endif
#ifndef KVC_DV
#define KVC_DV 8
#endif
constexpr int kDK = KVC_DK;   // K tiles (16 keys x 256 B) in flight per wave
constexpr int kDV = KVC_DV;   // V groups (4 keys x 256 B) in flight per wave
#ifndef KVC_WAVES_PER_EU
#define KVC_WAVES_PER_EU 4
#endif
constexpr int kWavesPerEU = KVC_WAVES_PER_EU;   // 4 workgroups of 4 waves per CU

struct FusedSmall {
    float m[kMaxGroup];      // row maxima of the logits
    float l[kMaxGroup];      // softmax normalisers
    float il[kMaxGroup];     // 1 / l
    float wred[kFWaves][kMaxGroup];
    int hist[256];
    int red[kFWaves * 2];
    int pmax[kFWaves];       // newest position seen by each wave
    int posmax;
    int r_nc[kFWaves], r_nd[kFWaves], r_ds[kFWaves], r_arg[kFWaves];
    uint32_t mn_hi[kFWaves], mn_lo[kFWaves];
    int sh[8];
};

__device__ inline bf16x8_t as_bf16x8(u16x8_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ inline void load_q(u16x8_t (&qa)[4], const uint16_t *qp, bool valid, int r) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
        if (valid) qa[c4] = *reinterpret_cast<const u16x8_t *>(qp + 32 * c4 + 8 * r);
        else qa[c4] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
}

__device__ inline void load_k(u16x8_t (&kb)[4], const uint16_t *kp, int r) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) kb[c4] = *reinterpret_cast<const u16x8_t *>(kp + 32 * c4 + 8 * r);
}

// Row (in head_dim units) of slot j in the fast path, without branches: a
// block id outside the pool is redirected to block 0 and remembered in 'bad'
// (reported once after the loops).  Paged block sizes are powers of two.
template <bool PAGED>
struct FastRows {
    size_t ubase;          // contiguous: first row of the unit
    const int32_t *bt;     // paged: block-table row of the sequence
    int stride, hoff, shift, mask, nblk;

    __device__ inline FastRows(const CacheDev &c, int b, int h) {
        ubase = ((size_t)b * c.Hkv + h) * (size_t)c.cap;
        bt = c.bt ? c.bt + (size_t)b * c.max_blocks : nullptr;
        stride = c.Hkv * c.bs;
        hoff = h * c.bs;
        shift = PAGED ? __ffs(c.bs) - 1 : 0;
        mask = c.bs - 1;
        nblk = c.num_blocks;
    }
    __device__ inline size_t row(int j, bool &bad) const {
        if constexpr (!PAGED) {
            return ubase + (size_t)j;
        } else {
            int blk = bt[j >> shift];
            const bool bb = (unsigned)blk >= (unsigned)nblk;
            bad |= bb;
            blk = bb ? 0 : blk;
            return (size_t)blk * stride + hoff + (j & mask);
        }
    }
};

// Bytes of the per-wave K staging tiles, or of the selection keys and flags
// that reuse them, whichever is larger.
constexpr size_t kStageBytes = 16 * 256;   // 16 rows x 256 B per wave
__host__ __device__ constexpr size_t stage_region_bytes(int tc) {
    return (size_t)kFWaves * kStageBytes > (size_t)tc * 5 ? (size_t)kFWaves * kStageBytes
                                                          : ((size_t)tc * 5 + 15) / 16 * 16;
}

// 64-bit ranking word: larger = better (kept first); unique inside a unit
__device__ inline uint64_t rank_word(uint32_t primary, int32_t pos) {
    return ((uint64_t)primary << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}

template <int MODE>
__device__ void fused_generic(const FusedArgs &fa, int u, unsigned char *smem) {
    attn_unit_generic<uint16_t, kHD>(fa.attn, u, 0, *reinterpret_cast<AttnLds<kHD> *>(smem));
    if (MODE == kModeAttn) return;
    __syncthreads();
    select_unit<1>(fa.sel, u, *reinterpret_cast<SelLds<1> *>(smem));
    __syncthreads();
    compact_unit<uint16_t, kHD>(fa.comp, u, *reinterpret_cast<CompLds *>(smem));
}

template <int MODE, bool PAGED, int TC>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void fused_kernel(FusedArgs fa) {
    // most K tiles / V groups one wave handles: fixed trip counts let the
    // loops unroll into straight-line code with exact load/wait pairing
    constexpr int kNTW = (TC / 16 + kFWaves - 1) / kFWaves;
    constexpr int kNGW = (TC / 4 + kFWaves - 1) / kFWaves;
    extern __shared__ __align__(16) unsigned char smem[];
    const AttnArgs &a = fa.attn;
    const CacheDev &c = a.c;
    const int u = blockIdx.x;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, col = lane & 15;
    const int G = c.G;

    const int n = load_count(c, u, tid == 0);
    const int T = n + 1;
    if (T > TC || n >= c.cap) {
        fused_generic<MODE>(fa, u, smem);
        return;
    }

    constexpr int LD = TC + 4;
    float *lg = reinterpret_cast<float *>(smem);
    int32_t *pos_s = reinterpret_cast<int32_t *>(lg + G * LD);
    float *sc_s = reinterpret_cast<float *>(pos_s + TC);
    // K staging (one 16-row tile per wave) while keys stream; the selection
    // keys and flags reuse the same bytes afterwards
    unsigned char *stage_all = reinterpret_cast<unsigned char *>(sc_s + TC);
    unsigned char *stage = stage_all + w * kStageBytes;
    uint32_t *key_s = reinterpret_cast<uint32_t *>(stage_all);
    uint8_t *flg_s = reinterpret_cast<uint8_t *>(key_s + TC);
    FusedSmall &sm = *reinterpret_cast<FusedSmall *>(stage_all + stage_region_bytes(TC));

    const uint16_t *K = static_cast<const uint16_t *>(c.k);
    const uint16_t *V = static_cast<const uint16_t *>(c.v);
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new) + (size_t)u * kHD;
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new) + (size_t)u * kHD;
    int32_t *P = c.pos + (size_t)u * c.cap;
    float *S = a.scores ? a.scores + (size_t)u * c.cap : nullptr;
    const bool h2o = S != nullptr;
    const int32_t npos = a.new_pos[b];

    int pmax = -1;
    for (int j = tid; j < T; j += kFThreads) {
        const int32_t pj = (j < n) ? P[j] : npos;
        pos_s[j] = pj;
        pmax = max(pmax, pj);
        sc_s[j] = (h2o && j < n) ? S[j] : 0.f;
    }

    // ---------------- logits: MFMA 16x16x32 bf16, A = queries, B = 16 keys
    u16x8_t qa[4];
    load_q(qa, static_cast<const uint16_t *>(a.q) + ((size_t)b * c.Hq + (size_t)h * G + col) * kHD,
           col < G, r);
    const int ntiles = (T + 15) >> 4;
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const FastRows<PAGED> rows(c, b, h);
    bool bad = false;
    // every tile index is loadable: slots at or past n read the new token's
    // row, so the loads need no branch (the results are masked by j < T)
    // K tile t = slots 16t .. 16t+15.  Loads are coalesced: instruction k of a
    // lane reads 16 B (chunk 'col') of row 4k + r, so one wave instruction
    // covers 4 whole rows.  The tile then goes through the wave's LDS staging
    // buffer, chunk c of row q stored at slot c ^ q (conflict-free on both
    // sides), and comes back in the MFMA B layout: key = col, 8 dims per
    // 16-lane group.
    auto krow = [&](int t, int k) -> const u16x8_t * {
        const int j = 16 * t + 4 * k + r;
        const size_t rr = rows.row(j < n ? j : 0, bad);
        return reinterpret_cast<const u16x8_t *>(((j < n) ? K + rr * kHD : kn) + 8 * col);
    };
    {
        u16x8_t kb[kDK][4];
#pragma unroll
        for (int d = 0; d < kDK; ++d)
#pragma unroll
            for (int k = 0; k < 4; ++k) kb[d][k] = *krow(w + kFWaves * d, k);
#pragma unroll
        for (int i = 0; i < kNTW; ++i) {
            const int t = w + kFWaves * i;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int q = 4 * k + r;
                *reinterpret_cast<u16x8_t *>(stage + q * 256 + ((col ^ q) << 4)) = kb[i % kDK][k];
            }
            if (i + kDK < kNTW)
#pragma unroll
                for (int k = 0; k < 4; ++k) kb[i % kDK][k] = *krow(t + kFWaves * kDK, k);
            u16x8_t kop[4];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                kop[c4] = *reinterpret_cast<const u16x8_t *>(stage + col * 256 +
                                                             (((4 * c4 + r) ^ col) << 4));
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[c4]), as_bf16x8(kop[c4]),
                                                              acc, 0, 0, 0);
            const int j = 16 * t + col;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int g = 4 * r + ii;
                const float z = (j < T) ? acc[ii] * a.scale : -INFINITY;
                if (g < G && j < T) lg[g * LD + j] = z;
                mx[ii] = fmaxf(mx[ii], z);
            }
        }
    }
    // V rows do not depend on the softmax: start streaming them now
    const int ngroups = (T + 3) >> 2;
    auto vptr = [&](int q4) -> const u16x8_t * {
        const int j = 4 * q4 + r;
        const size_t rr = rows.row(j < n ? j : 0, bad);
        return reinterpret_cast<const u16x8_t *>(((j < n) ? V + rr * kHD : vn) + 8 * col);
    };
    u16x8_t vb[kDV];
#pragma unroll
    for (int d = 0; d < kDV; ++d) vb[d] = *vptr(w + kFWaves * d);
    (void)ngroups;
    // row maxima (16-lane groups share a query head set, then across waves),
    // and the newest position of the unit
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float m = mx[i];
        m = fmaxf(m, __shfl_xor(m, 8, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        if (col == 0 && 4 * r + i < G) sm.wred[w][4 * r + i] = m;
    }
    pmax = wave_max_i(pmax);
    if (lane == 0) sm.pmax[w] = pmax;
    __syncthreads();
    if (tid < G) {
        float m = sm.wred[0][tid];
        for (int v = 1; v < kFWaves; ++v) m = fmaxf(m, sm.wred[v][tid]);
        sm.m[tid] = m;
    }
    if (tid == 64) {
        int pm = sm.pmax[0];
        for (int v = 1; v < kFWaves; ++v) pm = max(pm, sm.pmax[v]);
        sm.posmax = pm;
    }
    __syncthreads();

    // ---------------- P.V: MFMA 16x16x4 f32, A = probabilities, B = 4 V rows.
    // The lane that feeds weight (g = col, key j) to the MFMA computes it:
    // w = exp(z - m_g), stored back for the H2O update, summed for l_g.
    f32x4_t oacc[8];
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) oacc[t8] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    const float mcol = (col < G) ? sm.m[col] : 0.f;
#pragma unroll
    for (int i = 0; i < kNGW; ++i) {
        const int q4 = w + kFWaves * i;
        const int j = 4 * q4 + r;
        // groups past the end carry p = 0 and read valid rows
        float p = 0.f;
        if (col < G && j < T) {
            p = __expf(lg[col * LD + j] - mcol);
            lg[col * LD + j] = p;
        }
        lsum += p;
        const u16x8_t cur = vb[i % kDV];
        if (i + kDV < kNGW) vb[i % kDV] = *vptr(q4 + kFWaves * kDV);
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
            oacc[t8] = __builtin_amdgcn_mfma_f32_16x16x4f32(p, bf16_to_f32(cur[t8]), oacc[t8], 0,
                                                             0, 0);
    }
    if (bad) raise_flag(c, KVC_FLAG_BAD_BLOCK);
    // lanes col, col+16, col+32, col+48 hold partial sums of query head col
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (lane < G) sm.wred[w][lane] = lsum;
    __syncthreads();   // weights in lg are final, partial row sums written
    if (tid < G) {
        float l = 0.f;
        for (int v = 0; v < kFWaves; ++v) l += sm.wred[v][tid];
        sm.l[tid] = l;
        sm.il[tid] = 1.f / l;
    }
    __syncthreads();

    // ---------------- H2O: accumulated attention with the final normaliser
    if (h2o) {
        for (int j = tid; j < T; j += kFThreads) {
            float ps = 0.f;
            for (int g = 0; g < G; ++g) ps += lg[g * LD + j] * sm.il[g];
            sc_s[j] = (j < n) ? sc_s[j] + ps : ps;
        }
    }

    // ---------------- output: sum the four waves' partial P.V, normalise.
    // The partials go to the staging bytes when they fit (G <= 8), else to
    // the weights' bytes once the H2O pass is done with them.
    {
        const bool in_stage = G * kHD * kFWaves * 4 <= (int)(kFWaves * kStageBytes);
        float *opart = in_stage ? reinterpret_cast<float *>(stage_all) : lg;
        if (!in_stage) __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * r + i;
            if (g < G) {
                float *dst = opart + ((size_t)w * G + g) * kHD + 8 * col;
#pragma unroll
                for (int t8 = 0; t8 < 8; ++t8) dst[t8] = oacc[t8][i];
            }
        }
        __syncthreads();
        float *outp = a.out + ((size_t)b * c.Hq + (size_t)h * G) * kHD;
        for (int e = tid; e < G * kHD; e += kFThreads) {
            const int g = e / kHD;
            float o = opart[e];
            for (int v = 1; v < kFWaves; ++v) o += opart[(size_t)v * G * kHD + e];
            outp[e] = o / sm.l[g];
        }
    }

    uint16_t *Kw = static_cast<uint16_t *>(c.k);
    uint16_t *Vw = static_cast<uint16_t *>(c.v);

    if (MODE == kModeAttn) {
        // append the new token at slot n, write every score back
        if (h2o)
            for (int j = tid; j < T; j += kFThreads) S[j] = sc_s[j];
        if (tid < 16) {
            const size_t rw = row_of(c, b, h, n) * kHD;
            reinterpret_cast<uint4 *>(Kw + rw)[tid] = reinterpret_cast<const uint4 *>(kn)[tid];
            reinterpret_cast<uint4 *>(Vw + rw)[tid] = reinterpret_cast<const uint4 *>(vn)[tid];
        }
        if (tid == 0) {
            P[n] = npos;
            c.n_slots[u] = n + 1;
        }
        return;
    }

    // ================= selection on the LDS copies =================
    // One pass classifies every entry, draws the candidates' ranking keys and
    // finds the worst candidate (smallest ranking word) and a dropped entry.
    const SelectArgs &sa = fa.sel;
    __syncthreads();   // the output pass is done with the staging bytes
    const int L = sm.posmax + 1;
    int ncand = 0, ndrop = 0, dslot = -1, barg = -1;
    uint64_t best = ~0ull;
    for (int j = tid; j < T; j += kFThreads) {
        const int32_t p = pos_s[j];
        uint8_t k = kKeep;
        if (sa.kind == KVC_POLICY_STREAMING)
            k = (p < sa.n_sink || (int64_t)p >= (int64_t)L - sa.n_recent) ? kKeep : kDrop;
        else if (sa.kind == KVC_POLICY_H2O)
            k = ((int64_t)p >= (int64_t)L - sa.n_recent) ? kKeep : kCand;
        else if (sa.kind == KVC_POLICY_RANDOM)
            k = (p < sa.prompt_len) ? kKeep : kCand;
        if (k == kCand) {
            const uint32_t key = (sa.kind == KVC_POLICY_H2O)
                                     ? float_order_bits(sc_s[j])
                                     : ~philox_word0((uint32_t)p, sa.step, (uint32_t)h, (uint32_t)b,
                                                     (uint32_t)(sa.seed & 0xFFFFFFFFu),
                                                     (uint32_t)(sa.seed >> 32));
            key_s[j] = key;
            ++ncand;
            const uint64_t wd = rank_word(key, p);
            if (wd < best) {
                best = wd;
                barg = j;
            }
        } else if (k == kDrop) {
            ++ndrop;
            dslot = max(dslot, j);
        }
        flg_s[j] = k;
    }
    ncand = wave_sum_i(ncand);
    ndrop = wave_sum_i(ndrop);
    dslot = wave_max_i(dslot);
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
        const uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
        const int oa = __shfl_xor(barg, o, 64);
        const uint64_t ob = ((uint64_t)hi << 32) | lo;
        if (ob < best) {
            best = ob;
            barg = oa;
        }
    }
    if (lane == 0) {
        sm.r_nc[w] = ncand;
        sm.r_nd[w] = ndrop;
        sm.r_ds[w] = dslot;
        sm.r_arg[w] = barg;
        sm.mn_hi[w] = (uint32_t)(best >> 32);
        sm.mn_lo[w] = (uint32_t)best;
    }
    __syncthreads();
    ncand = 0;
    ndrop = 0;
    dslot = -1;
    barg = -1;
    best = ~0ull;
    for (int v = 0; v < kFWaves; ++v) {
        ncand += sm.r_nc[v];
        ndrop += sm.r_nd[v];
        dslot = max(dslot, sm.r_ds[v]);
        const uint64_t ob = ((uint64_t)sm.mn_hi[v] << 32) | sm.mn_lo[v];
        if (sm.r_arg[v] >= 0 && ob < best) {
            best = ob;
            barg = sm.r_arg[v];
        }
    }
    const int want = (sa.kind == KVC_POLICY_H2O) ? sa.n_heavy : sa.n_keep;
    const int extra = (ncand > want) ? (want <= 0 ? ncand : ncand - want) : 0;

    if (ndrop + extra <= 1) {
        // ---- at most one eviction (the steady state): no scans.  With one
        // evicted slot e, n_out = n and the new token fills e when e < n
        // (the hole-fill pairing of a single hole with source slot n).
        const int e = (extra == 1) ? barg : (ndrop == 1 ? dslot : -1);
        const int n_out = (e < 0) ? T : n;
        const int dst_new = (e < 0) ? n : (e < n ? e : -1);
        if (dst_new >= 0 && tid < 16) {
            const size_t rw = row_of(c, b, h, dst_new) * kHD;
            reinterpret_cast<uint4 *>(Kw + rw)[tid] = reinterpret_cast<const uint4 *>(kn)[tid];
            reinterpret_cast<uint4 *>(Vw + rw)[tid] = reinterpret_cast<const uint4 *>(vn)[tid];
        }
        if (h2o)
            for (int j = tid; j < n; j += kFThreads)
                if (j != e) S[j] = sc_s[j];
        if (tid == 0) {
            if (dst_new >= 0) {
                P[dst_new] = npos;
                if (h2o) S[dst_new] = sc_s[n];
            }
            c.n_slots[u] = n_out;
        }
        return;
    }

    // ---- general case: finish the candidates' flags, then hole-fill
    if (extra > 0) {
        if (want <= 0) {
            for (int j = tid; j < T; j += kFThreads)
                if (flg_s[j] == kCand) flg_s[j] = kDrop;
        } else {
            // radix select of the 'want' largest ranking words among candidates
            uint64_t prefix = 0, mask = 0;
            int krem = want;
            for (int shift = 56; shift >= 0; shift -= 8) {
                sm.hist[tid] = 0;   // kFThreads == 256 bins
                __syncthreads();
                for (int j = tid; j < T; j += kFThreads)
                    if (flg_s[j] == kCand) {
                        const uint64_t wd = rank_word(key_s[j], pos_s[j]);
                        if ((wd & mask) == prefix) atomicAdd(&sm.hist[(wd >> shift) & 255], 1);
                    }
                __syncthreads();
                if (tid == 0) {
                    int cum = 0, dsel = 0;
                    for (int d = 255; d >= 0; --d) {
                        if (cum + sm.hist[d] >= krem) {
                            dsel = d;
                            break;
                        }
                        cum += sm.hist[d];
                    }
                    sm.sh[0] = dsel;
                    sm.sh[1] = krem - cum;
                    sm.sh[2] = (sm.hist[dsel] == krem - cum);
                }
                __syncthreads();
                krem = sm.sh[1];
                prefix |= (uint64_t)sm.sh[0] << shift;
                mask |= (uint64_t)255 << shift;
                const int done = sm.sh[2];
                __syncthreads();
                if (done) break;
            }
            for (int j = tid; j < T; j += kFThreads)
                if (flg_s[j] == kCand)
                    flg_s[j] = ((rank_word(key_s[j], pos_s[j]) & mask) >= prefix) ? kKeep : kDrop;
        }
    } else {
        for (int j = tid; j < T; j += kFThreads)
            if (flg_s[j] == kCand) flg_s[j] = kKeep;
    }
    __syncthreads();

    // ================= compaction =================
    // n_out kept; holes = dropped slots below n_out, sources = kept slots at or
    // above n_out (slot n is the new token), paired in ascending order.
    int kc = 0;
    int tot;
    for (int j = tid; j < T; j += kFThreads) kc += (flg_s[j] == kKeep);
    (void)block_excl_scan(kc, sm.red, &tot);
    const int n_out = tot;
    int32_t *hole = reinterpret_cast<int32_t *>(key_s);   // reuse: ranks are final
    int32_t *srcl = reinterpret_cast<int32_t *>(lg);
    int nh = 0, ns = 0;
    for (int j0 = 0; j0 < T; j0 += kFThreads) {
        const int j = j0 + tid;
        const int isHole = (j < n_out) && flg_s[j] != kKeep;
        const int isSrc = (j >= n_out) && (j < T) && flg_s[j] == kKeep;
        int th, ts;
        const int rh = block_excl_scan(isHole, sm.red, &th);
        const int rs = block_excl_scan(isSrc, sm.red + kFWaves, &ts);
        if (isHole) hole[nh + rh] = j;
        if (isSrc) srcl[ns + rs] = j;
        nh += th;
        ns += ts;
    }
    __syncthreads();
    const int moves = min(nh, ns);
    for (int e = tid; e < moves * 16; e += kFThreads) {
        const int i = e >> 4, part = e & 15;
        const int d = hole[i], s = srcl[i];
        const size_t rd = row_of(c, b, h, d) * kHD;
        const uint4 *ks = reinterpret_cast<const uint4 *>((s == n) ? kn : K + row_of(c, b, h, s) * kHD);
        const uint4 *vs = reinterpret_cast<const uint4 *>((s == n) ? vn : V + row_of(c, b, h, s) * kHD);
        reinterpret_cast<uint4 *>(Kw + rd)[part] = ks[part];
        reinterpret_cast<uint4 *>(Vw + rd)[part] = vs[part];
    }
    for (int i = tid; i < moves; i += kFThreads) {
        const int d = hole[i], s = srcl[i];
        P[d] = pos_s[s];
        if (h2o) S[d] = sc_s[s];
    }
    // kept slots that stay: new scores; the new token kept in place (no eviction)
    for (int j = tid; j < n_out; j += kFThreads)
        if (flg_s[j] == kKeep) {
            if (h2o) S[j] = sc_s[j];
            if (j == n) P[n] = npos;
        }
    if (n < n_out && tid < 16) {
        const size_t rw = row_of(c, b, h, n) * kHD;
        reinterpret_cast<uint4 *>(Kw + rw)[tid] = reinterpret_cast<const uint4 *>(kn)[tid];
        reinterpret_cast<uint4 *>(Vw + rw)[tid] = reinterpret_cast<const uint4 *>(vn)[tid];
    }
    if (tid == 0) c.n_slots[u] = n_out;
}

size_t fused_smem_bytes(int G, int tcap) {
    const size_t ld = (size_t)tcap + 4;
    size_t fast = (size_t)G * ld * 4 + (size_t)tcap * (4 + 4) + stage_region_bytes(tcap) +
                  sizeof(FusedSmall) + 16;
    size_t gen = sizeof(AttnLds<kHD>);
    if (sizeof(SelLds<1>) > gen) gen = sizeof(SelLds<1>);
    if (sizeof(CompLds) > gen) gen = sizeof(CompLds);
    return fast > gen ? fast : gen;
}

template <int TC>
static hipError_t launch_tc(const FusedArgs &fa, int mode, size_t smem, hipStream_t s) {
    const int units = fa.attn.c.B * fa.attn.c.Hkv;
    const bool paged = fa.attn.c.bs > 0;
    static hipError_t attr = [smem] {
        (void)smem;
        const int most = (int)fused_smem_bytes(kMaxGroup, TC);
        const void *fns[4] = {(const void *)fused_kernel<kModeAttn, false, TC>,
                              (const void *)fused_kernel<kModeStep, false, TC>,
                              (const void *)fused_kernel<kModeAttn, true, TC>,
                              (const void *)fused_kernel<kModeStep, true, TC>};
        hipError_t e = hipSuccess;
        for (const void *f : fns)
            if (e == hipSuccess)
                e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, most);
        return e;
    }();
    if (attr != hipSuccess) return attr;
    if (mode == kModeAttn && !paged)
        hipLaunchKernelGGL((fused_kernel<kModeAttn, false, TC>), dim3(units), dim3(kFThreads), smem,
                           s, fa);
    else if (mode == kModeAttn)
        hipLaunchKernelGGL((fused_kernel<kModeAttn, true, TC>), dim3(units), dim3(kFThreads), smem,
                           s, fa);
    else if (!paged)
        hipLaunchKernelGGL((fused_kernel<kModeStep, false, TC>), dim3(units), dim3(kFThreads), smem,
                           s, fa);
    else
        hipLaunchKernelGGL((fused_kernel<kModeStep, true, TC>), dim3(units), dim3(kFThreads), smem,
                           s, fa);
    return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs &fa, int mode, hipStream_t s) {
    const size_t smem = fused_smem_bytes(fa.attn.c.G, fa.tcap);
    if (fa.tcap == kFusedSmallT) return launch_tc<kFusedSmallT>(fa, mode, smem, s);
    if (fa.tcap == kFusedMaxT) return launch_tc<kFusedMaxT>(fa, mode, smem, s);
    return hipErrorInvalidValue;
}

}  // namespace kvc
