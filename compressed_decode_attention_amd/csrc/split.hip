// split.hip -- decode attention over long units on the matrix cores: one
// workgroup per (unit, chunk of consecutive slots), partial results merged by
// attn_combine_kernel (attn.hip).
//
// What it computes (KV cache compression guide, section 16, "prefill, decode,
// TP": a decode step reads all kept history; FlashAttention-style splitting of
// long rows across workgroups, same guide, section 2): for the chunk's slots
// j (the new token included when its index n falls in the chunk),
//   z_gj = scale * q_g . k_j,  m_g = max_j z_gj,  w_gj = exp(z_gj - m_g),
//   l_g = sum_j w_gj,  o_g = sum_j w_gj v_j   (not normalised),
// written as the split's partial (o, m, l); with H2O scores requested the
// weights w go to the logit scratch, where the combine pass turns them into
// probabilities with the global max and normaliser.  The workgroup whose
// chunk holds index n appends the new token.
//
// The tile machinery is the one-workgroup kernel's (fused.hip): QK^T on
// v_mfma_f32_16x16x32_bf16 through a swizzled per-wave LDS tile, the chunk's
// logits resident in LDS, P.V on v_mfma_f32_16x16x16_bf16 with the register
// repack and P as a bf16 high/low pair, bounded buffer-resource loads (here
// bounded by the chunk, so no wave reads past it), bf16 or E5M2 rows.
// Chunks start at multiples of 16 slots, so tiles never straddle two chunks.
#include "mfma_tiles.h"

namespace kvc {

struct SplitSmall {
    float m[kMaxGroup];              // chunk maxima of the logits
    float wred[kFWaves][kMaxGroup];
    int blk[kFusedMaxT / 16 + 2];    // paged: block ids of the chunk's slots
    u16x8_t knew[kHD / 8];           // the new token's key row (as attended)
};

template <int TC>
__host__ __device__ constexpr size_t split_smem_bytes_tc(int G) {
    return (size_t)G * (TC + 4) * 4 + (size_t)kFWaves * kStageBytes + sizeof(SplitSmall);
}

size_t split_smem_bytes(int G, int tc) {
    size_t fast = tc <= kFusedSmallT ? split_smem_bytes_tc<kFusedSmallT>(G)
                                     : split_smem_bytes_tc<kFusedMaxT>(G);
    // a chunk longer than the launch's capacity runs the generic routine
    return fast > sizeof(AttnLds<kHD>) ? fast : sizeof(AttnLds<kHD>);
}

// The random-eviction share of split s of unit u over the slots [j0, jsel)
// it holds after this step (the new token's slot n included when it was
// stored): candidates are the slots whose position is past the pinned
// prompt, ranked by the same composite key as the selection (blog, "scorers
// are overrated": per-head uniform draws; the key is the inverted Philox word
// of (position, step, kv head, sequence), then the inverted position).
// Positions are loaded early (presel_load, KPS per thread) so that ranking
// them at the end of the kernel waits for no memory.
template <int KPS>
__device__ inline void presel_load(const AttnArgs &a, int u, int b, int j0, int jsel, int n,
                                   int32_t (&p)[KPS]) {
    const int32_t *P = a.c.pos + (size_t)u * a.c.cap;
    const int32_t np = a.new_pos[b];
#pragma unroll
    for (int k = 0; k < KPS; ++k) {
        const int j = j0 + (int)threadIdx.x + k * kFThreads;
        p[k] = 0;
        if (j < jsel) p[k] = (j == n) ? np : P[j];
    }
}

static_assert(kPreselWaves == kFWaves, "one random-eviction record per wave of a split");

// A thread's running minimum of the candidates' keys and their count.
struct PreselAcc {
    uint32_t cnt = 0;
    uint64_t best = ~0ull;
    int arg = -1;
};

__device__ inline void presel_add(const AttnArgs &a, int b, int h, int j, int32_t p,
                                  PreselAcc &acc) {
    if (p < a.presel_prompt_len) return;
    ++acc.cnt;
    const uint32_t pr = ~philox_word0((uint32_t)p, a.presel_step, (uint32_t)h, (uint32_t)b,
                                      (uint32_t)(a.presel_seed & 0xFFFFFFFFu),
                                      (uint32_t)(a.presel_seed >> 32));
    const uint64_t key = ((uint64_t)pr << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
    if (acc.arg < 0 || key < acc.best) {
        acc.best = key;
        acc.arg = j;
    }
}

// Wave reduction of the threads' shares (equal keys: the lower slot); each
// wave writes its own record, so the split needs no barrier (one waiting for
// its output stores) to publish them.
__device__ inline void presel_write(const AttnArgs &a, int u, int s, PreselAcc acc) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    auto step = [&](uint32_t hi, uint32_t lo, int oa) {
        const uint64_t ok = ((uint64_t)hi << 32) | lo;
        if (ok < acc.best || (ok == acc.best && (unsigned)oa < (unsigned)acc.arg)) {
            acc.best = ok;
            acc.arg = oa;
        }
    };
    acc.cnt = wave_sum_iv(acc.cnt);
#define KVC_PRESEL_STEP(M) \
    step(lane_xor<M>((uint32_t)(acc.best >> 32)), lane_xor<M>((uint32_t)acc.best), \
         (int)lane_xor<M>((uint32_t)acc.arg))
    KVC_PRESEL_STEP(32);
    KVC_PRESEL_STEP(16);
    KVC_PRESEL_STEP(8);
    KVC_PRESEL_STEP(4);
    KVC_PRESEL_STEP(2);
    KVC_PRESEL_STEP(1);
#undef KVC_PRESEL_STEP
    if (lane == 0) {
        PreselRecord rec;
        rec.ncand = acc.cnt;
        rec.key_hi = (uint32_t)(acc.best >> 32);
        rec.key_lo = (uint32_t)acc.best;
        rec.slot = acc.arg;
        reinterpret_cast<PreselRecord *>(a.presel)[((size_t)u * a.nsplit + s) * kPreselWaves + w] =
            rec;
    }
}

template <int KPS>
__device__ inline void presel_rank(const AttnArgs &a, int u, int s, int b, int h, int j0, int jsel,
                                   const int32_t (&p)[KPS]) {
    PreselAcc acc;
#pragma unroll
    for (int k = 0; k < KPS; ++k) {
        const int j = j0 + (int)threadIdx.x + k * kFThreads;
        if (j < jsel) presel_add(a, b, h, j, p[k], acc);
    }
    presel_write(a, u, s, acc);
}

// Both steps over a chunk of any length (the generic routine's chunks).
__device__ inline void presel_chunk(const AttnArgs &a, int u, int s, int b, int h, int j0,
                                    int jsel, int n) {
    const int32_t *P = a.c.pos + (size_t)u * a.c.cap;
    PreselAcc acc;
    for (int j = j0 + (int)threadIdx.x; j < jsel; j += kFThreads)
        presel_add(a, b, h, j, (j == n) ? a.new_pos[b] : P[j], acc);
    presel_write(a, u, s, acc);
}

template <bool PAGED, int TC, bool PACK2, bool F8>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void split_kernel(AttnArgs a) {
    using Row = typename KvRow<F8>::type;
    constexpr int RB = F8 ? kHD : 2 * kHD;   // bytes of one cached K or V row
    constexpr int DK = F8 ? kDK8 : kDK;
    constexpr int DV = F8 ? kDV8 : kDV;
    constexpr int kNTW = (TC / 16 + kFWaves - 1) / kFWaves;   // tiles per wave, at most
    constexpr int LD = TC + 4;
    extern __shared__ __align__(16) unsigned char smem[];
    const CacheDev &c = a.c;
    const int ns = a.nsplit;
    const int u = blockIdx.x / ns, s = blockIdx.x % ns;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane >> 4, col = lane & 15;
    const int G = c.G;

    u16x8_t qa[4];
    load_q(qa, static_cast<const uint16_t *>(a.q) + ((size_t)b * c.Hq + (size_t)h * G + col) * kHD,
           col < G, r);
    const int n = __builtin_amdgcn_readfirstlane(load_count(c, u, s == 0 && tid == 0));
    const int T = n + 1;
    const int chunk = split_chunk(T, ns, a.max_len);
    if (s >= split_count(T, ns, a.max_len)) return;   // past the unit's entries: nothing to attend
    if (chunk > TC) {   // longer than the launch promised: the generic routine
        using TK = typename std::conditional<F8, e5m2_t, uint16_t>::type;
        attn_unit_generic<TK, kHD>(a, u, s, *reinterpret_cast<AttnLds<kHD> *>(smem));
        if (a.presel) {
            const int j0 = min(s * chunk, T), j1 = min(T, j0 + chunk);
            presel_chunk(a, u, s, b, h, j0, (a.append && n < c.cap) ? j1 : min(j1, n), n);
        }
        return;
    }
    const bool can_store = a.append && n < c.cap;
    if (a.append && !can_store && s == 0 && tid == 0) raise_flag(c, KVC_FLAG_FULL);
    const int j0 = min(s * chunk, T), j1 = min(T, j0 + chunk);   // attended slots
    const int jend = min(j1, n);                                   // of them cached

    float *lg = reinterpret_cast<float *>(smem);
    unsigned char *stage_all = reinterpret_cast<unsigned char *>(lg + G * LD);
    unsigned char *stage = stage_all + w * kStageBytes;
    SplitSmall &sm = *reinterpret_cast<SplitSmall *>(stage_all + kFWaves * kStageBytes);

    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new) + (size_t)u * kHD;
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new) + (size_t)u * kHD;
    const u16x8_t knr = reinterpret_cast<const u16x8_t *>(kn)[lane & 15];
    int blk0 = 0;
    if constexpr (PAGED) {
        // block ids of the cached slots [j0, jend), checked once (an id
        // outside the pool is reported and replaced by block 0)
        const int shift = __ffs(c.bs) - 1;
        blk0 = j0 >> shift;
        const int nb = jend > j0 ? ((jend - 1) >> shift) - blk0 + 1 : 0;
        const int32_t *bt = c.bt + (size_t)b * c.max_blocks;
        for (int i = tid; i < nb; i += kFThreads) {
            int blk = bt[blk0 + i];
            if ((unsigned)blk >= (unsigned)c.num_blocks) {
                raise_flag(c, KVC_FLAG_BAD_BLOCK);
                blk = 0;
            }
            sm.blk[i] = blk;
        }
        __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---------------- logits of the chunk: tile t = slots j0 + 16t .. + 15
    const int ntiles = (j1 - j0 + 15) >> 4;
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const TileSrc<PAGED, RB> src(c, b, h, j0, jend, sm.blk, blk0);
    const int lane_off = r * RB + KvRow<F8>::kBytes * col;
    auto kload = [&](int t, int k) -> Row {
        __amdgpu_buffer_rsrc_t rs;
        int toff;
        src.tile(t, false, rs, toff);
        return buffer_row<F8, PAGED, true>(rs, lane_off + toff + 4 * RB * k);
    };
    // the new token's tile and row inside the chunk (none when n is outside)
    const int tn = (j0 <= n && n < j1) ? (n - j0) >> 4 : -1, qn = n & 15;
    // the scale as a vector register: held across the K loop, it would
    // otherwise pin a scalar register group that the loop keeps reloading
    float scale;
    asm volatile("v_mov_b32 %0, %1" : "=v"(scale) : "s"(a.scale));
    // where this lane stores logit row 4r + ii of tile t: lgp[ii] + 16 t.  The
    // padding rows (4r + ii >= G) store into this wave's own staging tile
    // instead, every such lane to the same word (free at that point: LDS
    // operations of a wave complete in order), so the stores need no mask
    static_assert(16 * (TC / 16) * 4 <= (int)kStageBytes, "dummy logit stores stay in the wave's tile");
    float *lgp[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int g = 4 * r + ii;
        lgp[ii] = (g < G) ? lg + g * LD + (((col & 3) << 2) | (col >> 2))
                          : reinterpret_cast<float *>(stage) + ii;
    }
    {
        Row kb[DK][4];
#pragma unroll
        for (int d = 0; d < DK; ++d)
#pragma unroll
            for (int k = 0; k < 4; ++k) kb[d][k] = kload(w + kFWaves * d, k);
        if (tid < kHD / 8) {
            if constexpr (F8) sm.knew[tid] = e5m2x8_to_bf16(e5m2x8_encode(knr));
            else sm.knew[tid] = knr;
        }
        __syncthreads();   // the new key row is in LDS
#pragma unroll
        for (int i = 0; i < kNTW; ++i) {
            const int t = w + kFWaves * i;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int q = 4 * k + r;
                *reinterpret_cast<u16x8_t *>(stage + q * 256 + ((col ^ q) << 4)) =
                    as_bf16_row(kb[i % DK][k]);
            }
            if (t == tn && lane < 16)   // row n read as zeros: put the new key there
                *reinterpret_cast<u16x8_t *>(stage + qn * 256 + ((lane ^ qn) << 4)) = sm.knew[lane];
            if (i + DK < kNTW)
#pragma unroll
                for (int k = 0; k < 4; ++k) kb[i % DK][k] = kload(t + kFWaves * DK, k);
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
            // tiles past the chunk hold no key (uniform test); inside the
            // last tile, keys past j1 get -inf, so they weigh 0
            if (t < ntiles) {
                const int jr = 16 * t + col;   // slot j0 + jr
                const bool live = j0 + jr < j1;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const float z = live ? acc[ii] * scale : -INFINITY;
                    lgp[ii][16 * t] = z;
                    mx[ii] = z > mx[ii] ? z : mx[ii];
                }
            }
        }
    }
    // V rows of the same tiles, requested before the max is known
    auto vload = [&](int t, int k) -> Row {
        __amdgpu_buffer_rsrc_t rs;
        int toff;
        src.tile(t, true, rs, toff);
        return buffer_row<F8, PAGED, true>(rs, lane_off + toff + 4 * RB * k);
    };
    u16x8_t vnc = *reinterpret_cast<const u16x8_t *>(vn + 8 * col);
    if constexpr (F8) vnc = e5m2x8_to_bf16(e5m2x8_encode(vnc));
    Row vb[DV][4];
#pragma unroll
    for (int d = 0; d < DV; ++d)
#pragma unroll
        for (int k = 0; k < 4; ++k) vb[d][k] = vload(w + kFWaves * d, k);
    // random eviction: the chunk's positions, ranked after P.V
    constexpr int kPS = (TC + kFThreads - 1) / kFThreads;
    const int jsel = can_store ? j1 : jend;
    int32_t psel[kPS];
    if (a.presel) presel_load<kPS>(a, u, b, j0, jsel, n, psel);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float m = mx[i];
        m = fmaxf(m, lane_xor_f<8>(m));
        m = fmaxf(m, lane_xor_f<4>(m));
        m = fmaxf(m, lane_xor_f<2>(m));
        m = fmaxf(m, lane_xor_f<1>(m));
        if (col == 0 && 4 * r + i < G) sm.wred[w][4 * r + i] = m;
    }
    __syncthreads();
    if (tid < G) {
        float m = sm.wred[0][tid];
        for (int v = 1; v < kFWaves; ++v) m = fmaxf(m, sm.wred[v][tid]);
        sm.m[tid] = m;
    }
    __syncthreads();

    // ---------------- P.V over the chunk's tiles (weights relative to the chunk max)
    f32x4_t oacc[8];
#pragma unroll
    for (int m8 = 0; m8 < 8; ++m8) oacc[m8] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    constexpr bool pack2 = PACK2;
    const int ga = pack2 ? (col & 7) : col;
    const bool arow = ga < G;
    const bool hi_lane = !pack2 || col < 8;
    const float mrow = arow ? sm.m[ga] : 0.f;
    // an empty chunk has m = -inf: every weight is 0
    const bool any = mrow != -INFINITY;
    float *lrow = lg + (arow ? ga : 0) * LD;
#pragma unroll
    for (int i = 0; i < kNTW; ++i) {
        const int t = w + kFWaves * i;
        const int c0 = 16 * t + 4 * r;
        // logits past j1 are -inf (weight 0); tiles past the chunk (uniform
        // test), the padding rows of A and an empty chunk weigh nothing
        f32x4_t p = {0.f, 0.f, 0.f, 0.f};
        if (t < ntiles) {
            const f32x4_t z = *reinterpret_cast<const f32x4_t *>(lrow + c0);
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = (arow && any) ? __expf(z[e] - mrow) : 0.f;
        }
        s16x4_t ahi, alo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ahi[e] = bf16_bits(p[e]);
            alo[e] = bf16_bits(p[e] - bf16_value(ahi[e]));
        }
        if (hi_lane) {
            lsum += (p[0] + p[1]) + (p[2] + p[3]);
            if (t < ntiles && arow) *reinterpret_cast<f32x4_t *>(lrow + c0) = p;
        }
        const s16x4_t a0 = (pack2 && !hi_lane) ? alo : ahi;
        // row n (read as zeros) is the new token's, in tile tn only
        u16x8_t vr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[e] = as_bf16_row(vb[i % DV][e]);
        if (t == tn)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * e + r == qn) vr[e] = vnc;
        s16x4_t bop[8];
#pragma unroll
        for (int m8 = 0; m8 < 8; ++m8)
            bop[m8] = s16x4_t{(short)vr[0][m8], (short)vr[1][m8], (short)vr[2][m8], (short)vr[3][m8]};
        if (i + DV < kNTW)
#pragma unroll
            for (int k = 0; k < 4; ++k) vb[i % DV][k] = vload(t + kFWaves * DV, k);
#pragma unroll
        for (int m8 = 0; m8 < 8; ++m8)
            oacc[m8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, bop[m8], oacc[m8], 0, 0, 0);
        if (!pack2)
#pragma unroll
            for (int m8 = 0; m8 < 8; ++m8)
                oacc[m8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bop[m8], oacc[m8], 0, 0, 0);
    }
    if (pack2)
#pragma unroll
        for (int m8 = 0; m8 < 8; ++m8)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) oacc[m8][ii] = pair_sum32(oacc[m8][ii]);
    lsum = pair_sum16(lsum);
    lsum = pair_sum32(lsum);
    if (lane < G) sm.wred[w][lane] = lsum;
    __syncthreads();   // weights in lg are final, partial row sums written

    // ---------------- weights for the H2O update of the combine pass
    if (a.scores) {
        const size_t ld = (size_t)c.cap + 1;
        float *lw = a.logits + (size_t)u * G * ld;
        const int len = j1 - j0;
        for (int e = tid; e < G * len; e += kFThreads) {
            const int g = e / len, jr = e % len;
            lw[g * ld + j0 + jr] = lg[g * LD + lg_col(jr)];
        }
    }

    // ---------------- partial (o, m, l) of this split.  The four waves'
    // partial P.V go to the staging bytes when they fit (G <= 8), else to the
    // weights' bytes once the copy above is done with them.
    const bool in_stage = G * kHD * kFWaves * 4 <= (int)(kFWaves * kStageBytes);
    float *opart = in_stage ? reinterpret_cast<float *>(stage_all) : lg;
    if (!in_stage) __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * r + i;
        if (g < G && (!pack2 || r < 2)) {
            float *dst = opart + ((size_t)w * G + g) * kHD + 8 * col;
#pragma unroll
            for (int m8 = 0; m8 < 8; ++m8) dst[m8] = oacc[m8][i];
        }
    }
    __syncthreads();
    float *pp = a.part + ((size_t)u * ns + s) * G * (kHD + 2);
    for (int e = tid; e < G * kHD; e += kFThreads) {
        float o = opart[e];
        for (int v = 1; v < kFWaves; ++v) o += opart[(size_t)v * G * kHD + e];
        pp[(e / kHD) * (kHD + 2) + (e % kHD)] = o;
    }
    if (tid < G) {
        float l = 0.f;
        for (int v = 0; v < kFWaves; ++v) l += sm.wred[v][tid];
        pp[tid * (kHD + 2) + kHD] = sm.m[tid];
        pp[tid * (kHD + 2) + kHD + 1] = l;
    }

    // ---------------- append the new token (the split whose chunk holds n)
    if (can_store && j0 <= n && n < j1) {
        const size_t rw = row_of(c, b, h, n);
        if constexpr (F8) {
            if (tid < kHD / 8) {
                reinterpret_cast<u32x2_t *>(static_cast<unsigned char *>(c.k) + rw * RB)[tid] =
                    e5m2x8_encode(knr);
                reinterpret_cast<u32x2_t *>(static_cast<unsigned char *>(c.v) + rw * RB)[tid] =
                    e5m2x8_encode(*reinterpret_cast<const u16x8_t *>(vn + 8 * tid));
            }
        } else {
            if (tid < kHD / 8) {
                reinterpret_cast<uint4 *>(static_cast<uint16_t *>(c.k) + rw * kHD)[tid] =
                    reinterpret_cast<const uint4 *>(kn)[tid];
                reinterpret_cast<uint4 *>(static_cast<uint16_t *>(c.v) + rw * kHD)[tid] =
                    reinterpret_cast<const uint4 *>(vn)[tid];
            }
        }
        if (tid == 0) c.pos[(size_t)u * c.cap + n] = a.new_pos[b];
    }

    // ---------------- random eviction: rank this chunk's candidates
    if (a.presel) presel_rank<kPS>(a, u, s, b, h, j0, jsel, psel);
}

template <bool PAGED, int TC, bool F8>
static void launch_split_pk(const AttnArgs &a, bool pack2, size_t smem, hipStream_t s) {
    const dim3 grid(a.c.B * a.c.Hkv * a.nsplit), block(kFThreads);
    if (pack2)
        hipLaunchKernelGGL((split_kernel<PAGED, TC, true, F8>), grid, block, smem, s, a);
    else
        hipLaunchKernelGGL((split_kernel<PAGED, TC, false, F8>), grid, block, smem, s, a);
}

template <int TC, bool F8>
static hipError_t allow_split_smem(int most) {
    const void *fns[4] = {(const void *)split_kernel<false, TC, true, F8>,
                          (const void *)split_kernel<true, TC, true, F8>,
                          (const void *)split_kernel<false, TC, false, F8>,
                          (const void *)split_kernel<true, TC, false, F8>};
    hipError_t e = hipSuccess;
    for (const void *f : fns)
        if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, most);
    return e;
}

template <int TC>
static hipError_t launch_split_tc(const AttnArgs &a, bool e5m2, hipStream_t s) {
    static hipError_t attr = [] {
        const int most = (int)split_smem_bytes(kMaxGroup, TC);
        hipError_t e = allow_split_smem<TC, false>(most);
        return e == hipSuccess ? allow_split_smem<TC, true>(most) : e;
    }();
    if (attr != hipSuccess) return attr;
    const size_t smem = split_smem_bytes(a.c.G, TC);
    const bool pack2 = a.c.G <= 8, paged = a.c.bs > 0;
    if (e5m2)
        paged ? launch_split_pk<true, TC, true>(a, pack2, smem, s)
              : launch_split_pk<false, TC, true>(a, pack2, smem, s);
    else
        paged ? launch_split_pk<true, TC, false>(a, pack2, smem, s)
              : launch_split_pk<false, TC, false>(a, pack2, smem, s);
    return hipGetLastError();
}

hipError_t launch_split(const AttnArgs &a, bool e5m2, int max_len, hipStream_t s) {
    const int chunk = split_chunk(max_len, a.nsplit, max_len);
    if (chunk <= kFusedSmallT) return launch_split_tc<kFusedSmallT>(a, e5m2, s);
    // chunks longer than the large instance holds (attended lengths above
    // 64 splits of 1,024, the last slot of the largest capacity) take the
    // generic routine inside its workgroups
    return launch_split_tc<kFusedMaxT>(a, e5m2, s);
}

}  // namespace kvc
