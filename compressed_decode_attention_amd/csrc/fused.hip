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
//    K rows are loaded coalesced (4 rows x 256 B per wave instruction) and
//    turned into the B layout through a small swizzled LDS tile per wave;
//    bf16 x bf16 products are exact in fp32.
//  * the logits of the whole unit stay in LDS ([G][n+1] fp32), so the softmax
//    is exact (no online rescaling) and the H2O update uses the final
//    normaliser without a second pass over K.
//  * P.V runs as v_mfma_f32_16x16x16_bf16 over 16-key tiles.  V rows are
//    loaded coalesced (4 rows x 256 B per wave instruction): lane (r, c)
//    holds dims 8c..8c+7 of keys 4e + r, e = 0..3.  Taking MFMA k-index 4r + e
//    as key 4e + r and output column c of MFMA m as dim 8c + m, the B operand
//    of MFMA m is element m of the lane's four rows: a repack in registers.
//    P enters as a bf16 pair: rows 0..7 carry bf16(p), rows 8..15 the bf16
//    rounding of the remainder (G <= 8; two MFMAs per tile above that), so
//    their sum carries p to about 2^-17 relative and every product is exact
//    in the fp32 accumulator.
//  * selection runs on the LDS copies of pos / scores / random keys; the
//    common steady-state case (exactly one eviction) is an arg-min, the
//    general case an 8-bit radix select over 64-bit (key, position) words.
//  * compaction pairs evicted slots below n_out with kept slots at or above
//    n_out; the new token is written straight into its final slot.
// E5M2 caches (8-bit codes, bf16 activations) run the same kernel: a lane
// loads 8 codes (8 B) where it loads 8 bf16 values (16 B) for bf16, which
// keeps every lane's share of a row the same, and widens them to bf16 with
// the hardware conversion (exact: every E5M2 value is a bf16 value) before
// the staging and the repack.  The new token is rounded to E5M2 once, and
// that rounded row is what is attended and stored.
// Units longer than the launch's LDS capacity (or a full cache) take the
// generic per-unit routines inside the same workgroup, so results never
// depend on the length hint.
#include "mfma_tiles.h"

namespace kvc {

struct FusedSmall {
    float m[kMaxGroup];      // row maxima of the logits
    float l[kMaxGroup];      // softmax normalisers
    float il[kMaxGroup];     // 1 / l
    float wred[kFWaves][kMaxGroup];
    float wmax[kFWaves][kMaxGroup];   // each wave's logit maxima, then its output factors
    int hist[256];
    int red[kFWaves * 2];
    int pmax[kFWaves];       // newest position seen by each wave
    int posmax;
    int r_nc[kFWaves], r_nd[kFWaves], r_ds[kFWaves], r_arg[kFWaves];
    uint32_t mn_hi[kFWaves], mn_lo[kFWaves];
    int sh[8];
    int blk[kFusedMaxT / 16 + 1];   // paged: block ids of the attended slots
    u16x8_t knew[kHD / 8];          // the new token's key row (as attended)
    alignas(16) u32x2_t kenc[kHD / 8];   // E5M2: the new token's stored K row
    alignas(16) u32x2_t venc[kHD / 8];   // ... and V row
};

// Bytes of the per-wave K staging tiles, or of the selection keys and flags
// that reuse them, whichever is larger.
__host__ __device__ constexpr size_t stage_region_bytes(int tc) {
    return (size_t)kFWaves * kStageBytes > (size_t)tc * 5 ? (size_t)kFWaves * kStageBytes
                                                          : ((size_t)tc * 5 + 15) / 16 * 16;
}

// 64-bit ranking word: larger = better (kept first); unique inside a unit
__device__ inline uint64_t rank_word(uint32_t primary, int32_t pos) {
    return ((uint64_t)primary << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}

// What the step kernel reads from its arguments: one copy of the cache's
// description and the policy, nothing twice (the kernel's scalar registers
// hold what it keeps live; a duplicate would cost registers or spills).
struct FusedParams {
    CacheDev c;
    const int32_t *new_pos;
    const void *q, *k_new, *v_new;
    float *out;
    float *scores;        // may be null
    float *logits;        // scratch of the fallback routines
    int32_t *keep_slots, *n_out;
    float scale, decay;
    int kind, n_sink, n_heavy, n_recent, prompt_len, n_keep;
    uint32_t step;
    uint64_t seed;
};

// Units longer than the launch's LDS capacity (or a full cache): the generic
// per-unit routines, with their arguments rebuilt from the kernel's.
template <int MODE, bool F8>
__device__ void fused_generic(const FusedParams &p, int u, unsigned char *smem) {
    using TK = typename std::conditional<F8, e5m2_t, uint16_t>::type;
    AttnArgs a{};
    a.c = p.c;
    a.new_pos = p.new_pos;
    a.q = p.q;
    a.k_new = p.k_new;
    a.v_new = p.v_new;
    a.out = p.out;
    a.scores = p.scores;
    a.scale = p.scale;
    a.decay = p.decay;
    a.nsplit = 1;
    a.max_len = p.c.cap + 1;
    a.append = true;
    a.part = nullptr;
    a.logits = p.logits;
    attn_unit_generic<TK, kHD>(a, u, 0, *reinterpret_cast<AttnLds<kHD> *>(smem));
    if (MODE == kModeAttn) return;
    __syncthreads();
    SelectArgs sa{};
    sa.c = p.c;
    sa.kind = p.kind;
    sa.n_sink = p.n_sink;
    sa.n_heavy = p.n_heavy;
    sa.n_recent = p.n_recent;
    sa.prompt_len = p.prompt_len;
    sa.n_keep = p.n_keep;
    sa.seed = p.seed;
    sa.step = p.step;
    sa.scores = p.scores;
    sa.keep_slots = p.keep_slots;
    sa.n_out = p.n_out;
    select_unit<1>(sa, u, *reinterpret_cast<SelLds<1> *>(smem));
    __syncthreads();
    CompactArgs ca{};
    ca.c = p.c;
    ca.keep_slots = p.keep_slots;
    ca.n_out = p.n_out;
    ca.scores = p.scores;
    ca.ordered = false;
    ca.dst = p.c;
    compact_unit<TK, kHD>(ca, u, *reinterpret_cast<CompLds *>(smem));
}

// PACK2: G <= 8, so one P.V MFMA carries both bf16 parts of p (rows 0..7 and
// 8..15); otherwise each tile takes two MFMAs per dim block.  F8: E5M2 cache.
template <int MODE, bool PAGED, int TC, bool PACK2, bool F8>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void fused_kernel(FusedParams fp) {
    using Row = typename KvRow<F8>::type;
    constexpr int RB = F8 ? kHD : 2 * kHD;   // bytes of one cached K or V row
    constexpr int NP = RB / 16;                // its 16-byte parts
    constexpr int DK = F8 ? kDK8 : kDK;
    constexpr int DV = F8 ? kDV8 : kDV;
    // most K tiles / V groups one wave handles: fixed trip counts let the
    // loops unroll into straight-line code with exact load/wait pairing
    constexpr int kNTW = (TC / 16 + kFWaves - 1) / kFWaves;
    extern __shared__ __align__(16) unsigned char smem[];
    const FusedParams &a = fp;
    const CacheDev &c = fp.c;
    const int u = blockIdx.x;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane >> 4, col = lane & 15;
    const int G = c.G;

    // the queries do not depend on the slot count: their loads go first
    u16x8_t qa[4];
    load_q(qa, static_cast<const uint16_t *>(a.q) + ((size_t)b * c.Hq + (size_t)h * G + col) * kHD,
           col < G, r);
    // contiguous caches: the wave's first K tile goes out before the slot
    // count is known, through a resource over the whole capacity (rows at or
    // past n may hold old data: their logits are replaced by -inf, the new
    // token's row is overwritten in staging, and rows past the capacity read
    // zeros); a second early tile would spill
    using RowT = typename KvRow<F8>::type;
    constexpr int RBk = F8 ? kHD : 2 * kHD;
    constexpr int DK0 = 1;
    RowT kb0[DK0][4];
    if constexpr (!PAGED) {
        const TileSrc<false, RBk> src0(c, b, h, c.cap, nullptr);
        const int lane_off0 = (lane >> 4) * RBk + KvRow<F8>::kBytes * (lane & 15);
#pragma unroll
        for (int d = 0; d < DK0; ++d) {
            __amdgpu_buffer_rsrc_t rs;
            int toff;
            src0.tile(w + kFWaves * d, false, rs, toff);
#pragma unroll
            for (int k = 0; k < 4; ++k) kb0[d][k] = buffer_row<F8, false>(rs, lane_off0 + toff + 4 * RBk * k);
        }
    }
    const int n = __builtin_amdgcn_readfirstlane(load_count(c, u, tid == 0));
    const int T = n + 1;
    if (T > TC || n >= c.cap) {
        fused_generic<MODE, F8>(fp, u, smem);
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

    const unsigned char *K = static_cast<const unsigned char *>(c.k);
    const unsigned char *V = static_cast<const unsigned char *>(c.v);
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new) + (size_t)u * kHD;
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new) + (size_t)u * kHD;
    int32_t *P = c.pos + (size_t)u * c.cap;
    float *S = a.scores ? a.scores + (size_t)u * c.cap : nullptr;
    const bool h2o = S != nullptr;
    const int32_t npos = a.new_pos[b];

    // positions, old scores and the new key row are requested together, before
    // any of them is waited for and ahead of the first K tiles (fixed trip
    // count, in-bounds indexes; without scores the positions are read twice
    // and the copy is ignored, which keeps every load unconditional)
    constexpr int kNS = (TC + kFThreads - 1) / kFThreads;
    const float *Ssrc = h2o ? S : reinterpret_cast<const float *>(P);
    int32_t pst[kNS];
    float sst[kNS];
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
        const int j = tid + kFThreads * i;
        const int jj = j < n ? j : 0;   // cap >= 1
        pst[i] = P[jj];
        sst[i] = Ssrc[jj];
    }
    const u16x8_t knr = reinterpret_cast<const u16x8_t *>(kn)[lane & 15];
    if constexpr (PAGED) {
        // the sequence's block ids, checked once (an id outside the pool is
        // reported and replaced by block 0); every K load needs them
        const int nb = (n + c.bs - 1) / c.bs;
        const int32_t *bt = c.bt + (size_t)b * c.max_blocks;
        for (int i = tid; i < nb; i += kFThreads) {
            int blk = bt[i];
            if ((unsigned)blk >= (unsigned)c.num_blocks) {
                raise_flag(c, KVC_FLAG_BAD_BLOCK);
                blk = 0;
            }
            sm.blk[i] = blk;
        }
        __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---------------- logits: MFMA 16x16x32 bf16, A = queries, B = 16 keys
    const int ntiles = (T + 15) >> 4;
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const TileSrc<PAGED, RB> src(c, b, h, n, sm.blk);
    // K tile t = slots 16t .. 16t+15.  Loads are coalesced: instruction k of a
    // lane reads 16 B (chunk 'col') of row 4k + r, so one wave instruction
    // covers 4 whole rows; rows at or past n come back as zeros, and the lane
    // that holds row n takes the new token's chunk instead.  The tile then goes
    // through the wave's LDS staging buffer, chunk c of row q stored at slot
    // c ^ q (conflict-free on both sides), and comes back in the MFMA B
    // layout: key = col, 8 dims per 16-lane group.
    const int lane_off = r * RB + KvRow<F8>::kBytes * col;
    auto kload = [&](int t, int k) -> Row {
        __amdgpu_buffer_rsrc_t rs;
        int toff;
        src.tile(t, false, rs, toff);
        return buffer_row<F8, PAGED>(rs, lane_off + toff + 4 * RB * k);
    };
    const int tn = n >> 4, qn = n & 15;   // tile and row of the new token
    // the scale as a vector register: held across the K loop, it would
    // otherwise pin a scalar register group that the loop keeps reloading
    float scale;
    asm volatile("v_mov_b32 %0, %1" : "=v"(scale) : "s"(a.scale));
    // where this lane stores logit row 4r + ii of tile t: lgp[ii] + 16 t.  The
    // padding rows (4r + ii >= G) store into this wave's own staging tile
    // instead, every such lane to the same word (free at that point: LDS
    // operations of a wave complete in order; 16 t + ii < 1,024 words), so the
    // stores need no mask
    static_assert(16 * (TC / 16) * 4 <= (int)kStageBytes, "dummy logit stores stay in the wave's tile");
    float *lgp[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int g = 4 * r + ii;
        lgp[ii] = (g < G) ? lg + g * LD + (((col & 3) << 2) | (col >> 2))
                          : reinterpret_cast<float *>(stage) + ii;
    }
    int pmax = -1;
    {
        Row kb[DK][4];
#pragma unroll
        for (int d = 0; d < DK; ++d)
#pragma unroll
            for (int k = 0; k < 4; ++k) kb[d][k] = (!PAGED && d < DK0) ? kb0[d < DK0 ? d : 0][k] : kload(w + kFWaves * d, k);
        // the staged values land in LDS while the first K tiles are in flight.
        // No branch: every index at or past n writes slot n with the new
        // token's position and a zero score, the values slot n takes anyway.
#pragma unroll
        for (int i = 0; i < kNS; ++i) {
            const int j = tid + kFThreads * i;
            const bool old_slot = j < n;
            const int jw = old_slot ? j : n;
            const int32_t pj = old_slot ? pst[i] : npos;
            pos_s[jw] = pj;
            pmax = max(pmax, pj);
            sc_s[jw] = (h2o && old_slot) ? sst[i] : 0.f;
        }
        if (tid < kHD / 8) {
            if constexpr (F8) {
                const u32x2_t ke = e5m2x8_encode(knr);
                sm.kenc[tid] = ke;
                sm.knew[tid] = e5m2x8_to_bf16(ke);
            } else {
                sm.knew[tid] = knr;
            }
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
            // tiles past the unit hold no key (uniform test); inside the
            // last tile, keys past T get -inf, so the softmax weighs them 0
            if (t < ntiles) {
                const int j = 16 * t + col;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const float z = (j < T) ? acc[ii] * scale : -INFINITY;
                    lgp[ii][16 * t] = z;
                    mx[ii] = z > mx[ii] ? z : mx[ii];
                }
            }
        }
    }
    // V rows do not depend on the softmax: start streaming them now.  Wave w
    // takes the same tiles as for K; instruction k of a lane reads chunk col
    // of row 16t + 4k + r (zeros at or past n; row n is the new token's).
    auto vload = [&](int t, int k) -> Row {
        __amdgpu_buffer_rsrc_t rs;
        int toff;
        src.tile(t, true, rs, toff);
        return buffer_row<F8, PAGED>(rs, lane_off + toff + 4 * RB * k);
    };
    u16x8_t vnc = *reinterpret_cast<const u16x8_t *>(vn + 8 * col);
    if constexpr (F8) {
        const u32x2_t ve = e5m2x8_encode(vnc);
        if (tid < kHD / 8) sm.venc[tid] = ve;   // lanes 0..15: col = tid
        vnc = e5m2x8_to_bf16(ve);
    }
    Row vb[DV][4];
#pragma unroll
    for (int d = 0; d < DV; ++d)
#pragma unroll
        for (int k = 0; k < 4; ++k) vb[d][k] = vload(w + kFWaves * d, k);
    // row maxima (16-lane groups share a query head set, then across waves),
    // and the newest position of the unit
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float m = mx[i];
        m = fmaxf(m, lane_xor_f<8>(m));
        m = fmaxf(m, lane_xor_f<4>(m));
        m = fmaxf(m, lane_xor_f<2>(m));
        m = fmaxf(m, lane_xor_f<1>(m));
        if (col == 0 && 4 * r + i < G) sm.wmax[w][4 * r + i] = m;
    }
    pmax = wave_max_iv(pmax);
    if (lane == 0) sm.pmax[w] = pmax;
    // Each wave weighs its own tiles against its own maxima, so P.V starts
    // without waiting for the other waves; the waves' sums are rescaled to
    // the unit's maxima once P.V is done (the same exact softmax).  The
    // maxima above were written by lanes of this wave: LDS operations of a
    // wave complete in order.  E5M2 caches only: the bf16 instances gain
    // nothing measurable from it and the paged one would spill more, while
    // both modes and both layouts of a dtype must compute alike (their
    // results match bit for bit), so bf16 keeps one set of maxima per unit.
    constexpr bool kWaveMax = F8;
    if constexpr (kWaveMax) {
        __builtin_amdgcn_wave_barrier();
    } else {
        __syncthreads();
        if (tid < G) {
            float m = sm.wmax[0][tid];
            for (int v = 1; v < kFWaves; ++v) m = fmaxf(m, sm.wmax[v][tid]);
            sm.m[tid] = m;
        }
        __syncthreads();
    }

    // ---------------- P.V: MFMA 16x16x16 bf16 per 16-key tile.
    // A row (lane col) = query head ga; with G <= 8 rows 8..15 repeat heads
    // 0..7 and carry the low bf16 part of p.  The lane computes the weights
    // it feeds, w = exp(z - m_g) for keys 16t + 4e + r, stores them back for
    // the H2O update (high-part lanes only) and sums them for l_g.
    f32x4_t oacc[8];
#pragma unroll
    for (int m8 = 0; m8 < 8; ++m8) oacc[m8] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    constexpr bool pack2 = PACK2;
    const int ga = pack2 ? (col & 7) : col;
    const bool arow = ga < G;
    const bool hi_lane = !pack2 || col < 8;
    const float mrow = arow ? (kWaveMax ? sm.wmax[w][ga] : sm.m[ga]) : 0.f;
    float *lrow = lg + (arow ? ga : 0) * LD;
#pragma unroll
    for (int i = 0; i < kNTW; ++i) {
        const int t = w + kFWaves * i;
        const int c0 = 16 * t + 4 * r;         // lg_col of key 16t + r
        // logits of keys past T are -inf (weight 0); tiles past the unit
        // (uniform test) and the padding rows of A weigh nothing
        f32x4_t p = {0.f, 0.f, 0.f, 0.f};
        if (t < ntiles) {
            const f32x4_t z = *reinterpret_cast<const f32x4_t *>(lrow + c0);
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = arow ? __expf(z[e] - mrow) : 0.f;
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
        // B operand of MFMA m: element m of the four rows this lane loaded;
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
    if (pack2)   // rows 8..15 (lanes 32..63) hold the low parts of rows 0..7
#pragma unroll
        for (int m8 = 0; m8 < 8; ++m8)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) oacc[m8][ii] = pair_sum32(oacc[m8][ii]);
    // lanes col, col+16, col+32, col+48 hold partial sums of A row col
    lsum = pair_sum16(lsum);
    lsum = pair_sum32(lsum);
    if (lane < G) sm.wred[w][lane] = lsum;
    __syncthreads();   // weights in lg are final, partial row sums written
    if (tid < G && !kWaveMax) {
        // one maximum for the unit: every wave's factor is 1 / l
        float l = 0.f;
        for (int v = 0; v < kFWaves; ++v) l += sm.wred[v][tid];
        const float il = 1.f / l;
        for (int v = 0; v < kFWaves; ++v) sm.wmax[v][tid] = il;
        sm.l[tid] = l;
        sm.il[tid] = il;
    }
    if (tid < G && kWaveMax) {
        // the unit's maximum, each wave's factor exp(m_w - M), the
        // normaliser; the factor over the normaliser then scales both the
        // wave's weights (H2O) and its partial output
        float M = -INFINITY;
        for (int v = 0; v < kFWaves; ++v) M = fmaxf(M, sm.wmax[v][tid]);
        float l = 0.f;
        float f[kFWaves];
        for (int v = 0; v < kFWaves; ++v) {
            const float mv = sm.wmax[v][tid];
            f[v] = (mv == -INFINITY) ? 0.f : __expf(mv - M);
            l += sm.wred[v][tid] * f[v];
        }
        const float il = 1.f / l;
        for (int v = 0; v < kFWaves; ++v) sm.wmax[v][tid] = f[v] * il;
        sm.m[tid] = M;
        sm.l[tid] = l;
        sm.il[tid] = il;
    }
    if (tid == 64) {
        int pm = sm.pmax[0];
        for (int v = 1; v < kFWaves; ++v) pm = max(pm, sm.pmax[v]);
        sm.posmax = pm;
    }
    __syncthreads();

    // ---------------- H2O: accumulated attention with the final normaliser.
    // Contiguous caches, step mode: the same pass classifies every entry for
    // the selection and keeps the thread's counts and worst candidate in
    // registers (the staging bytes, where the flags and keys would go, still
    // hold the partial outputs); each wave's summary goes out before the
    // output pass's barrier, so the usual single eviction needs no pass and
    // no barrier of its own.  Paged caches classify after the output pass, as
    // the registers held across it would spill there; both orders select the
    // same entries.
    constexpr bool kFold = MODE != kModeAttn && !PAGED;
    const FusedParams &sa = fp;
    const int L = sm.posmax + 1;
    int ncand = 0, ndrop = 0, dslot = -1, barg = -1;
    uint64_t best = ~0ull;
    // the entry's class; a candidate's ranking key (smaller is evicted first)
    auto classify = [&](int j, float sj, uint32_t &key) -> uint8_t {
        const int32_t p = pos_s[j];
        uint8_t k = kKeep;
        if (sa.kind == KVC_POLICY_STREAMING)
            k = (p < sa.n_sink || (int64_t)p >= (int64_t)L - sa.n_recent) ? kKeep : kDrop;
        else if (sa.kind == KVC_POLICY_H2O)
            k = ((int64_t)p >= (int64_t)L - sa.n_recent) ? kKeep : kCand;
        else if (sa.kind == KVC_POLICY_RANDOM)
            k = (p < sa.prompt_len) ? kKeep : kCand;
        if (k == kCand)
            key = (sa.kind == KVC_POLICY_H2O)
                      ? float_order_bits(sj)
                      : ~philox_word0((uint32_t)p, sa.step, (uint32_t)h, (uint32_t)b,
                                      (uint32_t)(sa.seed & 0xFFFFFFFFu), (uint32_t)(sa.seed >> 32));
        return k;
    };
    auto tally = [&](int j, float sj) {
        uint32_t key = 0;
        const uint8_t k = classify(j, sj, key);
        if (k == kCand) {
            ++ncand;
            const uint64_t wd = rank_word(key, pos_s[j]);
            if (barg < 0 || wd < best) {
                best = wd;
                barg = j;
            }
        } else if (k == kDrop) {
            ++ndrop;
            dslot = max(dslot, j);
        }
    };
    if (h2o) {
        for (int j = tid; j < T; j += kFThreads) {
            float ps = 0.f;
            const int jc = lg_col(j);
            const int wj = (j >> 4) % kFWaves;   // the wave that weighed tile j / 16
            if constexpr (PACK2) {
                // G <= 8: every head's load in flight at once; heads past G
                // leave the sum as it is (the same fused multiply-adds in the
                // same order as the loop below)
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    const int gg = g < G ? g : 0;
                    const float t = __builtin_fmaf(lg[gg * LD + jc], sm.wmax[wj][gg], ps);
                    ps = g < G ? t : ps;
                }
            } else {
                for (int g = 0; g < G; ++g) ps += lg[g * LD + jc] * sm.wmax[wj][g];
            }
            const float sj = score_update((j < n) ? sc_s[j] : 0.f, ps, a.decay);
            sc_s[j] = sj;
            if constexpr (kFold) tally(j, sj);
        }
    } else if constexpr (kFold) {
        for (int j = tid; j < T; j += kFThreads) tally(j, sc_s[j]);
    }
    // each wave's counts and worst candidate into the small LDS block
    auto wave_summary = [&]() {
        ncand = wave_sum_iv(ncand);
        ndrop = wave_sum_iv(ndrop);
        dslot = wave_max_iv(dslot);
        auto arg_step = [&](uint32_t hi, uint32_t lo, int oa) {
            const uint64_t ob = ((uint64_t)hi << 32) | lo;
            if (ob < best || (ob == best && (unsigned)oa < (unsigned)barg)) {
                best = ob;
                barg = oa;
            }
        };
#define KVC_ARG_STEP(M) \
    arg_step(lane_xor<M>((uint32_t)(best >> 32)), lane_xor<M>((uint32_t)best), (int)lane_xor<M>((uint32_t)barg))
        KVC_ARG_STEP(32);
        KVC_ARG_STEP(16);
        KVC_ARG_STEP(8);
        KVC_ARG_STEP(4);
        KVC_ARG_STEP(2);
        KVC_ARG_STEP(1);
#undef KVC_ARG_STEP
        if (lane == 0) {
            sm.r_nc[w] = ncand;
            sm.r_nd[w] = ndrop;
            sm.r_ds[w] = dslot;
            sm.r_arg[w] = barg;
            sm.mn_hi[w] = (uint32_t)(best >> 32);
            sm.mn_lo[w] = (uint32_t)best;
        }
    };
    if constexpr (kFold) wave_summary();

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
            if (g < G && (!pack2 || r < 2)) {
                float *dst = opart + ((size_t)w * G + g) * kHD + 8 * col;
#pragma unroll
                for (int m8 = 0; m8 < 8; ++m8) dst[m8] = oacc[m8][i];
            }
        }
        __syncthreads();
        float *outp = a.out + ((size_t)b * c.Hq + (size_t)h * G) * kHD;
        // four consecutive elements of one head per thread (16-byte LDS
        // reads and global stores; the partials' bases are 16-byte aligned)
        for (int e = 4 * tid; e < G * kHD; e += 4 * kFThreads) {
            const int g = e / kHD;
            f32x4_t o = *reinterpret_cast<const f32x4_t *>(opart + e) * sm.wmax[0][g];
            for (int v = 1; v < kFWaves; ++v)
                o += *reinterpret_cast<const f32x4_t *>(opart + (size_t)v * G * kHD + e) * sm.wmax[v][g];
            *reinterpret_cast<f32x4_t *>(outp + e) = o;
        }
    }

    unsigned char *Kw = static_cast<unsigned char *>(c.k);
    unsigned char *Vw = static_cast<unsigned char *>(c.v);
    // 16-byte part p of the new token's stored K / V row
    auto knew_part = [&](int p) -> uint4 {
        if constexpr (F8) return reinterpret_cast<const uint4 *>(sm.kenc)[p];
        else return reinterpret_cast<const uint4 *>(kn)[p];
    };
    auto vnew_part = [&](int p) -> uint4 {
        if constexpr (F8) return reinterpret_cast<const uint4 *>(sm.venc)[p];
        else return reinterpret_cast<const uint4 *>(vn)[p];
    };
    auto store_new = [&](int slot) {   // lanes 0..NP-1
        const size_t rw = row_of(c, b, h, slot) * RB;
        reinterpret_cast<uint4 *>(Kw + rw)[tid] = knew_part(tid);
        reinterpret_cast<uint4 *>(Vw + rw)[tid] = vnew_part(tid);
    };

    if (MODE == kModeAttn) {
        // append the new token at slot n, write every score back
        if (h2o)
            for (int j = tid; j < T; j += kFThreads) S[j] = sc_s[j];
        if (tid < NP) store_new(n);
        if (tid == 0) {
            P[n] = npos;
            c.n_slots[u] = n + 1;
        }
        return;
    }

    // ================= selection =================
    if constexpr (!kFold) {
        __syncthreads();   // the output pass is done with the staging bytes
        for (int j = tid; j < T; j += kFThreads) {
            uint32_t key = 0;
            const uint8_t k = classify(j, sc_s[j], key);
            if (k == kCand) {
                key_s[j] = key;
                ++ncand;
                const uint64_t wd = rank_word(key, pos_s[j]);
                if (barg < 0 || wd < best) {
                    best = wd;
                    barg = j;
                }
            } else if (k == kDrop) {
                ++ndrop;
                dslot = max(dslot, j);
            }
            flg_s[j] = k;
        }
        wave_summary();
        __syncthreads();
    }
    // the waves' summaries
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
        if (sm.r_arg[v] >= 0 && (barg < 0 || ob < best)) {
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
        if (dst_new >= 0 && tid < NP) store_new(dst_new);
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

    // ---- general case: flags and keys into the staging bytes (once every
    // wave is done with them) when the tally did not write them; then finish
    // the candidates' flags and hole-fill
    if constexpr (kFold) {
        __syncthreads();
        for (int j = tid; j < T; j += kFThreads) {
            uint32_t key = 0;
            const uint8_t k = classify(j, sc_s[j], key);
            if (k == kCand) key_s[j] = key;
            flg_s[j] = k;
        }
        __syncthreads();
    }
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
                        if ((wd & mask) == prefix) hist_add_wave(sm.hist, (int)((wd >> shift) & 255));
                    }
                __syncthreads();
                if (tid < 64) radix_pick_bin(sm.hist, krem, sm.sh[0], sm.sh[1], sm.sh[2]);
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
    for (int e = tid; e < moves * NP; e += kFThreads) {
        const int i = e / NP, part = e % NP;
        const int d = hole[i], s = srcl[i];
        const size_t rd = row_of(c, b, h, d) * RB;
        const size_t rs = row_of(c, b, h, s) * RB;
        reinterpret_cast<uint4 *>(Kw + rd)[part] =
            (s == n) ? knew_part(part) : reinterpret_cast<const uint4 *>(K + rs)[part];
        reinterpret_cast<uint4 *>(Vw + rd)[part] =
            (s == n) ? vnew_part(part) : reinterpret_cast<const uint4 *>(V + rs)[part];
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
    if (n < n_out && tid < NP) store_new(n);
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

static FusedParams params_of(const FusedArgs &fa) {
    FusedParams p{};
    p.c = fa.attn.c;
    p.new_pos = fa.attn.new_pos;
    p.q = fa.attn.q;
    p.k_new = fa.attn.k_new;
    p.v_new = fa.attn.v_new;
    p.out = fa.attn.out;
    p.scores = fa.attn.scores;
    p.logits = fa.attn.logits;
    p.keep_slots = fa.sel.keep_slots;
    p.n_out = fa.sel.n_out;
    p.scale = fa.attn.scale;
    p.decay = fa.attn.decay;
    p.kind = fa.sel.kind;
    p.n_sink = fa.sel.n_sink;
    p.n_heavy = fa.sel.n_heavy;
    p.n_recent = fa.sel.n_recent;
    p.prompt_len = fa.sel.prompt_len;
    p.n_keep = fa.sel.n_keep;
    p.step = fa.sel.step;
    p.seed = fa.sel.seed;
    return p;
}

template <int MODE, bool PAGED, int TC, bool F8>
static void launch_pk(const FusedArgs &fa, bool pack2, size_t smem, hipStream_t s) {
    const dim3 grid(fa.attn.c.B * fa.attn.c.Hkv), block(kFThreads);
    const FusedParams p = params_of(fa);
    if (pack2)
        hipLaunchKernelGGL((fused_kernel<MODE, PAGED, TC, true, F8>), grid, block, smem, s, p);
    else
        hipLaunchKernelGGL((fused_kernel<MODE, PAGED, TC, false, F8>), grid, block, smem, s, p);
}

// every instantiation of one LDS capacity may use its largest LDS size
template <int TC, bool F8>
static hipError_t allow_smem(int most) {
    const void *fns[8] = {(const void *)fused_kernel<kModeAttn, false, TC, true, F8>,
                          (const void *)fused_kernel<kModeStep, false, TC, true, F8>,
                          (const void *)fused_kernel<kModeAttn, true, TC, true, F8>,
                          (const void *)fused_kernel<kModeStep, true, TC, true, F8>,
                          (const void *)fused_kernel<kModeAttn, false, TC, false, F8>,
                          (const void *)fused_kernel<kModeStep, false, TC, false, F8>,
                          (const void *)fused_kernel<kModeAttn, true, TC, false, F8>,
                          (const void *)fused_kernel<kModeStep, true, TC, false, F8>};
    hipError_t e = hipSuccess;
    for (const void *f : fns)
        if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, most);
    return e;
}

template <int TC, bool F8>
static void launch_mode(const FusedArgs &fa, int mode, bool pack2, size_t smem, hipStream_t s) {
    const bool paged = fa.attn.c.bs > 0;
    if (mode == kModeAttn)
        paged ? launch_pk<kModeAttn, true, TC, F8>(fa, pack2, smem, s)
              : launch_pk<kModeAttn, false, TC, F8>(fa, pack2, smem, s);
    else
        paged ? launch_pk<kModeStep, true, TC, F8>(fa, pack2, smem, s)
              : launch_pk<kModeStep, false, TC, F8>(fa, pack2, smem, s);
}

template <int TC>
static hipError_t launch_tc(const FusedArgs &fa, int mode, size_t smem, hipStream_t s) {
    static hipError_t attr = [] {
        const int most = (int)fused_smem_bytes(kMaxGroup, TC);
        hipError_t e = allow_smem<TC, false>(most);
        return e == hipSuccess ? allow_smem<TC, true>(most) : e;
    }();
    if (attr != hipSuccess) return attr;
    const bool pack2 = fa.attn.c.G <= 8;
    if (fa.e5m2)
        launch_mode<TC, true>(fa, mode, pack2, smem, s);
    else
        launch_mode<TC, false>(fa, mode, pack2, smem, s);
    return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs &fa, int mode, hipStream_t s) {
    const size_t smem = fused_smem_bytes(fa.attn.c.G, fa.tcap);
    if (fa.tcap == kFusedSmallT) return launch_tc<kFusedSmallT>(fa, mode, smem, s);
    if (fa.tcap == kFusedMaxT) return launch_tc<kFusedMaxT>(fa, mode, smem, s);
    return hipErrorInvalidValue;
}

}  // namespace kvc
