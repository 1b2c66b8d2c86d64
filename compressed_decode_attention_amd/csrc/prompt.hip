// prompt.hip -- H2O scores from a block of causal query rows, on the matrix
// cores (bf16, head_dim 128).
//
// What it computes (guide, sections 2 and 16, "the 4 methods" and "prefill,
// decode, TP": H2O accumulates the attention each cached token receives, and
// the prompt's own causal attention is where that starts):
//   for every unit (b, h), query row r of head g (g in h's group) and every
//   slot j with pos_j <= q_pos[b, r]:  p = softmax_j(scale q_{r,g} . k_j),
//   scores[b, h, j] += sum_{r, g} p.
// Rows are the (position, head) pairs r * G + g; a row that sees no slot adds
// nothing.
//
// Two passes, both exact (no approximation of the softmax):
//  1. statistics: one workgroup per 256 rows of a unit.  K tiles of 64 slots
//     are staged in LDS (XOR swizzle, conflict-free reads) and enter
//     v_mfma_f32_16x16x32_bf16 as the A operand; the rows are the B operand,
//     held in registers (64 rows per wave, so each A operand read from LDS
//     feeds four row tiles).  Each lane keeps a sum of exp2(c2 * dot + nb)
//     against a reference nb that moves only when a group of terms passes a
//     cap (2^64): no maximum or rescale per group, one wave-uniform test per
//     two 16-slot tiles instead (the scale is made positive, so references
//     follow the largest dot products); four lanes merge into the row's
//     log-sum-exp, written to the workspace.
//  2. scores: one workgroup per 256 slots of a unit.  The slots are the B
//     operand, held in registers (64 slots per wave); query tiles (64
//     consecutive positions of one head, so a tile's rows share one stride
//     through q) are staged in LDS.  Each lane sums exp2(c2 * dot - lse) over
//     its 16 rows of a tile in fp32, adds that to an fp64 column sum (a fixed
//     order: the scores are deterministic), and one lane per slot adds the
//     total to the score.  A wave skips the row tiles whose positions all
//     precede its own slots.
// Tiles that no row of a block can see (from the positions alone) are
// skipped, which halves the work of a causal prompt; tiles that every row sees
// whole (most of a causal triangle) run a mask-free variant of the tile's
// straight-line code (the choice is uniform per tile, so neither variant
// branches inside).  The softmax runs in base 2 (scale * log2(e) folded into
// one factor c2, the row statistic a base-2 log-sum-exp), so an element costs
// one multiply-add and one v_exp_f32.  Each slot tile's smallest and largest
// position come from a wave reduction (a wave's 64 lanes hold one tile).  All
// blocks of one unit run on one XCD (workgroups are dealt round-robin over the
// eight XCDs, so the rows they share can come from its L2), and both passes
// start every unit's longest block first: a causal prompt's blocks differ up
// to 32-fold in work, and a long block started last would run alone.  Per-tile
// loads are buffer loads with a scalar tile offset, their validity applied
// when the tile is staged, so the next tile's loads stay in flight through
// the current one.  Both kernels run three waves per SIMD: the larger
// register tiles halve the LDS reads and the per-tile fixed work (staging,
// barrier, next-tile search) per product, which pays more than a fourth wave.
#include "kvc_internal.h"

#include <limits.h>

#include <type_traits>

namespace kvc {

namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_p __attribute__((ext_vector_type(8)));

constexpr int kPThreads = 256;
constexpr int kPD = 128;          // head_dim of this path
constexpr int kRT = 4;            // pass 1: 16-row tiles per wave (B operands in registers)
constexpr int kStatRows = 64 * kRT;     // rows per workgroup, pass 1
constexpr int kST = 4;            // pass 2: 16-slot tiles per wave (B operands in registers)
constexpr int kScoreSlots = 64 * kST;   // slots per workgroup, pass 2
constexpr int kTile = 64;         // slots (pass 1) or rows (pass 2) staged per step
constexpr int kMaxRowTilesLds = 4096;   // pass 2: position tiles whose largest position fits in LDS
constexpr int kSG = 2;            // pass 1: 16-slot tiles per test of the references
constexpr float kLazyCap = 0x1p64f;   // pass 1: a group's sum past this moves the reference
constexpr float kNoRef = 0x1p100f;    // pass 1: offset before any slot is seen

__device__ inline bf16x8_p as_bf(u16x8_p x) { return __builtin_bit_cast(bf16x8_p, x); }

// Unit and block index of this workgroup; every block of a unit gets the same
// blockIdx % 8, hence the same XCD.  False for the padding of the last group.
// Workgroups start roughly in blockIdx order, so both passes deal them with
// the longest blocks first (for a causal prompt, a unit's last row block in
// the statistics pass and its first slot block in the scores pass), and the
// launch's tail is a short block.  Both do so within windows of W units per
// XCD (all their blocks, longest first, then the next window), so that the
// units whose rows are read at a time fit the XCD's L2 (K rows in the
// statistics pass, query rows in the scores pass).
constexpr int kStatsWindow = 8;
constexpr int kScoresWindow = 16;
template <int W, bool LONG_LAST>
__device__ inline bool windowed_unit_block(int nblk, int units, int &u, int &blk) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int groups = (units + 7) / 8;   // units per XCD
    const int full = groups / W, wsize = W * nblk;
    const int win = slot / wsize;
    const int within = win < full ? slot % wsize : slot - full * wsize;
    const int wc = win < full ? W : groups - full * W;   // units in this window
    blk = LONG_LAST ? nblk - 1 - within / wc : within / wc;
    u = 8 * (win * W + within % wc) + xcd;
    return u < units;
}

// byte offset of 16-byte chunk c of row q in a swizzled 64 x 256 B tile
__device__ inline int tile_off(int q, int c) { return q * 256 + ((c ^ (q & 15)) << 4); }

__device__ inline int block_max(int v, int *red) {
    v = wave_max_i(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
    for (int i = 1; i < kPThreads / 64; ++i) v = max(v, red[i]);
    __syncthreads();
    return v;
}

__device__ inline int block_min(int v, int *red) {
    v = wave_min_i(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
    for (int i = 1; i < kPThreads / 64; ++i) v = min(v, red[i]);
    __syncthreads();
    return v;
}

__device__ inline const uint16_t *q_row(const PromptArgs &a, int b, int h, int R) {
    const CacheDev &c = a.c;
    const int rr = R / c.G, g = R % c.G;
    return static_cast<const uint16_t *>(a.q_rows) +
           (((size_t)b * a.m_rows + rr) * c.Hq + (size_t)h * c.G + g) * kPD;
}

__device__ inline int row_pos(const PromptArgs &a, int b, int R) {
    return a.q_pos ? a.q_pos[(size_t)b * a.m_rows + R / a.c.G] : INT_MAX;
}

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }   // v_exp_f32

}  // namespace

// ---------------------------------------------------------------------------
// pass 1: log-sum-exp of every row over the slots it sees
// ---------------------------------------------------------------------------
// Software pipeline over the 64-slot tiles that some row of the block sees
// (found up front from each tile's smallest position): while the MFMAs run on
// one LDS buffer, the next active tile's K rows are already in registers on
// their way; one barrier per tile.
template <bool kPaged>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(3)))
void prompt_stats_kernel(PromptArgs a) {
    __shared__ __align__(16) unsigned char ktile[2][kTile * 256];
    __shared__ int kpos[2][kTile];
    __shared__ int red[kPThreads / 64];
    extern __shared__ int tile_pos[];   // [2][tiles of the capacity]: min, max position
    const CacheDev &c = a.c;
    const int nrows = a.m_rows * c.G;
    const int nblk = (nrows + kStatRows - 1) / kStatRows;
    int u, blk;
    if (!windowed_unit_block<kStatsWindow, true>(nblk, c.B * c.Hkv, u, blk)) return;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, col = lane & 15;
    const int n = load_count(c, u, tid == 0);
    const uint16_t *K = static_cast<const uint16_t *>(c.k);
    const int32_t *P = c.pos + (size_t)u * c.cap;
    const int ntile = (n + kTile - 1) / kTile;
    int *tmin_s = tile_pos, *tmax_s = tile_pos + (c.cap + kTile - 1) / kTile;
    // contiguous caches: buffer resources over the unit's n filled rows and
    // positions (loads past them return zeros; such slots are masked), so a
    // tile's loads take a scalar offset and one per-lane offset fixed for the
    // whole kernel
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(kPaged ? K : K + (size_t)u * c.cap * kPD, kPaged ? 0u : (uint32_t)n * (kPD * 2));
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(P, kPaged ? 0u : (uint32_t)n * 4);
    const int koff = (tid >> 4) * (kPD * 2) + 16 * (tid & 15);

    // B operands: kRT 16-row tiles per wave; lane (col, r) holds dims
    // 32c + 8r .. 32c + 8r + 7 of row col
    u16x8_p qb[kRT][4];
    int qp[kRT], Rw[kRT];
    int qmax = INT_MIN;
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
        const int R = blk * kStatRows + 16 * kRT * w + 16 * t + col;
        Rw[t] = R;
        const bool ok = R < nrows;
        const uint16_t *qr = q_row(a, b, h, ok ? R : 0);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            qb[t][c4] = ok ? *reinterpret_cast<const u16x8_p *>(qr + 32 * c4 + 8 * r)
                           : u16x8_p{0, 0, 0, 0, 0, 0, 0, 0};
        qp[t] = ok ? row_pos(a, b, R) : INT_MIN;
        qmax = max(qmax, qp[t]);
    }
    // smallest and largest position of every slot tile
    // (a wave's 64 lanes cover exactly one 64-slot tile: lanes past n
    // contribute nothing)
    static_assert(kTile == 64, "one wave per slot tile");
    for (int kt = w; kt < ntile; kt += kPThreads / 64) {
        const int j = kt * kTile + lane;
        const int p = j < n ? P[j] : INT_MAX;
        const int lo = wave_min_i(p);
        const int hi = wave_max_i(j < n ? p : INT_MIN);
        if (lane == 0) {
            tmin_s[kt] = lo;
            tmax_s[kt] = hi;
        }
    }
    qmax = block_max(qmax, red);   // (its barriers also publish the tile bounds)
    // smallest position of each 16-row tile of the wave, and whether the tile
    // holds no padding row (only such tiles may skip the mask)
    int qmin[kRT];
    bool rows_full[kRT];
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
        qmin[t] = __builtin_amdgcn_readfirstlane(wave_min_i(qp[t]));
        rows_full[t] = blk * kStatRows + 16 * kRT * w + 16 * t + 15 < nrows;
    }
    // a negative scale: the same logits from the negated query rows and
    // |scale|, so the running maxima of the raw dot products stay maxima of
    // the logits (bf16 negation is exact); a zero scale: every logit 0, from
    // zero rows and a positive factor (masked slots stay -inf, never -inf * 0)
    if (a.scale <= 0.f)
#pragma unroll
        for (int t = 0; t < kRT; ++t)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                qb[t][c4] = a.scale < 0.f ? qb[t][c4] ^ (uint16_t)0x8000 : u16x8_p{0, 0, 0, 0, 0, 0, 0, 0};
    const float c2 = (a.scale == 0.f ? 1.f : fabsf(a.scale)) * kLog2e;
    // next tile (from kt on) that some row of the block sees (uniform)
    auto next_active = [&](int kt) {
        while (kt < ntile && tmin_s[kt] > qmax) ++kt;
        return kt;
    };
    // the tile's K rows and positions into registers, unconditionally and in
    // bounds (paged caches read row n - 1 for slots past n, contiguous ones
    // zeros); such slots are masked.  Nothing reads the loaded values before
    // the next tile is staged, so the loads stay in flight while this tile
    // computes (the position of a slot past n is set when it is staged).
    u16x8_p pre[kTile / 16];
    int ppos = 0;
    auto fetch = [&](int kt) {
        const int j0 = kt * kTile;
        if constexpr (kPaged) {
#pragma unroll
            for (int pass = 0; pass < kTile / 16; ++pass) {
                const int j = min(j0 + 16 * pass + (tid >> 4), n - 1);
                pre[pass] = *reinterpret_cast<const u16x8_p *>(K + row_of(c, b, h, j) * kPD +
                                                               8 * (tid & 15));
            }
            ppos = P[min(j0 + (tid & (kTile - 1)), n - 1)];
        } else {
#pragma unroll
            for (int pass = 0; pass < kTile / 16; ++pass)
                pre[pass] = __builtin_bit_cast(
                    u16x8_p, __builtin_amdgcn_raw_buffer_load_b128(
                                 krs, koff, (j0 + 16 * pass) * (kPD * 2), 0));
            ppos = __builtin_amdgcn_raw_buffer_load_b32(prs, 4 * (tid & (kTile - 1)), 4 * j0, 0);
        }
    };

    // per lane and row tile: the sum of exp2(c2 * dot + nb) over the slots
    // seen, nb the base-2 offset of a reference that moves only when a
    // group's sum passes kLazyCap (a row's first visible group, or a logit
    // far above the reference); the log-sum-exp is log2(sum) - nb.  Before the
    // first visible group nb is kNoRef, so every visible term overflows and
    // sets the reference.
    float nb[kRT], ll[kRT];
#pragma unroll
    for (int t = 0; t < kRT; ++t) { nb[t] = kNoRef; ll[t] = 0.f; }
    int cur = next_active(0);
    if (cur < ntile) fetch(cur);
    int buf = 0;
    while (cur < ntile) {
        const int j0 = cur * kTile;
#pragma unroll
        for (int pass = 0; pass < kTile / 16; ++pass)
            *reinterpret_cast<u16x8_p *>(ktile[buf] + tile_off(16 * pass + (tid >> 4), tid & 15)) =
                pre[pass];
        if (tid < kTile) kpos[buf][tid] = j0 + tid < n ? ppos : INT_MAX;
        __syncthreads();
        const int nxt = next_active(cur + 1);
        if (nxt < ntile) fetch(nxt);   // lands while this tile computes
        // every row of a 16-row tile sees every slot of a filled 64-slot tile:
        // no mask (positions alone cannot tell padding, so fullness is checked)
        const bool slots_full = j0 + kTile <= n;
        const int kmax = tmax_s[cur];
        bool inner[kRT];
#pragma unroll
        for (int t = 0; t < kRT; ++t) inner[t] = slots_full && rows_full[t] && kmax <= qmin[t];
        // two 16-slot tiles' dot products at a time (8 per lane and row
        // tile, for each of the wave's row tiles), their terms against the
        // current references, and one wave-uniform test whether a reference
        // has to move.  The mask decision is uniform per tile, so each
        // variant is straight-line code.
        auto tile_body = [&](auto masked_c) {
            constexpr bool kMasked = decltype(masked_c)::value;
#pragma unroll
            for (int s0 = 0; s0 < kTile / 16; s0 += kSG) {
                f32x4_p acc[kRT][kSG];
#pragma unroll
                for (int s = 0; s < kSG; ++s) {
                    // A operand: lane (col, r) holds dims 32c + 8r.. of slot 16(s0+s) + col
                    const int q = 16 * (s0 + s) + col;
                    u16x8_p ka[4];
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4)
                        ka[c4] = *reinterpret_cast<const u16x8_p *>(ktile[buf] + tile_off(q, 4 * c4 + r));
                    // C[slot 4r + i][row col]
#pragma unroll
                    for (int t = 0; t < kRT; ++t) {
                        acc[t][s] = f32x4_p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4)
                            acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf(ka[c4]), as_bf(qb[t][c4]), acc[t][s], 0, 0, 0);
                    }
                }
                if constexpr (kMasked) {
                    // slots a row does not see (or past n) weigh nothing
#pragma unroll
                    for (int s = 0; s < kSG; ++s)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int jj = 16 * (s0 + s) + 4 * r + i;
                            const int kp = kpos[buf][jj];
                            const bool live = j0 + jj < n;
#pragma unroll
                            for (int t = 0; t < kRT; ++t)
                                acc[t][s][i] = (live && kp <= qp[t]) ? acc[t][s][i] : -INFINITY;
                        }
                }
                // the group's terms against the current reference (a masked
                // slot's term is exp2(-inf) = 0)
                float gs[kRT];
                bool move = false;
#pragma unroll
                for (int t = 0; t < kRT; ++t) {
                    float e[kSG][4];
#pragma unroll
                    for (int s = 0; s < kSG; ++s)
#pragma unroll
                        for (int i = 0; i < 4; ++i) e[s][i] = exp2_hw(fmaf(acc[t][s][i], c2, nb[t]));
                    gs[t] = ((e[0][0] + e[0][1]) + (e[0][2] + e[0][3])) +
                            ((e[1][0] + e[1][1]) + (e[1][2] + e[1][3]));
                    move = move || !(gs[t] < kLazyCap);
                }
                if (__builtin_amdgcn_ballot_w64(move) != 0) {
                    // some lane's group passed the cap: those lanes take the
                    // group's largest dot product as the new reference,
                    // rescale their sum and recount the group's terms
#pragma unroll
                    for (int t = 0; t < kRT; ++t) {
                        if (!(gs[t] < kLazyCap)) {
                            float gm = acc[t][0][0];
#pragma unroll
                            for (int s = 0; s < kSG; ++s)
#pragma unroll
                                for (int i = 0; i < 4; ++i) gm = fmaxf(gm, acc[t][s][i]);
                            const float nbn = -gm * c2;
                            float g2 = 0.f;
#pragma unroll
                            for (int s = 0; s < kSG; ++s)
#pragma unroll
                                for (int i = 0; i < 4; ++i) g2 += exp2_hw(fmaf(acc[t][s][i], c2, nbn));
                            ll[t] = ll[t] * exp2_hw(nbn - nb[t]) + g2;
                            nb[t] = nbn;
                        } else {
                            ll[t] += gs[t];
                        }
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < kRT; ++t) ll[t] += gs[t];
                }
            }
        };
        bool all_inner = true;
#pragma unroll
        for (int t = 0; t < kRT; ++t) all_inner = all_inner && inner[t];
        if (all_inner)
            tile_body(std::integral_constant<bool, false>());
        else
            tile_body(std::integral_constant<bool, true>());
        buf ^= 1;
        cur = nxt;
    }
    // merge the four lanes of each row (references as base-2 logits -nb),
    // then the log-sum-exp: the sum's binary exponent is split off exactly,
    // so the logarithm is taken of a mantissa in [1, 2)
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
        float ref = -nb[t], l = ll[t];
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float ro = __shfl_xor(ref, off, 64), lo = __shfl_xor(l, off, 64);
            const float rn = fmaxf(ref, ro);
            l = l * exp2_hw(ref - rn) + lo * exp2_hw(ro - rn);
            ref = rn;
        }
        if (r == 0 && Rw[t] < nrows) {
            int ex;
            const float mant = frexpf(l, &ex);   // l = mant * 2^ex, mant in [0.5, 1)
            a.lse[(size_t)u * nrows + Rw[t]] =
                (l > 0.f) ? (ref + (float)(ex - 1)) + log2f(2.f * mant) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// pass 2: every slot's score receives the probabilities of all rows
// ---------------------------------------------------------------------------
// Software pipeline over the query tiles that see some slot of the block
// (from the largest position of each 64-position tile, found up front when
// the number of such tiles fits the LDS table; otherwise every tile is
// visited and the masks alone decide; a position tile that sees nothing is
// skipped for all heads of the group at once): the next active tile's rows
// load into registers while the MFMAs run on the current LDS buffer.
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(3)))
void prompt_scores_kernel(PromptArgs a) {
    __shared__ __align__(16) unsigned char qtile[2][kTile * 256];
    __shared__ int rpos[2][kTile];
    __shared__ __align__(16) float rlse[2][kTile];
    __shared__ int red[kPThreads / 64];
    extern __shared__ int rtile_max[];   // [position tiles] largest position, when tracked
    const CacheDev &c = a.c;
    const int nrows = a.m_rows * c.G;
    int u, blk;
    const int nblk = (c.cap + kScoreSlots - 1) / kScoreSlots;
    if (!windowed_unit_block<kScoresWindow, false>(nblk, c.B * c.Hkv, u, blk)) return;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, col = lane & 15;
    const int n = load_count(c, u, false);
    if (blk * kScoreSlots >= n) return;   // the whole block is past the filled slots
    const uint16_t *K = static_cast<const uint16_t *>(c.k);
    const int32_t *P = c.pos + (size_t)u * c.cap;
    // row tiles: 64 consecutive positions of one head, head-minor (tile rt
    // holds positions 64 (rt / G) .. + 63 of head rt % G), so a tile's rows
    // are consecutive query rows of one head
    const int G = c.G;
    const int nrt_g = (a.m_rows + kTile - 1) / kTile;   // position tiles
    const int nrt = nrt_g * G;
    const bool track = nrt_g <= a.row_tiles_lds;

    // B operands: kST 16-slot tiles per wave; lane (col, r) holds dims
    // 32c + 8r .. of slot col
    u16x8_p kb[kST][4];
    int kp[kST], jw[kST];
    bool kv[kST];
    int kmin = INT_MAX;
#pragma unroll
    for (int t = 0; t < kST; ++t) {
        const int j = blk * kScoreSlots + 16 * kST * w + 16 * t + col;
        jw[t] = j;
        kv[t] = j < n;
        const size_t row = row_of(c, b, h, kv[t] ? j : 0);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            kb[t][c4] = kv[t] ? *reinterpret_cast<const u16x8_p *>(K + row * kPD + 32 * c4 + 8 * r)
                              : u16x8_p{0, 0, 0, 0, 0, 0, 0, 0};
        kp[t] = kv[t] ? P[j] : INT_MAX;
        kmin = min(kmin, kp[t]);
    }
    // largest position of every position tile (a wave's 64 lanes hold one)
    if (track)
        for (int k = w; k < nrt_g; k += kPThreads / 64) {
            const int rr = kTile * k + lane;
            const int p = rr < a.m_rows ? (a.q_pos ? a.q_pos[(size_t)b * a.m_rows + rr] : INT_MAX)
                                        : INT_MIN;
            const int hi = wave_max_i(p);
            if (lane == 0) rtile_max[k] = hi;
        }
    // smallest position among the wave's slots (a row tile whose positions
    // all precede it adds nothing to this wave's slots)
    const int kmin_w = __builtin_amdgcn_readfirstlane(wave_min_i(kmin));
    kmin = block_min(kmin, red);   // (its barriers also publish the tile bounds)
    // largest position of each 16-slot tile of the wave, and whether all its
    // slots are filled (only such tiles may skip the mask)
    int kmaxw[kST];
    bool slots_full[kST];
#pragma unroll
    for (int t = 0; t < kST; ++t) {
        kmaxw[t] = __builtin_amdgcn_readfirstlane(wave_max_i(kp[t]));
        slots_full[t] = blk * kScoreSlots + 16 * kST * w + 16 * t + 15 < n;
    }
    // a negative or zero scale: negated or zero slot rows and a positive
    // factor, as the statistics pass does with the query rows
    if (a.scale <= 0.f)
#pragma unroll
        for (int t = 0; t < kST; ++t)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                kb[t][c4] = a.scale < 0.f ? kb[t][c4] ^ (uint16_t)0x8000 : u16x8_p{0, 0, 0, 0, 0, 0, 0, 0};
    const float c2 = (a.scale == 0.f ? 1.f : fabsf(a.scale)) * kLog2e;
    auto next_active = [&](int rt) {
        if (track)
            while (rt < nrt) {
                const int k = rt / G;
                if (rtile_max[k] >= kmin) break;
                rt = (k + 1) * G;   // no row of this position tile sees the block
            }
        return rt;
    };
    // the tile's query rows, positions and base-2 log-sum-exps into
    // registers.  Position rr of head g (of this kv head's group) is query row
    // (b m + rr) Hq + h G + g of q_rows and statistic rr G + g of the unit;
    // buffer resources end at the sequence's last row, its last position and
    // the unit's last statistic, so rows past m_rows read zeros (such rows
    // are masked: their position and statistic are set when the tile is
    // staged).  Nothing reads the loaded values before then, so the loads stay
    // in flight while the current tile computes.
    u16x8_p pre[kTile / 16];
    int ppos = 0;
    float plse = 0.f;
    const size_t q_first = ((size_t)b * a.m_rows * c.Hq + (size_t)h * G) * kPD;
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(static_cast<const uint16_t *>(a.q_rows) + q_first,
                  (uint32_t)(((size_t)a.m_rows * c.Hq - (size_t)h * G) * (kPD * 2)));
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.lse + (size_t)u * nrows, (uint32_t)nrows * 4);
    const __amdgpu_buffer_rsrc_t prs =
        make_rsrc(a.q_pos ? a.q_pos + (size_t)b * a.m_rows : nullptr, a.q_pos ? (uint32_t)a.m_rows * 4 : 0u);
    const int qoff = (tid >> 4) * c.Hq * (kPD * 2) + 16 * (tid & 15);
    const int lane_row = tid & (kTile - 1);
    auto fetch = [&](int rt) {
        const int k = rt / G, g = rt - k * G;
        const int rr0 = kTile * k;
#pragma unroll
        for (int pass = 0; pass < kTile / 16; ++pass)
            pre[pass] = __builtin_bit_cast(
                u16x8_p, __builtin_amdgcn_raw_buffer_load_b128(
                             qrs, qoff, ((rr0 + 16 * pass) * c.Hq + g) * (kPD * 2), 0));
        ppos = __builtin_amdgcn_raw_buffer_load_b32(prs, 4 * lane_row, 4 * rr0, 0);
        plse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             lrs, 4 * G * lane_row, 4 * (rr0 * G + g), 0));
    };

    double cs[kST];
#pragma unroll
    for (int t = 0; t < kST; ++t) cs[t] = 0.0;
    int cur = next_active(0);
    if (cur < nrt) fetch(cur);
    int buf = 0;
    while (cur < nrt) {
#pragma unroll
        for (int pass = 0; pass < kTile / 16; ++pass)
            *reinterpret_cast<u16x8_p *>(qtile[buf] + tile_off(16 * pass + (tid >> 4), tid & 15)) =
                pre[pass];
        if (tid < kTile) {
            const bool row = kTile * (cur / G) + tid < a.m_rows;
            rpos[buf][tid] = row ? (a.q_pos ? ppos : INT_MAX) : INT_MIN;
            rlse[buf][tid] = row ? plse : -INFINITY;
        }
        __syncthreads();
        const int nxt = next_active(cur + 1);
        if (nxt < nrt) fetch(nxt);   // lands while this tile computes
        // every row of a filled 64-row tile sees the wave's whole 16-slot tile
        const int tmin = __builtin_amdgcn_readfirstlane(wave_min_i(rpos[buf][lane]));
        const bool rows_full = kTile * (cur / G) + kTile <= a.m_rows;
        bool inner[kST];
#pragma unroll
        for (int t = 0; t < kST; ++t) inner[t] = slots_full[t] && rows_full && kmaxw[t] <= tmin;
        // the tile's probabilities are summed in fp32 per lane (16 rows per
        // slot and lane, in a fixed order), then added to the fp64 total.
        // The mask decision is uniform per tile: straight-line variants.
        float ts[kST];
#pragma unroll
        for (int t = 0; t < kST; ++t) ts[t] = 0.f;
        auto tile_body = [&](auto masked_c) {
            constexpr bool kMasked = decltype(masked_c)::value;
#pragma unroll
            for (int s = 0; s < kTile / 16; ++s) {
                // A operand: lane (col, r) holds dims 32c + 8r.. of row 16s + col
                const int q = 16 * s + col;
                u16x8_p qa[4];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    qa[c4] = *reinterpret_cast<const u16x8_p *>(qtile[buf] + tile_off(q, 4 * c4 + r));
                // C[row 4r + i][slot col]
                const f32x4_p rl = *reinterpret_cast<const f32x4_p *>(&rlse[buf][16 * s + 4 * r]);   // base 2
                int rp[4];
                if constexpr (kMasked)
#pragma unroll
                    for (int i = 0; i < 4; ++i) rp[i] = rpos[buf][16 * s + 4 * r + i];
#pragma unroll
                for (int t = 0; t < kST; ++t) {
                    f32x4_p acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(qa[c4]), as_bf(kb[t][c4]),
                                                                      acc, 0, 0, 0);
                    float e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        e[i] = exp2_hw(fmaf(acc[i], c2, -rl[i]));
                        if constexpr (kMasked) e[i] = (kv[t] && kp[t] <= rp[i]) ? e[i] : 0.f;
                    }
                    ts[t] += (e[0] + e[1]) + (e[2] + e[3]);
                }
            }
        };
        bool all_inner = true;
#pragma unroll
        for (int t = 0; t < kST; ++t) all_inner = all_inner && inner[t];
        // (a causal prompt: the block's row tiles before this wave's first
        // slot are staged for the other waves but skipped here)
        const bool wave_sees = !track || rtile_max[cur / G] >= kmin_w;
        if (all_inner)
            tile_body(std::integral_constant<bool, false>());
        else if (wave_sees)
            tile_body(std::integral_constant<bool, true>());
#pragma unroll
        for (int t = 0; t < kST; ++t) cs[t] += (double)ts[t];
        buf ^= 1;
        cur = nxt;
    }
    // the four lanes of a slot hold different rows: add them, then the score
#pragma unroll
    for (int t = 0; t < kST; ++t) {
        double v = cs[t];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (r == 0 && kv[t]) a.scores[(size_t)u * c.cap + jw[t]] += (float)v;
    }
}

size_t prompt_workspace_bytes(int units, int m_rows, int G) {
    return (size_t)units * (size_t)m_rows * (size_t)G * sizeof(float);
}

hipError_t launch_prompt_scores(const PromptArgs &a, hipStream_t s) {
    const int units = a.c.B * a.c.Hkv;
    const int groups = (units + 7) / 8;
    const int nrows = a.m_rows * a.c.G;
    if (nrows == 0) return hipSuccess;
    const int nb1 = (nrows + kStatRows - 1) / kStatRows;
    const int nb2 = (a.c.cap + kScoreSlots - 1) / kScoreSlots;
    const size_t tile_bytes = 2 * (size_t)((a.c.cap + kTile - 1) / kTile) * sizeof(int);
    if (a.c.bs == 0)
        hipLaunchKernelGGL(prompt_stats_kernel<false>, dim3(groups * 8 * nb1), dim3(kPThreads),
                           tile_bytes, s, a);
    else
        hipLaunchKernelGGL(prompt_stats_kernel<true>, dim3(groups * 8 * nb1), dim3(kPThreads),
                           tile_bytes, s, a);
    // position tiles whose largest position is tracked in LDS (up to 16 KB)
    PromptArgs a2 = a;
    const int nrt_g = (a.m_rows + kTile - 1) / kTile;
    a2.row_tiles_lds = nrt_g <= kMaxRowTilesLds ? nrt_g : 0;
    hipLaunchKernelGGL(prompt_scores_kernel, dim3(groups * 8 * nb2), dim3(kPThreads),
                       (size_t)a2.row_tiles_lds * sizeof(int), s, a2);
    return hipGetLastError();
}

}  // namespace kvc
