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
//  1. statistics: one workgroup per 128 rows of a unit.  K tiles of 64 slots
//     are staged in LDS (XOR swizzle, conflict-free reads) and enter
//     v_mfma_f32_16x16x32_bf16 as the A operand; the rows are the B operand,
//     held in registers.  Each lane keeps a running max / sum over its four
//     slots of every 16-slot tile; four lanes merge into the row's
//     log-sum-exp, written to the workspace.
//  2. scores: one workgroup per 128 slots of a unit.  The slots are the B
//     operand, held in registers; 64-row query tiles are staged in LDS.  Each
//     lane sums exp(z - lse) over its four rows of every tile into fp64 column
//     sums (a fixed order: the scores are deterministic), and one lane per
//     slot adds the total to the score.
// Tiles that no row of a block can see (from the positions alone) are
// skipped, which halves the work of a causal prompt.  All blocks of one unit
// run on one XCD (workgroups are dealt round-robin over the eight XCDs), so
// the K (pass 1) or Q (pass 2) rows they share are read from that XCD's L2.
#include "kvc_internal.h"

#include <limits.h>

namespace kvc {

namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_p __attribute__((ext_vector_type(8)));

constexpr int kPThreads = 256;
constexpr int kPD = 128;          // head_dim of this path
constexpr int kStatRows = 128;    // rows per workgroup, pass 1 (32 per wave)
constexpr int kScoreSlots = 128;  // slots per workgroup, pass 2 (32 per wave)
constexpr int kTile = 64;         // slots (pass 1) or rows (pass 2) staged per step

__device__ inline bf16x8_p as_bf(u16x8_p x) { return __builtin_bit_cast(bf16x8_p, x); }

// Unit and block index of this workgroup; every block of a unit gets the same
// blockIdx % 8, hence the same XCD.  False for the padding of the last group.
__device__ inline bool unit_block(int nblk, int units, int &u, int &blk) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    u = 8 * (slot / nblk) + xcd;
    blk = slot % nblk;
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

}  // namespace

// ---------------------------------------------------------------------------
// pass 1: log-sum-exp of every row over the slots it sees
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPThreads) void prompt_stats_kernel(PromptArgs a) {
    __shared__ __align__(16) unsigned char ktile[kTile * 256];
    __shared__ int kpos[kTile];
    __shared__ int red[kPThreads / 64];
    const CacheDev &c = a.c;
    const int nrows = a.m_rows * c.G;
    const int nblk = (nrows + kStatRows - 1) / kStatRows;
    int u, blk;
    if (!unit_block(nblk, c.B * c.Hkv, u, blk)) return;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, col = lane & 15;
    const int n = load_count(c, u, tid == 0);
    const uint16_t *K = static_cast<const uint16_t *>(c.k);
    const int32_t *P = c.pos + (size_t)u * c.cap;

    // B operands: two 16-row tiles per wave; lane (col, r) holds dims
    // 32c + 8r .. 32c + 8r + 7 of row col
    u16x8_p qb[2][4];
    int qp[2], Rw[2];
    int qmax = INT_MIN;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int R = blk * kStatRows + 32 * w + 16 * t + col;
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
    qmax = block_max(qmax, red);

    float mm[2] = {-INFINITY, -INFINITY}, ll[2] = {0.f, 0.f};
    const int ntile = (n + kTile - 1) / kTile;
    for (int kt = 0; kt < ntile; ++kt) {
        const int j0 = kt * kTile;
        if (tid < kTile) kpos[tid] = (j0 + tid < n) ? P[j0 + tid] : INT_MAX;
        __syncthreads();
        // no row of this block sees a slot of the tile: skip it (uniform)
        const int kmin = wave_min_i(kpos[lane]);
        if (kmin > qmax) {
            __syncthreads();
            continue;
        }
#pragma unroll
        for (int pass = 0; pass < kTile / 16; ++pass) {
            const int q = 16 * pass + (tid >> 4), ch = tid & 15, j = j0 + q;
            u16x8_p v = {0, 0, 0, 0, 0, 0, 0, 0};
            if (j < n) v = *reinterpret_cast<const u16x8_p *>(K + row_of(c, b, h, j) * kPD + 8 * ch);
            *reinterpret_cast<u16x8_p *>(ktile + tile_off(q, ch)) = v;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kTile / 16; ++s) {
            // A operand: lane (col, r) holds dims 32c + 8r.. of slot 16s + col
            const int q = 16 * s + col;
            u16x8_p ka[4];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                ka[c4] = *reinterpret_cast<const u16x8_p *>(ktile + tile_off(q, 4 * c4 + r));
            // C[slot 4r + i][row col]
            int kp[4];
            bool kv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kp[i] = kpos[16 * s + 4 * r + i];
                kv[i] = j0 + 16 * s + 4 * r + i < n;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4_p acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ka[c4]), as_bf(qb[t][c4]), acc,
                                                                  0, 0, 0);
                float z[4], zmax = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    z[i] = (kv[i] && kp[i] <= qp[t]) ? acc[i] * a.scale : -INFINITY;
                    zmax = fmaxf(zmax, z[i]);
                }
                const float mnew = fmaxf(mm[t], zmax);
                if (mnew != -INFINITY) {
                    float sum = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) sum += __expf(z[i] - mnew);
                    ll[t] = ll[t] * __expf(mm[t] - mnew) + sum;
                    mm[t] = mnew;
                }
            }
        }
        __syncthreads();
    }
    // merge the four lanes of each row, then log-sum-exp
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float m = mm[t], l = ll[t];
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float mo = __shfl_xor(m, off, 64), lo = __shfl_xor(l, off, 64);
            const float mn = fmaxf(m, mo);
            if (mn != -INFINITY) {
                l = l * __expf(m - mn) + lo * __expf(mo - mn);
                m = mn;
            }
        }
        if (r == 0 && Rw[t] < nrows)
            a.lse[(size_t)u * nrows + Rw[t]] = (l > 0.f) ? m + logf(l) : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// pass 2: every slot's score receives the probabilities of all rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPThreads) void prompt_scores_kernel(PromptArgs a) {
    __shared__ __align__(16) unsigned char qtile[kTile * 256];
    __shared__ int rpos[kTile];
    __shared__ float rlse[kTile];
    __shared__ int red[kPThreads / 64];
    const CacheDev &c = a.c;
    const int nrows = a.m_rows * c.G;
    const int nblk = (c.cap + kScoreSlots - 1) / kScoreSlots;
    int u, blk;
    if (!unit_block(nblk, c.B * c.Hkv, u, blk)) return;
    const int b = u / c.Hkv, h = u % c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, col = lane & 15;
    const int n = load_count(c, u, false);
    if (blk * kScoreSlots >= n) return;   // the whole block is past the filled slots
    const uint16_t *K = static_cast<const uint16_t *>(c.k);
    const int32_t *P = c.pos + (size_t)u * c.cap;

    // B operands: two 16-slot tiles per wave; lane (col, r) holds dims
    // 32c + 8r .. of slot col
    u16x8_p kb[2][4];
    int kp[2], jw[2];
    bool kv[2];
    int kmin = INT_MAX;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int j = blk * kScoreSlots + 32 * w + 16 * t + col;
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
    kmin = block_min(kmin, red);

    double cs[2] = {0.0, 0.0};
    const int ntile = (nrows + kTile - 1) / kTile;
    for (int rt = 0; rt < ntile; ++rt) {
        const int R0 = rt * kTile;
        if (tid < kTile) {
            const int R = R0 + tid;
            const bool ok = R < nrows;
            rpos[tid] = ok ? row_pos(a, b, R) : INT_MIN;
            rlse[tid] = ok ? a.lse[(size_t)u * nrows + R] : -INFINITY;
        }
        __syncthreads();
        // no row of the tile sees a slot of this block: skip it (uniform)
        const int tmax = wave_max_i(rpos[lane]);
        if (tmax < kmin) {
            __syncthreads();
            continue;
        }
#pragma unroll
        for (int pass = 0; pass < kTile / 16; ++pass) {
            const int q = 16 * pass + (tid >> 4), ch = tid & 15, R = R0 + q;
            u16x8_p v = {0, 0, 0, 0, 0, 0, 0, 0};
            if (R < nrows) v = *reinterpret_cast<const u16x8_p *>(q_row(a, b, h, R) + 8 * ch);
            *reinterpret_cast<u16x8_p *>(qtile + tile_off(q, ch)) = v;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kTile / 16; ++s) {
            // A operand: lane (col, r) holds dims 32c + 8r.. of row 16s + col
            const int q = 16 * s + col;
            u16x8_p qa[4];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                qa[c4] = *reinterpret_cast<const u16x8_p *>(qtile + tile_off(q, 4 * c4 + r));
            // C[row 4r + i][slot col]
            int rp[4];
            float rl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rp[i] = rpos[16 * s + 4 * r + i];
                rl[i] = rlse[16 * s + 4 * r + i];
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4_p acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(qa[c4]), as_bf(kb[t][c4]), acc,
                                                                  0, 0, 0);
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    part += (kv[t] && kp[t] <= rp[i]) ? __expf(acc[i] * a.scale - rl[i]) : 0.f;
                cs[t] += (double)part;
            }
        }
        __syncthreads();
    }
    // the four lanes of a slot hold different rows: add them, then the score
#pragma unroll
    for (int t = 0; t < 2; ++t) {
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
    hipLaunchKernelGGL(prompt_stats_kernel, dim3(groups * 8 * nb1), dim3(kPThreads), 0, s, a);
    hipLaunchKernelGGL(prompt_scores_kernel, dim3(groups * 8 * nb2), dim3(kPThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvc
