/* Drives the host side of libkvc's C ABI (argument validation, workspace
 * layout, dispatch to the launchers, host helpers) with fake device pointers,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer against stub
 * launchers.  Exits 0 when every call returns the expected status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvc.h"

int kvc_stub_launches(void);

static int failures = 0;
#define EXPECT(call, want)                                                               \
    do {                                                                                 \
        int got_ = (int)(call);                                                          \
        if (got_ != (int)(want)) {                                                       \
            fprintf(stderr, "%s:%d: %s = %d, want %d (%s)\n", __FILE__, __LINE__, #call, \
                    got_, (int)(want), kvc_last_error());                                \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

static kvc_cache fake(int B, int Hq, int Hkv, int D, int cap, int dtype) {
    kvc_cache c;
    memset(&c, 0, sizeof c);
    c.batch = B;
    c.q_heads = Hq;
    c.kv_heads = Hkv;
    c.head_dim = D;
    c.capacity = cap;
    c.dtype = dtype;
    c.k = (void *)0x100000;
    c.v = (void *)0x200000;
    c.pos = (int32_t *)0x300000;
    c.n_slots = (int32_t *)0x400000;
    return c;
}

#define NP ((const int32_t *)0x1000)
#define Q ((const void *)0x2000)
#define KN ((const void *)0x3000)
#define VN ((const void *)0x4000)
#define OUT ((float *)0x5000)
#define SC ((float *)0x6000)
#define WS ((void *)0x10000000)

int main(void) {
    /* host helpers */
    EXPECT(kvc_bytes_per_token(80, 8, 128, 2) == 327680, 1);
    EXPECT(kvc_bytes_per_token(0, 8, 128, 2), 0);
    EXPECT(kvc_bytes_per_token(-3, 8, 128, 2), 0);
    EXPECT(kvc_n_keep(100, 0.29), 28);
    EXPECT(kvc_n_keep(0, 0.5), 0);
    EXPECT(kvc_n_keep(10, 7.0), 10);
    EXPECT(kvc_n_keep((int64_t)1 << 40, 1e-30), 1);
    for (int st = -1; st < 8; ++st) EXPECT(kvc_status_string(st) != NULL, 1);
    EXPECT(strcmp(kvc_status_string(-1), "unknown status"), 0);

    kvc_cache c = fake(2, 8, 2, 128, 64, KVC_BF16);
    size_t need = kvc_workspace_bytes(&c, 0);
    EXPECT(need > 0, 1);
    EXPECT(kvc_workspace_bytes(NULL, 0), 0);
    kvc_cache big = fake(512, 64, 8, 128, 65536, KVC_BF16);
    EXPECT(kvc_workspace_bytes(&big, 0) > ((size_t)1 << 32), 1);   /* 64-bit sizes */

    /* attention */
    EXPECT(kvc_decode_attn(NULL, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_decode_attn(&c, NP, NULL, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_decode_attn(&c, NP, (const void *)0x2008, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_decode_attn(&c, NP, Q, KN, VN, OUT, NULL, 1.0f / 0.0f, 0.f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_decode_attn(&c, NP, Q, KN, VN, OUT, NULL, 0.1f, 1.0f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_decode_attn(&c, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, NULL, 0, NULL), KVC_ERR_WORKSPACE);
    EXPECT(kvc_decode_attn(&c, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need - 1, NULL), KVC_ERR_WORKSPACE);
    EXPECT(kvc_decode_attn(&c, NP, Q, KN, VN, OUT, SC, 0.1f, 0.5f, 0, WS, need, NULL), KVC_OK);
    EXPECT(kvc_decode_attn(&c, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 33, WS, kvc_workspace_bytes(&c, 33), NULL), KVC_OK);
    kvc_cache f32 = fake(3, 12, 4, 64, 2000, KVC_F32);
    size_t nf = kvc_workspace_bytes(&f32, 0);
    EXPECT(kvc_decode_attn(&f32, NP, Q, KN, VN, OUT, SC, 0.1f, 0.f, 0, WS, nf, NULL), KVC_OK);
    kvc_cache e = fake(2, 8, 2, 128, 5000, KVC_FP8_E5M2);
    EXPECT(kvc_decode_attn(&e, NP, Q, KN, VN, OUT, SC, 0.1f, 0.f, 0, WS, kvc_workspace_bytes(&e, 0), NULL), KVC_OK);

    /* cache validation */
    kvc_cache bad = c;
    bad.q_heads = 7;
    EXPECT(kvc_decode_attn(&bad, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_SHAPE);
    bad = c;
    bad.head_dim = 96;
    EXPECT(kvc_decode_attn(&bad, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_UNSUPPORTED);
    bad = c;
    bad.capacity = 1 << 20;
    EXPECT(kvc_decode_attn(&bad, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_UNSUPPORTED);
    bad = c;
    bad.block_size = 16;   /* paged without a table */
    EXPECT(kvc_decode_attn(&bad, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);
    kvc_cache pg = c;
    pg.block_size = 16;
    pg.max_blocks = 4;
    pg.num_blocks = 9;
    pg.block_table = (const int32_t *)0x7000;
    EXPECT(kvc_decode_attn(&pg, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, kvc_workspace_bytes(&pg, 0), NULL), KVC_OK);
    pg.max_blocks = 3;
    EXPECT(kvc_decode_attn(&pg, NP, Q, KN, VN, OUT, NULL, 0.1f, 0.f, 0, WS, need, NULL), KVC_ERR_SHAPE);

    /* scoring, selection, compaction, whole steps */
    EXPECT(kvc_h2o_accumulate(&c, Q, -1, NULL, SC, 0.1f, NULL, 0, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_h2o_accumulate(&c, Q, 0, NULL, SC, 0.1f, NULL, 0, NULL), KVC_OK);
    size_t pw = kvc_h2o_accumulate_workspace_bytes(&c, 100);
    EXPECT(kvc_h2o_accumulate(&c, Q, 100, NP, SC, 0.1f, WS, pw, NULL), KVC_OK);
    EXPECT(kvc_h2o_accumulate(&c, Q, 100, NP, SC, 0.1f, WS, pw - 4, NULL), KVC_ERR_WORKSPACE);
    EXPECT(kvc_h2o_accumulate(&f32, Q, 7, NULL, SC, 0.1f, NULL, 0, NULL), KVC_OK);
    int32_t *keep = (int32_t *)0x8000, *nout = (int32_t *)0x9000;
    EXPECT(kvc_evict_streaming(&c, 64, 448, keep, nout, NULL), KVC_OK);
    EXPECT(kvc_evict_streaming(&c, -1, 448, keep, nout, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_evict_h2o(&c, SC, 64, 448, keep, nout, NULL), KVC_OK);
    EXPECT(kvc_evict_h2o(&c, NULL, 64, 448, keep, nout, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_evict_random(&c, 16, 100, 0xFFFFFFFFFFFFFFFFull, 7, keep, nout, NULL), KVC_OK);
    EXPECT(kvc_evict_random(&c, 16, -100, 0, 7, keep, nout, NULL), KVC_ERR_INVALID_ARG);
    EXPECT(kvc_compact(&c, keep, nout, SC, NULL, NULL), KVC_OK);
    kvc_cache dst = fake(2, 8, 2, 128, 64, KVC_BF16);
    dst.k = (void *)0x500000;
    dst.v = (void *)0x600000;
    EXPECT(kvc_compact(&c, keep, nout, NULL, &dst, NULL), KVC_OK);
    EXPECT(kvc_compact(&c, keep, nout, NULL, &c, NULL), KVC_ERR_INVALID_ARG);
    kvc_policy pol;
    memset(&pol, 0, sizeof pol);
    pol.kind = KVC_POLICY_H2O;
    pol.n_heavy = 64;
    pol.n_recent = 448;
    EXPECT(kvc_decode_step(&c, &pol, 1, NP, Q, KN, VN, OUT, SC, 0.1f, 0, WS, need, NULL), KVC_OK);
    EXPECT(kvc_decode_step(&c, &pol, 1, NP, Q, KN, VN, OUT, NULL, 0.1f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);
    pol.kind = KVC_POLICY_RANDOM;
    pol.prompt_len = 1024;
    pol.n_keep = 4096;
    kvc_cache r = fake(32, 40, 8, 128, 5121, KVC_BF16);
    EXPECT(kvc_decode_step(&r, &pol, 9, NP, Q, KN, VN, OUT, NULL, 0.1f, 5121, WS, kvc_workspace_bytes(&r, 5121), NULL), KVC_OK);
    pol.kind = 17;
    EXPECT(kvc_decode_step(&c, &pol, 1, NP, Q, KN, VN, OUT, SC, 0.1f, 0, WS, need, NULL), KVC_ERR_INVALID_ARG);

    /* the no-allocation step: oversize caches are rejected before any device call */
    pol.kind = KVC_POLICY_STREAMING;
    pol.n_sink = 64;
    pol.n_recent = 448;
    EXPECT(kvc_decode_step_noalloc(&big, &pol, 1, NP, Q, KN, VN, OUT, NULL, 0.1f, 0, NULL), KVC_ERR_WORKSPACE);
    EXPECT(kvc_decode_step_noalloc(&c, &pol, 1, NP, NULL, KN, VN, OUT, NULL, 0.1f, 0, NULL), KVC_ERR_INVALID_ARG);

    /* streaming-read helper */
    EXPECT(kvc_stream_read((const void *)0x1000, 4096, (uint32_t *)0x2000, NULL), KVC_OK);
    EXPECT(kvc_stream_read((const void *)0x1008, 4096, (uint32_t *)0x2000, NULL), KVC_ERR_INVALID_ARG);

    /* KIVI */
    kvc_kivi_cache kc;
    memset(&kc, 0, sizeof kc);
    kc.batch = 4;
    kc.q_heads = 32;
    kc.kv_heads = 8;
    kc.head_dim = 128;
    kc.max_quant = 2048;
    kc.bits = 4;
    kc.k_codes = (uint8_t *)0x100000;
    kc.v_codes = (uint8_t *)0x200000;
    kc.k_scale = (float *)0x300000;
    kc.k_lo = (float *)0x400000;
    kc.v_scale = (float *)0x500000;
    kc.v_lo = (float *)0x600000;
    kc.k_res = (void *)0x700000;
    kc.v_res = (void *)0x800000;
    kc.n_quant = (int32_t *)0x900000;
    kc.n_res = (int32_t *)0xA00000;
    size_t kw = kvc_kivi_workspace_bytes(&kc, 0);
    EXPECT(kvc_kivi_decode(&kc, Q, KN, VN, OUT, 0.1f, 0, WS, kw, NULL), KVC_OK);
    EXPECT(kvc_kivi_decode(&kc, Q, KN, VN, OUT, 0.1f, 0, WS, kw - 1, NULL), KVC_ERR_WORKSPACE);
    EXPECT(kvc_kivi_prefill(&kc, Q, KN, 2000, NP, NULL), KVC_OK);
    kc.bits = 2;
    EXPECT(kvc_kivi_decode(&kc, Q, KN, VN, OUT, 0.1f, 0, WS, kw, NULL), KVC_ERR_UNSUPPORTED);

    if (kvc_stub_launches() <= 0) {
        fprintf(stderr, "no launcher was reached\n");
        ++failures;
    }
    printf("abi host check: %d failure(s), %d launches reached the stubs\n", failures,
           kvc_stub_launches());
    return failures ? 1 : 0;
}
