"""Full-size parity at the workloads' real shapes and in the launch
configuration the benchmark times (length hint = capacity for the first,
over-budget step; budget + 1 afterwards).

Every step runs twice from identical states: the one-launch kvc_decode_step
that the benchmark times, and the three-call sequence decode_attn ->
evict -> compact.  The two must agree bit for bit over the whole live state
of every unit; the three-call sequence exposes the post-attention scores, so
sampled units are then checked against the oracle: outputs within 2e-3,
scores within 1e-5 relative, kept sets exactly (H2O on the GPU's own
post-attention scores; other policies on their own definition)."""
import math

import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle
import synth
from kvc_harness import OUT_ATOL, Snapshot, assert_scores_close, oracle_unit_attend, rows_by_pos

pytestmark = pytest.mark.gpu


def _clone(c: kvc.KvCache) -> kvc.KvCache:
    d = kvc.KvCache.__new__(kvc.KvCache)
    d.__dict__.update(c.__dict__)
    for name in ("k", "v", "pos", "n_slots", "flags"):
        setattr(d, name, getattr(c, name).clone())
    d._c = None
    return d


def _live_mask(c):
    idx = torch.arange(c.capacity, device="cuda").view(1, 1, -1)
    return idx < c.n_slots.unsqueeze(-1)


def _assert_live_equal(a, b, sa=None, sb=None):
    assert torch.equal(a.n_slots, b.n_slots)
    m = _live_mask(a)
    assert torch.equal(a.pos[m], b.pos[m])
    if a.block_size:
        live = int(a.n_slots.max().item())
        slots = torch.arange(live, device="cuda")
        blk = a.block_table.long()[:, slots // a.block_size]          # [B, live]
        mm = m[:, :, :live].permute(0, 2, 1)                          # [B, live, H]
        for x, y in ((a.k, b.k), (a.v, b.v)):
            xr = x[blk, :, slots % a.block_size]                      # [B, live, H, D]
            yr = y[blk, :, slots % a.block_size]
            assert torch.equal(xr[mm], yr[mm])
    else:
        assert torch.equal(a.k[m], b.k[m]) and torch.equal(a.v[m], b.v[m])
    if sa is not None:
        assert torch.equal(sa[m], sb[m])


def _policy_calls(pol, cache, scores, step, keep, nout):
    if pol.kind == kvc.POLICY_H2O:
        kvc.evict_h2o(cache, scores, pol.n_heavy, pol.n_recent, keep, nout)
    elif pol.kind == kvc.POLICY_STREAMING:
        kvc.evict_streaming(cache, pol.n_sink, pol.n_recent, keep, nout)
    elif pol.kind == kvc.POLICY_RANDOM:
        kvc.evict_random(cache, pol.prompt_len, pol.n_keep, pol.seed, step, keep, nout)


def _run(w, cache, lengths, pol, steps, hints, units, heavy_frac=0.0, seen0=None):
    """Fused vs three-call on full-size caches, oracle on sampled units."""
    B, G, D = cache.batch, cache.group, cache.head_dim
    twin = _clone(cache)
    h2o = pol.kind == kvc.POLICY_H2O
    sc_f = torch.zeros((B, cache.kv_heads, cache.capacity), device="cuda") if h2o else None
    sc_t = torch.zeros_like(sc_f) if h2o else None
    out_f = torch.empty((B, cache.q_heads, D), device="cuda")
    out_t = torch.empty_like(out_f)
    keep = torch.empty((B, cache.kv_heads, cache.capacity), dtype=torch.int32, device="cuda")
    nout = torch.empty((B, cache.kv_heads), dtype=torch.int32, device="cuda")
    ws = cache.workspace(max(hints))
    ws2 = cache.workspace(max(hints))
    seen = torch.tensor(lengths if seen0 is None else seen0, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    for t in range(1, steps + 1):
        hint = hints[min(t - 1, len(hints) - 1)]
        q = synth.device_normal((B, cache.q_heads, D), w.seed, w.wid, synth.T_Q, t)
        kn = synth.device_normal((B, cache.kv_heads, D), w.seed, w.wid, synth.T_KNEW, t,
                                 scale_rows_frac=heavy_frac)
        vn = synth.device_normal((B, cache.kv_heads, D), w.seed, w.wid, synth.T_VNEW, t)
        pre = Snapshot(twin, w.dtype, sc_t, units)
        kvc.decode_step(cache, pol, t, seen, q, kn, vn, out_f, sc_f, max_len_hint=hint,
                        workspace=ws)
        kvc.decode_attn(twin, seen, q, kn, vn, out_t, sc_t, max_len_hint=hint, workspace=ws2)
        mid = Snapshot(twin, w.dtype, sc_t, units)
        _policy_calls(pol, twin, sc_t, t, keep, nout)
        kk, mm = keep.cpu().numpy(), nout.cpu().numpy()
        if pol.kind != kvc.POLICY_FULL:
            kvc.compact(twin, keep, nout, sc_t)
        torch.cuda.synchronize()
        assert int(cache.flags.item()) == 0 and int(twin.flags.item()) == 0
        assert torch.equal(out_f, out_t), f"step {t}: fused and three-call outputs differ"
        _assert_live_equal(cache, twin, sc_f, sc_t)
        qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
        knh = kn.view(torch.int16).cpu().numpy().view(np.uint16)
        vnh = vn.view(torch.int16).cpu().numpy().view(np.uint16)
        o = out_t.cpu().numpy()
        sn = seen.cpu().numpy()
        for (b, h) in units:
            u0, u1 = pre.unit(b, h), mid.unit(b, h)
            ref, psum = oracle_unit_attend(w.dtype, qh[b, h * G:(h + 1) * G], u0, knh[b, h],
                                           vnh[b, h], scale)
            err = np.abs(o[b, h * G:(h + 1) * G] - ref).max()
            assert err <= OUT_ATOL, (t, b, h, err)
            n = u0["n"]
            if h2o:
                assert_scores_close(u1["s"][:n], u0["s"] + psum[:n])
                assert_scores_close(u1["s"][n:n + 1], psum[n:])
            L = int(sn[b]) + 1
            if pol.kind == kvc.POLICY_H2O:
                want = oracle.select_h2o(u1["pos"], u1["s"].astype(np.float64), L, pol.n_heavy,
                                         pol.n_recent)
            elif pol.kind == kvc.POLICY_STREAMING:
                want = oracle.select_streaming(u1["pos"], L, pol.n_sink, pol.n_recent)
            elif pol.kind == kvc.POLICY_RANDOM:
                want = oracle.select_random(u1["pos"], pol.prompt_len, pol.n_keep, pol.seed, b,
                                            h, t)
            else:
                want = np.ones(u1["pos"].size, bool)
            if pol.kind != kvc.POLICY_FULL:
                np.testing.assert_array_equal(kk[b, h, :mm[b, h]], np.flatnonzero(want),
                                              err_msg=f"step {t} unit {(b, h)}")
        seen += 1
    return cache


def _prefill(w, B, cap, fill, heavy_frac=0.0, paged=0, lengths=None):
    lengths = [fill] * B if lengths is None else lengths
    f8 = w.dtype == "e5m2"
    dt = kvc.FP8_E5M2 if f8 else kvc.BF16
    if paged:
        max_blocks = cap // paged
        nblk = B * max_blocks
        perm = torch.from_numpy(synth.block_permutation(nblk, w.seed, w.wid).reshape(B, max_blocks).copy())
        c = kvc.KvCache(B, w.q_heads, w.kv_heads, w.head_dim, cap, dt, block_size=paged,
                        num_blocks=nblk, block_table=perm)
    else:
        c = kvc.KvCache(B, w.q_heads, w.kv_heads, w.head_dim, cap, dt)
    # E5M2 caches hold the float32 draws truncated to codes (the seeded recipe)
    draw_dtype = torch.float32 if f8 else None
    stored = synth.device_e5m2_truncated if f8 else (lambda x: x)
    chunk = 32
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        L = max(lengths[b0:b1])
        k = stored(synth.device_normal((b1 - b0, w.kv_heads, L, w.head_dim), w.seed, w.wid,
                                       synth.T_K, b0, dtype=draw_dtype, scale_rows_frac=heavy_frac))
        v = stored(synth.device_normal((b1 - b0, w.kv_heads, L, w.head_dim), w.seed, w.wid,
                                       synth.T_V, b0, dtype=draw_dtype))
        for i, b in enumerate(range(b0, b1)):
            Lb = lengths[b]
            if paged:
                slots = torch.arange(Lb, device="cuda")
                blk = c.block_table[b, slots // paged].long()
                c.k[blk, :, slots % paged] = k[i, :, :Lb].permute(1, 0, 2)
                c.v[blk, :, slots % paged] = v[i, :, :Lb].permute(1, 0, 2)
            else:
                c.k[b, :, :Lb] = k[i, :, :Lb]
                c.v[b, :, :Lb] = v[i, :, :Lb]
            c.pos[b, :, :Lb] = torch.arange(Lb, dtype=torch.int32, device="cuda")
            c.n_slots[b] = Lb
        del k, v
    torch.cuda.synchronize()
    return c


def test_heavy_load_b512_l2048_h2o_full_size():
    # 512 sequences x 8 kv heads, 2,048-token prompts, 64 heavy + 448 recent:
    # step 1 trims 2,049 -> 512 on the split path, steps 2-3 run the fused kernel
    w = synth.workload("heavy_load_b512_l2048")
    P = w.prompt_len
    cache = _prefill(w, w.batch, P + 1, P)
    units = [(b, h) for b in (0, 97, 255, 256, 511) for h in (0, 3, 7)]
    _run(w, cache, [P] * w.batch, kvc.policy_h2o(64, 448), steps=3, hints=[P + 1, 513],
         units=units)


def test_heavy_load_b512_l2048_h2o_e5m2_full_size():
    # the same layer with an E5M2 (8-bit float) cache: the first step trims on
    # the split path, the others run the fused kernel's E5M2 instance
    w = synth.workload("heavy_load_b512_l2048", dtype="e5m2")
    P = w.prompt_len
    cache = _prefill(w, w.batch, P + 1, P)
    units = [(b, h) for b in (0, 200, 511) for h in (0, 6)]
    _run(w, cache, [P] * w.batch, kvc.policy_h2o(64, 448), steps=3, hints=[P + 1, 513],
         units=units)


def test_heavy_load_b512_l2048_streaming_full_size():
    w = synth.workload("heavy_load_b512_l2048")
    P = w.prompt_len
    cache = _prefill(w, w.batch, P + 1, P)
    units = [(b, h) for b in (1, 300, 510) for h in (0, 5)]
    _run(w, cache, [P] * w.batch, kvc.policy_streaming(64, 448), steps=3, hints=[P + 1, 513],
         units=units)


def test_llama3_8b_h2o_b64_heavy_hitters_full_size():
    w = synth.workload("llama3_8b_h2o_b64")
    P = w.prompt_len
    cache = _prefill(w, w.batch, P + 1, P, heavy_frac=w.heavy_frac)
    units = [(b, h) for b in (0, 31, 63) for h in (0, 2, 7)]
    _run(w, cache, [P] * w.batch, kvc.policy_h2o(64, 448), steps=4, hints=[P + 1, 513],
         units=units, heavy_frac=w.heavy_frac)


def test_reasoning_random_b32_steady_state_full_size():
    # 1,024 pinned + 4,096 kept generated per head, one over budget: every step
    # evicts exactly one generated token per head (the long-trace budget)
    w = synth.workload("reasoning_random_b32")
    fill = w.pinned + w.n_keep
    cache = _prefill(w, w.batch, fill + 1, fill)
    units = [(b, h) for b in (0, 17, 31) for h in (0, 4, 7)]
    _run(w, cache, [fill] * w.batch, kvc.policy_random(w.pinned, w.n_keep, w.seed), steps=3,
         hints=[fill + 1], units=units)


def test_mixed_paged_h2o_b128_trim_and_steady_full_size():
    # 128 sequences, log-uniform lengths in [512, 32768], paged blocks of 16 with
    # a shuffled table; step 1 trims every unit to 512, then fused steps
    w = synth.workload("mixed_paged_h2o_b128")
    lengths = [int(x) for x in synth.mixed_lengths(w)]
    Lmax = max(lengths)
    cap = (Lmax + 1 + 15) // 16 * 16
    cache = _prefill(w, w.batch, cap, None, paged=16, lengths=lengths)
    order = np.argsort(lengths)
    pick = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    units = [(b, h) for b in pick for h in (0, 7)]
    _run(w, cache, lengths, kvc.policy_h2o(64, 448), steps=3, hints=[Lmax + 1, 513], units=units)
