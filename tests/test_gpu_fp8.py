"""GPU parity of an E5M2 (8-bit float) KV cache against the oracle.

K and V are held as OCP E5M2 codes; q, k_new and v_new are bfloat16.  The new
token is stored as the nearest E5M2 value and attended as stored, so the
oracle attends over exactly the codes the GPU holds.  Checked as for the
bf16 cache: outputs within 2e-3, appended codes bit-exact against the
oracle's encoder, H2O scores within 1e-5 relative, kept sets exact over whole
trajectories, the one-launch step equal to the three calls bit for bit, and
the paged layout equal to the contiguous one.
"""
import math

import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle
import synth
from kvc_harness import (OUT_ATOL, Snapshot, assert_scores_close, dev, make_cache,
                         oracle_unit_attend, rows_by_pos)

pytestmark = pytest.mark.gpu


def _w(name, **kw):
    return synth.workload(name, dtype="e5m2", **kw)


def _act(x):
    return dev(x, "bf16")


def _stored(x_bf16):
    """E5M2 codes the cache must hold for bf16 activations x."""
    return oracle.encode_e5m2(oracle.decode(x_bf16, "bf16"))


def _path(path, lengths, capacity):
    """(capacity, hint): 'fused' = attended length within the one-workgroup
    kernel's limit of 1,024; 'split' = above it; 'fallback' = a hint smaller
    than some unit, which the one-workgroup launch must handle exactly."""
    if path == "fused":
        return capacity, max(lengths) + 1
    if path == "split":
        cap = max(capacity, 1104)
        return cap, cap + 1
    return capacity, 1


def _attn_once(w, lengths, capacity, path="fused", paged=0, with_scores=True, step=1):
    capacity, hint = _path(path, lengths, capacity)
    B, G, D = len(lengths), w.group, w.head_dim
    cache = make_cache(w, lengths, capacity, paged=paged)
    q, kn, vn = synth.batch_step_inputs(w, step, B)
    scores = None
    if with_scores:
        g = torch.Generator(device="cpu").manual_seed(7)
        scores = (torch.rand((B, w.kv_heads, capacity), generator=g) * 3).cuda()
    pre = Snapshot(cache, "e5m2", scores)
    out = torch.full((B, w.q_heads, D), float("nan"), device="cuda")
    new_pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    kvc.decode_attn(cache, new_pos, _act(q), _act(kn), _act(vn), out, scores, max_len_hint=hint,
                    workspace=cache.workspace(hint))
    post = Snapshot(cache, "e5m2", scores)
    assert int(cache.flags.item()) == 0
    o = out.cpu().numpy()
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(w.kv_heads):
            u0, u1 = pre.unit(b, h), post.unit(b, h)
            n = u0["n"]
            ref, psum = oracle_unit_attend("e5m2", q[b, h * G:(h + 1) * G], u0, kn[b, h],
                                           vn[b, h], scale)
            err = np.abs(o[b, h * G:(h + 1) * G] - ref).max()
            assert err <= OUT_ATOL, (b, h, err)
            assert u1["n"] == n + 1 and u1["pos"][n] == lengths[b]
            np.testing.assert_array_equal(u1["pos"][:n], u0["pos"])
            np.testing.assert_array_equal(u1["k"][:n], u0["k"])
            np.testing.assert_array_equal(u1["v"][:n], u0["v"])
            np.testing.assert_array_equal(u1["k"][n], _stored(kn[b, h]))
            np.testing.assert_array_equal(u1["v"][n], _stored(vn[b, h]))
            if with_scores:
                assert_scores_close(u1["s"][:n], u0["s"] + psum[:n])
                assert_scores_close(u1["s"][n:n + 1], psum[n:n + 1])
    return cache


W_GQA = _w("llama3_8b_h2o_b64", heavy_frac=0.0)
W_HEAVY = _w("llama3_8b_h2o_b64")
W_G5 = _w("reasoning_random_b32")
W_G8 = _w("heavy_load_b512_l2048")
W_D64 = _w("tiny_mha_streaming_f32")


@pytest.mark.parametrize("path", ["fused", "split", "fallback"])
@pytest.mark.parametrize("w", [W_HEAVY, W_G5, W_G8], ids=lambda w: w.name)
def test_attention_every_path_and_group(w, path):
    # ragged lengths over several tiles, an empty unit and a one-entry unit
    _attn_once(w, [129, 700, 0, 1], capacity=1000, path=path)


def test_head_dim_64_and_no_scores():
    _attn_once(W_D64, [90, 17], capacity=100, with_scores=False)
    _attn_once(W_GQA, [513, 64], capacity=520, with_scores=False)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_paged_layout(path):
    _attn_once(W_GQA, [17, 100, 300], capacity=320, paged=16, path=path)


def test_group_of_sixteen():
    w = _w("heavy_load_b512_l2048", q_heads=128)
    for path in ("fused", "split"):
        _attn_once(w, [300, 17], capacity=400, path=path)


@pytest.mark.parametrize("capacity", [64, 1100])
def test_new_token_encoding_over_every_bf16_pattern(capacity):
    # 64 sequences x 8 heads x 128 dims = every one of the 65,536 bf16 bit
    # patterns once in v_new (NaN and infinities included: v only enters the
    # weighted sum) and every finite pattern in k_new; each stored code must
    # be the oracle encoder's (nearest, ties to even, saturating, NaN kept).
    w = W_GQA
    B, H, D = 64, w.kv_heads, w.head_dim
    cache = make_cache(w, [3] * B, capacity=capacity)
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vn = pats.reshape(B, H, D)
    finite = pats[(pats & 0x7F80) != 0x7F80]
    kn = np.resize(finite, B * H * D).reshape(B, H, D)
    q = np.zeros((B, w.q_heads, D), np.uint16)     # zero query: logits 0 for finite keys
    out = torch.empty((B, w.q_heads, D), device="cuda")
    kvc.decode_attn(cache, torch.full((B,), 3, dtype=torch.int32, device="cuda"), _act(q),
                    _act(kn), _act(vn), out, None, workspace=cache.workspace())
    torch.cuda.synchronize()
    got_k = cache.k[:, :, 3].cpu().numpy()
    got_v = cache.v[:, :, 3].cpu().numpy()
    np.testing.assert_array_equal(got_k, _stored(kn))
    np.testing.assert_array_equal(got_v, _stored(vn))


def _policy_pair(w):
    if w.policy == "streaming":
        return (kvc.policy_streaming(w.n_sink, w.n_recent),
                oracle.Policy.streaming(w.n_sink, w.n_recent))
    if w.policy == "h2o":
        return kvc.policy_h2o(w.n_heavy, w.n_recent), oracle.Policy.h2o(w.n_heavy, w.n_recent)
    return (kvc.policy_random(w.pinned, w.n_keep, w.seed),
            oracle.Policy.random(w.pinned, w.n_keep, w.seed))


def _trajectory(w, lengths, capacity, steps, hint=None, paged=0):
    """Oracle trajectory against the one-launch step: kept sets exact, outputs
    within 2e-3, every step."""
    hint = capacity + 1 if hint is None else hint
    B = len(lengths)
    cache = make_cache(w, lengths, capacity, paged=paged)
    orc = oracle.Oracle(w.q_heads, w.kv_heads, w.head_dim, "e5m2")
    for b, L in enumerate(lengths):
        orc.load(b, *synth.prefill_kv(w, b, L))
    pol_gpu, pol_orc = _policy_pair(w)
    ws = cache.workspace(hint)
    out = torch.empty((B, w.q_heads, w.head_dim), device="cuda")
    scores = torch.zeros((B, w.kv_heads, capacity), device="cuda") if w.policy == "h2o" else None
    seen = list(lengths)
    for t in range(1, steps + 1):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        kvc.decode_step(cache, pol_gpu, t, torch.tensor(seen, dtype=torch.int32, device="cuda"),
                        _act(q), _act(kn), _act(vn), out, scores, max_len_hint=hint,
                        workspace=ws)
        snap = Snapshot(cache, "e5m2")
        o = out.cpu().numpy()
        for b in range(B):
            ref, _ = orc.step(b, q[b], kn[b], vn[b], pol_orc, step=t)
            assert np.abs(o[b] - ref).max() <= OUT_ATOL, (t, b)
            want = orc.kept_positions(b)
            for h in range(w.kv_heads):
                np.testing.assert_array_equal(np.sort(snap.unit(b, h)["pos"]), want[h],
                                              err_msg=f"step {t} seq {b} head {h}")
            seen[b] += 1
    assert int(cache.flags.item()) == 0


@pytest.mark.parametrize("capacity", [600, 1100])
def test_streaming_trajectory_heavy_load_shape(capacity):
    w = _w("heavy_load_b512_l2048", policy="streaming")
    _trajectory(w, [600, 512, 511, 40], capacity=capacity + 1, steps=3)


@pytest.mark.parametrize("capacity", [200, 1104])
def test_random_eviction_trajectory(capacity):
    w = _w("reasoning_random_b32", pinned=64, n_keep=96)
    _trajectory(w, [150, 170, 64], capacity=capacity, steps=12)


def test_streaming_trajectory_paged():
    w = _w("mixed_paged_h2o_b128", policy="streaming", n_sink=8, n_recent=40)
    _trajectory(w, [30, 47, 80, 200], capacity=208, steps=6, paged=16)


@pytest.mark.parametrize("capacity", [48, 1100])
def test_h2o_state_synchronised(capacity):
    """At every step the oracle attends over the GPU's pre-step entries and
    selects on the GPU's post-attention scores; the kept set, the scores and
    the compacted rows must match."""
    w = _w("llama3_8b_h2o_b64", n_heavy=6, n_recent=20)
    lengths, steps = [40, 26, 3], 12
    B, G = len(lengths), w.group
    cache = make_cache(w, lengths, capacity)
    hint = capacity + 1
    scores = torch.zeros((B, w.kv_heads, capacity), device="cuda")
    ws = cache.workspace(hint)
    out = torch.empty((B, w.q_heads, w.head_dim), device="cuda")
    keep = torch.empty((B, w.kv_heads, capacity), dtype=torch.int32, device="cuda")
    nout = torch.empty((B, w.kv_heads), dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    seen = list(lengths)
    for t in range(1, steps + 1):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        pre = Snapshot(cache, "e5m2", scores)
        kvc.decode_attn(cache, torch.tensor(seen, dtype=torch.int32, device="cuda"), _act(q),
                        _act(kn), _act(vn), out, scores, max_len_hint=hint, workspace=ws)
        mid = Snapshot(cache, "e5m2", scores)
        kvc.evict_h2o(cache, scores, w.n_heavy, w.n_recent, keep, nout)
        kk, mm = keep.cpu().numpy(), nout.cpu().numpy()
        kvc.compact(cache, keep, nout, scores)
        post = Snapshot(cache, "e5m2", scores)
        o = out.cpu().numpy()
        for (b, h) in pre.units:
            u0, u1, u2 = pre.unit(b, h), mid.unit(b, h), post.unit(b, h)
            ref, psum = oracle_unit_attend("e5m2", q[b, h * G:(h + 1) * G], u0, kn[b, h],
                                           vn[b, h], scale)
            assert np.abs(o[b, h * G:(h + 1) * G] - ref).max() <= OUT_ATOL
            n = u0["n"]
            assert_scores_close(u1["s"][:n], u0["s"] + psum[:n])
            want = oracle.select_h2o(u1["pos"], u1["s"].astype(np.float64), seen[b] + 1,
                                     w.n_heavy, w.n_recent)
            np.testing.assert_array_equal(kk[b, h, :int(mm[b, h])], np.flatnonzero(want))
            r1, r2 = rows_by_pos(u1), rows_by_pos(u2)
            assert set(r2) == set(int(p) for p in u1["pos"][want])
            for p in r2:
                assert r1[p] == r2[p]
        for b in range(B):
            seen[b] += 1


def _live_equal(c0, c1, s0=None, s1=None):
    assert torch.equal(c0.n_slots, c1.n_slots)
    n = c0.n_slots.cpu()
    for b in range(c0.batch):
        for h in range(c0.kv_heads):
            m = int(n[b, h])
            assert torch.equal(c0.pos[b, h, :m], c1.pos[b, h, :m])
            k0, v0 = c0.rows(b, h, range(m))
            k1, v1 = c1.rows(b, h, range(m))
            assert torch.equal(k0, k1) and torch.equal(v0, v1)
            if s0 is not None:
                assert torch.equal(s0[b, h, :m], s1[b, h, :m])


@pytest.mark.parametrize("cap", [160, 1100])
@pytest.mark.parametrize("policy", ["h2o", "h2o_decay", "streaming", "random"])
def test_one_launch_step_equals_three_calls(policy, cap):
    if policy.startswith("h2o"):
        w = _w("llama3_8b_h2o_b64", n_heavy=8, n_recent=40)
    else:
        w = _w("llama3_8b_h2o_b64", policy=policy, n_sink=4, n_recent=40, pinned=50, n_keep=30)
    lengths = [120, 60, 49, 0]
    B = len(lengths)
    caches = [make_cache(w, lengths, cap), make_cache(w, lengths, cap)]
    scs = [torch.zeros((B, w.kv_heads, cap), device="cuda") for _ in range(2)]
    outs = [torch.empty((B, w.q_heads, w.head_dim), device="cuda") for _ in range(2)]
    pol, _ = _policy_pair(w)
    decay = 0.99 if policy == "h2o_decay" else 0.0
    if decay:
        pol = kvc.policy_h2o(w.n_heavy, w.n_recent, decay=decay)
    wss = [c.workspace(cap + 1) for c in caches]
    keep = torch.empty((B, w.kv_heads, cap), dtype=torch.int32, device="cuda")
    nout = torch.empty((B, w.kv_heads), dtype=torch.int32, device="cuda")
    h2o = policy.startswith("h2o")
    for t in range(1, 7):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        new_pos = torch.tensor([L + t - 1 for L in lengths], dtype=torch.int32, device="cuda")
        args = (new_pos, _act(q), _act(kn), _act(vn))
        s0, s1 = (scs[0], scs[1]) if h2o else (None, None)
        kvc.decode_step(caches[0], pol, t, *args, outs[0], s0, max_len_hint=cap + 1,
                        workspace=wss[0])
        kvc.decode_attn(caches[1], *args, outs[1], s1, max_len_hint=cap + 1, workspace=wss[1],
                        score_decay=decay)
        if policy == "streaming":
            kvc.evict_streaming(caches[1], pol.n_sink, pol.n_recent, keep, nout)
        elif h2o:
            kvc.evict_h2o(caches[1], s1, pol.n_heavy, pol.n_recent, keep, nout)
        else:
            kvc.evict_random(caches[1], pol.prompt_len, pol.n_keep, pol.seed, t, keep, nout)
        kvc.compact(caches[1], keep, nout, s1)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        _live_equal(caches[0], caches[1], s0, s1)


def test_paged_equals_contiguous_over_steps():
    w = _w("mixed_paged_h2o_b128", n_heavy=16, n_recent=48)
    lengths, cap = [300, 64, 17, 200], 320
    a = make_cache(w, lengths, cap)
    p = make_cache(w, lengths, cap, paged=16, extra_blocks=7, seed_blocks=3)
    B = len(lengths)
    sa = torch.zeros((B, w.kv_heads, cap), device="cuda")
    sp = torch.zeros_like(sa)
    oa = torch.empty((B, w.q_heads, w.head_dim), device="cuda")
    op = torch.empty_like(oa)
    pol = kvc.policy_h2o(16, 48)
    for t in range(1, 5):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        new_pos = torch.tensor([L + t - 1 for L in lengths], dtype=torch.int32, device="cuda")
        args = (new_pos, _act(q), _act(kn), _act(vn))
        kvc.decode_step(a, pol, t, *args, oa, sa, max_len_hint=cap, workspace=a.workspace(cap))
        kvc.decode_step(p, pol, t, *args, op, sp, max_len_hint=cap, workspace=p.workspace(cap))
        torch.cuda.synchronize()
        assert torch.equal(oa, op)
        _live_equal(a, p, sa, sp)


def test_prompt_scoring_over_an_e5m2_cache():
    # bf16 query rows over E5M2 keys (vector path): scores against the oracle
    w = W_G8
    lengths, m = [150, 37], 60
    cache = make_cache(w, lengths, capacity=160)
    q = np.stack([np.stack([synth.step_inputs(w, b, 10_000 + r)[0] for r in range(m)])
                  for b in range(len(lengths))])
    g = torch.Generator(device="cpu").manual_seed(11)
    scores = (torch.rand((len(lengths), w.kv_heads, 160), generator=g) * 3).cuda()
    pre = Snapshot(cache, "e5m2", scores)
    qp = torch.arange(m, dtype=torch.int32, device="cuda").repeat(len(lengths), 1)
    scale = 1.0 / math.sqrt(w.head_dim)
    kvc.h2o_accumulate(cache, _act(q), m, scores, q_pos=qp, scale=scale)
    post = Snapshot(cache, "e5m2", scores)
    G, D = w.group, w.head_dim
    for (b, h), u0 in pre.units.items():
        n = u0["n"]
        qr = oracle.decode(q[b][:, h * G:(h + 1) * G], "bf16")
        K = oracle.decode(u0["k"], "e5m2").reshape(n, D)
        add = oracle.prompt_scores(qr, K, u0["pos"], np.arange(m), scale)
        assert_scores_close(post.unit(b, h)["s"], u0["s"] + add)
