"""Multi-step parity: whole decode steps (attention + eviction + compaction).

* StreamingLLM and random eviction depend only on positions (and the random
  keys), so the oracle runs its own full trajectory and every step's kept
  position sets must match bit-exactly and every step's outputs within 2e-3.
* H2O is checked state-synchronised: at every step the oracle attends over
  the GPU's pre-step entries, its selection runs on the GPU's post-attention
  score vector, and the kept set must match exactly (scores within 1e-5).
* The one-launch step (kvc_decode_step) must leave exactly the state of the
  three-call sequence; the paged layout exactly the state of the contiguous.
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


def _policy_pair(w):
    if w.policy == "streaming":
        return kvc.policy_streaming(w.n_sink, w.n_recent), oracle.Policy.streaming(w.n_sink,
                                                                                    w.n_recent)
    if w.policy == "h2o":
        return kvc.policy_h2o(w.n_heavy, w.n_recent), oracle.Policy.h2o(w.n_heavy, w.n_recent)
    if w.policy == "random":
        return (kvc.policy_random(w.pinned, w.n_keep, w.seed),
                oracle.Policy.random(w.pinned, w.n_keep, w.seed))
    return kvc.policy_full(), oracle.Policy.full()


def _trajectory(w, lengths, capacity, steps, fused=True, paged=0, hint=None):
    """Oracle trajectory vs GPU trajectory, kept sets and outputs every step.

    hint None = the capacity bound: up to 1024 attended entries that is the
    one-workgroup fused kernel (bf16, head_dim 128), above it the split path."""
    hint = capacity + 1 if hint is None else hint
    B = len(lengths)
    cache = make_cache(w, lengths, capacity, paged=paged)
    orc = oracle.Oracle(w.q_heads, w.kv_heads, w.head_dim, w.dtype)
    for b, L in enumerate(lengths):
        k, v = synth.prefill_kv(w, b, L)
        orc.load(b, k, v)
    pol_gpu, pol_orc = _policy_pair(w)
    ws = cache.workspace(hint)
    out = torch.empty((B, w.q_heads, w.head_dim), device="cuda")
    scores = torch.zeros((B, w.kv_heads, capacity), device="cuda") if w.policy == "h2o" else None
    seen = list(lengths)
    for t in range(1, steps + 1):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        new_pos = torch.tensor(seen, dtype=torch.int32, device="cuda")
        qd, knd, vnd = dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype)
        if fused:
            kvc.decode_step(cache, pol_gpu, t, new_pos, qd, knd, vnd, out, scores,
                            max_len_hint=hint, workspace=ws)
        else:
            _three_calls(cache, w, pol_gpu, t, new_pos, qd, knd, vnd, out, scores, ws, hint)
        snap = Snapshot(cache, w.dtype)
        o = out.cpu().numpy()
        for b in range(B):
            ref, _ = orc.step(b, q[b], kn[b], vn[b], pol_orc, step=t)
            err = np.abs(o[b] - ref).max()
            assert err <= OUT_ATOL, (t, b, err)
            want = orc.kept_positions(b)
            for h in range(w.kv_heads):
                got = np.sort(snap.unit(b, h)["pos"])
                np.testing.assert_array_equal(got, want[h], err_msg=f"step {t} seq {b} head {h}")
            seen[b] += 1
    assert int(cache.flags.item()) == 0
    return cache


def _three_calls(cache, w, pol, t, new_pos, q, kn, vn, out, scores, ws, hint):
    kvc.decode_attn(cache, new_pos, q, kn, vn, out, scores, max_len_hint=hint, workspace=ws,
                    score_decay=pol.decay if pol.kind == kvc.POLICY_H2O else 0.0)
    keep = torch.empty((cache.batch, cache.kv_heads, cache.capacity), dtype=torch.int32,
                       device="cuda")
    nout = torch.empty((cache.batch, cache.kv_heads), dtype=torch.int32, device="cuda")
    if pol.kind == kvc.POLICY_STREAMING:
        kvc.evict_streaming(cache, pol.n_sink, pol.n_recent, keep, nout)
    elif pol.kind == kvc.POLICY_H2O:
        kvc.evict_h2o(cache, scores, pol.n_heavy, pol.n_recent, keep, nout)
    elif pol.kind == kvc.POLICY_RANDOM:
        kvc.evict_random(cache, pol.prompt_len, pol.n_keep, pol.seed, t, keep, nout)
    else:
        return
    kvc.compact(cache, keep, nout, scores)


def test_tiny_streaming_fp32_workload_all_steps():
    # 1 sequence, 8 MHA heads, head_dim 64, 1024 cached fp32, 64 + 448, 16 steps
    w = synth.workload("tiny_mha_streaming_f32")
    _trajectory(w, [w.prompt_len], capacity=w.prompt_len + 1, steps=w.steps)


def test_tiny_streaming_three_call_path():
    w = synth.workload("tiny_mha_streaming_f32")
    _trajectory(w, [w.prompt_len], capacity=w.prompt_len + 1, steps=4, fused=False)


@pytest.mark.parametrize("capacity", [200, 1100])
def test_random_eviction_trajectory_reaches_steady_state(capacity):
    # reasoning-trace shape, shortened: pinned prompt 64, 96 kept generated
    w = synth.workload("reasoning_random_b32", pinned=64, n_keep=96)
    _trajectory(w, [150, 170, 64], capacity=capacity, steps=24)


def test_random_eviction_on_paged_cache_split_path():
    # paged blocks of 16 and a capacity above the one-workgroup limit: the
    # split kernels rank their chunks' candidates through the block table
    w = synth.workload("reasoning_random_b32", pinned=64, n_keep=96)
    _trajectory(w, [150, 170, 64], capacity=1104, steps=12, paged=16)


def test_random_eviction_three_call_path():
    w = synth.workload("reasoning_random_b32", pinned=64, n_keep=96)
    _trajectory(w, [150, 170], capacity=200, steps=6, fused=False)


def test_random_eviction_long_prompt_steady_state():
    # reasoning shape at its real budget: 1,024 pinned + 4,096 kept generated,
    # starting one token over budget so that every step evicts one per head
    w = synth.workload("reasoning_random_b32")
    _trajectory(w, [5120, 5000], capacity=5121, steps=3)


@pytest.mark.parametrize("capacity", [208, 1104])
def test_streaming_on_paged_cache(capacity):
    w = synth.workload("mixed_paged_h2o_b128", policy="streaming", n_sink=8, n_recent=40)
    _trajectory(w, [30, 47, 80, 200], capacity=capacity, steps=8, paged=16)


def test_streaming_heavy_load_shape_fused():
    # the heavy-load layer shape (G = 8) with its 64 + 448 budget, reduced batch
    w = synth.workload("heavy_load_b512_l2048", policy="streaming")
    _trajectory(w, [600, 512, 511, 900], capacity=901, steps=3, hint=901)


def test_undersized_hint_falls_back_inside_the_step_kernel():
    w = synth.workload("heavy_load_b512_l2048", policy="streaming")
    _trajectory(w, [900, 40, 700], capacity=901, steps=3, hint=2)


def _h2o_sync(w, lengths, capacity, steps, paged=0, check_units=None, hint=None, decay=0.0):
    hint = capacity + 1 if hint is None else hint
    B = len(lengths)
    G = w.group
    cache = make_cache(w, lengths, capacity, paged=paged)
    scores = torch.zeros((B, w.kv_heads, capacity), device="cuda")
    ws = cache.workspace(hint)
    out = torch.empty((B, w.q_heads, w.head_dim), device="cuda")
    keep = torch.empty((B, w.kv_heads, capacity), dtype=torch.int32, device="cuda")
    nout = torch.empty((B, w.kv_heads), dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    units = check_units or [(b, h) for b in range(B) for h in range(w.kv_heads)]
    seen = list(lengths)
    for t in range(1, steps + 1):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        pre = Snapshot(cache, w.dtype, scores, units)
        kvc.decode_attn(cache, torch.tensor(seen, dtype=torch.int32, device="cuda"),
                        dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype), out, scores,
                        max_len_hint=hint, workspace=ws, score_decay=decay)
        mid = Snapshot(cache, w.dtype, scores, units)
        kvc.evict_h2o(cache, scores, w.n_heavy, w.n_recent, keep, nout)
        kk, mm = keep.cpu().numpy(), nout.cpu().numpy()
        kvc.compact(cache, keep, nout, scores)
        post = Snapshot(cache, w.dtype, scores, units)
        o = out.cpu().numpy()
        for (b, h) in units:
            u0, u1, u2 = pre.unit(b, h), mid.unit(b, h), post.unit(b, h)
            ref, psum = oracle_unit_attend(w.dtype, q[b, h * G:(h + 1) * G], u0, kn[b, h],
                                           vn[b, h], scale)
            assert np.abs(o[b, h * G:(h + 1) * G] - ref).max() <= OUT_ATOL
            n = u0["n"]
            if decay == 0.0:
                assert_scores_close(u1["s"][:n], u0["s"] + psum[:n])
                assert_scores_close(u1["s"][n:n + 1], psum[n:])
            else:   # decayed activity: old score fades, this step's weight enters
                assert_scores_close(u1["s"][:n], decay * u0["s"] + (1 - decay) * psum[:n])
                assert_scores_close(u1["s"][n:n + 1], (1 - decay) * psum[n:])
            # oracle selection on the GPU's own post-attention scores
            L = seen[b] + 1
            want = oracle.select_h2o(u1["pos"], u1["s"].astype(np.float64), L, w.n_heavy,
                                     w.n_recent)
            m = int(mm[b, h])
            np.testing.assert_array_equal(kk[b, h, :m], np.flatnonzero(want))
            # compaction: exactly the kept rows, bit-exact, with their scores
            r1, r2 = rows_by_pos(u1), rows_by_pos(u2)
            assert set(r2) == set(int(p) for p in u1["pos"][want])
            for p in r2:
                assert r1[p] == r2[p]
        for b in range(B):
            seen[b] += 1


def test_h2o_state_synchronised_with_heavy_hitters():
    # LLaMA-3-8B shape with 2% heavy keys, 64 + 448, a 2,048-token prompt
    w = synth.workload("llama3_8b_h2o_b64")
    _h2o_sync(w, [2048, 2048, 700], capacity=2049, steps=4)


@pytest.mark.parametrize("capacity", [48, 1100])
def test_h2o_small_budget_many_steps(capacity):
    w = synth.workload("llama3_8b_h2o_b64", n_heavy=6, n_recent=20)
    _h2o_sync(w, [40, 26, 3], capacity=capacity, steps=30)


def test_h2o_on_paged_mixed_lengths():
    w = synth.workload("mixed_paged_h2o_b128", n_heavy=16, n_recent=48)
    _h2o_sync(w, [600, 64, 1000, 17], capacity=1008, steps=5, paged=16)


@pytest.mark.parametrize("decay", [0.5, 0.99])
@pytest.mark.parametrize("capacity", [48, 1100])
def test_h2o_decayed_activity_small_budget(decay, capacity):
    # both paths (one-workgroup step kernel at 48, split kernels at 1,100)
    w = synth.workload("llama3_8b_h2o_b64", n_heavy=6, n_recent=20)
    _h2o_sync(w, [40, 26, 3], capacity=capacity, steps=20, decay=decay)


def test_h2o_decayed_activity_heavy_load_shape():
    w = synth.workload("heavy_load_b512_l2048")
    _h2o_sync(w, [512, 512, 300, 700], capacity=701, steps=3, decay=0.99)


def test_h2o_heavy_load_shape_fused_steady_state():
    # heavy-load layer (G = 8), 64 + 448, units starting at and below budget
    w = synth.workload("heavy_load_b512_l2048")
    _h2o_sync(w, [512, 512, 300, 700], capacity=701, steps=3)


def _state(cache, scores, dn):
    s = Snapshot(cache, dn, scores)
    return {k: rows_by_pos(v) for k, v in s.units.items()}, s


def _live_equal(c0, c1, s0=None, s1=None):
    """Same live state: slot counts, and per unit the live slots' K, V, pos
    (and scores) bit for bit.  Slots at or above n_slots are not state."""
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
@pytest.mark.parametrize("policy", ["h2o", "h2o_decay", "streaming", "random", "full"])
def test_fused_step_equals_three_calls(policy, cap):
    w = synth.workload("llama3_8b_h2o_b64", policy=policy, n_heavy=8, n_recent=40,
                       n_sink=4, pinned=50, n_keep=30) if not policy.startswith("h2o") else \
        synth.workload("llama3_8b_h2o_b64", n_heavy=8, n_recent=40)
    lengths = [120, 60, 49, 0]
    caches = [make_cache(w, lengths, cap), make_cache(w, lengths, cap)]
    B = len(lengths)
    scs = [torch.zeros((B, w.kv_heads, cap), device="cuda") for _ in range(2)]
    outs = [torch.empty((B, w.q_heads, w.head_dim), device="cuda") for _ in range(2)]
    pol, _ = _policy_pair(w)
    if policy == "h2o_decay":
        pol = kvc.policy_h2o(w.n_heavy, w.n_recent, decay=0.99)
    wss = [c.workspace(cap + 1) for c in caches]
    for t in range(1, 7):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        new_pos = torch.tensor([L + t - 1 for L in lengths], dtype=torch.int32, device="cuda")
        args = (new_pos, dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype))
        sc0 = scs[0] if policy.startswith("h2o") else None
        sc1 = scs[1] if policy.startswith("h2o") else None
        kvc.decode_step(caches[0], pol, t, *args, outs[0], sc0, max_len_hint=cap + 1,
                        workspace=wss[0])
        _three_calls(caches[1], w, pol, t, *args, outs[1], sc1, wss[1], cap + 1)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        _live_equal(caches[0], caches[1], sc0, sc1)


def test_paged_and_contiguous_give_identical_results():
    w = synth.workload("mixed_paged_h2o_b128", n_heavy=16, n_recent=48)
    lengths, cap = [300, 64, 17, 200], 320
    a = make_cache(w, lengths, cap)
    p = make_cache(w, lengths, cap, paged=16, extra_blocks=7, seed_blocks=3)
    B = len(lengths)
    sa = torch.zeros((B, w.kv_heads, cap), device="cuda")
    sp = torch.zeros((B, w.kv_heads, cap), device="cuda")
    oa = torch.empty((B, w.q_heads, w.head_dim), device="cuda")
    op = torch.empty_like(oa)
    pol = kvc.policy_h2o(16, 48)
    for t in range(1, 6):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        new_pos = torch.tensor([L + t - 1 for L in lengths], dtype=torch.int32, device="cuda")
        args = (new_pos, dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype))
        kvc.decode_step(a, pol, t, *args, oa, sa, max_len_hint=cap, workspace=a.workspace(cap))
        kvc.decode_step(p, pol, t, *args, op, sp, max_len_hint=cap, workspace=p.workspace(cap))
        torch.cuda.synchronize()
        assert torch.equal(oa, op)
        _live_equal(a, p, sa, sp)


def test_h2o_at_maximum_capacity():
    # one unit at the library's capacity limit (65,536 slots: 64 splits of
    # 1,024) beside a short one; the first step ranks 65,088 candidates from
    # global memory, the second is a steady step
    w = synth.workload("llama3_8b_h2o_b64")
    _h2o_sync(w, [65535, 3000], capacity=65536, steps=2)


@pytest.mark.parametrize("policy", ["h2o", "random", "streaming"])
def test_whole_step_equals_three_calls_at_maximum_capacity(policy):
    w = synth.workload("llama3_8b_h2o_b64", policy=policy, pinned=1024, n_keep=4096)
    lengths, cap = [65535, 0], 65536
    caches = [make_cache(w, lengths, cap), make_cache(w, lengths, cap)]
    B = len(lengths)
    h2o = policy == "h2o"
    scs = [torch.zeros((B, w.kv_heads, cap), device="cuda") for _ in range(2)]
    outs = [torch.empty((B, w.q_heads, w.head_dim), device="cuda") for _ in range(2)]
    pol, _ = _policy_pair(w)
    wss = [c.workspace(cap) for c in caches]
    for t in range(1, 3):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        new_pos = torch.tensor([L + t - 1 for L in lengths], dtype=torch.int32, device="cuda")
        args = (new_pos, dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype))
        kvc.decode_step(caches[0], pol, t, *args, outs[0], scs[0] if h2o else None,
                        max_len_hint=cap, workspace=wss[0])
        _three_calls(caches[1], w, pol, t, *args, outs[1], scs[1] if h2o else None, wss[1], cap)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        _live_equal(caches[0], caches[1], scs[0] if h2o else None, scs[1] if h2o else None)
    assert int(caches[0].flags.item()) == 0 and int(caches[1].flags.item()) == 0


@pytest.mark.parametrize("policy", ["h2o", "random"])
def test_whole_step_on_a_full_cache_equals_three_calls(policy):
    # every slot of the cache in use: the new token is attended but not stored
    # (KVC_FLAG_FULL), and the one slot that leaves is chosen among the cached
    # ones only; split path (capacity above the one-workgroup limit)
    cap = 1100
    w = synth.workload("llama3_8b_h2o_b64", policy=policy, n_heavy=8, n_recent=cap - 9,
                       pinned=50, n_keep=cap - 51)
    lengths = [cap, cap]
    caches = [make_cache(w, lengths, cap), make_cache(w, lengths, cap)]
    B = len(lengths)
    h2o = policy == "h2o"
    scs = [torch.zeros((B, w.kv_heads, cap), device="cuda") for _ in range(2)]
    outs = [torch.empty((B, w.q_heads, w.head_dim), device="cuda") for _ in range(2)]
    pol, _ = _policy_pair(w)
    wss = [c.workspace(cap + 1) for c in caches]
    q, kn, vn = synth.batch_step_inputs(w, 1, B)
    new_pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    args = (new_pos, dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype))
    kvc.decode_step(caches[0], pol, 1, *args, outs[0], scs[0] if h2o else None,
                    max_len_hint=cap + 1, workspace=wss[0])
    _three_calls(caches[1], w, pol, 1, *args, outs[1], scs[1] if h2o else None, wss[1], cap + 1)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    _live_equal(caches[0], caches[1], scs[0] if h2o else None, scs[1] if h2o else None)
    assert bool((caches[0].n_slots == cap - 1).all())
    for c in caches:
        assert int(c.flags.item()) & kvc.FLAG_FULL


@pytest.mark.parametrize("cap", [700, 1100])
def test_h2o_ties_keep_the_lowest_positions(cap):
    # q = 0: every attended slot gets probability 1 / (n + 1) from every head,
    # so every candidate ties and the 64 heavy hitters are the lowest
    # positions.  Slots hold shuffled positions, so a tie broken by slot
    # instead of position would keep other tokens.  One-workgroup step
    # (capacity 700) and the split path (1,100).
    w = synth.workload("llama3_8b_h2o_b64", n_heavy=64, n_recent=448)
    lengths = [cap - 1, 600]
    cache = make_cache(w, lengths, cap)
    rng = np.random.default_rng(5)
    for b, L in enumerate(lengths):
        perm = torch.from_numpy(rng.permutation(L).astype(np.int32)).cuda()
        cache.pos[b, :, :L] = perm
    B = len(lengths)
    scores = torch.zeros((B, w.kv_heads, cap), device="cuda")
    out = torch.empty((B, w.q_heads, w.head_dim), device="cuda")
    _, kn, vn = synth.batch_step_inputs(w, 1, B)
    q = torch.zeros((B, w.q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    new_pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    kvc.decode_step(cache, kvc.policy_h2o(64, 448), 1, new_pos, q, dev(kn, w.dtype),
                    dev(vn, w.dtype), out, scores, max_len_hint=cap, workspace=cache.workspace(cap))
    torch.cuda.synchronize()
    n = cache.n_slots.cpu().numpy()
    pos = cache.pos.cpu().numpy()
    for b, L in enumerate(lengths):
        seen = L + 1   # positions 0..L after the step
        want = np.array(list(range(64)) + list(range(seen - 448, seen)), dtype=np.int32)
        for h in range(w.kv_heads):
            assert n[b, h] == 512
            np.testing.assert_array_equal(np.sort(pos[b, h, :512]), want)
    assert int(cache.flags.item()) == 0
