"""GPU parity of kvc_h2o_accumulate (H2O scores from a block of query rows)
against the oracle's prompt scoring.

Each case fills a cache, draws m query rows per sequence, starts from random
scores and checks every slot: new score within 1e-5 relative of old score +
the oracle's probability sum (rows see the slots with pos <= their own
position; every slot when no positions are given).  The matrix-core path
(bf16, head_dim 128, any group size) and the VALU path (fp32 / head_dim 64)
are both covered, with ragged row and slot counts that span several tiles,
paged and shuffled caches, empty units, and the full prompt of the LLaMA-3-8B
workload (sampled units against the oracle, every unit against the mass
invariant).
"""
import math

import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle
import synth
from kvc_harness import Snapshot, assert_scores_close, dev, host, make_cache

pytestmark = pytest.mark.gpu


def _rows(w, B, m):
    """Query rows [B, m, Hq, D] (storage): row r of sequence b is the step-r
    query of the workload's generator."""
    return np.stack([np.stack([synth.step_inputs(w, b, 10_000 + r)[0] for r in range(m)])
                     for b in range(B)])


def _check(w, cache, q_rows, q_pos, scale=None, units=None, check_mass=False):
    B, m = q_rows.shape[0], q_rows.shape[1]
    G, D = w.group, w.head_dim
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    g = torch.Generator(device="cpu").manual_seed(11)
    scores = (torch.rand((B, w.kv_heads, cache.capacity), generator=g) * 3).cuda()
    pre = Snapshot(cache, w.dtype, scores, units)
    qd = dev(q_rows, w.dtype)
    qp = None if q_pos is None else torch.tensor(q_pos, dtype=torch.int32, device="cuda")
    kvc.h2o_accumulate(cache, qd, m, scores, q_pos=qp, scale=scale)
    post = Snapshot(cache, w.dtype, scores, units)
    for (b, h), u0 in pre.units.items():
        u1 = post.unit(b, h)
        n = u0["n"]
        if n == 0:
            continue
        qr = oracle.decode(q_rows[b][:, h * G:(h + 1) * G], w.dtype)
        K = oracle.decode(u0["k"], w.dtype).reshape(n, D)
        add = oracle.prompt_scores(qr, K, u0["pos"], None if q_pos is None else q_pos[b], scale)
        assert_scores_close(u1["s"], u0["s"] + add)
        if check_mass:
            assert abs((u1["s"] - u0["s"]).sum() - G * m) < 1e-4 * G * m
    return scores


W_G4 = synth.workload("llama3_8b_h2o_b64", heavy_frac=0.0)
W_HEAVY = synth.workload("llama3_8b_h2o_b64")
W_G5 = synth.workload("reasoning_random_b32")
W_G8 = synth.workload("heavy_load_b512_l2048")
W_F32 = synth.workload("tiny_mha_streaming_f32")


@pytest.mark.parametrize("w", [W_G4, W_HEAVY, W_G5, W_G8], ids=lambda w: w.name)
@pytest.mark.parametrize("m", [37, 150])
def test_causal_prompt_rows(w, m):
    # the prompt's own rows over the prompt: slots = positions 0..m-1
    lengths = [m, m]
    cache = make_cache(w, lengths, capacity=m + 5)
    q = _rows(w, len(lengths), m)
    _check(w, cache, q, [np.arange(m), np.arange(m)])


@pytest.mark.parametrize("w", [W_G4, W_G8, W_F32], ids=lambda w: w.name)
@pytest.mark.parametrize("scale", [-0.18, 0.0])
def test_negative_and_zero_scale(w, scale):
    # any finite scale: a negative one flips which slots dominate, zero spreads
    # every row evenly over the slots it sees
    m = 150
    cache = make_cache(w, [m, m], capacity=m + 5)
    q = _rows(w, 2, m)
    _check(w, cache, q, [np.arange(m), np.arange(m)], scale=scale, check_mass=True)


def test_group_of_sixteen_and_one():
    for q_heads in (128, 8):   # G = 16, G = 1
        w = synth.workload("heavy_load_b512_l2048", q_heads=q_heads)
        cache = make_cache(w, [70, 131], capacity=140)
        _check(w, cache, _rows(w, 2, 131), [np.arange(131), np.arange(131)])


def test_rows_without_positions_see_every_slot():
    w = W_G4
    cache = make_cache(w, [130, 64, 1], capacity=140)
    _check(w, cache, _rows(w, 3, 50), None)


def test_shuffled_slots_and_arbitrary_positions():
    # slots hold a random subset of positions in random order; rows at random
    # positions, some before every slot (they add nothing)
    w = W_G4
    B, n, m = 2, 180, 70
    cache = make_cache(w, [n] * B, capacity=n)
    rng = np.random.default_rng(4)
    for b in range(B):
        for h in range(w.kv_heads):
            cache.pos[b, h, :n] = torch.tensor(rng.permutation(600)[:n], dtype=torch.int32)
    q_pos = [np.sort(rng.integers(-20, 620, m)) for _ in range(B)]
    _check(w, cache, _rows(w, B, m), q_pos)


def test_several_blocks_ragged_tails_and_unsorted_rows():
    # more slots than one workgroup's block (256) with a ragged last block,
    # rows in ragged 64-position tiles: sequence 0 at every other position
    # (a row tile sees slots of several blocks), sequence 1 at unsorted
    # positions, some past every slot (whole position tiles of mixed rows)
    w = W_G5
    lengths, m = [600, 517], 333
    cache = make_cache(w, lengths, capacity=600)
    rng = np.random.default_rng(9)
    q_pos = [np.arange(m) * 2, rng.permutation(700)[:m]]
    _check(w, cache, _rows(w, len(lengths), m), q_pos)


def test_partial_windows_of_the_block_order():
    # 160 units = 20 per XCD: the statistics pass's windows of 8 units and the
    # scores pass's windows of 16 both end with a partial window of 4; units
    # sampled from full and partial windows of several XCDs, each against the
    # oracle and the probability mass
    w = W_G4
    B, L = 20, 300
    cache = make_cache(w, [L] * B, capacity=L)
    units = [divmod(u, w.kv_heads) for u in (0, 7, 8 * 8 + 3, 8 * 15 + 6, 8 * 16 + 5, 8 * 17 + 1, 159)]
    _check(w, cache, _rows(w, B, L), [np.arange(L)] * B, units=units, check_mass=True)


def test_paged_cache_matches_contiguous_bit_for_bit():
    w = W_G8
    lengths, m = [200, 33, 129], 160
    q = _rows(w, len(lengths), m)
    q_pos = [np.arange(m)] * len(lengths)
    s_paged = _check(w, make_cache(w, lengths, capacity=208, paged=16), q, q_pos)
    s_flat = _check(w, make_cache(w, lengths, capacity=208), q, q_pos)
    for b, L in enumerate(lengths):
        assert torch.equal(s_paged[b, :, :L], s_flat[b, :, :L])


def test_empty_units_and_zero_rows():
    w = W_G4
    cache = make_cache(w, [0, 40], capacity=48)
    _check(w, cache, _rows(w, 2, 20), [np.arange(20)] * 2)
    scores = torch.ones((2, w.kv_heads, 48), device="cuda")
    kvc.h2o_accumulate(cache, torch.empty(0, dtype=torch.bfloat16, device="cuda"), 0, scores)
    assert bool((scores == 1).all())


@pytest.mark.parametrize("w", [W_F32, synth.workload("tiny_mha_streaming_f32", dtype="bf16")],
                         ids=["f32_d64", "bf16_d64"])
def test_vector_path_for_other_shapes(w):
    cache = make_cache(w, [90, 17], capacity=96)
    _check(w, cache, _rows(w, 2, 90), [np.arange(90)] * 2)


def test_deterministic_across_calls():
    w = W_G8
    cache = make_cache(w, [300, 300], capacity=300)
    qd = dev(_rows(w, 2, 300), w.dtype)
    qp = torch.arange(300, dtype=torch.int32, device="cuda").repeat(2, 1)
    outs = []
    for _ in range(2):
        s = torch.zeros((2, w.kv_heads, 300), device="cuda")
        kvc.h2o_accumulate(cache, qd, 300, s, q_pos=qp)
        outs.append(s)
    assert torch.equal(outs[0], outs[1])


def test_full_prompt_of_the_llama3_workload():
    # 64 sequences x 2,048-token prompts, 32 q / 8 kv heads: every row of the
    # prompt scores the prompt (the seed of H2O before the first trim).  Two
    # units against the oracle; every unit carries mass G per row.
    w = W_HEAVY
    B, P, G, D = 64, 2048, w.group, w.head_dim
    cache = kvc.KvCache(B, w.q_heads, w.kv_heads, D, P, kvc.BF16)
    cache.k.copy_(synth.device_normal(cache.k.shape, w.seed, w.wid, 1, scale_rows_frac=0.02))
    cache.v.copy_(synth.device_normal(cache.v.shape, w.seed, w.wid, 2))
    cache.pos.copy_(torch.arange(P, dtype=torch.int32, device="cuda").expand(B, w.kv_heads, P))
    cache.n_slots.fill_(P)
    q = synth.device_normal((B, P, w.q_heads, D), w.seed, w.wid, 3)
    qp = torch.arange(P, dtype=torch.int32, device="cuda").repeat(B, 1)
    scores = torch.zeros((B, w.kv_heads, P), device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    kvc.h2o_accumulate(cache, q, P, scores, q_pos=qp)
    e1.record()
    torch.cuda.synchronize()
    print(f"[prompt scoring] B={B} P={P} Hq={w.q_heads}: {e0.elapsed_time(e1):.2f} ms", flush=True)
    mass = scores.double().sum(dim=2)
    assert bool(((mass - G * P).abs() < 1e-3 * G * P).all())
    scale = 1.0 / math.sqrt(D)
    for (b, h) in [(0, 0), (B - 1, w.kv_heads - 1)]:
        K = oracle.decode(host(cache.k[b, h], "bf16"), "bf16")
        qr = oracle.decode(host(q[b, :, h * G:(h + 1) * G].contiguous(), "bf16"), "bf16")
        want = oracle.prompt_scores(qr, K, np.arange(P), np.arange(P), scale)
        assert_scores_close(scores[b, h].cpu().numpy(), want)
