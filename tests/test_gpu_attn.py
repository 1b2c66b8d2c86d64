"""GPU parity of kvc_decode_attn against the oracle, call by call.

Each case builds a cache from the seeded generators, runs one decode_attn,
and checks every unit: outputs within 2e-3 of the oracle's fp64 attention
over the same entries, the append (slot n holds the new token bit-exactly,
its position, n_slots + 1, nothing else moved), and -- with scores -- every
slot's new score within 1e-5 relative of old score + oracle probability sum.
"""
import math

import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import synth
from kvc_harness import (OUT_ATOL, Snapshot, assert_scores_close, dev, make_cache,
                         oracle_unit_attend)

pytestmark = pytest.mark.gpu


def _path(path, lengths, capacity):
    """(capacity, hint) that route a bf16 / head_dim 128 call to a given path:
    'fused' = one workgroup per unit with LDS-resident logits, 'split' = the
    generic split kernels (attended length above the fused limit of 1024),
    'fallback' = fused launch whose hint is too small for some units."""
    if path == "fused":
        return capacity, max(lengths) + 1
    if path == "split":
        cap = max(capacity, 1104)   # a multiple of the paged block size
        return cap, cap + 1
    if path == "fallback":
        assert max(lengths) + 1 > 512
        return capacity, 1
    return capacity, 0


def _run(w, lengths, capacity, with_scores=True, hint=0, paged=0, step=1, q_zero=False,
         path=None, scale=None):
    if path is not None:
        capacity, hint = _path(path, lengths, capacity)
    B = len(lengths)
    G, D = w.group, w.head_dim
    cache = make_cache(w, lengths, capacity, paged=paged)
    q, kn, vn = synth.batch_step_inputs(w, step, B)
    if q_zero:
        q = np.zeros_like(q)
    scores = None
    if with_scores:
        g = torch.Generator(device="cpu").manual_seed(7)
        scores = (torch.rand((B, w.kv_heads, capacity), generator=g) * 3).cuda()
    pre = Snapshot(cache, w.dtype, scores)
    out = torch.full((B, w.q_heads, D), float("nan"), device="cuda")
    new_pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    ws = cache.workspace(hint)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    kvc.decode_attn(cache, new_pos, dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype), out,
                    scores, scale=scale, max_len_hint=hint, workspace=ws)
    post = Snapshot(cache, w.dtype, scores)
    assert int(cache.flags.item()) == 0
    out_h = out.cpu().numpy()
    worst = 0.0
    for b in range(B):
        for h in range(w.kv_heads):
            u0, u1 = pre.unit(b, h), post.unit(b, h)
            n = u0["n"]
            ref, psum = oracle_unit_attend(w.dtype, q[b, h * G:(h + 1) * G], u0, kn[b, h],
                                           vn[b, h], scale)
            err = np.abs(out_h[b, h * G:(h + 1) * G] - ref).max()
            worst = max(worst, err)
            assert err <= OUT_ATOL, (b, h, err)
            assert u1["n"] == n + 1
            np.testing.assert_array_equal(u1["pos"][:n], u0["pos"])
            assert u1["pos"][n] == lengths[b]
            np.testing.assert_array_equal(u1["k"][:n], u0["k"])
            np.testing.assert_array_equal(u1["v"][:n], u0["v"])
            np.testing.assert_array_equal(u1["k"][n], kn[b, h])
            np.testing.assert_array_equal(u1["v"][n], vn[b, h])
            if with_scores:
                assert_scores_close(u1["s"][:n], u0["s"] + psum[:n])
                assert_scores_close(u1["s"][n:n + 1], psum[n:n + 1])
                assert abs(psum.sum() - G) < 1e-9 * G
    return worst


W_GQA = synth.workload("llama3_8b_h2o_b64", heavy_frac=0.0)
W_HEAVY = synth.workload("llama3_8b_h2o_b64")
W_G5 = synth.workload("reasoning_random_b32")
W_G8 = synth.workload("heavy_load_b512_l2048")
W_F32 = synth.workload("tiny_mha_streaming_f32")


PATHS = ["fused", "split"]


@pytest.mark.parametrize("hint", [0, 1, 600, 2000])
def test_ragged_lengths_every_split_mode(hint):
    # lengths span several tiles and a ragged tail, plus an empty unit
    _run(W_GQA, [0, 37, 300, 511], capacity=512 if hint < 1024 else 1500, hint=hint)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", [W_HEAVY, W_G5, W_G8, W_F32], ids=lambda w: w.name)
def test_group_sizes_dtypes_and_heavy_hitters(w, path):
    _run(w, [129, 700, 2], capacity=1000, path=path)


@pytest.mark.parametrize("path", PATHS)
def test_without_scores(path):
    _run(W_G8, [513, 64], capacity=520, with_scores=False, path=path)


@pytest.mark.parametrize("path", PATHS)
def test_zero_query_spreads_probability_uniformly(path):
    _run(W_GQA, [100, 255], capacity=300, q_zero=True, path=path)


@pytest.mark.parametrize("path", PATHS + ["fallback"])
@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_negative_and_zero_scale(path, scale):
    # any finite scale: the masked rows and slots still weigh nothing
    _run(W_G5, [129, 700, 2], capacity=1000, path=path, scale=scale)


def test_long_units_split_across_workgroups():
    _run(W_G5, [5120, 3000], capacity=5121, hint=5121)


def test_fused_launch_with_too_small_hint_falls_back_exactly():
    _run(W_G8, [900, 40, 513, 1000], capacity=1001, path="fallback")


def test_split_launch_with_too_small_hint_falls_back_exactly():
    # a length bound of 1,100 sizes the split launch for chunks of at most 144
    # slots; the one unit of 4,401 entries needs 560 per split and must take
    # the generic routine inside the same launch, the short units the fast one
    _run(W_GQA, [4400] + [3] * 63, capacity=4401, hint=1100)


def test_group_of_sixteen_query_heads():
    w = synth.workload("heavy_load_b512_l2048", q_heads=128)
    for path in PATHS:
        _run(w, [300, 17], capacity=400, path=path)


@pytest.mark.parametrize("path", PATHS)
def test_paged_layout_matches_contiguous_results(path):
    _run(W_GQA, [17, 100, 300], capacity=320, paged=16, path=path)


@pytest.mark.parametrize("capacity", [4, 1100])
def test_empty_cache_returns_the_new_value(capacity):
    w = W_GQA
    cache = make_cache(w, [0, 0], capacity=capacity)
    q, kn, vn = synth.batch_step_inputs(w, 1, 2)
    out = torch.empty((2, w.q_heads, w.head_dim), device="cuda")
    kvc.decode_attn(cache, torch.zeros(2, dtype=torch.int32, device="cuda"), dev(q, w.dtype),
                    dev(kn, w.dtype), dev(vn, w.dtype), out, None, workspace=cache.workspace())
    vf = synth.bf16_to_f32(vn)
    o = out.cpu().numpy()
    for b in range(2):
        for i in range(w.q_heads):
            np.testing.assert_array_equal(o[b, i], vf[b, i // w.group])


@pytest.mark.parametrize("capacity", [8, 1100])
def test_full_cache_sets_flag_and_does_not_store(capacity):
    w = W_GQA
    cache = make_cache(w, [capacity, 3], capacity=capacity)
    q, kn, vn = synth.batch_step_inputs(w, 1, 2)
    out = torch.empty((2, w.q_heads, w.head_dim), device="cuda")
    before = cache.k.clone()
    kvc.decode_attn(cache, torch.tensor([capacity, 3], dtype=torch.int32, device="cuda"),
                    dev(q, w.dtype), dev(kn, w.dtype), dev(vn, w.dtype), out, None,
                    workspace=cache.workspace())
    torch.cuda.synchronize()
    assert int(cache.flags.item()) & kvc.FLAG_FULL
    assert cache.n_slots[0].tolist() == [capacity] * w.kv_heads
    assert cache.n_slots[1].tolist() == [4] * w.kv_heads
    assert torch.equal(cache.k[0], before[0])
    assert torch.isfinite(out).all()
