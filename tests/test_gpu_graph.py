"""Whole decode steps captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

libkvc enqueues kernels only (no allocation, no memset, no synchronisation),
so a step can be captured once and replayed as new tokens arrive.  Each case
captures one kvc_decode_step on one cache, then replays it several times,
with eager work and host synchronisations between the replays, while a twin
cache takes the same steps eagerly; after every replay the two must hold the
same output and live state bit for bit.
"""
import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import synth
from kvc_harness import dev, make_cache

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("case", ["h2o_one_workgroup", "random_split", "streaming_paged"])
def test_captured_step_replays_like_eager_steps(case):
    if case == "h2o_one_workgroup":
        w = synth.workload("llama3_8b_h2o_b64", n_heavy=8, n_recent=40)
        pol, lengths, cap, paged = kvc.policy_h2o(8, 40), [60, 49, 30], 64, 0
    elif case == "random_split":
        w = synth.workload("reasoning_random_b32", pinned=64, n_keep=96)
        pol, lengths, cap, paged = kvc.policy_random(64, 96, w.seed), [160, 170, 64], 1104, 0
    else:
        w = synth.workload("mixed_paged_h2o_b128", policy="streaming", n_sink=8, n_recent=40)
        pol, lengths, cap, paged = kvc.policy_streaming(8, 40), [30, 47, 80], 208, 16
    h2o = pol.kind == kvc.POLICY_H2O
    B = len(lengths)
    eager, graphed = make_cache(w, lengths, cap, paged=paged), make_cache(w, lengths, cap, paged=paged)
    sc = [torch.zeros((B, w.kv_heads, cap), device="cuda") if h2o else None for _ in range(2)]
    outs = [torch.empty((B, w.q_heads, w.head_dim), device="cuda") for _ in range(2)]
    ws = [eager.workspace(cap + 1), graphed.workspace(cap + 1)]
    # static inputs of the captured step
    q_s = torch.zeros((B, w.q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    kn_s = torch.zeros((B, w.kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    vn_s = torch.zeros_like(kn_s)
    pos_s = torch.zeros((B,), dtype=torch.int32, device="cuda")
    step = 7   # the step number is baked into the capture (random keys use it)

    def run(cache, q, kn, vn, new_pos, out, scores, wsp):
        kvc.decode_step(cache, pol, step, new_pos, q, kn, vn, out, scores, max_len_hint=cap + 1,
                        workspace=wsp)

    # an eager call on a scratch copy first, so that one-time setup (kernel
    # attributes) happens outside the capture
    scratch = make_cache(w, lengths, cap, paged=paged)
    run(scratch, q_s, kn_s, vn_s, pos_s, torch.empty_like(outs[1]),
        torch.zeros_like(sc[1]) if h2o else None, scratch.workspace(cap + 1))
    torch.cuda.synchronize()
    del scratch

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(graphed, q_s, kn_s, vn_s, pos_s, outs[1], sc[1], ws[1])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    seen = list(lengths)
    for t in range(1, 5):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        new_pos = torch.tensor(seen, dtype=torch.int32, device="cuda")
        # eager step on the twin
        run(eager, dev(q, "bf16"), dev(kn, "bf16"), dev(vn, "bf16"), new_pos, outs[0], sc[0], ws[0])
        # some unrelated eager work, then the replay with this step's inputs
        _ = (torch.randn(1 << 16, device="cuda") * 2).sum()
        q_s.copy_(dev(q, "bf16"))
        kn_s.copy_(dev(kn, "bf16"))
        vn_s.copy_(dev(vn, "bf16"))
        pos_s.copy_(new_pos)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), t
        _live_equal(eager, graphed, sc[0], sc[1])
        seen = [L + 1 for L in seen]
    assert int(eager.flags.item()) == 0 and int(graphed.flags.item()) == 0
