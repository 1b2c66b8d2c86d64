"""Checkpoint and resume: a cache's whole state (K, V, positions, slot counts,
H2O scores) copied to host memory after some decode steps and loaded into
freshly allocated device buffers continues exactly like the original --
the same outputs and the same live state bit for bit at every later step.
Random eviction draws its keys from (seed, sequence, kv head, step), so a
resumed run makes the same draws (online compaction study, section 5.3:
compaction decisions must be reproducible)."""
import pytest
import torch

import compressed_decode_attention_amd as kvc
import synth
from test_gpu_fullsize import _assert_live_equal, _prefill

pytestmark = pytest.mark.gpu


def _snapshot(cache, scores):
    names = ("k", "v", "pos", "n_slots", "flags")
    host = {n: getattr(cache, n).cpu() for n in names}
    if cache.block_size:
        host["block_table"] = cache.block_table.cpu()
    return host, (scores.cpu() if scores is not None else None)


def _restore(like, host, scores_host):
    bs = like.block_size
    c = kvc.KvCache(like.batch, like.q_heads, like.kv_heads, like.head_dim, like.capacity,
                    like.dtype, block_size=bs, num_blocks=like.num_blocks,
                    block_table=host.get("block_table"))
    for n in ("k", "v", "pos", "n_slots", "flags"):
        getattr(c, n).copy_(host[n])
    sc = scores_host.cuda() if scores_host is not None else None
    torch.cuda.synchronize()
    return c, sc


def _run(w, cache, pol, h2o, seen0, before, after, hint0, hint):
    B, Hq, Hkv, D = cache.batch, cache.q_heads, cache.kv_heads, cache.head_dim
    scores = torch.zeros((B, Hkv, cache.capacity), device="cuda") if h2o else None
    seen = torch.tensor(seen0, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ws = cache.workspace(max(hint0, hint))

    def inputs(t):
        return (synth.device_normal((B, Hq, D), w.seed, w.wid, synth.T_Q, t),
                synth.device_normal((B, Hkv, D), w.seed, w.wid, synth.T_KNEW, t),
                synth.device_normal((B, Hkv, D), w.seed, w.wid, synth.T_VNEW, t))

    for t in range(1, before + 1):
        kvc.decode_step(cache, pol, t, seen + (t - 1), *inputs(t), out, scores,
                        max_len_hint=hint0 if t == 1 else hint, workspace=ws)
    host, sc_host = _snapshot(cache, scores)
    # the original continues ...
    outs = []
    for t in range(before + 1, before + after + 1):
        kvc.decode_step(cache, pol, t, seen + (t - 1), *inputs(t), out, scores,
                        max_len_hint=hint, workspace=ws)
        outs.append(out.clone())
    # ... and so does a copy restored into new buffers (and a new workspace)
    fresh, sc2 = _restore(cache, host, sc_host)
    ws2 = fresh.workspace(max(hint0, hint))
    out2 = torch.empty_like(out)
    for i, t in enumerate(range(before + 1, before + after + 1)):
        kvc.decode_step(fresh, pol, t, seen + (t - 1), *inputs(t), out2, sc2,
                        max_len_hint=hint, workspace=ws2)
        torch.cuda.synchronize()
        assert torch.equal(out2, outs[i]), f"step {t}: resumed output differs"
    assert int(cache.flags.item()) == 0 and int(fresh.flags.item()) == 0
    _assert_live_equal(cache, fresh, scores, sc2)


def test_resume_h2o_fused_steps():
    w = synth.workload("llama3_8b_h2o_b64", batch=8)
    P = 700
    cache = _prefill(w, 8, P + 1, P, heavy_frac=w.heavy_frac)
    _run(w, cache, kvc.policy_h2o(64, 448), True, [P] * 8, 4, 6, P + 1, 513)


def test_resume_random_eviction_split_path():
    # 1,024 + 1,500 entries: the split path, one eviction per head per step
    w = synth.workload("reasoning_random_b32", batch=4)
    fill = 1024 + 1500
    cache = _prefill(w, 4, fill + 1, fill)
    _run(w, cache, kvc.policy_random(1024, 1500, 77), False, [fill] * 4, 3, 5, fill + 1,
         fill + 1)


def test_resume_random_eviction_fused_path():
    w = synth.workload("reasoning_random_b32", batch=4)
    fill = 96 + 300
    cache = _prefill(w, 4, fill + 1, fill)
    _run(w, cache, kvc.policy_random(96, 300, 5), False, [fill] * 4, 3, 5, fill + 1, fill + 1)


def test_resume_paged_h2o():
    w = synth.workload("mixed_paged_h2o_b128", batch=6)
    lengths = [600, 513, 900, 1200, 700, 520]
    cap = 1216
    cache = _prefill(w, 6, cap, None, paged=16, lengths=lengths)
    _run(w, cache, kvc.policy_h2o(64, 448), True, lengths, 3, 5, cap, 513)
