"""kvc_decode_step_noalloc (static per-GPU scratch, no allocation) against
kvc_decode_step with a caller workspace, through the C ABI: two calls in a
row on the same GPU, the second with a smaller input, must give the same
outputs and the same cache state bit for bit."""
import math

import pytest
import torch

import compressed_decode_attention_amd as kvc
import synth
from test_gpu_fullsize import _assert_live_equal, _clone, _prefill

pytestmark = pytest.mark.gpu


def _both(w, cache, pol, step, lengths, hint, h2o, heavy_frac=0.0):
    B, Hq, Hkv, D = cache.batch, cache.q_heads, cache.kv_heads, cache.head_dim
    twin = _clone(cache)
    sc_a = torch.zeros((B, Hkv, cache.capacity), device="cuda") if h2o else None
    sc_b = torch.zeros_like(sc_a) if h2o else None
    q = synth.device_normal((B, Hq, D), w.seed, w.wid, synth.T_Q, step)
    kn = synth.device_normal((B, Hkv, D), w.seed, w.wid, synth.T_KNEW, step,
                             scale_rows_frac=heavy_frac)
    vn = synth.device_normal((B, Hkv, D), w.seed, w.wid, synth.T_VNEW, step)
    seen = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    out_a = torch.empty((B, Hq, D), device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    kvc.decode_step(cache, pol, step, seen, q, kn, vn, out_a, sc_a, max_len_hint=hint,
                    workspace=cache.workspace(hint))
    assert twin.workspace_bytes(hint) <= kvc.NOALLOC_SCRATCH_BYTES
    kvc.decode_step_noalloc(twin, pol, step, seen, q, kn, vn, out_b, sc_b, max_len_hint=hint)
    torch.cuda.synchronize()
    assert int(cache.flags.item()) == 0 and int(twin.flags.item()) == 0
    assert torch.equal(out_a, out_b)
    _assert_live_equal(cache, twin, sc_a, sc_b)
    return twin


def test_noalloc_step_equals_the_workspace_step_twice_second_smaller():
    # call 1: 32 units over a 2,048-token prompt, H2O trim on the split path
    # (partials, logits and keep lists all live in the scratch)
    w = synth.workload("llama3_8b_h2o_b64", batch=8)
    P = w.prompt_len
    c1 = _prefill(w, 8, P + 1, P, heavy_frac=w.heavy_frac)
    _both(w, c1, kvc.policy_h2o(64, 448), 1, [P] * 8, P + 1, True, w.heavy_frac)
    # call 2: a smaller batch on the one-workgroup kernel (random eviction,
    # several evictions per unit), over the scratch the first call left
    w2 = synth.workload("llama3_8b_h2o_b64", batch=2)
    c2 = _prefill(w2, 2, 301, 300)
    _both(w2, c2, kvc.policy_random(100, 150, 5), 2, [300] * 2, 301, False)


def test_noalloc_step_continues_a_run():
    # the same cache stepped by both entry points alternately stays identical
    w = synth.workload("heavy_load_b512_l2048", batch=16)
    P = 600
    c = _prefill(w, 16, P + 1, P)
    twin = _clone(c)
    pol = kvc.policy_streaming(64, 448)
    B, Hq, Hkv, D = c.batch, c.q_heads, c.kv_heads, c.head_dim
    seen = torch.full((B,), P, dtype=torch.int32, device="cuda")
    out_a = torch.empty((B, Hq, D), device="cuda")
    out_b = torch.empty_like(out_a)
    ws = c.workspace(P + 1)
    for t in range(1, 5):
        q = synth.device_normal((B, Hq, D), w.seed, w.wid, synth.T_Q, t)
        kn = synth.device_normal((B, Hkv, D), w.seed, w.wid, synth.T_KNEW, t)
        vn = synth.device_normal((B, Hkv, D), w.seed, w.wid, synth.T_VNEW, t)
        kvc.decode_step(c, pol, t, seen, q, kn, vn, out_a, max_len_hint=P + 1, workspace=ws)
        kvc.decode_step_noalloc(twin, pol, t, seen, q, kn, vn, out_b, max_len_hint=P + 1)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"step {t}"
        _assert_live_equal(c, twin)
        seen += 1
