"""GPU parity of the KIVI-style quantized cache (kvc_kivi_prefill,
kvc_kivi_decode) against the oracle's Kivi model.

Quantized state is compared bit for bit after the prefill and after every
decode step: counts, every group's 4-bit codes (unpacked from the layout
kvc.h states) and its binary32 scale / lo, and the residual rows.  Outputs
must lie within 2e-3 of the oracle's float64 attention over the dequantized
tokens, the residual and the new token.  Cases: ragged prompts around the
residual size, several group sizes, conversions during the steps, shares
longer than one LDS piece (online rescaling), a full quantized store, and the
LLaMA-3-8B and heavy-load shapes.
"""
import math

import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle
import synth
from kvc_harness import OUT_ATOL, dev, host

pytestmark = pytest.mark.gpu

D = 128


def _nibble_index():
    """(byte, shift) of each dim's code in a 64-byte K row; for V, of each
    (token, dim) of a 32-token group in its two 1,024-byte tiles (kvc.h)."""
    def place(word, elem):
        slot = elem // 2 if elem % 2 == 0 else 4 + elem // 2
        return 4 * word + slot // 2, 4 * (slot % 2)
    kb, ks = [], []
    for d in range(D):
        b, s = place(4 * ((d % 32) // 8) + d // 32, d % 8)
        kb.append(b)
        ks.append(s)
    vb = np.zeros((32, D), np.int64)
    vs = np.zeros((32, D), np.uint8)
    for i in range(32):
        t, q = divmod(i, 16)
        r, e = q % 4, q // 4          # token 4e + r of its tile
        for d in range(D):
            c, m = d % 16, d // 16
            w = 2 * (e // 2) + m % 2   # words 0/1: tokens r, r+4; 2/3: r+8, r+12
            bit = 16 * (e % 2) + 4 * (m // 2)
            vb[i, d] = 1024 * t + 16 * (16 * r + c) + 4 * w + bit // 8
            vs[i, d] = bit % 8
    return (np.array(kb), np.array(ks, np.uint8)), (vb, vs)


K_IDX, V_IDX = _nibble_index()
# residual V rows keep dim d at element 8 (d % 16) + d // 16 (kvc.h)
V_RES_ELEM = np.array([8 * (d % 16) + d // 16 for d in range(D)])


def _unpack(rows: np.ndarray, idx) -> np.ndarray:
    b, s = idx
    return (rows[..., b] >> s) & 0xF


def _prompts(w, lengths):
    L = max(max(lengths), 1)
    k = np.zeros((len(lengths), w.kv_heads, L, D), np.uint16)
    v = np.zeros_like(k)
    parts = []
    for b, n in enumerate(lengths):
        kb, vb = synth.prefill_kv(w, b, n)
        k[b, :, :n], v[b, :, :n] = kb, vb
        parts.append((kb, vb))
    return k, v, parts


def _check_state(cache, orc, B, Hkv):
    torch.cuda.synchronize()
    nq = cache.n_quant.cpu().numpy()
    nr = cache.n_res.cpu().numpy()
    kc = cache.k_codes.cpu().numpy()
    vc = cache.v_codes.cpu().numpy()
    ks, kl = cache.k_scale.cpu().numpy(), cache.k_lo.cpu().numpy()
    vs, vl = cache.v_scale.cpu().numpy(), cache.v_lo.cpu().numpy()
    kr = host(cache.k_res, "bf16")
    vr = host(cache.v_res, "bf16")[..., V_RES_ELEM]
    for b in range(B):
        for h in range(Hkv):
            u, ou = b * Hkv + h, orc.units[b][h]
            assert (nq[b, h], nr[b, h]) == (ou.n_quant, ou.n_res), (b, h)
            for g, grp in enumerate(ou.groups):
                t = slice(32 * g, 32 * g + 32)
                np.testing.assert_array_equal(_unpack(kc[u, t], K_IDX), grp.k_codes)
                vgrp = vc[u].reshape(-1)[2048 * g:2048 * (g + 1)]
                np.testing.assert_array_equal((vgrp[V_IDX[0]] >> V_IDX[1]) & 0xF, grp.v_codes)
                np.testing.assert_array_equal(ks[u, g], grp.k_scale)
                np.testing.assert_array_equal(kl[u, g], grp.k_lo)
                np.testing.assert_array_equal(vs[u, t], grp.v_scale)
                np.testing.assert_array_equal(vl[u, t], grp.v_lo)
            n = ou.n_res
            np.testing.assert_array_equal(oracle.decode(kr[u, :n], "bf16"), ou.res_k)
            np.testing.assert_array_equal(oracle.decode(vr[u, :n], "bf16"), ou.res_v)


def _run(w, lengths, steps, max_quant=None, hint=0, check_every=1, scale=None):
    B, Hq, Hkv = len(lengths), w.q_heads, w.kv_heads
    k, v, parts = _prompts(w, lengths)
    longest = max(lengths) + steps
    mq = max_quant if max_quant is not None else oracle.kivi_split(longest)[0]
    cache = kvc.KiviCache(B, Hq, Hkv, D, mq)
    kvc.kivi_prefill(cache, dev(k, "bf16"), dev(v, "bf16"),
                     torch.tensor(lengths, dtype=torch.int32, device="cuda"))
    orc = oracle.Kivi(Hq, Hkv, D, scale=scale)
    for b in range(B):
        orc.load(b, *parts[b])
    _check_state(cache, orc, B, Hkv)
    ws = cache.workspace(hint)
    out = torch.empty((B, Hq, D), device="cuda")
    worst = 0.0
    for t in range(1, steps + 1):
        q, kn, vn = synth.batch_step_inputs(w, t, B)
        kvc.kivi_decode(cache, dev(q, "bf16"), dev(kn, "bf16"), dev(vn, "bf16"), out,
                        scale=scale, max_quant_hint=hint, workspace=ws)
        o = out.cpu().numpy()
        for b in range(B):
            ref = orc.step(b, q[b], kn[b], vn[b])
            err = float(np.abs(o[b] - ref).max())
            worst = max(worst, err)
            assert err <= OUT_ATOL, (t, b, err)
        if t % check_every == 0 or t == steps:
            _check_state(cache, orc, B, Hkv)
    assert int(cache.flags.item()) == 0
    return worst


W4 = synth.workload("llama3_8b_h2o_b64", heavy_frac=0.0)       # G = 4
W5 = synth.workload("reasoning_random_b32")                     # G = 5
W8 = synth.workload("heavy_load_b512_l2048")                    # G = 8


def test_prefill_ragged_lengths_around_the_residual():
    # nothing quantized (0, 20, 128), one group (129, 160), several (200, 700)
    _run(W4, [0, 20, 128, 129, 160, 200, 700], steps=0)


def test_short_prompts_decode_from_the_residual_alone():
    # units with no quantized group (an empty one included) attend the residual
    # and the new token only; the 128-token unit converts its first group at
    # the first step
    _run(W4, [0, 1, 20, 127, 128], steps=3)


@pytest.mark.parametrize("w", [W4, W5, W8], ids=lambda w: w.name)
def test_decode_steps_with_conversions(w):
    # units at 128 convert on step 1, at 127 on step 2; 40 steps cross a
    # conversion in every unit
    _run(w, [127, 128, 300, 45], steps=40, check_every=5)


def test_single_query_head_group():
    w = synth.workload("heavy_load_b512_l2048", q_heads=8)     # G = 1
    _run(w, [129, 600], steps=6)


def test_long_share_runs_in_pieces():
    # a length bound of one group gives one share per unit, so a unit of
    # 2,100 tokens (61 groups) runs in one workgroup whose waves each walk
    # about 15 groups on their own running softmax
    _run(W8, [2100, 700, 129], steps=3, hint=32)


@pytest.mark.parametrize("scale", [-0.07, 0.0])
@pytest.mark.parametrize("hint", [0, 32])
def test_negative_and_zero_scale(scale, hint):
    # any finite scale: the heads past G and the keys past the residual must
    # still weigh nothing when the logits flip sign or vanish, with one share
    # per unit (the output written by the attention) and with several
    _run(W5, [150, 400, 620], steps=3, hint=hint, scale=scale)


def test_many_splits_and_empty_splits():
    # a small batch spreads the groups over many workgroups; short units leave
    # most of their splits empty
    _run(W4, [1500, 140, 3], steps=4)


def test_full_quantized_store_sets_flag_and_keeps_state():
    w = W4
    lengths = [256, 100]                     # unit 0: 128 quantized + 128 residual
    B, Hq, Hkv = len(lengths), w.q_heads, w.kv_heads
    k, v, parts = _prompts(w, lengths)
    cache = kvc.KiviCache(B, Hq, Hkv, D, 128)
    kvc.kivi_prefill(cache, dev(k, "bf16"), dev(v, "bf16"),
                     torch.tensor(lengths, dtype=torch.int32, device="cuda"))
    before = (cache.n_quant.clone(), cache.n_res.clone(), cache.k_res.clone())
    q, kn, vn = synth.batch_step_inputs(w, 1, B)
    out = torch.empty((B, Hq, D), device="cuda")
    kvc.kivi_decode(cache, dev(q, "bf16"), dev(kn, "bf16"), dev(vn, "bf16"), out)
    torch.cuda.synchronize()
    assert int(cache.flags.item()) & kvc.FLAG_FULL
    assert torch.equal(cache.n_quant[0], before[0][0]) and torch.equal(cache.n_res[0], before[1][0])
    assert torch.equal(cache.k_res[:Hkv], before[2][:Hkv])
    # the attention of the step is still exact, and unit 1 went on normally
    orc = oracle.Kivi(Hq, Hkv, D)
    for b in range(B):
        orc.load(b, *parts[b])
    o = out.cpu().numpy()
    for b in range(B):
        assert np.abs(o[b] - orc.step(b, q[b], kn[b], vn[b])).max() <= OUT_ATOL
    assert cache.n_res[1].tolist() == [101] * Hkv


@pytest.mark.parametrize("w,B,hinted", [(W4, 64, False), (W8, 512, True)],
                         ids=["llama3_8b_b64", "heavy_load_b512"])
def test_full_batch_sampled(w, B, hinted):
    # every sequence x 2,048-token prompts at the workload's heads: a sample of
    # units' outputs against the oracle for two steps (the first converts a
    # full residual) and every unit's counts.  Batch 64 (32 q / 8 kv heads)
    # runs several shares per unit and the combine; the heavy-load layer
    # (batch 512, 64 q / 8 kv heads) with the length bound the benchmark
    # passes runs one share per unit, the single-launch step.
    P = 2048
    lengths = [P] * B
    k = synth.device_normal((B, w.kv_heads, P, D), 0, 977, 1)
    v = synth.device_normal((B, w.kv_heads, P, D), 0, 977, 2)
    mq = oracle.kivi_split(P + 211)[0] if hinted else oracle.kivi_split(P + 8)[0]
    hint = mq if hinted else 0
    cache = kvc.KiviCache(B, w.q_heads, w.kv_heads, D, mq)
    kvc.kivi_prefill(cache, k, v, torch.tensor(lengths, dtype=torch.int32, device="cuda"))
    sample = [0, 17, B - 1]
    orc = oracle.Kivi(w.q_heads, w.kv_heads, D)
    kh, vh = host(k, "bf16"), host(v, "bf16")
    del k, v
    for b in sample:
        orc.load(b, kh[b], vh[b])
    ws = cache.workspace(hint)
    out = torch.empty((B, w.q_heads, D), device="cuda")
    for t in range(1, 3):
        q = synth.device_normal((B, w.q_heads, D), 0, 978, t)
        kn = synth.device_normal((B, w.kv_heads, D), 0, 979, t)
        vn = synth.device_normal((B, w.kv_heads, D), 0, 980, t)
        kvc.kivi_decode(cache, q, kn, vn, out, max_quant_hint=hint, workspace=ws)
        o = out.cpu().numpy()
        qh, knh, vnh = host(q, "bf16"), host(kn, "bf16"), host(vn, "bf16")
        for b in sample:
            assert np.abs(o[b] - orc.step(b, qh[b], knh[b], vnh[b])).max() <= OUT_ATOL, (t, b)
    assert int(cache.flags.item()) == 0
    nq = cache.n_quant.cpu().numpy()
    assert (nq == 1952).all() and (cache.n_res.cpu().numpy() == 98).all()
