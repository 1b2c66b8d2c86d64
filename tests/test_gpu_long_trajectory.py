"""Parity over the workloads' whole decode runs at their real shapes.

* H2O (the heavy-load layer: batch 512, 128 steps; the LLaMA-3-8B-shaped
  layer with heavy-hitter keys: batch 64, 256 steps; the mixed-length paged
  batch: 128 sequences, 64 steps): every step runs the one-launch
  kvc_decode_step that the benchmark times and, on a twin cache, the
  three-call sequence decode_attn -> evict_h2o -> compact; the two must agree
  bit for bit over the whole live state.  A stratified subset of sequences
  (every kv head) is checked against the oracle at every step -- outputs
  within 2e-3, scores within 1e-5 relative, kept sets exactly on the GPU's own
  post-attention scores (state-synchronised H2O parity) -- and every sequence
  at the first two and the last step.
* Random eviction over the reasoning-trace schedule (batch 32, 40 q / 8 kv
  heads, 1,024 pinned prompt tokens, n_keep 4,096, 16,384 decode steps: the
  cache grows from 1,024 to 5,120 entries, then loses one generated token per
  head per step): the kept position set of eight units is compared with the
  oracle's positions-only replay after every step, and their outputs with
  oracle attention over the oracle's own kept entries at sampled steps."""
import concurrent.futures as cf
import math

import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle
import synth
from kvc_harness import OUT_ATOL, assert_scores_close
from test_gpu_fullsize import _assert_live_equal, _clone, _prefill

pytestmark = pytest.mark.gpu

_POOL = cf.ThreadPoolExecutor(max_workers=8)


def _bf16_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class _Bulk:
    """Host copy of the live state of whole sequences: pos, n, scores and
    (optionally) K / V rows, transferred in one piece per tensor."""

    def __init__(self, cache, seqs, scores=None, rows=True):
        torch.cuda.synchronize()
        self.seqs = list(seqs)
        idx = torch.tensor(self.seqs, device="cuda")
        n = cache.n_slots[idx]
        nmax = int(n.max().item())
        self.n = n.cpu().numpy()
        self.pos = cache.pos[idx, :, :nmax].cpu().numpy()
        self.s = scores[idx, :, :nmax].cpu().numpy() if scores is not None else None
        self.k = self.v = None
        if rows:
            if cache.block_size:
                slots = torch.arange(nmax, device="cuda")
                blk = cache.block_table[idx][:, slots // cache.block_size].long()   # [b, n]
                off = slots % cache.block_size
                k = cache.k[blk, :, off.expand_as(blk)]                              # [b, n, H, D]
                v = cache.v[blk, :, off.expand_as(blk)]
                self.k = _bf16_host(k.permute(0, 2, 1, 3))
                self.v = _bf16_host(v.permute(0, 2, 1, 3))
            else:
                self.k = _bf16_host(cache.k[idx, :, :nmax])
                self.v = _bf16_host(cache.v[idx, :, :nmax])
        self.row = {b: i for i, b in enumerate(self.seqs)}

    def unit(self, b, h):
        i = self.row[b]
        n = int(self.n[i, h])
        u = dict(n=n, pos=self.pos[i, h, :n])
        u["s"] = None if self.s is None else self.s[i, h, :n]
        if self.k is not None:
            u["k"], u["v"] = self.k[i, h, :n], self.v[i, h, :n]
        return u


def _check_unit(args):
    """Oracle check of one unit at one step (runs in a worker thread)."""
    (t, b, h, G, scale, qg, knh, vnh, o, u0, u1, keep, L, pol) = args
    kn, vn = oracle.decode(knh, "bf16"), oracle.decode(vnh, "bf16")
    K = np.vstack([oracle.decode(u0["k"], "bf16"), kn[None]])
    V = np.vstack([oracle.decode(u0["v"], "bf16"), vn[None]])
    ref, p = oracle.attend(oracle.decode(qg, "bf16"), K, V, scale, want_p=True)
    err = float(np.abs(o - ref).max())
    assert err <= OUT_ATOL, f"step {t} unit {(b, h)}: output error {err}"
    psum = p.sum(axis=0)
    n = u0["n"]
    assert_scores_close(u1["s"][:n], u0["s"] + psum[:n])
    assert_scores_close(u1["s"][n:n + 1], psum[n:])
    want = oracle.select_h2o(u1["pos"], u1["s"].astype(np.float64), L, pol.n_heavy, pol.n_recent)
    np.testing.assert_array_equal(keep, np.flatnonzero(want),
                                  err_msg=f"step {t} unit {(b, h)}: kept set")
    return err


def _run_h2o(w, cache, lengths, steps, hints, seqs, full_steps, heavy_frac=0.0):
    pol = kvc.policy_h2o(64, 448)
    B, G, D, H = cache.batch, cache.group, cache.head_dim, cache.kv_heads
    twin = _clone(cache)
    sc_f = torch.zeros((B, H, cache.capacity), device="cuda")
    sc_t = torch.zeros_like(sc_f)
    out_f = torch.empty((B, cache.q_heads, D), device="cuda")
    out_t = torch.empty_like(out_f)
    keep = torch.empty((B, H, cache.capacity), dtype=torch.int32, device="cuda")
    nout = torch.empty((B, H), dtype=torch.int32, device="cuda")
    ws, ws2 = cache.workspace(max(hints)), cache.workspace(max(hints))
    seen = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    worst, checked = 0.0, 0
    for t in range(1, steps + 1):
        hint = hints[min(t - 1, len(hints) - 1)]
        q = synth.device_normal((B, cache.q_heads, D), w.seed, w.wid, synth.T_Q, t)
        kn = synth.device_normal((B, H, D), w.seed, w.wid, synth.T_KNEW, t,
                                 scale_rows_frac=heavy_frac)
        vn = synth.device_normal((B, H, D), w.seed, w.wid, synth.T_VNEW, t)
        chk = list(range(B)) if t in full_steps else seqs
        pre = _Bulk(twin, chk, sc_t)
        kvc.decode_step(cache, pol, t, seen, q, kn, vn, out_f, sc_f, max_len_hint=hint,
                        workspace=ws)
        kvc.decode_attn(twin, seen, q, kn, vn, out_t, sc_t, max_len_hint=hint, workspace=ws2)
        mid = _Bulk(twin, chk, sc_t, rows=False)
        kvc.evict_h2o(twin, sc_t, pol.n_heavy, pol.n_recent, keep, nout)
        idx = torch.tensor(chk, device="cuda")
        kk, mm = keep[idx].cpu().numpy(), nout[idx].cpu().numpy()
        kvc.compact(twin, keep, nout, sc_t)
        torch.cuda.synchronize()
        assert int(cache.flags.item()) == 0 and int(twin.flags.item()) == 0
        assert torch.equal(out_f, out_t), f"step {t}: fused and three-call outputs differ"
        _assert_live_equal(cache, twin, sc_f, sc_t)
        qh, knh, vnh = _bf16_host(q[idx]), _bf16_host(kn[idx]), _bf16_host(vn[idx])
        o = out_t[idx].cpu().numpy()
        sn = seen[idx].cpu().numpy()
        jobs = []
        for i, b in enumerate(chk):
            for h in range(H):
                jobs.append((t, b, h, G, scale, qh[i, h * G:(h + 1) * G], knh[i, h], vnh[i, h],
                             o[i, h * G:(h + 1) * G], pre.unit(b, h), mid.unit(b, h),
                             kk[i, h, :mm[i, h]], int(sn[i]) + 1, pol))
        for err in _POOL.map(_check_unit, jobs):
            worst = max(worst, err)
            checked += 1
        seen += 1
        if t % 32 == 0:
            print(f"  step {t}: {checked} unit-steps checked, worst {worst:.2e}", flush=True)
    return worst, checked


def _stratified(B, k):
    return sorted({int(round(i * (B - 1) / (k - 1))) for i in range(k)})


@pytest.mark.timeout(1200)
def test_heavy_load_b512_l2048_h2o_all_128_steps():
    # step 1 trims 2,049 -> 512 on the split path, steps 2..128 run the fused
    # kernel at the benchmark's launch configuration (hint 513)
    w = synth.workload("heavy_load_b512_l2048")
    P = w.prompt_len
    cache = _prefill(w, w.batch, P + 1, P)
    worst, checked = _run_h2o(w, cache, [P] * w.batch, w.steps, [P + 1, 513],
                              _stratified(w.batch, 16), {1, 2, w.steps})
    assert checked == (16 * (w.steps - 3) + 3 * w.batch) * w.kv_heads
    print(f"heavy-load H2O, {w.steps} steps: {checked} unit-steps checked, worst |out - oracle| {worst:.2e}")


@pytest.mark.timeout(1200)
def test_llama3_8b_h2o_b64_heavy_hitters_all_256_steps():
    w = synth.workload("llama3_8b_h2o_b64")
    P = w.prompt_len
    cache = _prefill(w, w.batch, P + 1, P, heavy_frac=w.heavy_frac)
    worst, checked = _run_h2o(w, cache, [P] * w.batch, w.steps, [P + 1, 513],
                              _stratified(w.batch, 16), {1, 2, w.steps}, heavy_frac=w.heavy_frac)
    print(f"LLaMA-3-8B-shaped H2O, {w.steps} steps: {checked} unit-steps checked, worst {worst:.2e}")


@pytest.mark.timeout(1200)
def test_mixed_paged_h2o_b128_all_64_steps():
    w = synth.workload("mixed_paged_h2o_b128")
    lengths = [int(x) for x in synth.mixed_lengths(w)]
    Lmax = max(lengths)
    cap = (Lmax + 1 + 15) // 16 * 16
    cache = _prefill(w, w.batch, cap, None, paged=16, lengths=lengths)
    order = np.argsort(lengths)
    seqs = sorted({int(order[i]) for i in _stratified(w.batch, 16)})
    worst, checked = _run_h2o(w, cache, lengths, w.steps, [Lmax + 1, 513], seqs,
                              {1, 2, w.steps})
    print(f"mixed paged H2O, {w.steps} steps: {checked} unit-steps checked, worst {worst:.2e}")


# ---------------------------------------------------------------------------
# random eviction over the whole reasoning-trace schedule
# ---------------------------------------------------------------------------

def _gpu_evictions(hist, nhist, n0, new_pos):
    """Per step, the position a unit lost, from its slot-ordered positions
    after every step (hist [steps, cap], counts nhist [steps]): growth steps
    append the new token at slot n and change nothing else (-1: nothing
    evicted); steady steps either change exactly one slot, which then holds
    the new token (the old position there was evicted), or change none (the
    new token itself was evicted)."""
    steps = hist.shape[0]
    ev = np.full(steps, -1, np.int64)
    prev = None
    n_prev = n0[0]
    prev = n0[1]
    for t in range(steps):
        cur, n_cur = hist[t], int(nhist[t])
        same = cur[:n_prev] == prev[:n_prev]
        changed = np.flatnonzero(~same)
        if n_cur == n_prev + 1:
            assert changed.size == 0 and cur[n_prev] == new_pos[t], f"growth step {t + 1}"
        elif n_cur == n_prev:
            assert changed.size <= 1, f"step {t + 1}: {changed.size} slots changed"
            if changed.size == 1:
                s = int(changed[0])
                assert cur[s] == new_pos[t], f"step {t + 1}: slot {s} holds {cur[s]}"
                ev[t] = prev[s]
            else:
                ev[t] = new_pos[t]
        else:
            raise AssertionError(f"step {t + 1}: count {n_prev} -> {n_cur}")
        prev, n_prev = cur, n_cur
    return ev


@pytest.mark.timeout(1200)
def test_reasoning_random_b32_whole_trace_schedule():
    w = synth.workload("reasoning_random_b32")
    P, NK, steps = w.pinned, w.n_keep, w.steps
    B, H, G, D = w.batch, w.kv_heads, w.group, w.head_dim
    cap = P + NK + 1
    cache = _prefill(w, B, cap, P)
    pol = kvc.policy_random(P, NK, w.seed)
    units = [(0, 0), (4, 1), (9, 2), (13, 3), (18, 4), (22, 5), (27, 6), (31, 7)]
    ub = torch.tensor([b for b, _ in units], device="cuda")
    uh = torch.tensor([h for _, h in units], device="cuda")
    U = len(units)
    sample = sorted({1, 2, 3, 1000, NK - 1, NK, NK + 1, NK + 2, 8192, 12000, steps - 1, steps})
    # prompt rows of the checked units (the prefill's draws, as cached)
    k0, v0 = _bf16_host(cache.k[ub, uh, :P]), _bf16_host(cache.v[ub, uh, :P])
    hist = torch.empty((steps, U, cap), dtype=torch.int32, device="cuda")
    nhist = torch.empty((steps, U), dtype=torch.int32, device="cuda")
    knh = torch.empty((steps, U, D), dtype=torch.bfloat16, device="cuda")
    vnh = torch.empty_like(knh)
    qs, outs = {}, {}
    out = torch.empty((B, w.q_heads, D), device="cuda")
    ws = cache.workspace(cap)
    seen = torch.full((B,), P, dtype=torch.int32, device="cuda")
    gidx = (uh.view(-1, 1) * G + torch.arange(G, device="cuda").view(1, -1))   # [U, G]
    for t in range(1, steps + 1):
        q = synth.device_normal((B, w.q_heads, D), w.seed, w.wid, synth.T_Q, t)
        kn = synth.device_normal((B, H, D), w.seed, w.wid, synth.T_KNEW, t)
        vn = synth.device_normal((B, H, D), w.seed, w.wid, synth.T_VNEW, t)
        # the split path from the first step on (every unit above 1,024 entries)
        kvc.decode_step(cache, pol, t, seen, q, kn, vn, out, max_len_hint=cap, workspace=ws)
        hist[t - 1] = cache.pos[ub, uh]
        nhist[t - 1] = cache.n_slots[ub, uh]
        knh[t - 1] = kn[ub, uh]
        vnh[t - 1] = vn[ub, uh]
        if t in sample:
            qs[t] = _bf16_host(q[ub.view(-1, 1), gidx])
            outs[t] = out[ub.view(-1, 1), gidx].cpu().numpy()
        seen += 1
        if t % 2048 == 0:
            torch.cuda.synchronize()
            assert int(cache.flags.item()) == 0
            print(f"  step {t}", flush=True)
    torch.cuda.synchronize()
    assert int(cache.flags.item()) == 0
    new_pos = np.arange(P, P + steps, dtype=np.int64)
    # the oracle's replays, one thread per unit (positions and keys only)
    replays = list(_POOL.map(
        lambda bh: oracle.random_replay(np.arange(P), cap, steps, P, 1, P, NK, w.seed, bh[0],
                                        bh[1]), units))
    knh_h, vnh_h = _bf16_host(knh), _bf16_host(vnh)
    for i, (b, h) in enumerate(units):
        nev, ev_want, fin = replays[i]
        hu = hist[:, i].cpu().numpy()
        nu = nhist[:, i].cpu().numpy()
        ev_gpu = _gpu_evictions(hu, nu, (P, np.arange(P, dtype=np.int32)), new_pos)
        # growth then one eviction per step, as the schedule says
        assert np.all(nev[:NK] == 0) and np.all(nev[NK:] == 1)
        np.testing.assert_array_equal(ev_gpu[:NK], -1)
        np.testing.assert_array_equal(ev_gpu[NK:], ev_want, err_msg=f"unit {(b, h)}: evictions")
        np.testing.assert_array_equal(np.sort(hu[-1, :nu[-1]]), fin)
        # outputs at sampled steps: oracle attention over the oracle's kept
        # entries (the set before step t plus the new token), rows by position
        kept = set(range(P))
        evs = iter(ev_want)
        rows_k = lambda p: k0[i, p] if p < P else knh_h[p - P, i]
        rows_v = lambda p: v0[i, p] if p < P else vnh_h[p - P, i]
        for t in range(1, steps + 1):
            kept.add(P + t - 1)
            if t in sample:
                ps = sorted(kept)
                K = oracle.decode(np.stack([rows_k(p) for p in ps]), "bf16")
                V = oracle.decode(np.stack([rows_v(p) for p in ps]), "bf16")
                ref = oracle.attend(oracle.decode(qs[t][i], "bf16"), K, V, 1.0 / math.sqrt(D))
                err = float(np.abs(outs[t][i] - ref).max())
                assert err <= OUT_ATOL, f"step {t} unit {(b, h)}: output error {err}"
            if nev[t - 1]:
                kept.discard(int(next(evs)))
    print(f"reasoning trace: {U} units x {steps} steps of kept sets, outputs at {len(sample)} steps")
