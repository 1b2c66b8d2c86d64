"""GPU parity of the eviction choice (kvc_evict_*) and of the compaction.

Kept sets must equal the oracle's bit-exactly (slot indices), for random slot
orders, ties, every policy, units with fewer candidates than the budget, and
units large enough to leave the LDS path.  H2O runs on the same fp32 score
vector on both sides."""
import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle
from kvc_harness import Snapshot, host, rows_by_pos

pytestmark = pytest.mark.gpu


def _pos_cache(units_pos, cap, Hkv, D=64, dtype=kvc.BF16, fill_kv=False, seed=0):
    """Cache whose unit (b, h) holds the given positions in its slots."""
    B = len(units_pos) // Hkv
    cache = kvc.KvCache(B, Hkv, Hkv, D, cap, dtype)
    pos = np.zeros((B, Hkv, cap), np.int32)
    n = np.zeros((B, Hkv), np.int32)
    for i, p in enumerate(units_pos):
        b, h = divmod(i, Hkv)
        pos[b, h, :len(p)] = p
        n[b, h] = len(p)
    cache.pos.copy_(torch.from_numpy(pos))
    cache.n_slots.copy_(torch.from_numpy(n))
    if fill_kv:
        g = torch.Generator(device="cuda").manual_seed(seed)
        cache.k.copy_(torch.randn(cache.k.shape, generator=g, device="cuda").to(cache.k.dtype))
        cache.v.copy_(torch.randn(cache.v.shape, generator=g, device="cuda").to(cache.v.dtype))
    torch.cuda.synchronize()
    return cache


def _units(rng, count, max_n, span, recent_full=0):
    out = []
    for _ in range(count):
        n = int(rng.integers(0, max_n + 1))
        L = int(rng.integers(max(n, 1), span + 1))
        if recent_full and n >= recent_full:
            # keep the recent window complete, the rest a random subset
            rest = rng.permutation(max(L - recent_full, 0))[:n - recent_full]
            p = np.concatenate([np.arange(L - recent_full, L), rest])
        else:
            p = rng.permutation(L)[:n]
        out.append(rng.permutation(p).astype(np.int32))
    return out


def _gpu_keep(cache, call):
    units = cache.batch * cache.kv_heads
    keep = torch.full((cache.batch, cache.kv_heads, cache.capacity), -7, dtype=torch.int32,
                      device="cuda")
    nout = torch.full((cache.batch, cache.kv_heads), -7, dtype=torch.int32, device="cuda")
    call(keep, nout)
    torch.cuda.synchronize()
    k = keep.cpu().numpy().reshape(units, -1)
    m = nout.cpu().numpy().reshape(units)
    res = []
    for u in range(units):
        sl = k[u, :m[u]]
        assert np.all(np.diff(sl) > 0), "keep_slots must be ascending"
        res.append(sl)
    return res


def _flags_to_slots(flags):
    return np.flatnonzero(flags)


@pytest.mark.parametrize("trial", range(4))
def test_h2o_select_matches_oracle(trial):
    rng = np.random.default_rng(trial)
    Hkv, cap = 4, 700
    units_pos = _units(rng, 8 * Hkv, 690, 3000, recent_full=60 if trial % 2 else 0)
    cache = _pos_cache(units_pos, cap, Hkv)
    # coarse fp32 scores so that many ties occur
    sc = (rng.integers(0, 16, (8, Hkv, cap)) / 8.0).astype(np.float32)
    scores = torch.from_numpy(sc).cuda()
    n_heavy, n_recent = [(5, 60), (64, 448), (0, 30), (700, 0)][trial]
    got = _gpu_keep(cache, lambda k, m: kvc.evict_h2o(cache, scores, n_heavy, n_recent, k, m))
    for u, p in enumerate(units_pos):
        b, h = divmod(u, Hkv)
        L = int(p.max()) + 1 if len(p) else 0
        want = _flags_to_slots(oracle.select_h2o(p, sc[b, h, :len(p)].astype(np.float64), L,
                                                 n_heavy, n_recent))
        np.testing.assert_array_equal(got[u], want)


@pytest.mark.parametrize("trial", range(4))
def test_random_select_matches_oracle(trial):
    rng = np.random.default_rng(100 + trial)
    Hkv, cap = 4, 900
    units_pos = _units(rng, 6 * Hkv, 880, 2000)
    cache = _pos_cache(units_pos, cap, Hkv)
    prompt_len, n_keep = [(100, 50), (0, 1), (300, 0), (50, 2000)][trial]
    seed, step = 0x1234_5678_9ABC_DEF0 + trial, 17 + trial
    got = _gpu_keep(cache, lambda k, m: kvc.evict_random(cache, prompt_len, n_keep, seed, step,
                                                          k, m))
    for u, p in enumerate(units_pos):
        b, h = divmod(u, Hkv)
        want = _flags_to_slots(oracle.select_random(p, prompt_len, n_keep, seed, b, h, step))
        np.testing.assert_array_equal(got[u], want)


@pytest.mark.parametrize("trial", range(3))
def test_streaming_select_matches_oracle(trial):
    rng = np.random.default_rng(200 + trial)
    Hkv, cap = 2, 1100
    units_pos = _units(rng, 10 * Hkv, 1090, 1500)
    cache = _pos_cache(units_pos, cap, Hkv)
    n_sink, n_recent = [(64, 448), (0, 100), (4, 0)][trial]
    got = _gpu_keep(cache, lambda k, m: kvc.evict_streaming(cache, n_sink, n_recent, k, m))
    for u, p in enumerate(units_pos):
        L = int(p.max()) + 1 if len(p) else 0
        want = _flags_to_slots(oracle.select_streaming(p, L, n_sink, n_recent))
        np.testing.assert_array_equal(got[u], want)


def test_large_units_leave_the_lds_path():
    rng = np.random.default_rng(300)
    Hkv, cap = 2, 12000
    units_pos = [rng.permutation(20000)[:n].astype(np.int32) for n in (12000, 9000, 8193, 100)]
    cache = _pos_cache(units_pos, cap, Hkv)
    sc = rng.random((2, Hkv, cap)).astype(np.float32)
    sc[0, 0, :500] = 0.5   # ties
    scores = torch.from_numpy(sc).cuda()
    got = _gpu_keep(cache, lambda k, m: kvc.evict_h2o(cache, scores, 300, 2000, k, m))
    for u, p in enumerate(units_pos):
        b, h = divmod(u, Hkv)
        want = _flags_to_slots(oracle.select_h2o(p, sc[b, h, :len(p)].astype(np.float64),
                                                 int(p.max()) + 1, 300, 2000))
        np.testing.assert_array_equal(got[u], want)
    got = _gpu_keep(cache, lambda k, m: kvc.evict_random(cache, 1000, 2500, 5, 9, k, m))
    for u, p in enumerate(units_pos):
        b, h = divmod(u, Hkv)
        want = _flags_to_slots(oracle.select_random(p, 1000, 2500, 5, b, h, 9))
        np.testing.assert_array_equal(got[u], want)
    # dropped slots (no ranking) on the same path
    got = _gpu_keep(cache, lambda k, m: kvc.evict_streaming(cache, 64, 3000, k, m))
    for u, p in enumerate(units_pos):
        want = _flags_to_slots(oracle.select_streaming(p, int(p.max()) + 1, 64, 3000))
        np.testing.assert_array_equal(got[u], want)


# every row size of the copy (64 to 512 bytes: 4 to 32 parts of 16 bytes, so
# 16 to 2 moves per wave step)
@pytest.mark.parametrize("dtype,D", [(kvc.BF16, 128), (kvc.F32, 128), (kvc.BF16, 64), (kvc.F32, 64),
                                     (kvc.FP8_E5M2, 128), (kvc.FP8_E5M2, 64)])
def test_compaction_moves_survivors_bit_exactly(dtype, D):
    rng = np.random.default_rng(400)
    Hkv, cap = 2, 600
    units_pos = _units(rng, 4 * Hkv, 590, 1500)
    cache = _pos_cache(units_pos, cap, Hkv, D=D, dtype=dtype, fill_kv=True)
    sc = rng.random((4, Hkv, cap)).astype(np.float32)
    scores = torch.from_numpy(sc).cuda()
    dn = {kvc.BF16: "bf16", kvc.F32: "f32", kvc.FP8_E5M2: "e5m2"}[dtype]
    pre = Snapshot(cache, dn, scores)
    keep = torch.empty((4, Hkv, cap), dtype=torch.int32, device="cuda")
    nout = torch.empty((4, Hkv), dtype=torch.int32, device="cuda")
    kvc.evict_h2o(cache, scores, 40, 100, keep, nout)
    kk = keep.cpu().numpy()
    mm = nout.cpu().numpy()
    kvc.compact(cache, keep, nout, scores)
    post = Snapshot(cache, dn, scores)
    for b in range(4):
        for h in range(Hkv):
            u0, u1 = pre.unit(b, h), post.unit(b, h)
            m = int(mm[b, h])
            assert u1["n"] == m
            kept = set(u0["pos"][kk[b, h, :m]].tolist())
            assert set(u1["pos"].tolist()) == kept
            r0, r1 = rows_by_pos(u0), rows_by_pos(u1)
            for p in kept:
                assert r0[p] == r1[p]
            # slots below n_out that were kept did not move
            for s in kk[b, h, :m]:
                if s < m:
                    assert u1["pos"][s] == u0["pos"][s]


def test_ordered_gather_is_the_hook_layout():
    rng = np.random.default_rng(500)
    Hkv, cap, prompt = 4, 400, 100
    units_pos = [rng.permutation(np.arange(350)).astype(np.int32) for _ in range(2 * Hkv)]
    cache = _pos_cache(units_pos, cap, Hkv, fill_kv=True)
    n_keep = kvc.n_keep(250, 0.5)
    keep = torch.empty((2, Hkv, cap), dtype=torch.int32, device="cuda")
    nout = torch.empty((2, Hkv), dtype=torch.int32, device="cuda")
    kvc.evict_random(cache, prompt, n_keep, 3, 1, keep, nout)
    dst = kvc.KvCache(2, Hkv, Hkv, 64, prompt + n_keep, kvc.BF16)
    pre = Snapshot(cache, "bf16")
    kvc.compact(cache, keep, nout, None, ordered_dst=dst)
    out = Snapshot(dst, "bf16")
    for b in range(2):
        for h in range(Hkv):
            u = out.unit(b, h)
            p = units_pos[b * Hkv + h]
            want = np.sort(p[oracle.select_random(p, prompt, n_keep, 3, b, h, 1)])
            np.testing.assert_array_equal(u["pos"], want)
            assert u["pos"][:prompt].tolist() == list(range(prompt))
            r0 = rows_by_pos(pre.unit(b, h))
            for i, pp in enumerate(u["pos"]):
                assert r0[int(pp)][0] == u["k"][i].tobytes()
                assert r0[int(pp)][1] == u["v"][i].tobytes()
    # the source cache is untouched
    assert Snapshot(cache, "bf16").n.tolist() == pre.n.tolist()
