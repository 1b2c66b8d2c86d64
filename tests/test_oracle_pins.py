"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, a published known-answer
vector, a brute-force enumeration on tiny inputs, a figure the pages print, or
a statistical law -- never against a retyped copy of its own formula.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = [t.strip() for t in line.split("=")]
                out[k] = float(v)
    return out


# ---------------------------------------------------------------------------
# Philox4x32-10: known-answer vectors of the generator's authors
# ---------------------------------------------------------------------------

def test_philox_known_answers():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(t, 16) for t in line.split()])
    assert len(rows) == 3
    for r in rows:
        got = oracle.philox4x32_10(r[0:4], r[4:6])
        assert [int(x) for x in got] == r[6:10]


def test_random_key_uses_documented_counter_layout():
    # counter = (pos, step, kv head, sequence), key = (seed low, seed high)
    seed = 0x0123456789ABCDEF
    got = oracle.random_key(pos=77, seed=seed, seq=5, head=3, step=9)
    ref = oracle.philox4x32_10([77, 9, 3, 5], [seed & 0xFFFFFFFF, seed >> 32])[0]
    assert got == int(ref)


# ---------------------------------------------------------------------------
# bytes per token: the capacity formula (guide, section 16) and its examples
# ---------------------------------------------------------------------------

def test_bytes_per_token_closed_forms():
    assert oracle.bytes_per_token(1, 8, 128, 2) == 4096
    # 80 attention layers, 8 kv heads, head_dim 128, 2-byte elements
    per_tok = oracle.bytes_per_token(80, 8, 128, 2)
    assert per_tok == 327_680
    # batch 512 x prompt 2048: the formula gives 343.6 GB (the guide's "about
    # 512 GB" does not follow from its own formula; the formula is pinned)
    assert per_tok * 2048 * 512 == 343_597_383_680
    # hybrid models: only attention layers hold KV (16 of 64 layers)
    assert oracle.bytes_per_token(16, 8, 128, 2) * 4 == oracle.bytes_per_token(64, 8, 128, 2)
    for bad in [(0, 8, 128, 2), (1, 0, 128, 2), (1, 8, -1, 2), (1, 8, 128, 0)]:
        assert oracle.bytes_per_token(*bad) == 0


# ---------------------------------------------------------------------------
# exact bf16 decoding
# ---------------------------------------------------------------------------

def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2.0 - 2.0 ** -7) * 2.0 ** 127, -0.0,
            3.140625]
    got = oracle.decode(bits, "bf16")
    assert list(got) == want


def test_bf16_rounding_of_the_input_generator_is_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    got = oracle.decode(synth.bf16_bits(x), "bf16")
    assert list(got) == [1.0, 1.0 + 2 * 2.0 ** -7, 1.0 + 2.0 ** -7]


# ---------------------------------------------------------------------------
# attention: closed forms
# ---------------------------------------------------------------------------

def test_attention_worked_example_closed_form():
    # D = 2, scale = 1/sqrt(2), q = (1, 0).  Keys chosen so that the logits
    # are (ln 2, 0, ln 3): probabilities are exactly (2, 1, 3) / 6, and with
    # V rows (6,0), (0,6), (-6,6) the output is (2 - 3, 1 + 3) = (-1, 4).
    r2 = math.sqrt(2.0)
    q = np.array([[1.0, 0.0]])
    K = np.array([[r2 * math.log(2.0), 5.0], [0.0, -7.0], [r2 * math.log(3.0), 0.25]])
    V = np.array([[6.0, 0.0], [0.0, 6.0], [-6.0, 6.0]])
    o, p = oracle.attend(q, K, V, want_p=True)
    np.testing.assert_allclose(p[0], [2 / 6, 1 / 6, 3 / 6], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0], [-1.0, 4.0], rtol=0, atol=1e-14)


def test_attention_scale_is_inverse_sqrt_head_dim():
    # D = 4 -> scale 1/2; q.k1 = 2 -> z1 = 1, z2 = 0 -> p1 = e / (1 + e)
    q = np.array([[1.0, 0, 0, 0]])
    K = np.array([[2.0, 0, 0, 0], [0, 0, 0, 0]])
    V = np.array([[1.0, 0, 0, 0], [0, 0, 0, 0]])
    _, p = oracle.attend(q, K, V, want_p=True)
    assert abs(p[0, 0] - math.e / (1 + math.e)) < 1e-15


def test_attention_single_entry_returns_its_value():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((3, 5, 16))
    o = oracle.attend(q, k[:1], v[:1])
    np.testing.assert_array_equal(o, np.repeat(v[:1], 5, axis=0))


def test_attention_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 32))
    K = np.repeat(rng.standard_normal((1, 32)), 9, axis=0)
    V = rng.standard_normal((9, 32))
    o, p = oracle.attend(q, K, V, want_p=True)
    np.testing.assert_allclose(p, 1 / 9, rtol=1e-14)
    np.testing.assert_allclose(o, np.repeat(V.mean(0, keepdims=True), 4, axis=0), atol=1e-14)


def test_attention_large_logits_stay_finite_and_one_hot():
    q = np.array([[1.0, 0.0]])
    K = np.array([[3000.0, 0.0], [1000.0, 0.0], [-5000.0, 0.0]])
    V = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    o, p = oracle.attend(q, K, V, want_p=True)
    assert np.all(np.isfinite(o))
    np.testing.assert_array_equal(p[0], [1.0, 0.0, 0.0])
    np.testing.assert_array_equal(o[0], [1.0, 2.0])


def test_attention_probabilities_sum_to_one_and_permutation_invariance():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((8, 64))
    K = rng.standard_normal((37, 64)) * 3
    V = rng.standard_normal((37, 64))
    o, p = oracle.attend(q, K, V, want_p=True)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    perm = rng.permutation(37)
    o2, p2 = oracle.attend(q, K[perm], V[perm], want_p=True)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(p2, p[:, perm], atol=1e-15)
    # linear in V
    V2 = rng.standard_normal((37, 64))
    np.testing.assert_allclose(oracle.attend(q, K, 2 * V - V2),
                               2 * o - oracle.attend(q, K, V2), atol=1e-12)


def test_gqa_head_mapping_is_contiguous_groups():
    # 2 kv heads, G = 3: q heads 0..2 read kv head 0, q heads 3..5 kv head 1
    D = 8
    orc = oracle.Oracle(q_heads=6, kv_heads=2, head_dim=D, dtype="f32")
    K = np.zeros((2, 4, D), np.float32)
    V = np.zeros((2, 4, D), np.float32)
    V[0] = 1.0
    V[1] = -2.0
    orc.load(0, K, V)
    q = np.random.default_rng(4).standard_normal((6, D)).astype(np.float32)
    out, _ = orc.step(0, q, np.zeros((2, D), np.float32),
                      np.stack([np.ones(D), -2 * np.ones(D)]).astype(np.float32),
                      oracle.Policy.full())
    np.testing.assert_allclose(out[:3], 1.0, atol=1e-15)
    np.testing.assert_allclose(out[3:], -2.0, atol=1e-15)


# ---------------------------------------------------------------------------
# H2O scores: mass conservation and the uniform case
# ---------------------------------------------------------------------------

def _small_h2o_oracle(G=4, D=16, n=20, seed=5, scale_keys=1.0):
    rng = np.random.default_rng(seed)
    orc = oracle.Oracle(q_heads=2 * G, kv_heads=2, head_dim=D, dtype="f32")
    K = (rng.standard_normal((2, n, D)) * scale_keys).astype(np.float32)
    V = rng.standard_normal((2, n, D)).astype(np.float32)
    orc.load(0, K, V)
    return orc, rng


def test_h2o_score_mass_is_group_size_per_step():
    G = 4
    orc, rng = _small_h2o_oracle(G=G)
    pol = oracle.Policy.h2o(n_heavy=100, n_recent=100)  # no eviction
    total = np.zeros(2)
    for t in range(1, 6):
        q = rng.standard_normal((2 * G, 16)).astype(np.float32)
        kn = rng.standard_normal((2, 16)).astype(np.float32)
        _, post = orc.step(0, q, kn, kn, pol, step=t)
        for h in range(2):
            total[h] = post[h][1].sum()
            assert abs(total[h] - G * t) < 1e-12 * G * t


def test_h2o_zero_query_spreads_mass_uniformly():
    G = 3
    orc, rng = _small_h2o_oracle(G=G, n=9)
    q = np.zeros((2 * G, 16), np.float32)
    kn = rng.standard_normal((2, 16)).astype(np.float32)
    _, post = orc.step(0, q, kn, kn, oracle.Policy.h2o(100, 100))
    for h in range(2):
        np.testing.assert_allclose(post[h][1], G / 10, rtol=1e-14)


@pytest.mark.parametrize("lam", [0.5, 0.9, 0.99])
def test_decayed_activity_matches_the_geometric_closed_form(lam):
    # Zero queries attend uniformly: every entry's step weight is exactly G/T_k
    # (T_k entries attended at step k).  An entry appended at step s then holds
    # A = sum_{k=s..t} (1-lam) lam^(t-k) G/T_k -- the unrolled decayed update of
    # the online compaction study (sections 3.1, 4.1) -- and the n0 prompt
    # entries, present from the start with A = 0, the same sum from k = 1.
    G, n0, steps = 3, 9, 7
    orc, rng = _small_h2o_oracle(G=G, n=n0)
    pol = oracle.Policy.h2o(n_heavy=100, n_recent=100, decay=lam)  # no eviction
    q = np.zeros((2 * G, 16), np.float32)
    for t in range(1, steps + 1):
        kn = rng.standard_normal((2, 16)).astype(np.float32)
        _, post = orc.step(0, q, kn, kn, pol, step=t)
    T = [n0 + k for k in range(1, steps + 1)]        # attended count at step k
    def closed(first):
        return sum((1 - lam) * lam ** (steps - k) * G / T[k - 1] for k in range(first, steps + 1))
    for h in range(2):
        pos, score = post[h]
        assert pos.size == n0 + steps
        for i, p in enumerate(pos):
            first = 1 if p < n0 else p - n0 + 1      # the step that appended position p
            assert abs(score[i] - closed(first)) < 1e-14, (lam, p)


def test_decay_zero_is_plain_accumulation():
    G = 2
    a, rng = _small_h2o_oracle(G=G)
    b, _ = _small_h2o_oracle(G=G)
    for t in range(1, 5):
        q = rng.standard_normal((2 * G, 16)).astype(np.float32)
        kn = rng.standard_normal((2, 16)).astype(np.float32)
        _, pa = a.step(0, q, kn, kn, oracle.Policy.h2o(100, 100), step=t)
        _, pb = b.step(0, q, kn, kn, oracle.Policy.h2o(100, 100, decay=0.0), step=t)
        for h in range(2):
            np.testing.assert_array_equal(pa[h][1], pb[h][1])


# ---------------------------------------------------------------------------
# H2O selection: brute force over all subsets on tiny inputs
# ---------------------------------------------------------------------------

def _better(a, b):
    """(score desc, pos asc) total order."""
    return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])


def _brute_h2o(pos, score, L, n_heavy, n_recent):
    n = len(pos)
    recent = [i for i in range(n) if pos[i] >= L - n_recent]
    cand = [i for i in range(n) if pos[i] < L - n_recent]
    k = min(n_heavy, len(cand))
    winners = []
    for S in itertools.combinations(cand, k):
        rest = [j for j in cand if j not in S]
        if all(_better((score[i], pos[i]), (score[j], pos[j])) for i in S for j in rest):
            winners.append(set(S))
    assert len(winners) == 1, "the kept set must be unique under the total order"
    keep = np.zeros(n, bool)
    keep[recent] = True
    keep[list(winners[0])] = True
    return keep


@pytest.mark.parametrize("trial", range(40))
def test_h2o_select_matches_brute_force(trial):
    rng = np.random.default_rng(100 + trial)
    n = int(rng.integers(1, 13))
    pos = rng.permutation(40)[:n].astype(np.int32)
    # coarse scores so that ties occur
    score = rng.integers(0, 4, n).astype(np.float64) / 4
    L = int(pos.max()) + 1 + int(rng.integers(0, 3))
    n_recent = int(rng.integers(0, 5))
    n_heavy = int(rng.integers(0, 6))
    got = oracle.select_h2o(pos, score, L, n_heavy, n_recent)
    want = _brute_h2o(pos, score, L, n_heavy, n_recent)
    np.testing.assert_array_equal(got, want)


def test_h2o_ties_go_to_lower_position_and_zero_heavy_is_a_window():
    pos = np.arange(20, dtype=np.int32)[::-1].copy()
    score = np.ones(20)
    keep = oracle.select_h2o(pos, score, 20, n_heavy=3, n_recent=5)
    assert sorted(pos[keep]) == [0, 1, 2, 15, 16, 17, 18, 19]
    keep = oracle.select_h2o(pos, np.arange(20.0), 20, n_heavy=0, n_recent=5)
    assert sorted(pos[keep]) == [15, 16, 17, 18, 19]


def test_h2o_budget_figures_from_the_guide():
    fig = _read_kv("page_figures.txt")
    assert fig["h2o_heavy"] + fig["h2o_recent"] == fig["h2o_budget"] == 512
    rng = np.random.default_rng(7)
    L = 2049
    pos = rng.permutation(L).astype(np.int32)
    keep = oracle.select_h2o(pos, rng.random(L), L, 64, 448)
    assert keep.sum() == 512
    assert set(range(L - 448, L)) <= set(pos[keep].tolist())


# ---------------------------------------------------------------------------
# StreamingLLM: the closed-form kept set along a trajectory
# ---------------------------------------------------------------------------

def test_streaming_trajectory_closed_form():
    # 1 sequence, 2 MHA heads, D = 4, cache of positions 0..1023, 64 + 448.
    fig = _read_kv("page_figures.txt")
    n_sink, n_recent = int(fig["streaming_sink"]), int(fig["streaming_recent"])
    assert n_sink + n_recent == fig["streaming_budget"]
    D = 4
    orc = oracle.Oracle(q_heads=2, kv_heads=2, head_dim=D, dtype="f32")
    rng = np.random.default_rng(8)
    orc.load(0, rng.standard_normal((2, 1024, D)).astype(np.float32),
             rng.standard_normal((2, 1024, D)).astype(np.float32))
    for t in range(1, 17):
        q, kn, vn = rng.standard_normal((3, 2, D)).astype(np.float32)
        orc.step(0, q, kn, vn, oracle.Policy.streaming(n_sink, n_recent), step=t)
        want = list(range(64)) + list(range(576 + t, 1024 + t))
        for h in range(2):
            assert orc.units[0][h].pos.tolist() == want


def test_streaming_keeps_all_while_under_budget():
    pos = np.arange(300, dtype=np.int32)
    assert oracle.select_streaming(pos, 300, 64, 448).all()
    # exactly at the boundary: L = 512 -> all kept; L = 513 -> position 64 leaves
    pos = np.arange(513, dtype=np.int32)
    keep = oracle.select_streaming(pos, 513, 64, 448)
    assert keep.sum() == 512 and not keep[64]


# ---------------------------------------------------------------------------
# per-head random eviction with the prompt pinned
# ---------------------------------------------------------------------------

def test_n_keep_follows_the_hook_rounding():
    assert oracle.n_keep(100, 0.29) == 28          # 0.29 * 100 = 28.999... -> 28
    assert oracle.n_keep(3, 0.1) == 1               # max(1, 0)
    assert oracle.n_keep(16384, 0.25) == 4096
    assert oracle.n_keep(10, 1.0) == 10
    assert oracle.n_keep(10, 1.7) == 10             # slicing a permutation clamps
    assert oracle.n_keep(0, 0.5) == 0


def _random_unit_keep(n_tokens, prompt, k, seed, head, step=1, seq=0):
    pos = np.arange(n_tokens, dtype=np.int32)
    return oracle.select_random(pos, prompt, k, seed, seq, head, step)


def test_random_pins_prompt_equal_counts_and_is_not_a_no_op():
    n_tokens, prompt = 1000, 200
    k = oracle.n_keep(n_tokens - prompt, 0.25)
    keeps = [_random_unit_keep(n_tokens, prompt, k, seed=11, head=h) for h in range(8)]
    for kp in keeps:
        assert kp[:prompt].all()
        assert kp.sum() == prompt + k < n_tokens
    # heads draw different sets
    assert len({tuple(np.flatnonzero(kp)) for kp in keeps}) == 8


def test_random_identity_when_nothing_follows_the_prompt():
    for n_tokens in (0, 5, 256):
        kp = _random_unit_keep(n_tokens, 256, 1, seed=3, head=0)
        assert kp.all()
    kp = _random_unit_keep(300, 256, 44, seed=3, head=0)   # 44 candidates, keep 44
    assert kp.all()


def test_random_keeps_the_smallest_keys():
    pos = np.arange(50, 90, dtype=np.int32)
    kp = oracle.select_random(pos, 50, 10, 99, 2, 1, 7)
    keys = np.array([oracle.random_key(int(p), 99, 2, 1, 7) for p in pos], np.uint64)
    thr = np.sort(keys)[9]
    assert set(pos[kp]) == set(pos[keys <= thr])


def test_random_equal_keys_go_to_the_lower_position():
    # Word 0 of the generator is 32 bits: among 2^18 positions of one (seed,
    # sequence, head, step) several pairs share a key.  With the pair at the
    # edge of the kept set, the lower position is kept and the higher one
    # evicted, whatever their slot order (a total order on (key, position)).
    from key_ties import find_ties
    seed, seq, head, step, prompt = 0x5EED, 3, 5, 41, 16
    pos, keys, pairs = find_ties(seed, seq, head, step, prompt)
    assert pairs, "a 2^18-position search holds a tied pair"
    for W, lo, hi in pairs[:3]:
        assert oracle.random_key(lo, seed, seq, head, step) == W
        assert oracle.random_key(hi, seed, seq, head, step) == W and lo < hi
        below = pos[keys < W][:40]
        above = pos[keys > W][:7]
        pinned = np.arange(prompt, dtype=np.int32)
        for order in ("lo_first", "hi_first"):
            pair = [lo, hi] if order == "lo_first" else [hi, lo]
            cand = np.concatenate([pinned, above, pair, below]).astype(np.int32)
            k = oracle.select_random(cand, prompt, below.size + 1, seed, seq, head, step)
            kept = set(cand[k].tolist())
            assert lo in kept and hi not in kept, (order, W, lo, hi)
            assert set(pinned.tolist()) | set(below.tolist()) <= kept
            assert not (set(above.tolist()) & kept)
            # one more kept slot keeps both, one fewer keeps neither
            k2 = oracle.select_random(cand, prompt, below.size + 2, seed, seq, head, step)
            assert {lo, hi} <= set(cand[k2].tolist())
            k0 = oracle.select_random(cand, prompt, below.size, seed, seq, head, step)
            assert not ({lo, hi} & set(cand[k0].tolist()))


def test_random_replay_schedule_and_survival():
    # Positions-only replay of the long-trace schedule (prompt pinned, a fixed
    # budget of n_keep generated tokens, one token per step): nothing leaves
    # while the cache is under budget, then exactly one generated token per
    # step, the one with the largest key of that step; the prompt never
    # leaves.  Each steady step evicts one of n_keep + 1 candidates uniformly,
    # so a token present at the start of the steady phase survives S more
    # steps with probability (n_keep / (n_keep + 1))^S.
    prompt, n_keep, grow, S = 32, 64, 64, 64
    surv = []
    for seed in range(60):
        nev, ev, fin = oracle.random_replay(np.arange(prompt), prompt + n_keep + 1, grow + S,
                                            prompt, 1, prompt, n_keep, seed, 2, 1)
        assert nev[:grow].sum() == 0 and np.all(nev[grow:] == 1)
        assert fin.size == prompt + n_keep and np.all(fin[:prompt] == np.arange(prompt))
        assert np.all(ev >= prompt)
        if seed < 3:
            # the evicted token has the largest key of its step's candidates
            kept = list(range(prompt + grow))
            for t, e in zip(range(grow, grow + S), ev):
                kept.append(prompt + t)
                c = np.array([p for p in kept if p >= prompt], np.int32)
                kk = oracle.random_keys(c, seed, 2, 1, t + 1).astype(np.int64)
                assert int(c[kk == kk.max()].max()) == int(e)
                kept.remove(int(e))
            assert sorted(kept) == fin.tolist()
        surv.append(int(((fin >= prompt) & (fin < prompt + grow)).sum()))
    want = grow * (n_keep / (n_keep + 1)) ** S
    sd = math.sqrt(grow * 0.37 * 0.63 / len(surv)) * 2   # loose: survivals are not independent
    assert abs(np.mean(surv) - want) < 4 * sd, (np.mean(surv), want)


def test_random_inclusion_frequency_is_uniform():
    # over many seeds each candidate survives with probability k / N
    N, k, trials = 40, 10, 2000
    counts = np.zeros(N)
    for s in range(trials):
        counts += _random_unit_keep(N, 0, k, seed=s, head=0)
    p = k / N
    sd = math.sqrt(trials * p * (1 - p))
    assert np.all(np.abs(counts - trials * p) < 5 * sd)
    # chi-square over positions with N-1 degrees of freedom, loose 1e-4 bound
    chi2 = float(((counts - trials * p) ** 2 / (trials * p * (1 - p))).sum())
    assert chi2 < 90.0


def test_random_head_overlap_and_union_fraction():
    # E|S_h n S_h'| = k^2 / N;  union over H heads keeps 1 - (1 - k/N)^H
    N, k, H, trials = 200, 50, 6, 300
    overl, union = [], []
    for s in range(trials):
        ks = [_random_unit_keep(N, 0, k, seed=s, head=h) for h in range(H)]
        overl.append((ks[0] & ks[1]).sum())
        union.append(np.logical_or.reduce(ks).mean())
    assert abs(np.mean(overl) - k * k / N) < 0.3
    assert abs(np.mean(union) - (1 - (1 - k / N) ** H)) < 0.005


def test_union_figure_of_the_blog():
    # the blog's warning: union over 32 heads at keep ratio 0.5 keeps about
    # 99.9999998% of the tokens; the expected union fraction is 1 - 0.5^32
    fig = _read_kv("page_figures.txt")
    H, r = int(fig["union_heads"]), fig["union_keep_ratio"]
    expected = 1 - (1 - r) ** H
    assert abs(100 * expected - fig["union_kept_percent"]) < 5e-7


def test_hook_shape_prompt_first_ascending():
    # one-shot use: [heads, prompt + n_keep] kept positions, prompt first, ascending
    Hkv, n_tokens, prompt, D = 4, 300, 100, 8
    k = oracle.n_keep(n_tokens - prompt, 0.5)
    orc = oracle.Oracle(q_heads=Hkv, kv_heads=Hkv, head_dim=D, dtype="f32")
    rng = np.random.default_rng(9)
    orc.load(0, rng.standard_normal((Hkv, n_tokens, D)).astype(np.float32),
             rng.standard_normal((Hkv, n_tokens, D)).astype(np.float32))
    for h, u in enumerate(orc.units[0]):
        keep = oracle.Oracle.select(u, n_tokens, oracle.Policy.random(prompt, k, seed=1), 0, 0, h)
        kept = u.pos[keep]
        assert kept.size == prompt + k
        assert kept[:prompt].tolist() == list(range(prompt))
        assert np.all(np.diff(kept) > 0)


# ---------------------------------------------------------------------------
# a budget at least the length is plain full attention
# ---------------------------------------------------------------------------

def test_budget_above_length_equals_full_attention():
    D, G = 16, 2
    rng = np.random.default_rng(10)
    K0 = rng.standard_normal((1, 30, D)).astype(np.float32)
    V0 = rng.standard_normal((1, 30, D)).astype(np.float32)
    a = oracle.Oracle(q_heads=G, kv_heads=1, head_dim=D, dtype="f32")
    b = oracle.Oracle(q_heads=G, kv_heads=1, head_dim=D, dtype="f32")
    a.load(0, K0, V0)
    b.load(0, K0, V0)
    for t in range(1, 6):
        q, kn, vn = (rng.standard_normal((G, D)).astype(np.float32),
                     rng.standard_normal((1, D)).astype(np.float32),
                     rng.standard_normal((1, D)).astype(np.float32))
        oa, _ = a.step(0, q, kn, vn, oracle.Policy.h2o(64, 448), step=t)
        ob, _ = b.step(0, q, kn, vn, oracle.Policy.full(), step=t)
        np.testing.assert_array_equal(oa, ob)
    assert a.units[0][0].pos.tolist() == list(range(35))


# ---------------------------------------------------------------------------
# prompt scoring (H2O scores from the prompt's own causal attention)
# ---------------------------------------------------------------------------

def test_prompt_scores_zero_queries_give_the_harmonic_tail():
    # uniform causal attention: row r spreads G over r + 1 slots, so slot j
    # collects G * sum_{r >= j} 1 / (r + 1) = G * (H_m - H_j)
    m, G, D = 37, 3, 16
    K = np.random.default_rng(1).standard_normal((m, D))
    s = oracle.prompt_scores(np.zeros((m, G, D)), K, np.arange(m), np.arange(m))
    harmonic = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, m + 1))])
    np.testing.assert_allclose(s, G * (harmonic[m] - harmonic[:m]), rtol=1e-13)


def test_prompt_scores_mass_is_group_size_per_row_that_sees_a_slot():
    rng = np.random.default_rng(2)
    m, n, G, D = 20, 30, 4, 16
    pos = rng.permutation(100)[:n]
    q_pos = rng.integers(-5, 100, m)
    s = oracle.prompt_scores(rng.standard_normal((m, G, D)), rng.standard_normal((n, D)), pos,
                             q_pos)
    rows_seeing = sum(int((pos <= qp).any()) for qp in q_pos)
    assert abs(s.sum() - G * rows_seeing) < 1e-12 * G * m
    assert (s[pos > q_pos.max()] == 0).all()


def test_prompt_scores_two_key_logistic_closed_form():
    q = np.array([[[0.5, -1.0, 2.0, 0.25]]])          # one row, one head
    K = np.array([[1.0, 0.0, -1.0, 2.0], [0.0, 1.0, 0.5, -1.0]])
    scale = 0.5
    dz = scale * (q[0, 0] @ (K[1] - K[0]))
    p0 = 1.0 / (1.0 + math.exp(dz))
    s = oracle.prompt_scores(q, K, np.array([3, 7]), None, scale)
    np.testing.assert_allclose(s, [p0, 1.0 - p0], rtol=1e-14)
    # the row at position 5 sees only the slot at position 3
    s = oracle.prompt_scores(q, K, np.array([3, 7]), np.array([5]), scale)
    np.testing.assert_array_equal(s, [1.0, 0.0])


def test_prompt_scores_follow_a_permutation_of_the_slots():
    rng = np.random.default_rng(3)
    m, n, G, D = 12, 25, 2, 16
    q = rng.standard_normal((m, G, D))
    K = rng.standard_normal((n, D))
    pos = np.arange(n)
    q_pos = np.sort(rng.integers(0, n, m))
    perm = rng.permutation(n)
    a = oracle.prompt_scores(q, K, pos, q_pos)
    b = oracle.prompt_scores(q, K[perm], pos[perm], q_pos)
    np.testing.assert_allclose(b, a[perm], rtol=1e-13)


# ---------------------------------------------------------------------------
# E5M2 (fp8 KV cache): values from the OCP 8-bit floating point specification
# ---------------------------------------------------------------------------

E5M2_TABLE = {   # code -> value (sign, 5-bit exponent with bias 15, 2-bit mantissa)
    0x00: 0.0, 0x01: 2.0 ** -16, 0x02: 2.0 ** -15, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14,
    0x3C: 1.0, 0x3D: 1.25, 0x3E: 1.5, 0x3F: 1.75, 0x40: 2.0, 0x7B: 57344.0,
    0xBC: -1.0, 0xFB: -57344.0, 0x7C: math.inf, 0xFC: -math.inf,
}


def test_e5m2_decodes_the_specification_values():
    codes = np.array(list(E5M2_TABLE), np.uint8)
    np.testing.assert_array_equal(oracle.decode(codes, "e5m2"), list(E5M2_TABLE.values()))
    nan = oracle.decode(np.array([0x7D, 0x7E, 0x7F, 0xFF], np.uint8), "e5m2")
    assert np.isnan(nan).all()
    neg0 = oracle.decode(np.array([0x80], np.uint8), "e5m2")[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0


def test_e5m2_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)
    np.testing.assert_array_equal(oracle.encode_e5m2(oracle.decode(codes, "e5m2")), codes)


@pytest.mark.parametrize("x,code", [
    (1.125, 0x3C), (1.375, 0x3E), (1.625, 0x3E), (1.875, 0x40),   # ties to the even code
    (1.1, 0x3C), (1.2, 0x3D),                                        # nearest
    (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02), (5 * 2.0 ** -17, 0x02),   # subnormal ties
    (57344.0, 0x7B), (60000.0, 0x7B), (1e9, 0x7B), (-1e9, 0xFB), (math.inf, 0x7B),  # saturation
    (-1.0, 0xBC), (-0.0, 0x80),
])
def test_e5m2_rounding_and_saturation(x, code):
    assert int(oracle.encode_e5m2(np.array([x]))[0]) == code


def test_e5m2_encoding_is_monotone_and_within_half_a_step():
    x = np.linspace(-70000, 70000, 200001)
    c = oracle.encode_e5m2(x)
    v = oracle.decode(c, "e5m2")
    assert (np.diff(v) >= 0).all()
    inside = np.abs(x) <= 57344
    # relative error of the nearest code: at most 2^-3 of the value (2 mantissa bits)
    err = np.abs(v[inside] - x[inside])
    assert (err <= np.maximum(np.abs(x[inside]) * 2.0 ** -3, 2.0 ** -17)).all()


# ---------------------------------------------------------------------------
# KIVI-style quantized cache (guide page: "2. cost structure of the 4
# baselines", group 32 and residual 128; "16. -- the 4 methods step by step",
# K along channels and V along tokens; "16. -- limits and conclusion",
# periodic conversion when the residual fills)
# ---------------------------------------------------------------------------

def test_quantizer_reproduces_values_on_an_exact_grid():
    # values lo + k * s with s a power of two and both ends present: the grid
    # is exactly those values, so the codes are k and the values come back
    rng = np.random.default_rng(0)
    for bits in (2, 4):
        top = (1 << bits) - 1
        k = rng.integers(0, top + 1, size=(50, 32))
        k[:, 0], k[:, 1] = 0, top
        lo = rng.integers(-64, 64, size=(50, 1)) * 0.125
        s = 2.0 ** rng.integers(-6, 2, size=(50, 1))
        x = (lo + k * s).astype(np.float32)
        c, sc, l = oracle.quantize_groups(x, bits)
        np.testing.assert_array_equal(c, k)
        np.testing.assert_array_equal(sc, s[:, 0].astype(np.float32))
        np.testing.assert_array_equal(oracle.dequantize_groups(c, sc, l), x)


def test_quantizer_ties_go_to_the_even_code():
    # grid 0, 1, .., 15 (scale 1): a value half-way between two levels takes
    # the even one
    base = np.arange(16, dtype=np.float32)
    x = np.concatenate([base, np.array([0.5, 1.5, 2.5, 3.5, 12.5, 13.5, 14.5, 7.25], np.float32),
                        np.zeros(8, np.float32)])[None]
    c, sc, _ = oracle.quantize_groups(x, 4)
    assert sc[0] == 1.0
    np.testing.assert_array_equal(c[0, 16:24], [0, 2, 2, 4, 12, 14, 14, 7])


def test_quantizer_constant_group_and_error_bound():
    c, sc, lo = oracle.quantize_groups(np.full((1, 32), 3.5, np.float32), 4)
    assert sc[0] == 0 and lo[0] == 3.5 and (c == 0).all()
    assert (oracle.dequantize_groups(c, sc, lo) == 3.5).all()
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((400, 32)) * rng.uniform(0.01, 100, (400, 1))).astype(np.float32)
    for bits in (2, 4):
        c, sc, lo = oracle.quantize_groups(x, bits)
        v = oracle.dequantize_groups(c, sc, lo)
        # every value within half a grid step; the ends land on the ends
        assert (np.abs(v - x) <= 0.5 * sc[:, None].astype(np.float64) * (1 + 1e-6)).all()
        assert (c.max(axis=1) == (1 << bits) - 1).all() and (c.min(axis=1) == 0).all()
        np.testing.assert_array_equal(c[np.arange(400), x.argmin(axis=1)], 0)
        # order is kept
        order = np.argsort(x, axis=1, kind="stable")
        assert (np.diff(np.take_along_axis(c.astype(int), order, axis=1), axis=1) >= 0).all()


def test_kivi_keys_quantize_per_channel_and_values_per_token():
    # keys constant along tokens within each channel, values constant along
    # each token's 32-channel groups: the stated granularities reproduce them
    # exactly, the transposed ones would not
    rng = np.random.default_rng(2)
    D = 128
    K = np.repeat(rng.standard_normal((1, D)), 32, axis=0)
    V = np.repeat(rng.standard_normal((32, D // 32)), 32, axis=1)
    g = oracle.KiviGroup(K, V, bits=4, cgroup=32)
    np.testing.assert_array_equal(g.keys(), K.astype(np.float32))
    np.testing.assert_array_equal(g.values(), V.astype(np.float32))
    # swapped, each tensor meets the other granularity and is not reproduced
    g2 = oracle.KiviGroup(V, K, bits=4, cgroup=32)
    assert np.abs(g2.keys() - V).max() > 1e-3 and np.abs(g2.values() - K).max() > 1e-3
    # an outlier channel of the keys does not widen the other channels' grids
    K2 = rng.standard_normal((32, D))
    K2[:, 0] *= 1000
    err = np.abs(oracle.KiviGroup(K2, V, 4, 32).keys() - K2)
    rng_ch = K2.max(axis=0) - K2.min(axis=0)
    assert (err[:, 1:] <= rng_ch[1:] / 30 * (1 + 1e-6)).all()


def _kivi_bf16(shape, seed):
    return synth.bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("L", [20, 128, 129, 200, 2050])
def test_kivi_residual_schedule_closed_form(L):
    # after t steps from a prompt of L tokens the cache holds N = L + t tokens:
    # ceil((N - 128) / 32) whole groups of the oldest (none while N <= 128) and
    # the rest, the newest 97 .. 128 once N > 128, in the residual, in order
    H, D = 2, 64
    kv = oracle.Kivi(2, H, D)
    kp = _kivi_bf16((H, L, D), 3)
    kv.load(0, kp, _kivi_bf16((H, L, D), 4))
    seen = [oracle.decode(kp, "bf16")[0]]
    for t in range(1, 80):
        kn = _kivi_bf16((H, D), 100 + t)
        kv.step(0, _kivi_bf16((2, D), 200 + t), kn, _kivi_bf16((H, D), 300 + t))
        seen.append(oracle.decode(kn, "bf16")[0][None])
        N = L + t
        q = 32 * max(0, -(-(N - 128) // 32))
        u = kv.units[0][0]
        assert (u.n_quant, u.n_res) == (q, N - q)
        if N > 128:
            assert 97 <= u.n_res <= 128
        allk = np.vstack(seen)
        np.testing.assert_array_equal(u.res_k, allk[q:])


def test_kivi_attention_without_quantized_tokens_is_plain_attention():
    H, G, D, L = 2, 4, 64, 90
    kv = oracle.Kivi(H * G, H, D)
    k, v = _kivi_bf16((H, L, D), 5), _kivi_bf16((H, L, D), 6)
    kv.load(0, k, v)
    q, kn, vn = _kivi_bf16((H * G, D), 7), _kivi_bf16((H, D), 8), _kivi_bf16((H, D), 9)
    out = kv.step(0, q, kn, vn)
    K = np.concatenate([oracle.decode(k, "bf16"), oracle.decode(kn, "bf16")[:, None]], axis=1)
    V = np.concatenate([oracle.decode(v, "bf16"), oracle.decode(vn, "bf16")[:, None]], axis=1)
    Q = oracle.decode(q, "bf16")
    for h in range(H):
        z = Q[h * G:(h + 1) * G] @ K[h].T / math.sqrt(D)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(out[h * G:(h + 1) * G], p @ V[h], rtol=0, atol=1e-12)


def test_kivi_attention_is_exact_on_inputs_the_grids_represent():
    # every group's keys constant per channel and values constant per token
    # group: the quantized cache holds the values exactly, so the step equals
    # plain attention over them
    H, G, D, L = 1, 2, 64, 300
    rng = np.random.default_rng(10)
    Kf = np.repeat(rng.standard_normal((L // 32 + 1, 1, D)), 32, axis=1).reshape(-1, D)[:L]
    Vf = np.repeat(rng.standard_normal((L, D // 32, 1)), 32, axis=2).reshape(L, D)
    k = synth.bf16_bits(Kf.astype(np.float32))[None]
    v = synth.bf16_bits(Vf.astype(np.float32))[None]
    kv = oracle.Kivi(G, H, D)
    kv.load(0, k, v)
    assert kv.units[0][0].n_quant == 192
    q, kn, vn = _kivi_bf16((G, D), 11), _kivi_bf16((H, D), 12), _kivi_bf16((H, D), 13)
    out = kv.step(0, q, kn, vn)
    K = np.vstack([oracle.decode(k, "bf16")[0], oracle.decode(kn, "bf16")])
    V = np.vstack([oracle.decode(v, "bf16")[0], oracle.decode(vn, "bf16")])
    z = oracle.decode(q, "bf16") @ K.T / math.sqrt(D)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, p @ V, rtol=0, atol=1e-12)
