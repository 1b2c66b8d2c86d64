"""Equal random keys at the edge of the kept set, on every GPU path that ranks
random-eviction candidates.

Two positions of one unit whose Philox word 0 is equal (found with the
oracle's key function, tests/key_ties.py) sit exactly at the kept set's edge:
keeping the n_keep smallest keys must keep the lower position and evict the
higher one (equal keys go to the lower position; the eviction-in-practice
blog's per-head draw made reproducible with a total order).  Paths covered:
the selection kernel behind kvc_evict_random (arg-min and radix select, with
the unit's keys in LDS and read from global memory), the one-workgroup step
kernel (single eviction and radix select, both LDS capacities), and the split
step path (the split kernel's per-wave records when one slot leaves, the
finish pass's radix select otherwise), with the pair in one wave's share or
in different chunks, in both slot orders."""
import numpy as np
import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle
from key_ties import boundary_unit

pytestmark = pytest.mark.gpu

SEED = 0x00C0_FFEE_1234_5678
PROMPT = 16


def _units(step, Hkv, B, n_below, n_above, tag, layout=None):
    """Per unit (b, h): slot-ordered positions (pinned prompt first, then the
    candidates) and its tied pair.  layout(unit index, positions, pair) may
    move the pair to chosen slots."""
    rng = np.random.default_rng(tag)
    units, pairs = [], []
    for b in range(B):
        for h in range(Hkv):
            cand, pair = boundary_unit(SEED, b, h, step, PROMPT, n_below, n_above, rng)
            p = np.concatenate([np.arange(PROMPT, dtype=np.int32), cand])
            if layout is not None:
                p = layout(b * Hkv + h, p, pair)
            units.append(p.astype(np.int32))
            pairs.append(pair)
    return units, pairs


def _place(p, pair, slot_lo, slot_hi):
    """Positions p with the pair moved to the given slots (order kept otherwise)."""
    rest = [int(x) for x in p if int(x) not in pair]
    n = len(p)
    out = [None] * n
    out[slot_lo], out[slot_hi] = pair[0], pair[1]
    it = iter(rest)
    for i in range(n):
        if out[i] is None:
            out[i] = next(it)
    return np.array(out, np.int32)


def _cache(units, Hkv, G, cap, D=128, dtype=kvc.BF16):
    B = len(units) // Hkv
    c = kvc.KvCache(B, Hkv * G, Hkv, D, cap, dtype)
    pos = np.zeros((B, Hkv, cap), np.int32)
    n = np.zeros((B, Hkv), np.int32)
    for i, p in enumerate(units):
        b, h = divmod(i, Hkv)
        pos[b, h, :p.size] = p
        n[b, h] = p.size
    c.pos.copy_(torch.from_numpy(pos))
    c.n_slots.copy_(torch.from_numpy(n))
    g = torch.Generator(device="cuda").manual_seed(7)
    c.k.copy_(torch.randn(c.k.shape, generator=g, device="cuda").to(c.k.dtype))
    c.v.copy_(torch.randn(c.v.shape, generator=g, device="cuda").to(c.v.dtype))
    torch.cuda.synchronize()
    return c


def _check_pairs(kept_sets, pairs, wants):
    for i, (kept, (lo, hi), want) in enumerate(zip(kept_sets, pairs, wants)):
        assert lo in want and hi not in want, f"unit {i}: the pair is not at the edge"
        assert kept == want, (f"unit {i}: kept set differs from the oracle's "
                              f"(lower {lo} kept: {lo in kept}, higher {hi} kept: {hi in kept})")


@pytest.mark.parametrize("n_below,n_above", [(300, 0), (300, 5), (9000, 0), (9000, 5)],
                         ids=["lds-argmin", "lds-radix", "global-argmin", "global-radix"])
def test_evict_random_equal_keys_keep_the_lower_position(n_below, n_above):
    Hkv, B, step = 2, 2, 23
    units, pairs = _units(step, Hkv, B, n_below, n_above, tag=n_below + n_above)
    cap = max(p.size for p in units)
    cache = _cache(units, Hkv, 1, cap, D=64)
    keep = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
    nout = torch.full((B, Hkv), -1, dtype=torch.int32, device="cuda")
    kvc.evict_random(cache, PROMPT, n_below + 1, SEED, step, keep, nout)
    torch.cuda.synchronize()
    kk, mm = keep.cpu().numpy(), nout.cpu().numpy()
    kept, wants = [], []
    for i, p in enumerate(units):
        b, h = divmod(i, Hkv)
        w = oracle.select_random(p, PROMPT, n_below + 1, SEED, b, h, step)
        np.testing.assert_array_equal(kk[b, h, :mm[b, h]], np.flatnonzero(w))
        kept.append(set(p[kk[b, h, :mm[b, h]]].tolist()))
        wants.append(set(p[w].tolist()))
    _check_pairs(kept, pairs, wants)


def _step_inputs(n_below, n_above, layout=None, tag=0, Hkv=2, B=2):
    """Units, tied pairs, new positions and step of one random-eviction step
    case (host only)."""
    step = 57 + tag
    units, pairs = _units(step, Hkv, B, n_below, n_above, tag=1000 + tag, layout=layout)
    # the new token of sequence b: one position, a low key in both of its heads
    new_pos = []
    for b in range(B):
        used = set()
        for h in range(Hkv):
            used |= set(units[b * Hkv + h].tolist())
        lim = [oracle.random_key(pairs[b * Hkv + h][0], SEED, b, h, step) for h in range(Hkv)]
        p = 1 << 20
        while p in used or any(oracle.random_key(p, SEED, b, h, step) >= lim[h]
                               for h in range(Hkv)):
            p += 1
        new_pos.append(p)
    return units, pairs, new_pos, step


def _step_wants(units, pairs, new_pos, step, n_keep, Hkv=2):
    """The oracle's kept positions of every unit after the step."""
    wants = []
    for i, p in enumerate(units):
        b, h = divmod(i, Hkv)
        post = np.append(p, np.int32(new_pos[b]))
        w = oracle.select_random(post, PROMPT, n_keep, SEED, b, h, step)
        wants.append(set(post[w].tolist()))
        lo, hi = pairs[i]
        assert lo in wants[-1] and hi not in wants[-1] and new_pos[b] in wants[-1]
    return wants


def _step_case(n_below, n_above, hint_pad, layout=None, G=8, tag=0):
    """One kvc_decode_step under random eviction.  Every unit holds the pinned
    prompt, n_below + n_above candidates and the tied pair; the new token's
    position has a key below every pair's, so n_keep = n_below + 2 keeps it,
    the n_below low keys and the pair's lower position."""
    Hkv, B = 2, 2
    units, pairs, new_pos, step = _step_inputs(n_below, n_above, layout, tag, Hkv, B)
    n_keep = n_below + 2
    wants = _step_wants(units, pairs, new_pos, step, n_keep, Hkv)
    n = max(p.size for p in units)
    cap = n + 1
    cache = _cache(units, Hkv, G, cap)
    D = cache.head_dim
    g = torch.Generator(device="cuda").manual_seed(11)
    q = torch.randn((B, Hkv * G, D), generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn((B, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((B, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, Hkv * G, D), device="cuda")
    hint = n + 1 + hint_pad
    kvc.decode_step(cache, kvc.policy_random(PROMPT, n_keep, SEED), step,
                    torch.tensor(new_pos, dtype=torch.int32, device="cuda"), q, kn, vn, out,
                    max_len_hint=hint, workspace=cache.workspace(hint))
    torch.cuda.synchronize()
    assert int(cache.flags.item()) == 0
    pos, ns = cache.pos.cpu().numpy(), cache.n_slots.cpu().numpy()
    kept = []
    for i, p in enumerate(units):
        b, h = divmod(i, Hkv)
        got = pos[b, h, :ns[b, h]]
        assert got.size == np.unique(got).size
        kept.append(set(got.tolist()))
    _check_pairs(kept, pairs, wants)


@pytest.mark.parametrize("n_above", [0, 3], ids=["single", "radix"])
def test_fused_step_equal_keys_keep_the_lower_position(n_above):
    # one workgroup per unit, 528-entry LDS instance (about 420 attended entries)
    _step_case(400, n_above, 0, tag=n_above)


@pytest.mark.parametrize("n_above", [0, 3], ids=["single", "radix"])
def test_fused_step_1024_instance_equal_keys_keep_the_lower_position(n_above):
    # about 700 attended entries: the 1,024-entry LDS instance
    _step_case(680, n_above, 0, tag=10 + n_above)


@pytest.mark.parametrize("n_above", [0, 3], ids=["single", "radix"])
@pytest.mark.parametrize("where", ["same-wave", "other-chunk", "other-chunk-reversed"])
def test_split_step_equal_keys_keep_the_lower_position(where, n_above):
    # about 1,520 attended entries: split kernel + finish pass; the pair in
    # adjacent slots (one wave's share of one chunk) or in far apart chunks
    _step_case(1500, n_above, 0, layout=_split_layout(where),
               tag=20 + n_above + 3 * len(where))


def _split_layout(where):
    def layout(i, p, pair):
        if where == "same-wave":
            return _place(p, pair, 600 + i, 601 + i)
        if where == "other-chunk":
            return _place(p, pair, 40 + i, p.size - 30 - i)
        return _place(p, (pair[1], pair[0]), 40 + i, p.size - 30 - i)
    return layout
