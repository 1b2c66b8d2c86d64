"""Equal random-eviction keys, found with the oracle's key function.

Word 0 of Philox4x32-10 is 32 bits wide, so among a few hundred thousand
positions of one (seed, sequence, kv head, step) several pairs share a key
(about n^2 / 2^33 pairs for n positions).  The tie rule of the random policy
-- equal keys go to the lower position -- only shows on such pairs, and the
tests below place them at the edge of the kept set.  Test infrastructure:
nothing here ranks or selects, it only searches keys."""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

import oracle


def find_ties(seed: int, seq: int, head: int, step: int, start: int,
              span: int = 1 << 18) -> Tuple[np.ndarray, np.ndarray, List[Tuple[int, int, int]]]:
    """Keys of positions start .. start+span-1 and every pair of positions
    with an equal key, as (key, lower position, higher position), largest key
    first.  The span doubles until at least one pair turns up."""
    while True:
        pos = np.arange(start, start + span, dtype=np.int64).astype(np.int32)
        keys = oracle.random_keys(pos, seed, seq, head, step)
        order = np.argsort(keys, kind="stable")
        ks = keys[order]
        same = np.flatnonzero(ks[1:] == ks[:-1])
        pairs = []
        for i in same:
            a, b = int(pos[order[i]]), int(pos[order[i + 1]])
            pairs.append((int(ks[i]), min(a, b), max(a, b)))
        if pairs:
            pairs.sort(reverse=True)
            return pos, keys, pairs
        span *= 2


def boundary_unit(seed: int, seq: int, head: int, step: int, prompt_len: int, n_below: int,
                  n_above: int, rng: np.random.Generator):
    """Candidate positions (all >= prompt_len) for one unit with a tied pair at
    the edge of the kept set: the pair (key W), n_below positions with keys
    below W and n_above with keys above W.  Keeping the n_below + 1 smallest
    keys then keeps the pair's lower position and drops its higher one.
    Returns (positions in a shuffled order, the pair (lower, higher))."""
    pos, keys, pairs = find_ties(seed, seq, head, step, prompt_len)
    # a pair with room on both sides
    for W, lo, hi in pairs:
        below = pos[(keys < W)]
        above = pos[(keys > W)]
        if below.size >= n_below and above.size >= n_above:
            break
    else:
        raise AssertionError("no tied pair with enough keys on both sides")
    pick_b = rng.choice(below, n_below, replace=False) if n_below else np.zeros(0, np.int32)
    pick_a = rng.choice(above, n_above, replace=False) if n_above else np.zeros(0, np.int32)
    cand = np.concatenate([pick_b, pick_a, [lo, hi]]).astype(np.int32)
    return rng.permutation(cand).astype(np.int32), (lo, hi)


def low_key_position(seed: int, seq: int, head: int, step: int, start: int, below: int,
                     exclude) -> int:
    """A position >= start, not in exclude, whose key is below `below`."""
    ex = set(int(x) for x in exclude)
    p = start
    while True:
        if p not in ex and int(oracle.random_key(p, seed, seq, head, step)) < below:
            return p
        p += 1
