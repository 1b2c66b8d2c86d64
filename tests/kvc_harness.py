"""Helpers for the GPU parity tests: build device caches from the seeded
generators, read device state back as per-unit arrays, and compare with the
CPU oracle.  Nothing here computes attention or eviction itself."""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import compressed_decode_attention_amd as kvc
import oracle
import synth

DT = {"bf16": kvc.BF16, "f32": kvc.F32, "e5m2": kvc.FP8_E5M2}

# tolerances (outputs: bf16 inputs, fp32 accumulation vs fp64; scores: relative)
OUT_ATOL = 2e-3
SCORE_RTOL = 1e-5


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage array -> device tensor of the cache dtype (bit-exact)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x, np.uint16).view(np.int16)).view(
            torch.bfloat16).cuda()
    if dtype == "e5m2":
        return torch.from_numpy(np.ascontiguousarray(x, np.uint8)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def host(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> storage array (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if dtype == "e5m2":
        return t.contiguous().cpu().numpy().astype(np.uint8)
    return t.contiguous().cpu().numpy()


def make_cache(w: synth.Workload, lengths: Sequence[int], capacity: int, paged: int = 0,
               extra_blocks: int = 0, seed_blocks: int = 0) -> kvc.KvCache:
    """Cache holding the workload's prefill of each sequence (positions 0..L-1
    in slots 0..L-1 for every kv head)."""
    B = len(lengths)
    if paged:
        max_blocks = capacity // paged
        nblk = B * max_blocks + extra_blocks
        perm = synth.block_permutation(nblk, w.seed, w.wid, seed_blocks)
        table = torch.from_numpy(perm[:B * max_blocks].reshape(B, max_blocks).copy())
        cache = kvc.KvCache(B, w.q_heads, w.kv_heads, w.head_dim, capacity, DT[w.dtype],
                            block_size=paged, num_blocks=nblk, block_table=table)
    else:
        cache = kvc.KvCache(B, w.q_heads, w.kv_heads, w.head_dim, capacity, DT[w.dtype])
    for b, L in enumerate(lengths):
        k, v = synth.prefill_kv(w, b, L)
        kt, vt = dev(k, w.dtype), dev(v, w.dtype)
        slots = torch.arange(L, device="cuda")
        for h in range(w.kv_heads):
            if paged:
                blk = cache.block_table[b, slots // paged].long()
                cache.k[blk, h, slots % paged] = kt[h]
                cache.v[blk, h, slots % paged] = vt[h]
            else:
                cache.k[b, h, :L] = kt[h]
                cache.v[b, h, :L] = vt[h]
        cache.pos[b, :, :L] = torch.arange(L, dtype=torch.int32, device="cuda")
        cache.n_slots[b] = L
    torch.cuda.synchronize()
    return cache


class Snapshot:
    """Host copy of a cache: per unit, slot-ordered pos / K / V (storage) / score."""

    def __init__(self, cache: kvc.KvCache, dtype: str, scores: Optional[torch.Tensor] = None,
                 units: Optional[List[tuple]] = None):
        torch.cuda.synchronize()
        self.dtype = dtype
        self.n = cache.n_slots.cpu().numpy()
        pos = cache.pos.cpu().numpy()
        sc = scores.cpu().numpy() if scores is not None else None
        self.units: Dict[tuple, dict] = {}
        todo = units if units is not None else [(b, h) for b in range(cache.batch)
                                                for h in range(cache.kv_heads)]
        for (b, h) in todo:
            n = int(self.n[b, h])
            k, v = cache.rows(b, h, range(n)) if n else (None, None)
            self.units[(b, h)] = dict(
                n=n,
                pos=pos[b, h, :n].copy(),
                k=host(k, dtype) if n else np.zeros((0, cache.head_dim)),
                v=host(v, dtype) if n else np.zeros((0, cache.head_dim)),
                s=sc[b, h, :n].copy() if sc is not None else None,
            )

    def unit(self, b, h):
        return self.units[(b, h)]


def kept_positions(snap: Snapshot, b: int, h: int) -> np.ndarray:
    return np.sort(snap.unit(b, h)["pos"])


def oracle_unit_attend(dtype: str, q_store: np.ndarray, pre: dict, knew: np.ndarray,
                       vnew: np.ndarray, scale: float):
    """Oracle attention of one unit over its pre-step entries plus the new token.

    q_store [G, D], knew / vnew [D] (activation storage; an E5M2 cache takes
    bf16 activations and holds, hence attends, the new token rounded to
    E5M2).  Returns out [G, D], p-sum over the group for the n cached slots
    (slot order) and the new token.
    """
    act = oracle.act_dtype(dtype)
    kn, vn = oracle.decode(knew, act), oracle.decode(vnew, act)
    if dtype == "e5m2":
        kn = oracle.decode(oracle.encode_e5m2(kn), "e5m2")
        vn = oracle.decode(oracle.encode_e5m2(vn), "e5m2")
    K = np.vstack([oracle.decode(pre["k"], dtype).reshape(-1, q_store.shape[1]), kn[None]])
    V = np.vstack([oracle.decode(pre["v"], dtype).reshape(-1, q_store.shape[1]), vn[None]])
    out, p = oracle.attend(oracle.decode(q_store, act), K, V, scale, want_p=True)
    return out, p.sum(axis=0)


def assert_scores_close(got: np.ndarray, want: np.ndarray):
    """|got - want| <= 1e-5 * max(|want|, 1e-6) element-wise."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    tol = SCORE_RTOL * np.maximum(np.abs(want), 1e-6)
    bad = np.abs(got - want) > tol
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"score mismatch at {i}: got {got[i]!r} want {want[i]!r} "
                             f"({int(bad.sum())} of {bad.size})")


def rows_by_pos(u: dict) -> Dict[int, tuple]:
    return {int(p): (u["k"][i].tobytes(), u["v"][i].tobytes(),
                     None if u["s"] is None else float(u["s"][i]))
            for i, p in enumerate(u["pos"])}
