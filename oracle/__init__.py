"""CPU oracle for decode attention over a budget-limited per-head KV cache.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package; the HIP library never does.  The arithmetic
lives in ``oracle.c`` (plain C, double precision, one thread); this module
loads it with ctypes and keeps a canonical per-head state (entries in
ascending position order) for multi-step trajectories.

Pages cited in the C source: the KV-cache-compression guide (sections on the
capacity formula and on StreamingLLM / H2O) and the eviction-in-practice blog
(sections on per-head random eviction and its reference hook).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c to load (the sanitizer test
# runs the pins against an AddressSanitizer / UndefinedBehaviorSanitizer build)
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile oracle.c with gcc (strict IEEE double, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if "ORACLE_LIB" not in os.environ and (
                not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB)
        c_i32p = ctypes.POINTER(ctypes.c_int32)
        c_dp = ctypes.POINTER(ctypes.c_double)
        c_u8p = ctypes.POINTER(ctypes.c_uint8)
        L.orc_bytes_per_token.restype = ctypes.c_uint64
        L.orc_bytes_per_token.argtypes = [ctypes.c_int64] * 4
        L.orc_bf16_to_f64.restype = None
        L.orc_bf16_to_f64.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16), c_dp]
        L.orc_e5m2_to_f64.restype = None
        L.orc_e5m2_to_f64.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_uint8), c_dp]
        L.orc_f64_to_e5m2.restype = None
        L.orc_f64_to_e5m2.argtypes = [ctypes.c_int64, c_dp, ctypes.POINTER(ctypes.c_uint8)]
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        L.orc_random_key.restype = ctypes.c_uint32
        L.orc_random_key.argtypes = [ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32,
                                     ctypes.c_uint32, ctypes.c_uint32]
        L.orc_attend.restype = None
        L.orc_attend.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                 c_dp, c_dp, c_dp, c_dp, c_dp]
        L.orc_select_streaming.restype = None
        L.orc_select_streaming.argtypes = [ctypes.c_int32, c_i32p, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_int32, c_u8p]
        L.orc_select_h2o.restype = None
        L.orc_select_h2o.argtypes = [ctypes.c_int32, c_i32p, c_dp, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_int32, c_u8p]
        L.orc_select_random.restype = None
        L.orc_select_random.argtypes = [ctypes.c_int32, c_i32p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.c_uint32, c_u8p]
        L.orc_random_keys.restype = None
        L.orc_random_keys.argtypes = [ctypes.c_int64, c_i32p, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.POINTER(ctypes.c_uint32)]
        L.orc_random_replay.restype = ctypes.c_int32
        L.orc_random_replay.argtypes = [ctypes.c_int32, c_i32p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_uint32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint32,
                                        ctypes.c_uint32, c_i32p, c_i32p, ctypes.c_int64, c_i32p,
                                        c_i32p]
        L.orc_n_keep.restype = ctypes.c_int64
        L.orc_n_keep.argtypes = [ctypes.c_int64, ctypes.c_double]
        c_fp = ctypes.POINTER(ctypes.c_float)
        L.orc_quantize_groups.restype = None
        L.orc_quantize_groups.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, c_fp,
                                          c_u8p, c_fp, c_fp]
        L.orc_dequantize_groups.restype = None
        L.orc_dequantize_groups.argtypes = [ctypes.c_int64, ctypes.c_int32, c_u8p, c_fp, c_fp,
                                            c_dp]
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


# ----------------------------------------------------------------------------
# thin wrappers
# ----------------------------------------------------------------------------

def bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(lib().orc_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (bf16 bit patterns, E5M2 codes or float32) -> float64, exactly."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if dtype == "e5m2":
        codes = np.ascontiguousarray(x, dtype=np.uint8)
        out = np.empty(codes.shape, np.float64)
        lib().orc_e5m2_to_f64(codes.size, _p(codes, ctypes.c_uint8), _p(out, ctypes.c_double))
        return out
    bits = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().orc_bf16_to_f64(bits.size, _p(bits, ctypes.c_uint16), _p(out, ctypes.c_double))
    return out


def encode_e5m2(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest E5M2 codes (ties to even, saturating at +-57344)."""
    v = np.ascontiguousarray(x, np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_f64_to_e5m2(v.size, _p(v, ctypes.c_double), _p(out, ctypes.c_uint8))
    return out


def act_dtype(dtype: str) -> str:
    """Storage dtype of q, k_new and v_new for a cache of this dtype: an E5M2
    cache is fed bf16 activations."""
    return "bf16" if dtype == "e5m2" else dtype


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    o = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_p(c, ctypes.c_uint32), _p(k, ctypes.c_uint32), _p(o, ctypes.c_uint32))
    return o


def random_key(pos: int, seed: int, seq: int, head: int, step: int) -> int:
    return int(lib().orc_random_key(pos, seed, seq, head, step))


def random_keys(pos, seed: int, seq: int, head: int, step: int) -> np.ndarray:
    """Random-eviction key of every position in pos (uint32 array)."""
    p = np.ascontiguousarray(pos, np.int32)
    out = np.empty(p.size, np.uint32)
    lib().orc_random_keys(p.size, _p(p, ctypes.c_int32), seed, seq, head, step,
                          _p(out, ctypes.c_uint32))
    return out.reshape(np.shape(pos))


def random_replay(pos0, cap: int, steps: int, first_pos: int, first_step: int, prompt_len: int,
                  n_keep: int, seed: int, seq: int, head: int):
    """Positions-only replay of per-head random eviction over `steps` decode
    steps of one unit (see orc_random_replay): returns (n_evicted [steps],
    evicted positions in step order, final kept positions ascending)."""
    p0 = np.ascontiguousarray(pos0, np.int32)
    nev = np.zeros(steps, np.int32)
    ev_cap = max(steps + p0.size, 1)
    ev = np.empty(ev_cap, np.int32)
    out = np.empty(max(cap, 1), np.int32)
    n_out = np.zeros(1, np.int32)
    rc = lib().orc_random_replay(p0.size, _p(p0, ctypes.c_int32), cap, steps, first_pos,
                                 first_step, prompt_len, n_keep, seed, seq, head,
                                 _p(nev, ctypes.c_int32), _p(ev, ctypes.c_int32), ev_cap,
                                 _p(out, ctypes.c_int32), _p(n_out, ctypes.c_int32))
    if rc != 0:
        raise ValueError("random_replay: the kept set outgrew cap")
    return nev, ev[:int(nev.sum())].copy(), out[:int(n_out[0])].copy()


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: Optional[float] = None,
           want_p: bool = False):
    """q [G, D], K [n, D], V [n, D] float64 -> out [G, D] (and p [G, n])."""
    q = np.ascontiguousarray(q, np.float64)
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    G, D = q.shape
    n = K.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((G, D), np.float64)
    p = np.empty((G, max(n, 1)), np.float64) if want_p else None
    lib().orc_attend(n, G, D, scale, _p(q, ctypes.c_double),
                     _p(K if n else np.zeros((1, D)), ctypes.c_double),
                     _p(V if n else np.zeros((1, D)), ctypes.c_double),
                     _p(out, ctypes.c_double), _p(p, ctypes.c_double) if want_p else None)
    if want_p:
        return out, p[:, :n]
    return out


def select_streaming(pos, L: int, n_sink: int, n_recent: int) -> np.ndarray:
    pos = np.ascontiguousarray(pos, np.int32)
    keep = np.zeros(pos.size, np.uint8)
    lib().orc_select_streaming(pos.size, _p(pos, ctypes.c_int32), L, n_sink, n_recent,
                               _p(keep, ctypes.c_uint8))
    return keep.astype(bool)


def prompt_scores(q_rows: np.ndarray, K: np.ndarray, pos: np.ndarray,
                  q_pos: Optional[np.ndarray], scale: Optional[float] = None) -> np.ndarray:
    """H2O scores that a block of query rows leaves on one kv head's cache.

    q_rows [m, G, D] (the m query rows of the G query heads of this kv head),
    K [n, D], pos [n] slot positions, q_pos [m] row positions or None.  Row r
    of head g attends the slots with pos <= q_pos[r] (every slot when q_pos is
    None): p = softmax(scale q K^T) over them, and each slot's score receives
    the sum over rows and heads of its probability.  A row that sees no slot
    adds nothing.  This is how H2O accumulates attention scores over the
    prompt's own causal attention before eviction starts (guide, sections 2
    and 16, "the 4 methods" and "prefill, decode, TP").  float64.
    """
    q_rows = np.asarray(q_rows, np.float64)
    K = np.asarray(K, np.float64)
    pos = np.asarray(pos, np.int64)
    m, G, D = q_rows.shape
    s = np.zeros(K.shape[0])
    for r in range(m):
        vis = np.ones(pos.size, bool) if q_pos is None else pos <= int(q_pos[r])
        if not vis.any():
            continue
        idx = np.flatnonzero(vis)
        Kv = K[idx]
        _, p = attend(q_rows[r], Kv, Kv, scale, want_p=True)   # V unused: only p matters
        s[idx] += p[:, :idx.size].sum(axis=0)
    return s


def select_h2o(pos, score, L: int, n_heavy: int, n_recent: int) -> np.ndarray:
    pos = np.ascontiguousarray(pos, np.int32)
    score = np.ascontiguousarray(score, np.float64)
    keep = np.zeros(pos.size, np.uint8)
    lib().orc_select_h2o(pos.size, _p(pos, ctypes.c_int32), _p(score, ctypes.c_double), L,
                         n_heavy, n_recent, _p(keep, ctypes.c_uint8))
    return keep.astype(bool)


def select_random(pos, prompt_len: int, n_keep: int, seed: int, seq: int, head: int,
                  step: int) -> np.ndarray:
    pos = np.ascontiguousarray(pos, np.int32)
    keep = np.zeros(pos.size, np.uint8)
    lib().orc_select_random(pos.size, _p(pos, ctypes.c_int32), prompt_len, n_keep,
                            seed, seq, head, step, _p(keep, ctypes.c_uint8))
    return keep.astype(bool)


def n_keep(N: int, keep_ratio: float) -> int:
    return int(lib().orc_n_keep(N, keep_ratio))


# ----------------------------------------------------------------------------
# multi-step trajectories
# ----------------------------------------------------------------------------

class Policy(dict):
    """kind: 'full' | 'streaming' | 'h2o' | 'random' plus its parameters."""

    @staticmethod
    def streaming(n_sink=64, n_recent=448):
        return Policy(kind="streaming", n_sink=n_sink, n_recent=n_recent)

    @staticmethod
    def h2o(n_heavy=64, n_recent=448, decay=0.0):
        """decay 0: accumulated attention; 0 < decay < 1: decayed attention
        activity (online compaction study, sections 3.1 and 4.1)."""
        return Policy(kind="h2o", n_heavy=n_heavy, n_recent=n_recent, decay=decay)

    @staticmethod
    def random(prompt_len, n_keep, seed=0):
        return Policy(kind="random", prompt_len=prompt_len, n_keep=n_keep, seed=seed)

    @staticmethod
    def full():
        return Policy(kind="full")


class Unit:
    """Canonical state of one (sequence, kv head): entries in ascending position."""

    __slots__ = ("pos", "k", "v", "s")

    def __init__(self, pos, k, v, s=None):
        self.pos = np.asarray(pos, np.int32)
        self.k = np.asarray(k, np.float64)
        self.v = np.asarray(v, np.float64)
        self.s = np.zeros(self.pos.size) if s is None else np.asarray(s, np.float64)


class Oracle:
    """Whole-batch decode steps with eviction, one sequence at a time."""

    def __init__(self, q_heads: int, kv_heads: int, head_dim: int, dtype: str,
                 scale: Optional[float] = None):
        assert q_heads % kv_heads == 0
        self.Hq, self.Hkv, self.D, self.dtype = q_heads, kv_heads, head_dim, dtype
        self.G = q_heads // kv_heads
        self.scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
        self.units: Dict[int, List[Unit]] = {}
        self.seen: Dict[int, int] = {}

    def load(self, b: int, k_store: np.ndarray, v_store: np.ndarray, seen: Optional[int] = None,
             pos: Optional[np.ndarray] = None, scores: Optional[np.ndarray] = None):
        """Cache of sequence b: storage arrays [Hkv, n, D]; positions default to 0..n-1."""
        k = decode(k_store, self.dtype)
        v = decode(v_store, self.dtype)
        n = k.shape[1]
        units = []
        for h in range(self.Hkv):
            ph = np.arange(n, dtype=np.int32) if pos is None else np.asarray(pos[h], np.int32)
            sh = None if scores is None else np.asarray(scores[h], np.float64)
            order = np.argsort(ph, kind="stable")
            units.append(Unit(ph[order], k[h][order], v[h][order],
                              None if sh is None else sh[order]))
        self.units[b] = units
        self.seen[b] = int(n if seen is None else seen)

    def step(self, b: int, q_store, knew_store, vnew_store, policy: Policy, step: int = 0,
             seq_id: Optional[int] = None):
        """One decode step of sequence b: attend (new token included), then evict.

        Returns out [Hq, D] float64 and the per-head post-attention scores
        (before eviction, keyed by position) for H2O.
        """
        act = act_dtype(self.dtype)
        q = decode(q_store, act).reshape(self.Hq, self.D)
        kn = decode(knew_store, act).reshape(self.Hkv, self.D)
        vn = decode(vnew_store, act).reshape(self.Hkv, self.D)
        if self.dtype == "e5m2":
            # the new token is stored, and therefore attended, as E5M2
            kn = decode(encode_e5m2(kn), "e5m2")
            vn = decode(encode_e5m2(vn), "e5m2")
        p_new = self.seen[b]
        out = np.empty((self.Hq, self.D))
        post = []
        for h, u in enumerate(self.units[b]):
            u.pos = np.append(u.pos, np.int32(p_new))
            u.k = np.vstack([u.k, kn[h][None]])
            u.v = np.vstack([u.v, vn[h][None]])
            u.s = np.append(u.s, 0.0)
            o, p = attend(q[h * self.G:(h + 1) * self.G], u.k, u.v, self.scale, want_p=True)
            out[h * self.G:(h + 1) * self.G] = o
            if policy["kind"] == "h2o":
                # this step's attention weight of every entry, summed over the
                # group; the new entry's score starts at 0 (appended above)
                w_step = p.sum(axis=0)
                lam = policy.get("decay", 0.0)
                if lam == 0.0:
                    u.s = u.s + w_step           # H2O: accumulated attention
                else:
                    u.s = lam * u.s + (1.0 - lam) * w_step   # A <- lam*A + (1-lam)*w
            post.append((u.pos.copy(), u.s.copy()))
        self.seen[b] = p_new + 1
        L = self.seen[b]
        for h, u in enumerate(self.units[b]):
            keep = self.select(u, L, policy, step, b if seq_id is None else seq_id, h)
            u.pos, u.k, u.v, u.s = u.pos[keep], u.k[keep], u.v[keep], u.s[keep]
        return out, post

    @staticmethod
    def select(u: Unit, L: int, policy: Policy, step: int, seq: int, head: int) -> np.ndarray:
        kind = policy["kind"]
        if kind == "full":
            return np.ones(u.pos.size, bool)
        if kind == "streaming":
            return select_streaming(u.pos, L, policy["n_sink"], policy["n_recent"])
        if kind == "h2o":
            return select_h2o(u.pos, u.s, L, policy["n_heavy"], policy["n_recent"])
        if kind == "random":
            return select_random(u.pos, policy["prompt_len"], policy["n_keep"],
                                 policy.get("seed", 0), seq, head, step)
        raise ValueError(kind)

    def kept_positions(self, b: int) -> List[np.ndarray]:
        return [u.pos.copy() for u in self.units[b]]


# ----------------------------------------------------------------------------
# KIVI-style quantized cache (guide page, sections "2. cost structure of the 4
# baselines", "16. -- KV cache capacity formula", "16. -- the 4 methods step
# by step" and "16. -- limits and conclusion"; see oracle.c)
# ----------------------------------------------------------------------------

def quantize_groups(x: np.ndarray, bits: int):
    """Each row of x [n_groups, len] (float32 values) on its own min/max grid
    of 2^bits levels: codes uint8 [n_groups, len], scale and lo float32
    [n_groups].  Code decisions in binary32, as orc_quantize_groups states."""
    v = np.ascontiguousarray(x, np.float32)
    n, ln = v.shape
    codes = np.empty((n, ln), np.uint8)
    scale = np.empty(n, np.float32)
    lo = np.empty(n, np.float32)
    lib().orc_quantize_groups(n, ln, bits, _p(v, ctypes.c_float), _p(codes, ctypes.c_uint8),
                              _p(scale, ctypes.c_float), _p(lo, ctypes.c_float))
    return codes, scale, lo


def dequantize_groups(codes: np.ndarray, scale: np.ndarray, lo: np.ndarray) -> np.ndarray:
    """codes [n_groups, len] -> code * scale + lo in float64 (exact)."""
    c = np.ascontiguousarray(codes, np.uint8)
    sc = np.ascontiguousarray(scale, np.float32)
    lw = np.ascontiguousarray(lo, np.float32)
    n, ln = c.shape
    out = np.empty((n, ln), np.float64)
    lib().orc_dequantize_groups(n, ln, _p(c, ctypes.c_uint8), _p(sc, ctypes.c_float),
                                _p(lw, ctypes.c_float), _p(out, ctypes.c_double))
    return out


def kivi_split(n_tokens: int, group: int = 32, residual: int = 128):
    """(quantized, residual) token counts of a cache holding n_tokens: the
    residual keeps at most `residual` of the newest tokens and the quantized
    part is whole groups, as few as that allows."""
    over = max(n_tokens - residual, 0)
    q = group * ((over + group - 1) // group)
    return q, n_tokens - q


class KiviGroup:
    """One quantized group of `group` consecutive tokens of one kv head.

    K is quantized per channel: channel d of the group's tokens is one grid
    (k_scale[d], k_lo[d]).  V is quantized per token: each token's channels
    32c .. 32c + 31 form one grid (v_scale[t, c], v_lo[t, c]).
    k_codes, v_codes: [group tokens, D] uint8."""

    def __init__(self, K: np.ndarray, V: np.ndarray, bits: int, cgroup: int):
        t, D = K.shape
        kc, ks, kl = quantize_groups(K.T, bits)                       # D grids of t values
        self.k_codes, self.k_scale, self.k_lo = kc.T.copy(), ks, kl
        vc, vs, vl = quantize_groups(V.reshape(t * (D // cgroup), cgroup), bits)
        self.v_codes = vc.reshape(t, D)
        self.v_scale = vs.reshape(t, D // cgroup)
        self.v_lo = vl.reshape(t, D // cgroup)
        self.cgroup = cgroup

    def keys(self) -> np.ndarray:
        return dequantize_groups(self.k_codes.T, self.k_scale, self.k_lo).T

    def values(self) -> np.ndarray:
        t, D = self.v_codes.shape
        c = self.cgroup
        return dequantize_groups(self.v_codes.reshape(t * (D // c), c), self.v_scale.reshape(-1),
                                 self.v_lo.reshape(-1)).reshape(t, D)


class KiviUnit:
    def __init__(self):
        self.groups: List[KiviGroup] = []
        self.res_k = None   # [r, D] float64 (bf16 values)
        self.res_v = None

    @property
    def n_quant(self) -> int:
        return sum(g.k_codes.shape[0] for g in self.groups)

    @property
    def n_res(self) -> int:
        return self.res_k.shape[0]


class Kivi:
    """KIVI-style cache of one attention layer: per (sequence, kv head) whole
    groups of `group` quantized tokens, oldest first, then a residual of at
    most `residual` newest tokens kept as given (bf16).

    A decode step attends the G query heads of each kv head over the
    dequantized tokens, the residual and the new token (attention first, as
    for eviction); then, when the residual already holds `residual` tokens,
    its `group` oldest are quantized as the next group, and the new token
    joins the residual.  That keeps the residual between residual - group + 1
    and residual tokens once the cache is longer than the residual: the
    conversion the guide describes as periodic work when the residual fills.
    """

    def __init__(self, q_heads: int, kv_heads: int, head_dim: int, bits: int = 4,
                 group: int = 32, residual: int = 128, cgroup: int = 32,
                 scale: Optional[float] = None):
        self.Hq, self.Hkv, self.D = q_heads, kv_heads, head_dim
        self.G = q_heads // kv_heads
        self.bits, self.group, self.residual, self.cgroup = bits, group, residual, cgroup
        self.scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
        self.units: Dict[int, List[KiviUnit]] = {}

    def load(self, b: int, k_store: np.ndarray, v_store: np.ndarray):
        """Prefill of sequence b: bf16 storage [kv_heads, L, D]."""
        K = decode(k_store, "bf16")
        V = decode(v_store, "bf16")
        L = K.shape[1]
        q, _ = kivi_split(L, self.group, self.residual)
        units = []
        for h in range(self.Hkv):
            u = KiviUnit()
            for g0 in range(0, q, self.group):
                u.groups.append(KiviGroup(K[h, g0:g0 + self.group], V[h, g0:g0 + self.group],
                                          self.bits, self.cgroup))
            u.res_k, u.res_v = K[h, q:].copy(), V[h, q:].copy()
            units.append(u)
        self.units[b] = units

    def entries(self, b: int, h: int):
        """(K, V) float64 of every cached token of (b, h), oldest first."""
        u = self.units[b][h]
        ks = [g.keys() for g in u.groups] + [u.res_k]
        vs = [g.values() for g in u.groups] + [u.res_v]
        return np.vstack(ks), np.vstack(vs)

    def step(self, b: int, q_store, knew_store, vnew_store) -> np.ndarray:
        """One decode step of sequence b (bf16 storage: q [Hq, D], k_new / v_new
        [Hkv, D]); returns out [Hq, D] float64."""
        q = decode(q_store, "bf16").reshape(self.Hq, self.D)
        kn = decode(knew_store, "bf16").reshape(self.Hkv, self.D)
        vn = decode(vnew_store, "bf16").reshape(self.Hkv, self.D)
        out = np.empty((self.Hq, self.D))
        for h, u in enumerate(self.units[b]):
            K, V = self.entries(b, h)
            K = np.vstack([K, kn[h][None]])
            V = np.vstack([V, vn[h][None]])
            out[h * self.G:(h + 1) * self.G] = attend(q[h * self.G:(h + 1) * self.G], K, V,
                                                      self.scale)
            if u.n_res == self.residual:
                g = self.group
                u.groups.append(KiviGroup(u.res_k[:g], u.res_v[:g], self.bits, self.cgroup))
                u.res_k, u.res_v = u.res_k[g:], u.res_v[g:]
            u.res_k = np.vstack([u.res_k, kn[h][None]])
            u.res_v = np.vstack([u.res_v, vn[h][None]])
        return out
