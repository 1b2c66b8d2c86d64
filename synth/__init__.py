"""Seeded synthetic inputs for the decode-attention-with-eviction path.

This module only draws random numbers and lays them out; it holds none of the
attention or eviction arithmetic.  It is the one piece shared by the tests, the
benchmark and the smoke run: the HIP library and the CPU oracle both consume
exactly the arrays produced here, and neither imports the other.

Recipe (every workload):
  * numpy ``default_rng`` (PCG64) with ``SeedSequence([seed, workload_id,
    tensor_id, sequence, (step)])`` so that every sequence and every decode step
    has its own reproducible stream;
  * ``standard_normal(float32)``; for bf16 workloads the float32 values are
    rounded to bf16 with round-to-nearest-even, and the 16-bit patterns are the
    canonical input (the GPU sees them as bf16, the oracle decodes them exactly);
  * heavy-hitter keys (the LLaMA-3-8B-shaped H2O workload): each (sequence, kv
    head, position) key row is multiplied by 8 with probability 0.02 before the
    rounding, for prompt keys and for decode keys alike;
  * mixed-length batch: ``L_b = floor(exp(U(ln 512, ln 32768)))`` and a seeded
    permutation of the physical block ids;
  * E5M2 (fp8) caches: the cached K / V are the same float32 draws truncated to
    E5M2 codes (sign, exponent, the top two mantissa bits; magnitudes below
    2^-14 become zero), and q, k_new, v_new stay bf16 activations.

The workloads mirror the shapes the source pages talk about (a heavy-load
batch of 512 sequences with 2,048-token prompts, a 512-token budget of 64 + 448,
a roughly 4x random-eviction budget over a long reasoning trace); no dataset
item is reproduced, only shapes and value distributions.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# tensor ids inside a SeedSequence
T_K, T_V, T_Q, T_KNEW, T_VNEW, T_HEAVY, T_HEAVY_NEW, T_LENS, T_BLOCKS = range(1, 10)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, dtype and policy of one synthetic decode workload."""

    wid: int                 # workload id used in the seed sequences
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: str               # "bf16", "f32" or "e5m2" (cache; activations bf16)
    prompt_len: int          # cached tokens before the first decode step
    steps: int               # decode steps
    policy: str              # "streaming" | "h2o" | "random" | "full"
    n_sink: int = 64         # StreamingLLM attention sinks
    n_heavy: int = 64        # H2O heavy hitters
    n_recent: int = 448      # recent window (StreamingLLM and H2O)
    pinned: int = 0          # random policy: pinned prompt tokens
    n_keep: int = 0          # random policy: kept generated tokens per head
    heavy_frac: float = 0.0  # fraction of key rows scaled by heavy_scale
    heavy_scale: float = 8.0
    paged_block: int = 0     # 0 = contiguous cache, else block size
    min_len: int = 0         # mixed-length batches: log-uniform bounds
    max_len: int = 0
    seed: int = 0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def elem_bytes(self) -> int:
        return {"bf16": 2, "f32": 4, "e5m2": 1}[self.dtype]

    @property
    def act_dtype(self) -> str:
        """Storage of q, k_new and v_new."""
        return "bf16" if self.dtype == "e5m2" else self.dtype


WORKLOADS = {
    "tiny_mha_streaming_f32": Workload(
        wid=1, name="tiny_mha_streaming_f32", batch=1, q_heads=8, kv_heads=8,
        head_dim=64, dtype="f32", prompt_len=1024, steps=16, policy="streaming",
        pinned=256),
    "llama3_8b_h2o_b64": Workload(
        wid=2, name="llama3_8b_h2o_b64", batch=64, q_heads=32, kv_heads=8,
        head_dim=128, dtype="bf16", prompt_len=2048, steps=256, policy="h2o",
        heavy_frac=0.02),
    "reasoning_random_b32": Workload(
        wid=3, name="reasoning_random_b32", batch=32, q_heads=40, kv_heads=8,
        head_dim=128, dtype="bf16", prompt_len=1024, steps=16384,
        policy="random", pinned=1024, n_keep=4096),
    "heavy_load_b512_l2048": Workload(
        wid=4, name="heavy_load_b512_l2048", batch=512, q_heads=64, kv_heads=8,
        head_dim=128, dtype="bf16", prompt_len=2048, steps=128, policy="h2o"),
    "mixed_paged_h2o_b128": Workload(
        wid=5, name="mixed_paged_h2o_b128", batch=128, q_heads=32, kv_heads=8,
        head_dim=128, dtype="bf16", prompt_len=0, steps=64, policy="h2o",
        paged_block=16, min_len=512, max_len=32768),
}


# ----------------------------------------------------------------------------
# bf16 bit patterns
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Inputs are finite normal draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def e5m2_truncated(x: np.ndarray) -> np.ndarray:
    """float32 -> E5M2 codes by dropping the low mantissa bits (round toward
    zero; |x| < 2^-14 -> signed zero).  Only used to draw cache contents;
    draws here never reach the E5M2 overflow range (|x| >= 2^16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    sign = ((u >> np.uint32(31)) << np.uint32(7)).astype(np.uint8)
    e = ((u >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
    m = ((u >> np.uint32(21)) & np.uint32(3)).astype(np.int64)
    assert (e < 143).all(), "draw beyond the E5M2 range"
    code = np.where(e < 113, 0, ((e - 112) << 2) | m)
    return (sign | code.astype(np.uint8)).astype(np.uint8)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Canonical storage form: uint16 bf16 patterns, uint8 E5M2 codes, or float32."""
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "e5m2":
        return e5m2_truncated(x)
    raise ValueError(f"unknown dtype {dtype}")


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


# ----------------------------------------------------------------------------
# streams
# ----------------------------------------------------------------------------

def rng(*parts: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(p) for p in parts]))


def normal(shape, *parts: int) -> np.ndarray:
    return rng(*parts).standard_normal(shape, dtype=np.float32)


def _heavy_rows(w: Workload, x: np.ndarray, tensor: int, *parts: int) -> np.ndarray:
    """Scale a random 'heavy_frac' of the key rows (last axis = head_dim)."""
    if w.heavy_frac <= 0.0:
        return x
    mask = rng(w.seed, w.wid, tensor, *parts).random(x.shape[:-1]) < w.heavy_frac
    return np.where(mask[..., None], x * np.float32(w.heavy_scale), x).astype(np.float32)


def prefill_kv(w: Workload, b: int, length: Optional[int] = None):
    """Cached K and V of sequence b before the first decode step.

    Returns storage arrays shaped [kv_heads, length, head_dim] (positions
    0..length-1 in order).
    """
    L = w.prompt_len if length is None else length
    shape = (w.kv_heads, L, w.head_dim)
    k = normal(shape, w.seed, w.wid, T_K, b)
    k = _heavy_rows(w, k, T_HEAVY, b)
    v = normal(shape, w.seed, w.wid, T_V, b)
    return to_storage(k, w.dtype), to_storage(v, w.dtype)


def step_inputs(w: Workload, b: int, step: int):
    """q [q_heads, D], k_new [kv_heads, D], v_new [kv_heads, D] of decode step 'step'."""
    q = normal((w.q_heads, w.head_dim), w.seed, w.wid, T_Q, b, step)
    kn = normal((w.kv_heads, w.head_dim), w.seed, w.wid, T_KNEW, b, step)
    kn = _heavy_rows(w, kn, T_HEAVY_NEW, b, step)
    vn = normal((w.kv_heads, w.head_dim), w.seed, w.wid, T_VNEW, b, step)
    act = w.act_dtype
    return to_storage(q, act), to_storage(kn, act), to_storage(vn, act)


def batch_step_inputs(w: Workload, step: int, batch: Optional[int] = None):
    """Stacked step inputs for sequences 0..batch-1."""
    B = w.batch if batch is None else batch
    parts = [step_inputs(w, b, step) for b in range(B)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))


def mixed_lengths(w: Workload, batch: Optional[int] = None) -> np.ndarray:
    """Log-uniform cached lengths of a mixed-length batch (int64)."""
    B = w.batch if batch is None else batch
    u = rng(w.seed, w.wid, T_LENS).random(w.batch)[:B]
    lo, hi = math.log(w.min_len), math.log(w.max_len)
    return np.floor(np.exp(lo + u * (hi - lo))).astype(np.int64)


def block_permutation(n_blocks: int, *parts: int) -> np.ndarray:
    """Seeded permutation of physical block ids (int32)."""
    return rng(*parts, T_BLOCKS).permutation(n_blocks).astype(np.int32)


def workload(name: str, **overrides) -> Workload:
    """A registered workload, optionally with fields replaced (smaller test cases)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


# ----------------------------------------------------------------------------
# device-side draws for full-size workloads (torch's own generator, seeded from
# the same SeedSequence parts); the numbers differ from the numpy streams but
# follow the same recipe: N(0,1) float32 rounded to bf16 (round to nearest even)
# ----------------------------------------------------------------------------

def device_seed(*parts: int) -> int:
    return int(np.random.SeedSequence([int(p) for p in parts]).generate_state(1, np.uint64)[0]
               & np.uint64(0x7FFFFFFFFFFFFFFF))


def device_e5m2_truncated(x):
    """The recipe of e5m2_truncated on a float32 device tensor: E5M2 codes
    (torch.uint8) keeping sign, exponent and the top two mantissa bits."""
    import torch
    u = x.contiguous().view(torch.int32)
    sign = (u >> 24) & 0x80
    e = (u >> 23) & 0xFF
    assert bool((e < 143).all()), "draw beyond the E5M2 range"
    code = torch.where(e < 113, torch.zeros_like(u), ((e - 112) << 2) | ((u >> 21) & 3))
    return (sign | code).to(torch.uint8)


def device_normal(shape, *parts: int, device="cuda", dtype=None, scale_rows_frac: float = 0.0,
                  scale: float = 8.0):
    """N(0,1) draws on the device, rounded to `dtype` (bf16 by default); with
    scale_rows_frac > 0 a Bernoulli fraction of the rows (last axis) is scaled."""
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(*parts))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale_rows_frac > 0.0:
        m = torch.rand(shape[:-1], generator=g, device=device) < scale_rows_frac
        x = torch.where(m[..., None], x * scale, x)
    return x.to(dtype)
