"""Python binding of libkvc (decode attention over a budget-limited per-head KV
cache with StreamingLLM / H2O / per-head random eviction, for MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkvc.so; PyTorch provides device memory and the stream.  The functions carry
the C ABI's names without the ``kvc_`` prefix.  There is no CPU fallback: if
the library is missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libkvc.so not found at {LIB_PATH}; build it with "
        "`python compressed_decode_attention_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------------------
# C types
# ---------------------------------------------------------------------------
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_SHAPE, ERR_WORKSPACE, ERR_HIP = range(6)
BF16, F32, FP8_E5M2 = 0, 1, 2
FLAG_FULL, FLAG_BAD_COUNT, FLAG_BAD_BLOCK = 1, 2, 4
POLICY_FULL, POLICY_STREAMING, POLICY_H2O, POLICY_RANDOM = range(4)

EXPORTED = (
    "kvc_bytes_per_token", "kvc_n_keep", "kvc_status_string", "kvc_last_error",
    "kvc_workspace_bytes", "kvc_decode_attn", "kvc_h2o_accumulate", "kvc_evict_streaming",
    "kvc_evict_h2o", "kvc_evict_random", "kvc_compact", "kvc_decode_step", "kvc_stream_read",
    "kvc_h2o_accumulate_workspace_bytes", "kvc_kivi_workspace_bytes", "kvc_kivi_prefill",
    "kvc_kivi_decode", "kvc_decode_step_noalloc",
)


class kvc_cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("pos", ctypes.c_void_p), ("n_slots", ctypes.c_void_p), ("flags", ctypes.c_void_p),
    ]


class kvc_policy(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("n_heavy", ctypes.c_int32),
        ("n_recent", ctypes.c_int32), ("prompt_len", ctypes.c_int32), ("n_keep", ctypes.c_int32),
        ("seed", ctypes.c_uint64), ("decay", ctypes.c_float),
    ]


class kvc_kivi_cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_quant", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("k_lo", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p), ("v_lo", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
        ("n_quant", ctypes.c_void_p), ("n_res", ctypes.c_void_p), ("flags", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_CP = ctypes.POINTER(kvc_cache)
_KP = ctypes.POINTER(kvc_kivi_cache)
_lib.kvc_bytes_per_token.restype = ctypes.c_size_t
_lib.kvc_bytes_per_token.argtypes = [ctypes.c_int32] * 4
_lib.kvc_n_keep.restype = ctypes.c_int64
_lib.kvc_n_keep.argtypes = [ctypes.c_int64, ctypes.c_double]
_lib.kvc_status_string.restype = ctypes.c_char_p
_lib.kvc_status_string.argtypes = [ctypes.c_int]
_lib.kvc_last_error.restype = ctypes.c_char_p
_lib.kvc_last_error.argtypes = []
_lib.kvc_workspace_bytes.restype = ctypes.c_size_t
_lib.kvc_workspace_bytes.argtypes = [_CP, ctypes.c_int32]
_lib.kvc_decode_attn.restype = ctypes.c_int
_lib.kvc_decode_attn.argtypes = [_CP, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_int32, _P, ctypes.c_size_t, _P]
_lib.kvc_h2o_accumulate.restype = ctypes.c_int
_lib.kvc_h2o_accumulate.argtypes = [_CP, _P, ctypes.c_int32, _P, _P, ctypes.c_float, _P,
                                    ctypes.c_size_t, _P]
_lib.kvc_h2o_accumulate_workspace_bytes.restype = ctypes.c_size_t
_lib.kvc_h2o_accumulate_workspace_bytes.argtypes = [_CP, ctypes.c_int32]
_lib.kvc_evict_streaming.restype = ctypes.c_int
_lib.kvc_evict_streaming.argtypes = [_CP, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
_lib.kvc_evict_h2o.restype = ctypes.c_int
_lib.kvc_evict_h2o.argtypes = [_CP, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
_lib.kvc_evict_random.restype = ctypes.c_int
_lib.kvc_evict_random.argtypes = [_CP, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64,
                                  ctypes.c_uint32, _P, _P, _P]
_lib.kvc_compact.restype = ctypes.c_int
_lib.kvc_compact.argtypes = [_CP, _P, _P, _P, _CP, _P]
_lib.kvc_decode_step.restype = ctypes.c_int
_lib.kvc_decode_step.argtypes = [_CP, ctypes.POINTER(kvc_policy), ctypes.c_uint32, _P, _P, _P,
                                 _P, _P, _P, ctypes.c_float, ctypes.c_int32, _P,
                                 ctypes.c_size_t, _P]
_lib.kvc_decode_step_noalloc.restype = ctypes.c_int
_lib.kvc_decode_step_noalloc.argtypes = [_CP, ctypes.POINTER(kvc_policy), ctypes.c_uint32, _P,
                                         _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32, _P]
_lib.kvc_stream_read.restype = ctypes.c_int
_lib.kvc_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _P]
_lib.kvc_kivi_workspace_bytes.restype = ctypes.c_size_t
_lib.kvc_kivi_workspace_bytes.argtypes = [_KP, ctypes.c_int32]
_lib.kvc_kivi_prefill.restype = ctypes.c_int
_lib.kvc_kivi_prefill.argtypes = [_KP, _P, _P, ctypes.c_int32, _P, _P]
_lib.kvc_kivi_decode.restype = ctypes.c_int
_lib.kvc_kivi_decode.argtypes = [_KP, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32, _P,
                                 ctypes.c_size_t, _P]


class KvcError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_lib.kvc_status_string(status).decode()} ({status}): {detail}")
        self.status = status


def _check(status: int):
    if status != OK:
        raise KvcError(status, _lib.kvc_last_error().decode())


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib


def status_string(s: int) -> str:
    return _lib.kvc_status_string(s).decode()


def last_error() -> str:
    return _lib.kvc_last_error().decode()


def bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(_lib.kvc_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def n_keep(n_candidates: int, keep_ratio: float) -> int:
    return int(_lib.kvc_n_keep(n_candidates, keep_ratio))


# ---------------------------------------------------------------------------
# tensors -> pointers
# ---------------------------------------------------------------------------
# cache storage per dtype (an E5M2 cache holds its codes as bytes)
_TORCH_DTYPE = {BF16: torch.bfloat16, F32: torch.float32, FP8_E5M2: torch.uint8}
# storage of q, k_new and v_new for a cache of each dtype
ACT_TORCH_DTYPE = {BF16: torch.bfloat16, F32: torch.float32, FP8_E5M2: torch.bfloat16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libkvc must be contiguous")
    return t.data_ptr()


def _req(t: Optional[torch.Tensor], name: str, cache, dtype, numel: int,
         optional: bool = False) -> Optional[int]:
    """Pointer of a tensor argument after checking that it lives on the
    cache's device with the expected dtype and element count (the library
    reads and writes exactly that many elements through the pointer)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} must not be None")
    if t.device != cache.device:
        raise ValueError(f"{name} is on {t.device}, the cache on {cache.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return _ptr(t)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class KvCache:
    """Device buffers of one cache (contiguous or paged) and its C descriptor.

    The tensors belong to this object; libkvc only reads and writes them.
    """

    def __init__(self, batch: int, q_heads: int, kv_heads: int, head_dim: int, capacity: int,
                 dtype: int = BF16, device="cuda", block_size: int = 0,
                 num_blocks: int = 0, block_table: Optional[torch.Tensor] = None):
        self.batch, self.q_heads, self.kv_heads = batch, q_heads, kv_heads
        self.head_dim, self.capacity, self.dtype = head_dim, capacity, dtype
        self.block_size = block_size
        tdt = _TORCH_DTYPE[dtype]
        if block_size:
            assert capacity % block_size == 0
            self.max_blocks = capacity // block_size
            self.num_blocks = num_blocks
            shape = (num_blocks, kv_heads, block_size, head_dim)
            if block_table is None:
                raise ValueError("paged cache needs a block table")
            self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
        else:
            self.max_blocks = 0
            self.num_blocks = 0
            shape = (batch, kv_heads, capacity, head_dim)
            self.block_table = None
        self.k = torch.zeros(shape, dtype=tdt, device=device)
        self.v = torch.zeros(shape, dtype=tdt, device=device)
        self.pos = torch.zeros((batch, kv_heads, capacity), dtype=torch.int32, device=device)
        self.n_slots = torch.zeros((batch, kv_heads), dtype=torch.int32, device=device)
        self.flags = torch.zeros((1,), dtype=torch.int32, device=device)
        self._c = None

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def device(self) -> torch.device:
        return self.k.device

    def _step_ptrs(self, new_pos, q, k_new, v_new, out, scores):
        """Checked pointers of a decode step's tensors."""
        act = ACT_TORCH_DTYPE[self.dtype]
        B, Hq, Hkv, D = self.batch, self.q_heads, self.kv_heads, self.head_dim
        return (_req(new_pos, "new_pos", self, torch.int32, B),
                _req(q, "q", self, act, B * Hq * D),
                _req(k_new, "k_new", self, act, B * Hkv * D),
                _req(v_new, "v_new", self, act, B * Hkv * D),
                _req(out, "out", self, torch.float32, B * Hq * D),
                _req(scores, "scores", self, torch.float32, B * Hkv * self.capacity,
                     optional=True))

    def _keep_ptrs(self, keep_slots, n_out):
        B, H = self.batch, self.kv_heads
        return (_req(keep_slots, "keep_slots", self, torch.int32, B * H * self.capacity),
                _req(n_out, "n_out", self, torch.int32, B * H))

    def c(self) -> kvc_cache:
        if self._c is None:
            c = kvc_cache()
            c.batch, c.q_heads, c.kv_heads = self.batch, self.q_heads, self.kv_heads
            c.head_dim, c.capacity, c.dtype = self.head_dim, self.capacity, self.dtype
            c.block_size, c.max_blocks, c.num_blocks = self.block_size, self.max_blocks, \
                self.num_blocks
            c.k, c.v = _ptr(self.k), _ptr(self.v)
            c.block_table = _ptr(self.block_table)
            c.pos, c.n_slots, c.flags = _ptr(self.pos), _ptr(self.n_slots), _ptr(self.flags)
            self._c = c
        return self._c

    def rows(self, b: int, h: int, slots):
        """(k, v) rows of unit (b, h) at the given slots (for inspection)."""
        slots = torch.as_tensor(slots, dtype=torch.long, device=self.k.device)
        if not self.block_size:
            return self.k[b, h, slots], self.v[b, h, slots]
        blk = self.block_table[b, slots // self.block_size].long()
        off = slots % self.block_size
        return self.k[blk, h, off], self.v[blk, h, off]

    def workspace_bytes(self, max_len_hint: int = 0) -> int:
        return int(_lib.kvc_workspace_bytes(ctypes.byref(self.c()), max_len_hint))

    def workspace(self, max_len_hint: int = 0) -> torch.Tensor:
        n = self.workspace_bytes(max_len_hint)
        return torch.empty((max(n, 1),), dtype=torch.uint8, device=self.k.device)

    def prompt_workspace(self, m_rows: int) -> torch.Tensor:
        """Workspace of kvc_h2o_accumulate for m_rows query rows per sequence."""
        n = int(_lib.kvc_h2o_accumulate_workspace_bytes(ctypes.byref(self.c()), m_rows))
        return torch.empty((max(n, 1),), dtype=torch.uint8, device=self.k.device)


def _policy(kind: int, n_sink=0, n_heavy=0, n_recent=0, prompt_len=0, n_keep=0, seed=0,
            decay=0.0):
    p = kvc_policy()
    p.kind, p.n_sink, p.n_heavy, p.n_recent = kind, n_sink, n_heavy, n_recent
    p.prompt_len, p.n_keep, p.seed, p.decay = prompt_len, n_keep, seed, decay
    return p


def policy_full():
    return _policy(POLICY_FULL)


def policy_streaming(n_sink=64, n_recent=448):
    return _policy(POLICY_STREAMING, n_sink=n_sink, n_recent=n_recent)


def policy_h2o(n_heavy=64, n_recent=448, decay=0.0):
    """H2O: recent window + heavy hitters by score; decay 0 sums the attention,
    0 < decay < 1 keeps a decayed attention activity instead."""
    return _policy(POLICY_H2O, n_heavy=n_heavy, n_recent=n_recent, decay=decay)


def policy_random(prompt_len, n_keep, seed=0):
    return _policy(POLICY_RANDOM, prompt_len=prompt_len, n_keep=n_keep, seed=seed)


def _scale(cache: KvCache, scale):
    return 1.0 / math.sqrt(cache.head_dim) if scale is None else float(scale)


def _ws(workspace, cache=None):
    if workspace is None:
        return None, 0
    if cache is not None and workspace.device != cache.device:
        raise ValueError(f"workspace is on {workspace.device}, the cache on {cache.device}")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def decode_attn(cache: KvCache, new_pos, q, k_new, v_new, out, scores=None, scale=None,
                max_len_hint: int = 0, workspace=None, stream=None, score_decay: float = 0.0):
    wp, wn = _ws(workspace, cache)
    pp, qp, kp, vp, op, sp = cache._step_ptrs(new_pos, q, k_new, v_new, out, scores)
    _check(_lib.kvc_decode_attn(ctypes.byref(cache.c()), pp, qp, kp, vp, op, sp,
                                _scale(cache, scale), score_decay, max_len_hint, wp, wn,
                                _stream(stream)))


def h2o_accumulate(cache: KvCache, q_rows, m_rows: int, scores, q_pos=None, scale=None,
                   stream=None, workspace=None):
    """Add the group-summed softmax probabilities of m_rows query rows per
    sequence (causal when q_pos is given) to the scores.  The workspace holds
    one fp32 log-sum-exp per row and head; it is allocated here if not given."""
    if workspace is None:
        workspace = cache.prompt_workspace(m_rows)
    wp, wn = _ws(workspace, cache)
    B, Hq, D = cache.batch, cache.q_heads, cache.head_dim
    qr = _req(q_rows, "q_rows", cache, ACT_TORCH_DTYPE[cache.dtype], B * m_rows * Hq * D)
    qpp = _req(q_pos, "q_pos", cache, torch.int32, B * m_rows, optional=True)
    sp = _req(scores, "scores", cache, torch.float32, B * cache.kv_heads * cache.capacity)
    _check(_lib.kvc_h2o_accumulate(ctypes.byref(cache.c()), qr, m_rows, qpp, sp,
                                   _scale(cache, scale), wp, wn, _stream(stream)))


def evict_streaming(cache: KvCache, n_sink: int, n_recent: int, keep_slots, n_out, stream=None):
    kp, np_ = cache._keep_ptrs(keep_slots, n_out)
    _check(_lib.kvc_evict_streaming(ctypes.byref(cache.c()), n_sink, n_recent, kp, np_,
                                    _stream(stream)))


def evict_h2o(cache: KvCache, scores, n_heavy: int, n_recent: int, keep_slots, n_out,
              stream=None):
    kp, np_ = cache._keep_ptrs(keep_slots, n_out)
    sp = _req(scores, "scores", cache, torch.float32,
              cache.batch * cache.kv_heads * cache.capacity)
    _check(_lib.kvc_evict_h2o(ctypes.byref(cache.c()), sp, n_heavy, n_recent, kp, np_,
                              _stream(stream)))


def evict_random(cache: KvCache, prompt_len: int, n_keep: int, seed: int, step: int, keep_slots,
                 n_out, stream=None):
    kp, np_ = cache._keep_ptrs(keep_slots, n_out)
    _check(_lib.kvc_evict_random(ctypes.byref(cache.c()), prompt_len, n_keep, seed, step, kp,
                                 np_, _stream(stream)))


def compact(cache: KvCache, keep_slots, n_out, scores=None, ordered_dst: Optional[KvCache] = None,
            stream=None):
    dst = ctypes.byref(ordered_dst.c()) if ordered_dst is not None else None
    if ordered_dst is not None and ordered_dst.device != cache.device:
        raise ValueError(f"ordered_dst is on {ordered_dst.device}, the cache on {cache.device}")
    kp, np_ = cache._keep_ptrs(keep_slots, n_out)
    sp = _req(scores, "scores", cache, torch.float32,
              cache.batch * cache.kv_heads * cache.capacity, optional=True)
    _check(_lib.kvc_compact(ctypes.byref(cache.c()), kp, np_, sp, dst, _stream(stream)))


def decode_step(cache: KvCache, policy: kvc_policy, step: int, new_pos, q, k_new, v_new, out,
                scores=None, scale=None, max_len_hint: int = 0, workspace=None, stream=None):
    wp, wn = _ws(workspace, cache)
    pp, qp, kp, vp, op, sp = cache._step_ptrs(new_pos, q, k_new, v_new, out, scores)
    _check(_lib.kvc_decode_step(ctypes.byref(cache.c()), ctypes.byref(policy), step, pp, qp, kp,
                                vp, op, sp, _scale(cache, scale), max_len_hint, wp, wn,
                                _stream(stream)))


NOALLOC_SCRATCH_BYTES = 128 << 20   # KVC_NOALLOC_SCRATCH_BYTES of kvc.h


def decode_step_noalloc(cache: KvCache, policy: kvc_policy, step: int, new_pos, q, k_new, v_new,
                        out, scores=None, scale=None, max_len_hint: int = 0, stream=None):
    """decode_step without a workspace: the library's static per-GPU scratch
    (calls that overlap on one GPU race)."""
    pp, qp, kp, vp, op, sp = cache._step_ptrs(new_pos, q, k_new, v_new, out, scores)
    _check(_lib.kvc_decode_step_noalloc(ctypes.byref(cache.c()), ctypes.byref(policy), step, pp,
                                        qp, kp, vp, op, sp, _scale(cache, scale), max_len_hint,
                                        _stream(stream)))


def stream_read(buf, sink, nbytes: Optional[int] = None, stream=None):
    """Read `nbytes` (default: all) of device tensor `buf` once with the
    library's streaming kernel; `sink` is a one-element int32/uint32 device
    tensor that is written only for an impossible data pattern."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(_lib.kvc_stream_read(_ptr(buf), n, _ptr(sink), _stream(stream)))


# ---------------------------------------------------------------------------
# KIVI-style quantized cache
# ---------------------------------------------------------------------------
KIVI_GROUP, KIVI_RESIDUAL = 32, 128


class KiviCache:
    """Device buffers of a KIVI-style quantized cache (layout of kvc.h) and
    its C descriptor; max_quant quantized tokens per (sequence, kv head)."""

    def __init__(self, batch: int, q_heads: int, kv_heads: int, head_dim: int, max_quant: int,
                 bits: int = 4, device="cuda"):
        self.batch, self.q_heads, self.kv_heads = batch, q_heads, kv_heads
        self.head_dim, self.max_quant, self.bits = head_dim, max_quant, bits
        U, T, D = batch * kv_heads, max_quant, head_dim
        row = D * bits // 8
        self.k_codes = torch.zeros((U, T, row), dtype=torch.uint8, device=device)
        # 16-token tiles of 1,024 bytes (kvc.h): the same bytes as T rows of 64
        self.v_codes = torch.zeros((U, T // 16, 16 * row), dtype=torch.uint8, device=device)
        self.k_scale = torch.zeros((U, T // KIVI_GROUP, D), dtype=torch.float32, device=device)
        self.k_lo = torch.zeros_like(self.k_scale)
        self.v_scale = torch.zeros((U, T, D // 32), dtype=torch.float32, device=device)
        self.v_lo = torch.zeros_like(self.v_scale)
        self.k_res = torch.zeros((U, KIVI_RESIDUAL, D), dtype=torch.bfloat16, device=device)
        self.v_res = torch.zeros_like(self.k_res)
        self.n_quant = torch.zeros((batch, kv_heads), dtype=torch.int32, device=device)
        self.n_res = torch.zeros((batch, kv_heads), dtype=torch.int32, device=device)
        self.flags = torch.zeros((1,), dtype=torch.int32, device=device)
        self._c = None

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def device(self) -> torch.device:
        return self.k_codes.device

    def c(self) -> kvc_kivi_cache:
        if self._c is None:
            c = kvc_kivi_cache()
            c.batch, c.q_heads, c.kv_heads = self.batch, self.q_heads, self.kv_heads
            c.head_dim, c.max_quant, c.bits = self.head_dim, self.max_quant, self.bits
            for name in ("k_codes", "v_codes", "k_scale", "k_lo", "v_scale", "v_lo", "k_res",
                         "v_res", "n_quant", "n_res", "flags"):
                setattr(c, name, _ptr(getattr(self, name)))
            self._c = c
        return self._c

    def workspace_bytes(self, max_quant_hint: int = 0) -> int:
        return int(_lib.kvc_kivi_workspace_bytes(ctypes.byref(self.c()), max_quant_hint))

    def workspace(self, max_quant_hint: int = 0) -> torch.Tensor:
        n = self.workspace_bytes(max_quant_hint)
        return torch.empty((max(n, 1),), dtype=torch.uint8, device=self.k_codes.device)


def kivi_prefill(cache: KiviCache, k, v, lengths, stream=None):
    """k, v [batch, kv_heads, max_len, head_dim] bf16; lengths [batch] int32 (device)."""
    max_len = k.shape[2]
    n = cache.batch * cache.kv_heads * max_len * cache.head_dim
    kp = _req(k, "k", cache, torch.bfloat16, n)
    vp = _req(v, "v", cache, torch.bfloat16, n)
    lp = _req(lengths, "lengths", cache, torch.int32, cache.batch)
    _check(_lib.kvc_kivi_prefill(ctypes.byref(cache.c()), kp, vp, max_len, lp, _stream(stream)))


def kivi_decode(cache: KiviCache, q, k_new, v_new, out, scale=None, max_quant_hint: int = 0,
                workspace=None, stream=None):
    if workspace is None:
        workspace = cache.workspace(max_quant_hint)
    wp, wn = _ws(workspace, cache)
    sc = 1.0 / math.sqrt(cache.head_dim) if scale is None else float(scale)
    B, Hq, Hkv, D = cache.batch, cache.q_heads, cache.kv_heads, cache.head_dim
    qp = _req(q, "q", cache, torch.bfloat16, B * Hq * D)
    kp = _req(k_new, "k_new", cache, torch.bfloat16, B * Hkv * D)
    vp = _req(v_new, "v_new", cache, torch.bfloat16, B * Hkv * D)
    op = _req(out, "out", cache, torch.float32, B * Hq * D)
    _check(_lib.kvc_kivi_decode(ctypes.byref(cache.c()), qp, kp, vp, op, sc, max_quant_hint, wp,
                                wn, _stream(stream)))
