"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, its host-only helpers agree with the oracle, and argument errors
are reported before anything is enqueued (no compute call is made here)."""
import ctypes
import os
import re

import pytest
import torch

import compressed_decode_attention_amd as kvc
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="fake device pointers are only used where no GPU exists")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", text)))


def test_library_is_the_in_tree_hip_build():
    assert os.path.dirname(kvc.LIB_PATH) == os.path.join(ROOT, "compressed_decode_attention_amd")
    with open(kvc.LIB_PATH, "rb") as f:
        blob = f.read()
    # the shared object carries gfx950 device code
    assert b"gfx950" in blob


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    lib = kvc.library()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(kvc.EXPORTED) == names


def test_bytes_per_token_matches_oracle():
    for args in [(1, 8, 128, 2), (80, 8, 128, 2), (16, 4, 64, 4), (0, 8, 128, 2), (3, -1, 8, 2),
                 (64, 32, 256, 1)]:
        assert kvc.bytes_per_token(*args) == oracle.bytes_per_token(*args)


def test_n_keep_matches_oracle():
    for N in [0, 1, 3, 7, 100, 101, 16384, 99999]:
        for r in [0.0, 0.1, 0.25, 0.29, 0.5, 0.75, 0.999, 1.0, 1.5]:
            assert kvc.n_keep(N, r) == oracle.n_keep(N, r), (N, r)


def test_status_strings():
    for s in range(6):
        assert kvc.status_string(s)
    assert kvc.status_string(99) == "unknown status"


def _fake_cache(**kw):
    c = kvc.kvc_cache()
    c.batch, c.q_heads, c.kv_heads, c.head_dim, c.capacity, c.dtype = 2, 8, 2, 128, 64, kvc.BF16
    c.k, c.v, c.pos, c.n_slots = 0x10000, 0x20000, 0x30000, 0x40000
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _attn(c, ws=None, nbytes=0, **kw):
    args = dict(new_pos=0x1000, q=0x2000, k_new=0x3000, v_new=0x4000, out=0x5000, scores=None,
                scale=0.088, decay=0.0)
    args.update(kw)
    return kvc.library().kvc_decode_attn(ctypes.byref(c) if c is not None else None,
                                         args["new_pos"], args["q"], args["k_new"],
                                         args["v_new"], args["out"], args["scores"],
                                         args["scale"], args["decay"], 0, ws, nbytes, None)


@no_gpu
@pytest.mark.parametrize("change,status", [
    (dict(q_heads=9), kvc.ERR_SHAPE),
    (dict(head_dim=96), kvc.ERR_UNSUPPORTED),
    (dict(q_heads=34), kvc.ERR_UNSUPPORTED),          # group of 17
    (dict(dtype=7), kvc.ERR_UNSUPPORTED),
    (dict(capacity=0), kvc.ERR_INVALID_ARG),
    (dict(capacity=70000), kvc.ERR_UNSUPPORTED),
    (dict(batch=1 << 23, kv_heads=4, q_heads=8), kvc.ERR_UNSUPPORTED),   # 2^25 units
    (dict(k=None), kvc.ERR_INVALID_ARG),
    (dict(k=0x10008), kvc.ERR_INVALID_ARG),          # misaligned
    (dict(block_size=16, block_table=0x50000, max_blocks=3, num_blocks=10), kvc.ERR_SHAPE),
    (dict(block_size=16, block_table=None, max_blocks=4, num_blocks=10), kvc.ERR_INVALID_ARG),
])
def test_cache_validation_errors(change, status):
    assert _attn(_fake_cache(**change)) == status
    assert kvc.last_error()


@no_gpu
def test_attention_argument_errors():
    assert _attn(None) == kvc.ERR_INVALID_ARG
    assert _attn(_fake_cache(), q=None) == kvc.ERR_INVALID_ARG
    assert _attn(_fake_cache(), scale=float("inf")) == kvc.ERR_INVALID_ARG
    for bad in (1.0, -0.5, float("nan"), 2.0):
        assert _attn(_fake_cache(), decay=bad) == kvc.ERR_INVALID_ARG
    assert b"score_decay" in kvc.library().kvc_last_error()
    # workspace required but missing / too small
    assert _attn(_fake_cache()) == kvc.ERR_WORKSPACE
    need = kvc.library().kvc_workspace_bytes(ctypes.byref(_fake_cache()), 0)
    assert need > 0
    assert _attn(_fake_cache(), ws=0x100000, nbytes=need - 1) == kvc.ERR_WORKSPACE
    assert _attn(_fake_cache(), ws=0x100010, nbytes=need) == kvc.ERR_WORKSPACE  # misaligned
    # q, k_new, v_new and out are read and written in 16-byte pieces
    for name, addr in (("q", 0x2008), ("k_new", 0x3004), ("v_new", 0x4002), ("out", 0x5004)):
        assert _attn(_fake_cache(), ws=0x100000, nbytes=need, **{name: addr}) == \
            kvc.ERR_INVALID_ARG, name
        assert b"16-byte aligned" in kvc.library().kvc_last_error()


@no_gpu
def test_noalloc_step_rejects_caches_beyond_its_static_scratch():
    lib = kvc.library()
    pol = kvc.policy_streaming()
    # batch 512 x 8 kv heads at capacity 65,536: gigabytes of fallback scratch
    big = _fake_cache(batch=512, q_heads=64, kv_heads=8, capacity=65536)
    need = lib.kvc_workspace_bytes(ctypes.byref(big), 0)
    assert need > kvc.NOALLOC_SCRATCH_BYTES
    assert lib.kvc_decode_step_noalloc(ctypes.byref(big), ctypes.byref(pol), 1, 0x1000, 0x2000,
                                       0x3000, 0x4000, 0x5000, None, 0.1, 0, None) == \
        kvc.ERR_WORKSPACE
    assert b"static scratch" in lib.kvc_last_error()
    # argument errors come first, as for kvc_decode_step
    assert lib.kvc_decode_step_noalloc(ctypes.byref(_fake_cache()), ctypes.byref(pol), 1, 0x1000,
                                       None, 0x3000, 0x4000, 0x5000, None, 0.1, 0, None) == \
        kvc.ERR_INVALID_ARG
    h2o = kvc.policy_h2o()
    assert lib.kvc_decode_step_noalloc(ctypes.byref(_fake_cache()), ctypes.byref(h2o), 1, 0x1000,
                                       0x2000, 0x3000, 0x4000, 0x5000, None, 0.1, 0, None) == \
        kvc.ERR_INVALID_ARG


def test_binding_checks_tensor_dtype_and_size_before_the_call():
    # host tensors stand in for device ones: the checks run before any call
    c = kvc.KvCache(2, 8, 2, 128, 16, kvc.BF16, device="cpu")
    B, Hq, Hkv, D = 2, 8, 2, 128
    pos = torch.zeros(B, dtype=torch.int32)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16)
    kn = torch.zeros((B, Hkv, D), dtype=torch.bfloat16)
    out = torch.zeros((B, Hq, D), dtype=torch.float32)
    bad = [
        dict(q=q.float()),                                    # wrong dtype
        dict(q=q[:1]),                                        # too few elements
        dict(out=out.to(torch.bfloat16)),                     # a bf16 out would be overrun
        dict(new_pos=pos.long()),
        dict(k_new=torch.zeros((B, Hkv, D + 8), dtype=torch.bfloat16)),
        dict(scores=torch.zeros((B, Hkv, 8))),                # shorter than the capacity
    ]
    for change in bad:
        args = dict(new_pos=pos, q=q, k_new=kn, v_new=kn, out=out, scores=None)
        args.update(change)
        with pytest.raises(ValueError):
            kvc.decode_step(c, kvc.policy_streaming(), 1, args["new_pos"], args["q"],
                            args["k_new"], args["v_new"], args["out"], args["scores"])
    keep = torch.zeros((B, Hkv, 16), dtype=torch.int32)
    with pytest.raises(ValueError):
        kvc.evict_streaming(c, 4, 4, keep, torch.zeros((B, Hkv), dtype=torch.int64))
    with pytest.raises(ValueError):
        kvc.evict_streaming(c, 4, 4, keep[:, :, :8].contiguous(), torch.zeros((B, Hkv),
                                                                               dtype=torch.int32))


@no_gpu
def test_policy_and_selection_errors():
    lib = kvc.library()
    c = _fake_cache()
    assert lib.kvc_evict_h2o(ctypes.byref(c), None, 64, 448, 0x1000, 0x2000, None) == \
        kvc.ERR_INVALID_ARG
    assert lib.kvc_evict_h2o(ctypes.byref(c), 0x3000, -1, 448, 0x1000, 0x2000, None) == \
        kvc.ERR_INVALID_ARG
    assert lib.kvc_evict_random(ctypes.byref(c), 10, -5, 0, 0, 0x1000, 0x2000, None) == \
        kvc.ERR_INVALID_ARG
    assert lib.kvc_evict_streaming(ctypes.byref(c), 4, 8, None, 0x2000, None) == \
        kvc.ERR_INVALID_ARG
    assert lib.kvc_compact(ctypes.byref(c), 0x1000, None, None, None, None) == \
        kvc.ERR_INVALID_ARG
    d = _fake_cache(head_dim=64)
    assert lib.kvc_compact(ctypes.byref(c), 0x1000, 0x2000, None, ctypes.byref(d), None) == \
        kvc.ERR_SHAPE
    pol = kvc.policy_h2o()
    ws = 0x1000000
    need = lib.kvc_workspace_bytes(ctypes.byref(c), 0)
    assert lib.kvc_decode_step(ctypes.byref(c), ctypes.byref(pol), 1, 0x1, 0x2000, 0x3000, 0x4000,
                               0x5000, None, 0.1, 0, ws, need, None) == kvc.ERR_INVALID_ARG
    bad = kvc._policy(9)
    assert lib.kvc_decode_step(ctypes.byref(c), ctypes.byref(bad), 1, 0x1, 0x2000, 0x3000, 0x4000,
                               0x5000, None, 0.1, 0, ws, need, None) == kvc.ERR_INVALID_ARG
    for decay in (1.0, -0.1, float("nan")):
        pd = kvc.policy_h2o(decay=decay)
        assert lib.kvc_decode_step(ctypes.byref(c), ctypes.byref(pd), 1, 0x1, 0x2000, 0x3000,
                                   0x4000, 0x5000, 0x6000, 0.1, 0, ws, need, None) == \
            kvc.ERR_INVALID_ARG
        assert b"decay" in lib.kvc_last_error()
    assert lib.kvc_h2o_accumulate(ctypes.byref(c), 0x1000, -1, None, 0x2000, 0.1, None, 0,
                                  None) == kvc.ERR_INVALID_ARG
    assert lib.kvc_h2o_accumulate(ctypes.byref(c), 0x1000, 0, None, 0x2000, 0.1, None, 0,
                                  None) == kvc.OK
    # bf16 / head_dim 128 runs on the matrix cores and needs one fp32 per row and head
    need = lib.kvc_h2o_accumulate_workspace_bytes(ctypes.byref(c), 10)
    assert need >= c.batch * c.kv_heads * 10 * (c.q_heads // c.kv_heads) * 4
    assert lib.kvc_h2o_accumulate(ctypes.byref(c), 0x1000, 10, None, 0x2000, 0.1, None, 0,
                                  None) == kvc.ERR_WORKSPACE
    assert lib.kvc_h2o_accumulate(ctypes.byref(c), 0x1008, 10, None, 0x2000, 0.1, 0x100000,
                                  need, None) == kvc.ERR_INVALID_ARG   # q_rows misaligned
    assert lib.kvc_h2o_accumulate_workspace_bytes(ctypes.byref(_fake_cache(dtype=kvc.F32)),
                                                  10) == 0


def test_workspace_grows_with_the_split():
    lib = kvc.library()
    small = lib.kvc_workspace_bytes(ctypes.byref(_fake_cache(batch=1024, capacity=513)), 513)
    big = lib.kvc_workspace_bytes(ctypes.byref(_fake_cache(batch=2, capacity=8192)), 8192)
    assert small > 0 and big > 0
    assert lib.kvc_workspace_bytes(None, 0) == 0


@no_gpu
def test_stream_read_argument_errors():
    lib = kvc.library()
    assert lib.kvc_stream_read(None, 1024, 0x20000, None) == kvc.ERR_INVALID_ARG
    assert lib.kvc_stream_read(0x10000, 1024, None, None) == kvc.ERR_INVALID_ARG
    assert lib.kvc_stream_read(0x10008, 1024, 0x20000, None) == kvc.ERR_INVALID_ARG  # misaligned
    assert lib.kvc_stream_read(0x10000, 1000, 0x20000, None) == kvc.ERR_INVALID_ARG  # not x16
    assert lib.kvc_stream_read(0x10000, 0, 0x20000, None) == kvc.ERR_INVALID_ARG
    assert b"16-byte aligned" in lib.kvc_last_error()


def _fake_kivi(**kw):
    c = kvc.kvc_kivi_cache()
    c.batch, c.q_heads, c.kv_heads, c.head_dim, c.max_quant, c.bits = 2, 8, 2, 128, 256, 4
    for i, name in enumerate(("k_codes", "v_codes", "k_scale", "k_lo", "v_scale", "v_lo", "k_res",
                              "v_res", "n_quant", "n_res")):
        setattr(c, name, 0x100000 * (i + 1))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@no_gpu
@pytest.mark.parametrize("change,status", [
    (dict(head_dim=64), kvc.ERR_UNSUPPORTED),
    (dict(bits=2), kvc.ERR_UNSUPPORTED),
    (dict(q_heads=18), kvc.ERR_UNSUPPORTED),        # group of 9
    (dict(q_heads=9), kvc.ERR_SHAPE),
    (dict(max_quant=100), kvc.ERR_SHAPE),
    (dict(max_quant=-32), kvc.ERR_INVALID_ARG),
    (dict(k_res=None), kvc.ERR_INVALID_ARG),
    (dict(v_codes=0x100008), kvc.ERR_INVALID_ARG),  # misaligned
    (dict(batch=1 << 23, kv_heads=4, q_heads=8), kvc.ERR_UNSUPPORTED),   # 2^25 units
])
def test_kivi_cache_validation(change, status):
    lib = kvc.library()
    c = _fake_kivi(**change)
    ws = 0x4000000
    assert lib.kvc_kivi_decode(ctypes.byref(c), 0x1000, 0x2000, 0x3000, 0x4000, 0.1, 0, ws,
                               1 << 30, None) == status
    assert lib.kvc_kivi_workspace_bytes(ctypes.byref(c), 0) == 0
    assert kvc.last_error()


@no_gpu
def test_kivi_call_errors():
    lib = kvc.library()
    c = _fake_kivi()
    need = lib.kvc_kivi_workspace_bytes(ctypes.byref(c), 0)
    assert need > 0
    # workspace missing, short, misaligned; bad scale; NULL activations
    assert lib.kvc_kivi_decode(ctypes.byref(c), 0x1000, 0x2000, 0x3000, 0x4000, 0.1, 0, None, 0,
                               None) == kvc.ERR_WORKSPACE
    assert lib.kvc_kivi_decode(ctypes.byref(c), 0x1000, 0x2000, 0x3000, 0x4000, 0.1, 0,
                               0x4000000, need - 1, None) == kvc.ERR_WORKSPACE
    assert lib.kvc_kivi_decode(ctypes.byref(c), 0x1000, 0x2000, 0x3000, 0x4000, 0.1, 0,
                               0x4000010, need, None) == kvc.ERR_WORKSPACE
    assert lib.kvc_kivi_decode(ctypes.byref(c), 0x1000, 0x2000, 0x3000, 0x4000,
                               float("nan"), 0, 0x4000000, need, None) == kvc.ERR_INVALID_ARG
    assert lib.kvc_kivi_decode(ctypes.byref(c), None, 0x2000, 0x3000, 0x4000, 0.1, 0,
                               0x4000000, need, None) == kvc.ERR_INVALID_ARG
    # prefill: 256 quantized slots hold prompts up to 384 tokens
    assert lib.kvc_kivi_prefill(ctypes.byref(c), 0x1000, 0x2000, 385, 0x3000, None) == \
        kvc.ERR_SHAPE
    assert b"max_quant" in lib.kvc_last_error()
    assert lib.kvc_kivi_prefill(ctypes.byref(c), 0x1000, 0x2000, 100, None, None) == \
        kvc.ERR_INVALID_ARG
    assert lib.kvc_kivi_prefill(ctypes.byref(c), 0x1000, 0x2000, -1, 0x3000, None) == \
        kvc.ERR_INVALID_ARG
    assert lib.kvc_kivi_prefill(None, 0x1000, 0x2000, 10, 0x3000, None) == kvc.ERR_INVALID_ARG


def test_kivi_workspace_grows_with_the_split():
    lib = kvc.library()
    small = lib.kvc_kivi_workspace_bytes(ctypes.byref(_fake_kivi(batch=512, max_quant=2048)), 0)
    few = lib.kvc_kivi_workspace_bytes(ctypes.byref(_fake_kivi(batch=1, max_quant=2048)), 0)
    assert small > 0 and few > 0
    # a bound of one group gives one split per unit
    one = lib.kvc_kivi_workspace_bytes(ctypes.byref(_fake_kivi(batch=1, max_quant=2048)), 32)
    assert one < few
