"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import verify_step_amd as msk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msk.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(msk_[a-z_]+)\s*\(", text,
                                 re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("msk_attn_step", "msk_moe_route", "msk_expert_ffn", "msk_layer_step",
              "msk_workspace_size", "msk_last_error", "msk_abi_version", "msk_workspace_status"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = msk.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", msk.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (msk_\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert getattr(L, n) is not None
    assert L.msk_abi_version() == 1


def _spec(**kw):
    s = dict(hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=32, n_experts=16, top_k=2,
             ffn_dim=128, window=128, rms_eps=1e-6, softmax_shift=10.0, dense_dtype="f32",
             expert_dtype="f32", kv_dtype="f32")
    s.update(kw)
    return s


def test_workspace_size_scales_with_context():
    a = msk.workspace_size(_spec(window=0), [100], 1)
    b = msk.workspace_size(_spec(window=0), [1 << 20], 4)
    assert 0 < a < b


@pytest.mark.parametrize("bad,status", [
    (dict(n_q_heads=6, n_kv_heads=4), 1),
    (dict(top_k=17, n_experts=16), 1),
    (dict(window=-1), 1),
    (dict(head_dim=48), 2),
    (dict(hidden=100), 2),
    (dict(kv_dtype="nvfp4"), 2),
    (dict(dense_dtype="e4m3"), 2),
    (dict(rms_eps=0.0), 1),
    (dict(n_experts=300, top_k=2), 2),
    (dict(head_dim=128, n_q_heads=8, n_kv_heads=2), 2),   # fp32 cache at head_dim 128
])
def test_workspace_size_rejects_bad_config(bad, status):
    with pytest.raises(msk.MskError) as e:
        msk.workspace_size(_spec(**bad), [10], 1)
    assert msk.last_error()


def test_batch_limits():
    with pytest.raises(msk.MskError):
        msk.workspace_size(_spec(), [10] * 65, 1)
    with pytest.raises(msk.MskError):
        msk.workspace_size(_spec(), [10] * 8, 9)         # 72 tokens
    with pytest.raises(msk.MskError):
        msk.workspace_size(_spec(), [-1], 1)


def _call_attn(cfg, kv_cap, kv_len, ws_bytes, null_x=False):
    L = msk.lib()
    w = msk.LayerWeights(*([ctypes.c_void_p(16)] * 18))
    kv = msk.KV(ctypes.c_void_p(16), ctypes.c_void_p(16), kv_cap)
    b = msk.make_batch(kv_len, 1)
    x = None if null_x else ctypes.c_void_p(32)
    return L.msk_attn_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(b),
                           x, ctypes.c_void_p(64), None, None, ctypes.c_void_p(128), ws_bytes,
                           None)


def test_entry_points_validate_before_enqueue():
    # none of these may reach the GPU: each must fail on the host first
    cfg = msk.make_cfg(_spec())
    assert _call_attn(cfg, 10, [10], 1 << 30) == 1          # kv_len + 1 > cap
    assert "cap" in msk.last_error()
    assert _call_attn(cfg, 100, [10], 1 << 30, null_x=True) == 1
    assert _call_attn(cfg, 100, [10], 16) == 3               # workspace too small
    bad = msk.make_cfg(_spec(head_dim=40))
    assert _call_attn(bad, 100, [10], 1 << 30) == 2
    L = msk.lib()
    w = msk.LayerWeights(*([None] * 18))
    assert L.msk_moe_route(ctypes.byref(cfg), ctypes.byref(w), 1, ctypes.c_void_p(8),
                           ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8), None,
                           ctypes.c_void_p(8), 1 << 30, None) == 1
    assert L.msk_expert_ffn(ctypes.byref(cfg), ctypes.byref(w), 0, None, None, None, None, None,
                            None, 0, None) == 1
    assert L.msk_layer_step(None, None, None, 1, None, None, None, None, None, None, 0, None) == 1
    cfgs = (msk.LayerCfg * 5)(*([cfg] * 5))
    ws_ = (msk.LayerWeights * 5)()
    kvs = (msk.KV * 5)()
    b = msk.make_batch([10], 1)
    assert L.msk_layer_step(cfgs, ws_, kvs, 5, ctypes.byref(b), ctypes.c_void_p(8), None, None,
                            None, ctypes.c_void_p(8), 1 << 30, None) == 1
    # NVFP4 experts without their scales
    c4 = msk.make_cfg(_spec(expert_dtype="nvfp4"))
    w4 = msk.LayerWeights(*([ctypes.c_void_p(16)] * 12 + [None] * 6))
    assert L.msk_expert_ffn(ctypes.byref(c4), ctypes.byref(w4), 1, ctypes.c_void_p(8),
                            ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8),
                            ctypes.c_void_p(8), ctypes.c_void_p(8), 1 << 30, None) == 1
    assert "scales" in msk.last_error()


def test_misaligned_pointers_are_argument_errors():
    # 16-byte weights and caches, 4-byte NVFP4 scale arrays; checked on the
    # host before anything is enqueued
    L = msk.lib()
    cfg = msk.make_cfg(_spec())
    b = msk.make_batch([10], 1)
    ptrs = [ctypes.c_void_p(256)] * 18
    ptrs[4] = ctypes.c_void_p(264)                          # wq 8-byte aligned
    w = msk.LayerWeights(*ptrs)
    kv = msk.KV(ctypes.c_void_p(256), ctypes.c_void_p(256), 100)
    assert L.msk_attn_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(b),
                           ctypes.c_void_p(32), ctypes.c_void_p(64), None, None,
                           ctypes.c_void_p(128), 1 << 30, None) == 1
    assert "aligned" in msk.last_error()
    w = msk.LayerWeights(*([ctypes.c_void_p(256)] * 18))
    kv = msk.KV(ctypes.c_void_p(260), ctypes.c_void_p(256), 100)
    assert L.msk_attn_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(b),
                           ctypes.c_void_p(32), ctypes.c_void_p(64), None, None,
                           ctypes.c_void_p(128), 1 << 30, None) == 1
    assert "aligned" in msk.last_error()
    c4 = msk.make_cfg(_spec(expert_dtype="nvfp4"))
    ptrs = [ctypes.c_void_p(256)] * 18
    ptrs[12] = ctypes.c_void_p(258)                         # s_gate 2-byte aligned
    w4 = msk.LayerWeights(*ptrs)
    assert L.msk_expert_ffn(ctypes.byref(c4), ctypes.byref(w4), 1, ctypes.c_void_p(8),
                            ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8),
                            ctypes.c_void_p(8), ctypes.c_void_p(8), 1 << 30, None) == 1
    assert "aligned" in msk.last_error()


def test_noalloc_rejects_a_step_larger_than_its_scratch():
    """The allocation-free step refuses, before anything is enqueued, a step
    whose workspace exceeds the per-GPU scratch array (host-side check)."""
    big = _spec(hidden=65536, n_experts=16, top_k=16, ffn_dim=128)
    n = msk.workspace_size(big, [10] * 8, 8)
    assert n > msk.noalloc_scratch_bytes() == 64 << 20
    fake = ctypes.c_void_p(1 << 20)           # never dereferenced: rejected first
    cfg = msk.make_cfg(big)
    w = msk.LayerWeights(*([fake.value] * len(msk._WEIGHT_FIELDS)))
    kv = msk.KV(fake.value, fake.value, 64)
    b = msk.make_batch([10] * 8, 8)
    st = msk.lib().msk_layer_step_noalloc(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), 1,
                                          ctypes.byref(b), fake, None, None, None, None)
    assert st == 3, msk.last_error()
    assert "scratch" in msk.last_error()


def test_prefill_validates_before_enqueue():
    """msk_moe_prefill: sizes, token counts and expert formats are checked on
    the host; nothing is dereferenced (all pointers fake) when they fail."""
    L = msk.lib()
    ok = _spec(hidden=256, ffn_dim=128, expert_dtype="bf16", dense_dtype="bf16")
    assert L.msk_moe_prefill_workspace_size(ctypes.byref(msk.make_cfg(ok)), 100) > 0
    for bad, n, status in [(ok, 0, 1), (ok, 8193, 1), (dict(ok, expert_dtype="f32"), 4, 2),
                           (dict(ok, ffn_dim=96), 4, 2)]:
        cfg = msk.make_cfg(bad)
        assert L.msk_moe_prefill_workspace_size(ctypes.byref(cfg), n) == 0
        fake = ctypes.c_void_p(1 << 20)
        w = msk.LayerWeights(*([fake.value] * len(msk._WEIGHT_FIELDS)))
        st = L.msk_moe_prefill(ctypes.byref(cfg), ctypes.byref(w), n, fake, fake, fake, fake, fake,
                               fake, 1 << 40, None)
        assert st == status, msk.last_error()
