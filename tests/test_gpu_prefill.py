"""GPU parity of the prefill expert FFN (msk_moe_prefill, through the C ABI)
against the oracle's expert FFN on the same seeded inputs: many tokens, the
slots grouped by expert into chunks of up to 160 (NVFP4 experts) or 128
(bf16 experts) for the matrix cores (inputs
as fp16 with a power of two per row for NVFP4 experts, bf16 for bf16
experts).  Same tolerance as the other bf16/fp4 paths: the MoE delta out - h
within 2e-2 of its RMS (plus one fp32 ulp of out)."""
import numpy as np
import pytest
import torch

import synth
import verify_step_amd as msk
from oracle import layer as ol
from parity_util import LOWP_TOL, assert_close, fp32_store_floor

pytestmark = pytest.mark.gpu

_SMALL = dict(hidden=512, n_q_heads=12, n_kv_heads=2, head_dim=128, n_experts=32, top_k=8,
              ffn_dim=256)
# five k-tiles of the gate/up product and three of the down product (an odd
# count ends the two-tile pipeline early); the down product's last 256-row
# block has 128 rows, so two of its four waves hold no rows
_ODD = dict(_SMALL, hidden=640, ffn_dim=384)


def _layer(expert, dims):
    p = synth.make_problem("decode-bf16", device="cuda",
                           overrides=dict(dims=dims, expert=expert, kv_len=[64], windows=[128]))
    return p.specs[0], p.weights[0]


def _inputs(spec, T, seed, routing="random"):
    g = torch.Generator(device="cuda").manual_seed(seed)
    H, E, K = spec["hidden"], spec["n_experts"], spec["top_k"]
    u = torch.randn((T, H), generator=g, device="cuda")
    h = torch.randn((T, H), generator=g, device="cuda")
    if routing == "random":      # k distinct experts per token
        idx = torch.argsort(torch.rand((T, E), generator=g, device="cuda"), dim=1)[:, :K]
    elif routing == "skewed":    # every token to experts 0..k-1: blocks of 64, 64, ..., ragged
        idx = torch.arange(K, device="cuda").repeat(T, 1)
    else:                        # repeats within a token: expert j % 3 in slot j
        idx = (torch.arange(K, device="cuda") % 3).repeat(T, 1)
    wts = torch.softmax(torch.randn((T, K), generator=g, device="cuda"), dim=1)
    return u, h, idx.to(torch.int32).contiguous(), wts.contiguous()


def _oracle(spec, w, u, h, idx, wts, rows=None):
    sel = slice(None) if rows is None else rows
    return ol.expert_ffn(spec, synth.host_weights(w), u[sel].double().cpu().numpy(),
                         idx[sel].cpu().numpy(), wts[sel].double().cpu().numpy(),
                         h[sel].double().cpu().numpy())


def _check(name, out, h, ref, rows=None):
    sel = slice(None) if rows is None else rows
    got = out[sel].double().cpu().numpy()
    h0 = h[sel].double().cpu().numpy()
    assert_close(f"{name} moe delta", got - h0, ref - h0, LOWP_TOL, fp32_store_floor(ref))


# slots per expert: random 300 -> about 75 (chunks of 5 to 8 16-slot tiles),
# 200 -> 50 (4 tiles), 100 -> 25 (2), 1 -> 1; skewed T -> T for each of 8
# experts: 300 -> two NVFP4 chunks of 150 (ten tiles, the last one ragged),
# 160 -> one full chunk of ten tiles, 161 -> two chunks of 80 and 81, 40 -> one
# bf16 chunk; repeats 70 -> 210, 210, 140 (two bf16 chunks each)
CASES = [
    ("bf16", "random", 300, "small"),
    ("nvfp4", "random", 300, "small"),
    ("nvfp4", "skewed", 300, "small"),
    ("nvfp4", "skewed", 160, "small"),
    ("nvfp4", "skewed", 161, "odd"),
    ("bf16", "repeats", 70, "small"),
    ("nvfp4", "random", 1, "small"),
    ("nvfp4", "random", 200, "odd"),
    ("bf16", "random", 100, "odd"),
    ("bf16", "skewed", 40, "odd"),
]


@pytest.mark.parametrize("expert,routing,T,dims", CASES)
def test_prefill_matches_oracle(expert, routing, T, dims):
    print(f"[gpu-prefill] {expert} {routing} T={T} {dims}", flush=True)
    spec, w = _layer(expert, _SMALL if dims == "small" else _ODD)
    u, h, idx, wts = _inputs(spec, T, 11, routing)
    ws = msk.prefill_workspace(spec, T)
    out = msk.moe_prefill(spec, w, u, idx, wts, h, ws)
    again = msk.moe_prefill(spec, w, u, idx, wts, h, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "two runs differ"
    _check(f"{expert} {routing}", out, h, _oracle(spec, w, u, h, idx, wts))


def test_prefill_skips_out_of_range_slots():
    """A slot whose expert index is outside [0, E) adds nothing: the same as
    that slot with weight 0."""
    print("[gpu-prefill] out-of-range slots", flush=True)
    spec, w = _layer("bf16", _SMALL)
    T, E = 40, spec["n_experts"]
    u, h, idx, wts = _inputs(spec, T, 12)
    bad = idx.clone()
    bad[::3, 2] = -1
    bad[1::5, 5] = E
    ws = msk.prefill_workspace(spec, T)
    out = msk.moe_prefill(spec, w, u, bad, wts, h, ws)
    torch.cuda.synchronize()
    dropped = (bad < 0) | (bad >= E)
    w0 = torch.where(dropped, torch.zeros_like(wts), wts)
    _check("out-of-range", out, h, _oracle(spec, w, u, h, idx, w0))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("expert", ["bf16", "nvfp4"])
def test_prefill_full_size(expert):
    """Hidden 6144, 256 experts top-8, FFN 2048: 1024 tokens (8192 slots, about
    32 per expert), whole batch on the GPU; the oracle recomputes six
    tokens (tokens never interact)."""
    print(f"[gpu-prefill] full size {expert}", flush=True)
    spec, w = _layer(expert, synth._BIG)
    T = 1024
    u, h, idx, wts = _inputs(spec, T, 13)
    ws = msk.prefill_workspace(spec, T)
    out = msk.moe_prefill(spec, w, u, idx, wts, h, ws)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 257, 511, 900, 1023])
    _check(f"full {expert}", out, h, _oracle(spec, w, u, h, idx, wts, rows), rows)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("expert,routing", [("nvfp4", "random"), ("bf16", "skewed")])
def test_prefill_max_tokens(expert, routing):
    """The largest call: 8192 tokens (65536 slots) at hidden 6144, 256 experts,
    FFN 2048.  Random routing gives about 256 slots per expert (two chunks
    each); skewed routing puts every token on experts 0..7 (bf16: 64 chunks
    of 128 each).  The oracle recomputes six tokens."""
    print(f"[gpu-prefill] max tokens {expert} {routing}", flush=True)
    spec, w = _layer(expert, synth._BIG)
    T = 8192
    u, h, idx, wts = _inputs(spec, T, 14, routing)
    ws = msk.prefill_workspace(spec, T)
    out = msk.moe_prefill(spec, w, u, idx, wts, h, ws)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 4096, 8000, 8191])
    _check(f"max {expert} {routing}", out, h, _oracle(spec, w, u, h, idx, wts, rows), rows)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("expert", ["nvfp4", "bf16"])
def test_prefill_long_rows(expert):
    """Hidden 6272 and FFN 4224: rows longer than the gather (6144) and SwiGLU
    (4096) keep in registers, so both convert their rows in two passes; 49
    and 33 k-tiles, and a last 256-row block of the down product with 128
    rows.  16 experts top-4 over 64 tokens."""
    print(f"[gpu-prefill] long rows {expert}", flush=True)
    dims = dict(_SMALL, hidden=6272, ffn_dim=4224, n_experts=16, top_k=4)
    spec, w = _layer(expert, dims)
    T = 64
    u, h, idx, wts = _inputs(spec, T, 15)
    ws = msk.prefill_workspace(spec, T)
    out = msk.moe_prefill(spec, w, u, idx, wts, h, ws)
    torch.cuda.synchronize()
    rows = np.array([0, 7, 31, 63])
    _check(f"long rows {expert}", out, h, _oracle(spec, w, u, h, idx, wts, rows), rows)
