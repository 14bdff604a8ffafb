"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Needs an MI355X (gfx950)."""
import sys

import numpy as np
import pytest
import torch

import synth
import verify_step_amd as msk
from oracle import layer as ol
from parity_util import (assert_close, check_appended, check_routing, check_topk_of_gpu_logits,
                         StackDrift, near_mask,
                         fill_shift, fp32_store_floor, oracle_inputs, restore_kv, snapshot_kv,
                         tol_for)

pytestmark = pytest.mark.gpu

# Routing is compared bit for bit wherever the oracle's k-th / (k+1)-th logit
# gap exceeds this fraction of the logits' RMS; fp32 logits carry errors near
# 1e-6 of it, so only a token closer than that to a tie could flip.
ROUTE_MARGIN = 1e-5
# Layers after the first of a stack take inputs that differ from the oracle's
# chain by the earlier layers' rounding (layer outputs within ~3e-4 of their
# RMS in the low-precision paths): their logits may move by about as much.
DRIFT_MARGIN = 3e-3

_SMALL = dict(hidden=512, n_q_heads=12, n_kv_heads=2, head_dim=128, n_experts=32, top_k=8,
              ffn_dim=256)

# (workload, overrides): full-size where the oracle finishes in seconds,
# otherwise the same structure at reduced width with ragged lengths that span
# several 64-position blocks, several work items and partial tails.
CASES = {
    "tiny-fp32": ("tiny-fp32", None),
    "decode-bf16": ("decode-bf16", None),
    "verify-small": ("verify-bf16-128k", dict(dims=_SMALL, kv_len=[1000, 77])),
    "stack-small": ("stack4-nvfp4", dict(dims=_SMALL, kv_len=[700], windows=[128, 0, 128, 0])),
    "longctx-small": ("longctx-nvfp4", dict(dims=dict(_SMALL, top_k=4, n_experts=16),
                                            kv_len=[3000, 1500, 700, 64, 1, 0, 33, 200])),
    "d64-bf16kv": ("decode-bf16", dict(dims=dict(_SMALL, head_dim=64, n_q_heads=8),
                                       kv_len=[130, 5], windows=[64], tokens_per_req=3,
                                       n_req=2)),
    # 96 query rows per kv head (two row groups on the matrix cores), each
    # draft with its own sliding window, bf16 cache
    "verify-m96-bf16kv": ("verify-bf16-128k", dict(dims=_SMALL, kv="bf16", kv_len=[300],
                                                   n_req=1, tokens_per_req=16, windows=[100])),
    # 12 rows per kv head over a bf16 cache of head_dim 128 (two-wave items)
    "verify-tr2-bf16kv": ("verify-bf16-128k", dict(dims=_SMALL, kv="bf16", kv_len=[200, 129],
                                                   tokens_per_req=2)),
    # NVFP4 rows whose scale rows start on 2 mod 4 bytes (hidden 480, ffn 96:
    # 30- and 6-byte scale rows) and rows that end inside a 64-chunk step
    "decode-odd-nvfp4": ("decode-bf16", dict(dims=dict(_SMALL, hidden=480, ffn_dim=96),
                                              expert="nvfp4", kv_len=[300], windows=[128])),
    "stack-odd-nvfp4": ("stack4-nvfp4", dict(dims=dict(_SMALL, hidden=480, ffn_dim=96),
                                             kv_len=[300], windows=[128, 0])),
}


def _problem(case):
    name, ov = CASES[case]
    print(f"[gpu-parity] building {case}", flush=True)
    p = synth.make_problem(name, device="cuda", overrides=ov)
    fill_shift(p)
    return p


@pytest.fixture(scope="module", params=list(CASES))
def prob(request):
    p = _problem(request.param)
    yield request.param, p
    del p
    torch.cuda.empty_cache()


def test_layer_step_matches_oracle(prob):
    case, p = prob
    print(f"[gpu-parity] layer_step {case}", flush=True)
    n = len(p.specs)
    T, H, K = p.T, p.specs[0]["hidden"], p.specs[0]["top_k"]
    snaps = snapshot_kv(p)
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req)
    x = p.x.clone()
    layer_out = torch.empty((n, T, H), dtype=torch.float32, device="cuda")
    topk = torch.empty((n, T, K), dtype=torch.int32, device="cuda")
    win = torch.empty((n, T, 2), dtype=torch.int32, device="cuda")
    msk.layer_step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws,
                   layer_out=layer_out, topk_idx=topk, win=win)
    torch.cuda.synchronize()
    msk.workspace_status(ws)
    assert torch.equal(x, layer_out[-1])

    # free-running: the oracle chains its own layers from x (see StackDrift)
    cur = p.x.double().cpu().numpy()
    gpu_in = cur.copy()
    lo = layer_out.double().cpu().numpy()
    drift = StackDrift(len(p.kv_len), p.tokens_per_req, ROUTE_MARGIN, DRIFT_MARGIN)
    for l in range(n):
        spec, w, kv = oracle_inputs(p, l)
        ref = ol.layer_step(spec, w, kv, p.kv_len, p.tokens_per_req, cur)
        tol = tol_for(spec)
        alive = drift.alive.copy()
        check_appended(p, l, ref, tol, tokens=alive)
        assert np.array_equal(win[l].cpu().numpy(), ref["win"])
        here = drift.routing(l, topk[l].cpu().numpy(), ref["logits"], ref["idx"], K)
        assert_close(f"layer {l} out", lo[l][here], ref["out"][here], tol)
        assert_close(f"layer {l} delta", (lo[l] - gpu_in)[here], (ref["out"] - cur)[here], tol,
                     fp32_store_floor(ref["out"][here]))
        cur = ref["out"]
        gpu_in = lo[l]
    restore_kv(p, snaps)


def test_ops_match_oracle(prob):
    """msk_attn_step, msk_moe_route and msk_expert_ffn one by one on layer 0."""
    case, p = prob
    print(f"[gpu-parity] ops {case}", flush=True)
    spec, w, kv = p.specs[0], p.weights[0], p.kv[0]
    T, H, E, K = p.T, spec["hidden"], spec["n_experts"], spec["top_k"]
    tol = tol_for(spec)
    snaps = snapshot_kv(p)
    ws = msk.new_workspace(p.specs[:1], p.kv_len, p.tokens_per_req)
    attn_o = torch.empty((T, spec["n_q_heads"] * spec["head_dim"]), device="cuda")
    win = torch.empty((T, 2), dtype=torch.int32, device="cuda")
    h, _, _ = msk.attn_step(spec, w, kv, p.kv_len, p.tokens_per_req, p.x, ws, attn_o=attn_o,
                            win=win)
    torch.cuda.synchronize()

    so, wo, kvo = oracle_inputs(p, 0)
    x = p.x.double().cpu().numpy()
    att = ol.attention_block(so, wo, kvo, p.kv_len, p.tokens_per_req, x)
    check_appended(p, 0, att, tol)
    assert np.array_equal(win.cpu().numpy(), att["win"])
    assert_close("attn_o", attn_o.cpu().numpy(), att["attn_o"], tol)
    assert_close("h - x", h.double().cpu().numpy() - x, att["h"] - x, tol,
                 fp32_store_floor(att["h"]))

    # router and experts each on inputs both sides share: the oracle's h (its
    # attention output above), then the oracle's routing of it, handed to the
    # GPU calls as their inputs
    h32 = np.asarray(att["h"], dtype=np.float32).astype(np.float64)
    r = ol.route(so, wo, h32)
    h_dev = torch.from_numpy(h32.astype(np.float32)).to("cuda")
    logits = torch.empty((T, E), device="cuda")
    u, idx, wts, _ = msk.moe_route(spec, w, h_dev, ws, logits=logits)
    u_o = torch.from_numpy(np.asarray(r["u"], dtype=np.float32)).to("cuda")
    idx_o = torch.from_numpy(np.asarray(r["idx"], dtype=np.int32)).to("cuda")
    wts_o = torch.from_numpy(np.asarray(r["weights"], dtype=np.float32)).to("cuda")
    out = msk.expert_ffn(spec, w, u_o, idx_o, wts_o, h_dev, ws)
    torch.cuda.synchronize()
    msk.workspace_status(ws)

    assert_close("u", u.cpu().numpy(), r["u"], tol)
    assert_close("logits", logits.cpu().numpy(), r["logits"], tol)
    check_topk_of_gpu_logits(idx.cpu().numpy(), logits.cpu().numpy(), K)
    near = check_routing(idx.cpu().numpy(), r["logits"], r["idx"], K,
                         ROUTE_MARGIN * float(np.sqrt(np.mean(r["logits"] ** 2))))
    print(f"[gpu-parity] router: {near} tokens inside the routing margin", flush=True)
    far = ~near_mask(r["logits"], K, ROUTE_MARGIN * float(np.sqrt(np.mean(r["logits"] ** 2))))
    np.testing.assert_allclose(wts.cpu().numpy()[far], np.asarray(r["weights"])[far],
                               rtol=1e-5, atol=1e-6)
    ref_out = ol.expert_ffn(so, wo, u_o.double().cpu().numpy(),
                            np.asarray(r["idx"], dtype=np.int64),
                            wts_o.double().cpu().numpy(), h32)
    assert_close("moe delta", out.double().cpu().numpy() - h32, ref_out - h32, tol,
                 fp32_store_floor(ref_out))
    restore_kv(p, snaps)


def test_determinism_and_untouched_slots(prob):
    """Two runs give identical bits; cache slots outside [L_b, L_b + Tr)
    keep their contents (NaN poison past the appended drafts stays)."""
    case, p = prob
    print(f"[gpu-parity] determinism {case}", flush=True)
    snaps = snapshot_kv(p)
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req)
    before = [{n: c[n].clone() for n in ("k", "v")} for c in p.kv] if p.T * 0 == 0 and \
        sum(c["k"].numel() for c in p.kv) < 2e8 else None
    outs = []
    for _ in range(2):
        restore_kv(p, snaps)
        x = p.x.clone()
        msk.layer_step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws)
        outs.append(x)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    if before is not None:
        for c, bsnap in zip(p.kv, before):
            for n in ("k", "v"):
                a, b = c[n], bsnap[n]
                mask = torch.ones_like(a, dtype=torch.bool)
                for r, L in enumerate(p.kv_len):
                    mask[r, :, L:L + p.tokens_per_req] = False
                aa = a[mask].view(torch.uint8) if a.dtype != torch.uint8 else a[mask]
                bb = b[mask].view(torch.uint8) if b.dtype != torch.uint8 else b[mask]
                assert torch.equal(aa, bb)
    restore_kv(p, snaps)
