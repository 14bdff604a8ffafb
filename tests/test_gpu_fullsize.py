"""GPU parity at the full workload sizes, on sampled outputs.

The step runs whole on the GPU, as the benchmark runs it.  The oracle then
recomputes outputs it can afford one by one:
* a whole request: requests never interact, so the oracle runs request b
  alone (its own cache slice and tokens);
* a prefix of a request's draft tokens: drafts form a causal chain, so tokens
  0..t of every layer depend only on tokens 0..t.
"""
import numpy as np
import pytest
import torch

import synth
import verify_step_amd as msk
from oracle import layer as ol
from parity_util import (StackDrift, assert_close, fill_shift, fp32_store_floor, tol_for)

pytestmark = pytest.mark.gpu

ROUTE_MARGIN = 1e-5
DRIFT_MARGIN = 3e-3   # later layers of a stack (see StackDrift)


def _run_gpu(p):
    n = len(p.specs)
    T, H, K = p.T, p.specs[0]["hidden"], p.specs[0]["top_k"]
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req)
    x = p.x.clone()
    layer_out = torch.empty((n, T, H), dtype=torch.float32, device="cuda")
    topk = torch.empty((n, T, K), dtype=torch.int32, device="cuda")
    win = torch.empty((n, T, 2), dtype=torch.int32, device="cuda")
    msk.layer_step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws,
                   layer_out=layer_out, topk_idx=topk, win=win)
    torch.cuda.synchronize()
    msk.workspace_status(ws)
    return layer_out.double().cpu().numpy(), topk.cpu().numpy(), win.cpu().numpy()


def _sub_kv(c, b):
    return dict(k=synth.HostView(c["k"][b:b + 1]), v=synth.HostView(c["v"][b:b + 1]),
                cap=c["cap"])


def _check_request(p, gpu, b, n_tok):
    """Oracle for the first n_tok draft tokens of request b through every
    layer, against the GPU's rows of those tokens."""
    lo, topk, win = gpu
    Tr = p.tokens_per_req
    rows = slice(b * Tr, b * Tr + n_tok)
    # free-running: the oracle chains its own layers (see StackDrift)
    cur = p.x[rows].double().cpu().numpy()
    gpu_in = cur.copy()
    drift = StackDrift(1, n_tok, ROUTE_MARGIN, DRIFT_MARGIN)
    for l, spec in enumerate(p.specs):
        w = synth.host_weights(p.weights[l])
        ref = ol.layer_step(spec, w, _sub_kv(p.kv[l], b), [p.kv_len[b]], n_tok, cur)
        tol = tol_for(spec)
        alive = drift.alive.copy()
        assert np.array_equal(win[l][rows], ref["win"])
        here = drift.routing(l, topk[l][rows], ref["logits"], ref["idx"], spec["top_k"])
        assert_close(f"req {b} layer {l} out", lo[l][rows][here], ref["out"][here], tol)
        assert_close(f"req {b} layer {l} delta", (lo[l][rows] - gpu_in)[here],
                     (ref["out"] - cur)[here], tol, fp32_store_floor(ref["out"][here]))
        # the appended K/V of these tokens
        for name, key in (("k", "k_new_bits"), ("v", "v_new_bits")):
            L = p.kv_len[b]
            got = synth.to_numpy(p.kv[l][name][b, :, L:L + n_tok]).astype(np.int64)[:, alive]
            want = np.transpose(np.asarray(ref[key]), (1, 0, 2)).astype(np.int64)[:, alive]
            sign = 0x80
            gv = np.where(got & sign, -(got & 0x7F), got)
            wv = np.where(want & sign, -(want & 0x7F), want)
            assert np.abs(gv - wv).max(initial=0) <= 1, f"{name} append differs by more than one code"
        cur = ref["out"]
        gpu_in = lo[l][rows]


@pytest.mark.timeout(600)
def test_verify_bf16_128k():
    """2 requests x 8 drafts, full attention over 131072 e4m3 positions, bf16
    experts; request 1 checked whole."""
    print("[fullsize] verify-bf16-128k", flush=True)
    p = synth.make_problem("verify-bf16-128k", device="cuda")
    fill_shift(p)
    gpu = _run_gpu(p)
    _check_request(p, gpu, 1, 8)
    del p
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_stack4_nvfp4():
    """4-layer stack, SWA 2048 / full 65536 alternating, NVFP4 experts; the
    first 2 of 8 draft tokens checked through all four layers."""
    print("[fullsize] stack4-nvfp4", flush=True)
    p = synth.make_problem("stack4-nvfp4", device="cuda")
    fill_shift(p)
    gpu = _run_gpu(p)
    _check_request(p, gpu, 0, 2)
    del p
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_longctx_nvfp4():
    """8 requests x 4 drafts over e4m3 caches of 2^20 .. 2^13 positions; the
    shortest request checked whole and the 1M-position one on its first
    draft token."""
    print("[fullsize] longctx-nvfp4", flush=True)
    p = synth.make_problem("longctx-nvfp4", device="cuda")
    fill_shift(p)
    gpu = _run_gpu(p)
    _check_request(p, gpu, 7, 4)
    _check_request(p, gpu, 0, 1)
    del p
    torch.cuda.empty_cache()
