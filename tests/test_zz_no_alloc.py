"""The allocation-free layer step (msk_layer_step_noalloc) against
msk_layer_step on the same inputs: two calls in a row, the second on a
smaller problem, each bit for bit equal to the workspace call (both run the
same kernels).  Needs an MI355X (gfx950)."""
import numpy as np
import pytest
import torch

import synth
import verify_step_amd as msk
from parity_util import fill_shift, restore_kv, snapshot_kv

pytestmark = pytest.mark.gpu

_SMALL = dict(hidden=512, n_q_heads=12, n_kv_heads=2, head_dim=128, n_experts=32, top_k=8,
              ffn_dim=256)


def _both(p):
    """(x, layer_out, topk, win) of msk_layer_step and of the allocation-free
    call, from the same inputs and cache contents."""
    n, T, H, K = len(p.specs), p.T, p.specs[0]["hidden"], p.specs[0]["top_k"]
    snaps = snapshot_kv(p)
    outs = []
    for noalloc in (False, True):
        restore_kv(p, snaps)
        x = p.x.clone()
        lo = torch.full((n, T, H), float("nan"), device="cuda")
        tk = torch.full((n, T, K), -1, dtype=torch.int32, device="cuda")
        win = torch.full((n, T, 2), -1, dtype=torch.int32, device="cuda")
        if noalloc:
            msk.layer_step_noalloc(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x,
                                   layer_out=lo, topk_idx=tk, win=win)
        else:
            ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req)
            msk.layer_step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws,
                           layer_out=lo, topk_idx=tk, win=win)
        torch.cuda.synchronize()
        outs.append((x.cpu(), lo.cpu(), tk.cpu(), win.cpu()))
    restore_kv(p, snaps)
    return outs


def _check(name, outs):
    (x0, lo0, tk0, w0), (x1, lo1, tk1, w1) = outs
    print(f"[no-alloc] {name}: max|dx| = {float((x0 - x1).abs().max()):.3e}", flush=True)
    assert torch.isfinite(x1).all()
    assert torch.equal(x0, x1)
    assert torch.equal(lo0, lo1)
    assert torch.equal(tk0, tk1)
    assert torch.equal(w0, w1)


def test_noalloc_matches_workspace_call_twice():
    # first call: several tokens, two layers, e4m3 cache, NVFP4 experts
    print("[no-alloc] stack-small", flush=True)
    p = synth.make_problem("stack4-nvfp4", device="cuda",
                           overrides=dict(dims=_SMALL, kv_len=[700], windows=[128, 0]))
    fill_shift(p)
    assert msk.workspace_size(p.specs, p.kv_len, p.tokens_per_req) <= msk.noalloc_scratch_bytes()
    _check("stack-small", _both(p))
    del p
    # second call, smaller: one token, one fp32 layer
    print("[no-alloc] tiny-fp32", flush=True)
    q = synth.make_problem("tiny-fp32", device="cuda")
    fill_shift(q)
    _check("tiny-fp32", _both(q))
