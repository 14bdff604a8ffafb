"""The persistent whole-step kernel (the timeline call, which runs it for
one-token steps where an instantiation exists) against the oracle, and its
per-workgroup phase stamps present and in order.  Cases: the small fp32
layer, the full-size bf16 decode layer, a reduced-width layer with NVFP4
experts over an e4m3 cache, and a six-layer fp32 stack, which the kernel runs
as two launches (four layers, then two)."""
import numpy as np
import pytest
import torch

import synth
import verify_step_amd as msk
from oracle import layer as ol
from parity_util import (assert_close, fill_shift, fp32_store_floor, oracle_inputs, restore_kv,
                         snapshot_kv, tol_for)

pytestmark = pytest.mark.gpu

PHASES_PER_LAYER = 7  # QKV, attention, combine, Wo, router, gate/up, down
_SMALL = dict(hidden=512, n_q_heads=12, n_kv_heads=2, head_dim=128, n_experts=32, top_k=8,
              ffn_dim=256)

CASES = {
    "tiny-fp32": ("tiny-fp32", None),
    "decode-bf16": ("decode-bf16", None),
    "decode-nvfp4-e4m3": ("decode-bf16", dict(dims=_SMALL, expert="nvfp4", kv="e4m3",
                                              kv_len=[3000], windows=[2048])),
    "tiny-fp32-6layers": ("tiny-fp32", dict(windows=[128, 0, 128, 0, 128, 0])),
}


@pytest.mark.parametrize("case", list(CASES))
def test_persistent_kernel_matches_oracle(case):
    name, ov = CASES[case]
    print(f"[gpu-timeline] {case}", flush=True)
    p = synth.make_problem(name, device="cuda", overrides=ov)
    fill_shift(p)
    snaps = snapshot_kv(p)
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req)
    n_wg = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    stamps = torch.zeros((n_wg, 32), dtype=torch.int64, device="cuda")
    x = p.x.clone()
    msk.layer_step_timeline(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws, stamps)
    torch.cuda.synchronize()
    msk.workspace_status(ws)

    cur = p.x.double().cpu().numpy()
    x0 = cur.copy()
    for l in range(len(p.specs)):
        spec, w, kv = oracle_inputs(p, l)
        cur = ol.layer_step(spec, w, kv, p.kv_len, p.tokens_per_req, cur)["out"]
    tol = tol_for(p.specs[0])
    got = x.double().cpu().numpy()
    assert_close("out", got, cur, tol)
    assert_close("delta", got - x0, cur - x0, tol, fp32_store_floor(cur))

    # the persistent kernel ran (stamps written) and each workgroup's stamps
    # follow the phase order
    st = stamps.cpu().numpy()
    ran = st[:, 0] > 0
    assert ran.sum() >= torch.cuda.get_device_properties(0).multi_processor_count, \
        "persistent kernel did not run"
    n = min(32, 1 + PHASES_PER_LAYER * len(p.specs))
    assert (np.diff(st[ran, :n], axis=1) >= 0).all()
    restore_kv(p, snaps)


def test_a_wait_that_gives_up_is_reported_by_the_next_call():
    """The barrier waits of the persistent kernel bounded to one poll give up
    (forced from the host: every kernel still runs to its end, on whatever
    its inputs hold).  The next call on the same workspace, made after the
    launch has finished, returns MSK_ERR_TIMEOUT before it enqueues anything,
    and the call after that runs clean and matches the oracle."""
    print("[gpu-timeline] watchdog", flush=True)
    p = synth.make_problem("tiny-fp32", device="cuda")
    fill_shift(p)
    snaps = snapshot_kv(p)
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req)
    n_wg = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    stamps = torch.zeros((n_wg, 32), dtype=torch.int64, device="cuda")
    x = p.x.clone()
    msk.set_spin_limit(1)
    try:
        msk.layer_step_timeline(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws,
                                stamps)
    finally:
        msk.set_spin_limit(0)
    torch.cuda.synchronize()
    assert (stamps[:, 0] > 0).any(), "persistent kernel did not run"
    restore_kv(p, snaps)

    x = p.x.clone()
    with pytest.raises(msk.MskError) as e:
        msk.layer_step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws)
    assert e.value.status == 5, e.value
    torch.cuda.synchronize()
    assert torch.equal(x, p.x), "the reporting call enqueued work"

    msk.layer_step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws)
    torch.cuda.synchronize()
    msk.workspace_status(ws)
    spec, w, kv = oracle_inputs(p, 0)
    ref = ol.layer_step(spec, w, kv, p.kv_len, p.tokens_per_req, p.x.double().cpu().numpy())["out"]
    assert_close("out after the report", x.double().cpu().numpy(), ref, tol_for(spec))
    restore_kv(p, snaps)
