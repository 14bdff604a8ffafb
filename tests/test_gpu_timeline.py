"""The persistent whole-step kernel (the timeline call, which runs it for
one-token all-fp32 stacks) on the small fp32 workload: the same result as
the oracle, and every workgroup's phase stamps present and in order."""
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


def test_timeline_persistent_kernel_matches_oracle():
    print("[gpu-timeline] tiny-fp32", flush=True)
    p = synth.make_problem("tiny-fp32", device="cuda")
    fill_shift(p)
    snaps = snapshot_kv(p)
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req)
    n_wg = torch.cuda.get_device_properties(0).multi_processor_count
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
    n = 1 + PHASES_PER_LAYER * len(p.specs)
    assert (st[:, 0] > 0).all(), "persistent kernel did not run"
    assert (np.diff(st[:, :n], axis=1) >= 0).all()
    restore_kv(p, snaps)
