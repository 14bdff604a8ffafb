"""CPU checks of the seeded generator and of the oracle on generated inputs."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as fm
from oracle import layer as ol


def _oracle_inputs(p, layer=0):
    w = synth.host_weights(p.weights[layer], lazy_experts=False)
    kv = synth.host_kv(p.kv[layer])
    spec = dict(p.specs[layer])
    spec["softmax_shift"] = ol.score_shift(w["q_norm"], w["k_norm"], spec["head_dim"])
    return spec, w, kv


def test_generator_is_seeded_and_poisons_slack():
    a = synth.make_problem("tiny-fp32")
    b = synth.make_problem("tiny-fp32")
    for k in a.weights[0]:
        assert torch.equal(a.weights[0][k], b.weights[0][k]), k
    k = a.kv[0]["k"]
    assert torch.isnan(k[0, :, 512:]).all() and not torch.isnan(k[0, :, :512]).any()
    assert a.kv[0]["cap"] >= 513


def test_tiny_layer_runs_and_reads_no_poison():
    p = synth.make_problem("tiny-fp32")
    spec, w, kv = _oracle_inputs(p)
    r = ol.layer_step(spec, w, kv, p.kv_len, p.tokens_per_req, p.x.numpy())
    assert np.all(np.isfinite(r["out"]))
    assert r["win"].tolist() == [[385, 512]]
    assert r["idx"].shape == (1, 2)
    # the attention delta and the MoE delta are both non-trivial
    assert np.std(r["h"] - p.x.numpy()) > 1e-3
    assert np.std(r["out"] - r["h"]) > 1e-3


def test_nvfp4_quantiser_round_trip():
    torch.manual_seed(0)
    wt = torch.randn(64, 256) * 0.02
    packed, scales, g = synth.quantize_nvfp4(wt)
    dec = fm.nvfp4_to_f64(packed.numpy(), scales.numpy(), g)
    s = fm.e4m3_bits_to_f64(scales.numpy())
    step = np.repeat(s, 16, axis=1) * np.float32(g)
    # e2m1 spacing is at most 2 units of the block step (between 4 and 6), so
    # rounding error is at most one block step; typically far less
    err = np.abs(dec - wt.double().numpy())
    assert np.all(err <= step * 1.0 + 1e-12)
    rel = np.linalg.norm(dec - wt.double().numpy()) / np.linalg.norm(wt.double().numpy())
    assert rel < 0.15


@pytest.mark.parametrize("name", ["verify-bf16-128k", "stack4-nvfp4", "longctx-nvfp4"])
def test_shrunken_big_workloads_run(name):
    ov = dict(dims=dict(hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=32, n_experts=16,
                        top_k=4, ffn_dim=64),
              kv_len=[37, 70][: len(synth.WORKLOADS[name]["kv_len"]) or 1])
    if name == "longctx-nvfp4":
        ov["kv_len"] = [300, 150, 75, 20]
    p = synth.make_problem(name, overrides=ov)
    for layer in range(len(p.specs)):
        spec, w, kv = _oracle_inputs(p, layer)
        r = ol.layer_step(spec, w, kv, p.kv_len, p.tokens_per_req, p.x.numpy())
        assert np.all(np.isfinite(r["out"]))
