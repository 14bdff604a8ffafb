"""Benchmark of the MoE decode/verify layer step on one MI355X.

One step = one call of msk_layer_step over the workload's layer stack with
inputs already resident in HBM.  Prints one JSON line:
  value          microseconds per layer-step (lower is better)
  roofline       the step kernel's achieved HBM GB/s on its algorithmic bytes
                 (distinct dense + router + selected-expert + attended-KV bytes)
                 against MI355X's 8 TB/s
  cpu_baseline   the CPU oracle timed on the same workload on this host

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402
import verify_step_amd as msk  # noqa: E402

METRIC = "µs per MoE layer decode/verify step + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0
ES = {"f32": 4, "bf16": 2, "e4m3": 1}


def expert_bytes(spec):
    H, F = spec["hidden"], spec["ffn_dim"]
    n = 3 * H * F
    if spec["expert_dtype"] == "nvfp4":
        return n // 2 + n // 16 + 3 * 4
    return n * ES[spec["expert_dtype"]]


def algorithmic_bytes(specs, kv_len, Tr, topk):
    """Bytes the step must read at least once: every dense weight, norm gain
    and router row, each distinct selected expert once, and the K and V rows
    of the union of the draft tokens' windows per (request, kv head)."""
    total = 0
    parts = dict(dense=0, experts=0, kv=0)
    for l, spec in enumerate(specs):
        H, Hq, Hkv, D, E = (spec[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                               "n_experts"))
        es = ES[spec["dense_dtype"]]
        dense = (Hq * D + 2 * Hkv * D) * H * es + H * Hq * D * es + E * H * es + (2 * H + 2 * D) * 4
        n_exp = len(np.unique(topk[l]))
        experts = n_exp * expert_bytes(spec)
        kv = 0
        W = spec["window"]
        for L in kv_len:
            lo = max(0, L - W + 1) if W > 0 else 0
            hi = L + Tr - 1
            kv += (hi - lo + 1) * Hkv * D * ES[spec["kv_dtype"]] * 2
        parts["dense"] += dense
        parts["experts"] += experts
        parts["kv"] += kv
        total += dense + experts + kv
    return total, parts


def cpu_baseline(p, budget_s=30.0):
    """Time the CPU oracle on the same workload: the whole layer step when it
    fits the budget (it does for one decode token), else one layer."""
    from oracle import layer as ol
    specs = p.specs
    cores = len(os.sched_getaffinity(0))
    cur = p.x.double().cpu().numpy()
    t0 = time.perf_counter()
    done = 0
    for l in range(len(specs)):
        w = synth.host_weights(p.weights[l])
        kv = synth.host_kv(p.kv[l])
        ol.layer_step(specs[l], w, kv, p.kv_len, p.tokens_per_req, cur)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=dt / done * 1e6, unit="us per layer-step", cores=cores, kind="oracle",
                sample=f"{done} of {len(specs)} layer step(s) of the benchmarked workload, "
                       f"float64 NumPy, including the host copies of the selected experts")


def unfused_step(p, x, ws):
    """The same step as separate per-op calls (attention, router, experts)
    per layer: one launch sequence per phase group, no persistent kernel."""
    H = p.specs[0]["hidden"]
    h = torch.empty_like(x)
    u = torch.empty_like(x)
    idx = torch.empty((p.T, p.specs[0]["top_k"]), dtype=torch.int32, device=x.device)
    wts = torch.empty((p.T, p.specs[0]["top_k"]), dtype=torch.float32, device=x.device)

    def run(stream=None):
        for spec, w, kv in zip(p.specs, p.weights, p.kv):
            msk.attn_step(spec, w, kv, p.kv_len, p.tokens_per_req, x, ws, h=h, stream=stream)
            msk.lib().msk_moe_route(
                msk.ctypes.byref(msk.make_cfg(spec)), msk.ctypes.byref(msk.make_weights(w)), p.T,
                msk._ptr(h), msk._ptr(u), msk._ptr(idx), msk._ptr(wts), None, msk._ptr(ws),
                ws.numel(), msk._stream(stream))
            msk.expert_ffn(spec, w, u, idx, wts, h, ws, out=x, stream=stream)
    return run


def timeline(p, ws, x):
    """Per-phase times of one persistent-kernel step from the in-kernel
    real-time counter (100 MHz): phase k ends when the last workgroup has
    finished it; its time is measured from the previous phase's end."""
    nblk = torch.cuda.get_device_properties(0).multi_processor_count
    stamps = torch.zeros((nblk, 32), dtype=torch.int64, device=x.device)
    msk.layer_step_timeline(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws, stamps)
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().astype(np.float64) * 0.01      # us
    names = ["qkv", "attn", "combine", "wo", "router", "gateup", "down"]
    out = []
    t0 = st[:, 0].min()
    prev = t0
    for l in range(len(p.specs)):
        for i, nm in enumerate(names):
            k = 1 + l * len(names) + i
            if k >= 32 or st[:, k].max() == 0:
                break
            end = st[:, k].max()
            out.append(dict(layer=l, phase=nm, us=round(end - prev, 2),
                            spread_us=round(end - st[:, k].min(), 2)))
            prev = end
    return dict(total_us=round(prev - t0, 2), phases=out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode-bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["fused", "unfused"], default="fused",
                    help="fused: msk_layer_step (one persistent kernel); unfused: the "
                         "msk_attn_step -> msk_moe_route -> msk_expert_ffn calls per layer")
    ap.add_argument("--timeline", action="store_true",
                    help="also print per-phase times of the persistent kernel")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer step runs on a single MI355X "
              "(no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    dev = "cuda:0"
    torch.cuda.set_device(0)
    p = synth.make_problem(args.workload, device=dev)
    for spec, w in zip(p.specs, p.weights):
        spec["softmax_shift"] = msk.softmax_shift(w["q_norm"], w["k_norm"], spec["head_dim"])
    n_layers = len(p.specs)
    K = p.specs[0]["top_k"]
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req, device=dev)
    x = p.x.clone()
    topk = torch.zeros((n_layers, p.T, K), dtype=torch.int32, device=dev)
    probe = msk.Step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws, topk_idx=topk)
    step = msk.Step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws)
    if args.path == "unfused":
        step = unfused_step(p, x, ws)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()
    msk.workspace_status(ws)

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    msk.workspace_status(ws)
    ms_step = ms_total / args.steps
    us_layer = ms_step * 1e3 / n_layers

    # one more step that records its routing, for the distinct-expert bytes
    probe(stream)
    torch.cuda.synchronize()
    nbytes, parts = algorithmic_bytes(p.specs, p.kv_len, p.tokens_per_req, topk.cpu().numpy())
    gbs = nbytes / (ms_step * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(us_layer, 3),
        "unit": "us per layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.specs[0]["dense_dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "n_layers": n_layers, "n_req": p.n_req,
                   "tokens_per_req": p.tokens_per_req, "kv_len": p.kv_len,
                   "dense": p.specs[0]["dense_dtype"], "experts": p.specs[0]["expert_dtype"],
                   "kv": p.specs[0]["kv_dtype"]},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": nbytes,
        "bytes_breakdown": parts,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_step_t1 (persistent whole step)" if args.path == "fused"
                     else "whole layer step (per-phase kernels)"},
    }
    out["path"] = args.path
    if args.timeline and args.path == "fused":
        out["timeline"] = timeline(p, ws, x)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
