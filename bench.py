"""Benchmark of the MoE decode/verify layer step on one MI355X.

One step = one call of msk_layer_step over the workload's layer stack with
inputs already resident in HBM.  Prints one JSON line:
  value          microseconds per layer-step (lower is better)
  hbm_gbs        whole-step algorithmic bytes (distinct dense + router +
                 selected-expert + attended-KV bytes) per second
  roofline       the dominant kernel (the phase with the most kernel time in
                 a second pass of the same steps, each launch bracketed by
                 dispatch-stamped HIP events): its algorithmic bytes per
                 launch / its mean launch duration, against MI355X's 8 TB/s;
                 traffic = HBM bytes per launch from the committed counter
                 summary, if the kernel sources still match it
  kernels        the same figures for every phase
  cpu_baseline   the CPU oracle timed on the same workload on this host

The prefill workloads (prefill-nvfp4, prefill-bf16) time msk_moe_prefill
instead: one layer's expert FFN over 4096 tokens on the matrix cores; their
line gives µs per call, achieved TFLOP/s of the two products (2 x slots x
3 x hidden x FFN flops) and a roofline against the 2.5 PFLOP/s dense fp16/bf16
peak; dtype is fp16 for NVFP4 experts (decoded exactly to fp16), bf16 otherwise.

With no --workload, every workload is measured and printed on a line of its
own; the largest single-GPU decode/verify workload (verify-bf16-128k: 2 x 8 draft tokens
over 131072 e4m3 positions per request, bf16 experts) comes last and carries
the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]
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
from verify_step_amd import profsum  # noqa: E402

METRIC = "µs per MoE layer decode/verify step + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0
ES = {"f32": 4, "bf16": 2, "e4m3": 1}


def expert_bytes(spec):
    """(gate + up, down) bytes of one expert in its storage format."""
    H, F = spec["hidden"], spec["ffn_dim"]
    n = H * F
    if spec["expert_dtype"] == "nvfp4":
        one = n // 2 + n // 16 + 4          # codes, e4m3 block scales, fp32 matrix scale
    else:
        one = n * ES[spec["expert_dtype"]]
    return 2 * one, one


def union_kv_positions(spec, kv_len, Tr):
    """Cache positions the step must read per (request, kv head): the union of
    its draft tokens' windows, appended positions included."""
    W = spec["window"]
    n = 0
    for L in kv_len:
        lo = max(0, L - W + 1) if W > 0 else 0
        n += L + Tr - lo
    return n


def phase_bytes(spec, kv_len, Tr, topk_l):
    """Algorithmic bytes of one launch of each phase's kernel for one layer:
    the weights (each distinct selected expert once) or cache rows it must
    stream, plus its activation inputs and outputs."""
    T = len(kv_len) * Tr
    H, Hq, Hkv, D, E, K, F = (spec[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                                 "n_experts", "top_k", "ffn_dim"))
    es, kes = ES[spec["dense_dtype"]], ES[spec["kv_dtype"]]
    NR = (Hq + 2 * Hkv) * D
    n_exp = len(np.unique(topk_l))
    gu, dn = expert_bytes(spec)
    kv = union_kv_positions(spec, kv_len, Tr) * Hkv * D * kes * 2
    return dict(
        qkv=NR * H * es + (H + 2 * D) * 4 + T * H * 4 + T * NR * 4 + T * 2 * Hkv * D * kes,
        attn=kv + T * Hq * D * 4,
        combine=T * Hq * D * 4,
        wo=H * Hq * D * es + T * Hq * D * 4 + 2 * T * H * 4,
        router=E * H * es + H * 4 + 2 * T * H * 4 + T * E * 4,
        topk=T * E * 4 + 2 * T * K * 4,
        gateup=n_exp * gu + T * H * 4 + T * K * F * 4,
        down=n_exp * dn + T * K * F * 4 + (2 * T * H * 4 if T == 1 else T * K * H * 4),
        union=T * K * 4,
        prep=2 * (T * H * 4 + H * 4 + 3 * T * H * 2),
        dense_sum=0,
        moe_sum=2 * T * H * 4 + T * K * (H * 4 + 8),
    )


def algorithmic_bytes(specs, kv_len, Tr, topk):
    """Bytes the step must read at least once: every dense weight, norm gain
    and router row, each distinct selected expert once, and the K and V rows
    of the union of the draft tokens' windows per (request, kv head)."""
    parts = dict(dense=0, experts=0, kv=0)
    for l, spec in enumerate(specs):
        H, Hq, Hkv, D, E = (spec[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                               "n_experts"))
        es = ES[spec["dense_dtype"]]
        parts["dense"] += ((Hq * D + 2 * Hkv * D) * H * es + H * Hq * D * es + E * H * es
                           + (2 * H + 2 * D) * 4)
        parts["experts"] += len(np.unique(topk[l])) * sum(expert_bytes(spec))
        parts["kv"] += union_kv_positions(spec, kv_len, Tr) * Hkv * D * ES[spec["kv_dtype"]] * 2
    return sum(parts.values()), parts


def stored_traffic(kernel, workload):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration) from the committed counter summary of this kernel and
    workload, or None when there is none or the kernel sources have changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            kv[k.strip()] = v.strip().strip("`")
    if kv.get("sources_sha256") != profsum.sources_digest():
        return None
    return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))


def _blas_threads():
    """Threads the host BLAS actually runs with (what the oracle's products use)."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(p, budget_s=30.0):
    """Time the CPU oracle on the same workload: whole layers of the step
    until the budget is spent (at least one).  Every weight and cache byte a
    layer can read is copied to host memory before its timer starts, so the
    figure is the oracle's arithmetic, not the device-to-host copies."""
    from oracle import layer as ol
    specs = p.specs
    cur = p.x.double().cpu().numpy()
    spent = 0.0
    done = 0
    for l in range(len(specs)):
        w = synth.host_weights(p.weights[l], lazy_experts=False)
        kv = dict(k=synth.to_numpy(p.kv[l]["k"]), v=synth.to_numpy(p.kv[l]["v"]),
                  cap=p.kv[l]["cap"])
        t0 = time.perf_counter()
        ol.layer_step(specs[l], w, kv, p.kv_len, p.tokens_per_req, cur)
        spent += time.perf_counter() - t0
        done += 1
        del w, kv
        if spent > budget_s:
            break
    return dict(value=spent / done * 1e6, unit="us per layer-step", cores=_blas_threads(),
                kind="oracle",
                sample=f"{done} of {len(specs)} layer step(s) of the benchmarked workload, "
                       f"float64 NumPy on host copies of the weights and cache (copies "
                       f"made before the timer starts)")


def per_op_step(p, x, ws):
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


KERNEL_NAMES = {"qkv": "k_qkv", "attn": "k_attn", "combine": "k_combine", "wo": "k_wo",
                "router": "k_router", "topk": "k_topk", "gateup": "k_gateup", "down": "k_down",
                "step": "k_step_p", "union": "k_union", "moe_sum": "k_moe_sum",
                "prep": "k_sum_prep", "dense_sum": "k_dense_sum"}
ONE_TOKEN_KERNELS = ("qkv", "wo", "router", "gateup", "down")


def kernel_name(phase, spec, T, Tr):
    """The kernel a phase runs as, mirroring the library's choice of path."""
    base = KERNEL_NAMES[phase]
    if T == 1 and phase in ONE_TOKEN_KERNELS:
        return base + "_t1"
    if T > 1 and phase in ("gateup", "down"):
        return base + "_tn"
    if T > 1 and phase in ("qkv", "wo", "router") and spec["dense_dtype"] == "bf16":
        return "k_dense_mfma"
    if phase == "attn":
        G = spec["n_q_heads"] // spec["n_kv_heads"]
        if spec["kv_dtype"] in ("bf16", "e4m3") and G * Tr > 8:
            return "k_attn_mfma"
    return base


def kernel_pass(p, x, ws, steps, stream, stamps=None):
    """Run `steps` more steps with every phase kernel bracketed by HIP events
    (msk_timer_start), each step recording its routing.  Returns per phase
    the summed kernel time, the launch count and the algorithmic bytes of
    those launches, plus the mean whole-step bytes."""
    n_layers, K = len(p.specs), p.specs[0]["top_k"]
    topk = torch.zeros((steps, n_layers, p.T, K), dtype=torch.int32, device=x.device)
    runs = [msk.Step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws,
                     topk_idx=topk[i], stamps=stamps) for i in range(steps)]
    msk.timer_start()
    for r in runs:
        r(stream)
    torch.cuda.synchronize()
    res = {ph: dict(ms=0.0, launches=0, bytes=0) for ph in msk.PHASES}
    for ph in msk.PHASES:
        res[ph]["ms"], res[ph]["launches"] = msk.timer_read(ph)
    msk.timer_start(())
    tk = topk.cpu().numpy()
    step_bytes = []
    for i in range(steps):
        step_bytes.append(algorithmic_bytes(p.specs, p.kv_len, p.tokens_per_req, tk[i]))
        for l, spec in enumerate(p.specs):
            for ph, b in phase_bytes(spec, p.kv_len, p.tokens_per_req, tk[i][l]).items():
                res[ph]["bytes"] += b
    return res, step_bytes


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, run under the counter passes to
    scale FETCH_SIZE / WRITE_SIZE to bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


HEADLINE = "verify-bf16-128k"
# the prefill expert FFN of one layer at full width (hidden 6144, 256 experts
# top-8, FFN 2048) over 4096 tokens: 32768 slots, about 128 per expert
PREFILL = {"prefill-nvfp4": dict(expert="nvfp4", tokens=4096, seed=6),
           "prefill-bf16": dict(expert="bf16", tokens=4096, seed=7)}
ALL_WORKLOADS = ["tiny-fp32", "decode-bf16", "stack4-nvfp4", "longctx-nvfp4", "deep32-nvfp4",
                 "prefill-nvfp4", "prefill-bf16", HEADLINE]
MFMA_F16_PEAK_TFLOPS = 2500.0
PREFILL_METRIC = ("µs per MoE layer prefill expert FFN + achieved TFLOP/s "
                  "(% of the dense fp16/bf16 matrix peak)")


def prefill_accounting(spec, counts):
    """Algorithmic flops of the two products ({"gateup", "down"}), the bytes
    of the distinct experts' weights, and the weight bytes the chunked
    products stream, for counts[e] slots routed to expert e."""
    H, F = spec["hidden"], spec["ffn_dim"]
    slots = int(np.sum(counts))
    gu_b, dn_b = expert_bytes(spec)
    distinct = int((np.asarray(counts) > 0).sum()) * (gu_b + dn_b)
    # each chunk of an expert's slots (up to 160 for NVFP4 experts, 128 for
    # bf16 experts) streams the expert's rows
    cmax = 160 if spec["expert_dtype"] == "nvfp4" else 128
    streamed = int(((np.asarray(counts) + cmax - 1) // cmax).sum()) * (gu_b + dn_b)
    flops = {"gateup": 2.0 * slots * 2 * F * H, "down": 2.0 * slots * H * F}
    return flops, distinct, streamed


def measure_prefill(name, args):
    """Time msk_moe_prefill on one layer's experts: returns its JSON record.
    Routing: each token's top-8 of 256 synthetic unit logits."""
    cfg = PREFILL[name]
    dev = "cuda:0"
    p = synth.make_problem("decode-bf16", device=dev,
                           overrides=dict(expert=cfg["expert"], kv_len=[64], windows=[128],
                                          seed=cfg["seed"]))
    spec, w = p.specs[0], p.weights[0]
    T, H, F, E, K = (cfg["tokens"], spec["hidden"], spec["ffn_dim"], spec["n_experts"],
                     spec["top_k"])
    g = torch.Generator(device=dev).manual_seed(cfg["seed"])
    u = torch.randn((T, H), generator=g, device=dev)
    h = torch.randn((T, H), generator=g, device=dev)
    logits = torch.randn((T, E), generator=g, device=dev)
    top, idx = torch.topk(logits, K, dim=1)
    idx = idx.to(torch.int32).contiguous()
    wts = torch.softmax(top, dim=1).contiguous()
    ws = msk.prefill_workspace(spec, T, device=dev)
    out = torch.empty_like(h)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        msk.moe_prefill(spec, w, u, idx, wts, h, ws, out=out, stream=stream)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        msk.moe_prefill(spec, w, u, idx, wts, h, ws, out=out, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # the same calls again with every kernel bracketed by dispatch-stamped events
    msk.timer_start()
    for _ in range(args.steps):
        msk.moe_prefill(spec, w, u, idx, wts, h, ws, out=out, stream=stream)
    torch.cuda.synchronize()
    kt = {ph: msk.timer_read(ph) for ph in msk.PHASES}
    msk.timer_start(())
    slots = T * K
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=E)
    flops, distinct, streamed = prefill_accounting(spec, counts)
    total_flops = sum(flops.values())
    timed = {ph: v for ph, v in kt.items() if v[1]}
    dom = max(("gateup", "down"), key=lambda ph: timed[ph][0])
    avg_us = timed[dom][0] * 1e3 / timed[dom][1]
    achieved = flops[dom] / (avg_us * 1e-6) / 1e12
    # HBM bytes per gate/up launch (its counter summary covers that kernel)
    traffic = stored_traffic("k_pf_gemm", name) if dom == "gateup" else None
    return {
        "metric": PREFILL_METRIC,
        "value": round(ms * 1e3, 3),
        "unit": "us per prefill expert FFN",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        # the products' input type: NVFP4 weights decoded to fp16, else bf16
        "dtype": "fp16" if spec["expert_dtype"] == "nvfp4" else "bf16",
        "data": "synthetic",
        "config": {"workload": name, "tokens": T, "slots": slots, "hidden": H, "ffn": F,
                   "experts": E, "top_k": K, "expert_format": spec["expert_dtype"],
                   "distinct_experts": int((counts > 0).sum())},
        "tflops": round(total_flops / (ms * 1e-3) / 1e12, 1),
        "tflops_frac": round(total_flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        "hbm_gbs_distinct_weights": round(distinct / (ms * 1e-3) / 1e9, 1),
        "weight_bytes_distinct": distinct,
        "weight_bytes_streamed": streamed,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "k_pf_gemm", "phase": dom,
                     "flops_per_launch": flops[dom], "avg_launch_us": round(avg_us, 3),
                     "launches": timed[dom][1]},
        "kernels": {ph: {"avg_us": round(v[0] * 1e3 / v[1], 3), "launches": v[1]}
                    for ph, v in timed.items()},
        "path": "moe_prefill",
    }


def measure(name, args, with_cpu):
    """Time one workload: returns its JSON record."""
    dev = "cuda:0"
    p = synth.make_problem(name, device=dev)
    for spec in p.specs:
        spec["softmax_shift"] = 0.0     # the library derives the score bound from the gains
    n_layers = len(p.specs)
    ws = msk.new_workspace(p.specs, p.kv_len, p.tokens_per_req, device=dev)
    x = p.x.clone()
    stamps = None
    if args.path == "persistent":
        n_wg = 4 * torch.cuda.get_device_properties(0).multi_processor_count
        stamps = torch.zeros((n_wg, 32), dtype=torch.int64, device=dev)
    step = msk.Step(p.specs, p.weights, p.kv, p.kv_len, p.tokens_per_req, x, ws, stamps=stamps)
    if args.path == "per_op":
        step = per_op_step(p, x, ws)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()
    msk.workspace_status(ws)
    # Each step takes the previous step's output as its input, so the routing
    # (and with it the distinct experts a step streams) changes from step to
    # step.  The timed steps and the per-kernel pass below both start from
    # this state, so the bytes counted in the second are those of the first.
    x_start = x.clone()

    # the timed region: K steps back to back, nothing else on the stream
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

    # the same K steps again, each kernel bracketed by dispatch-stamped events
    x.copy_(x_start)
    torch.cuda.synchronize()
    kp, step_bytes = kernel_pass(p, x, ws, args.steps, stream, stamps)
    msk.workspace_status(ws)
    nbytes = int(np.mean([b for b, _ in step_bytes]))
    parts = {k: int(np.mean([pp[k] for _, pp in step_bytes])) for k in step_bytes[0][1]}
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    timed = {ph: r for ph, r in kp.items() if r["launches"]}
    dom = max(timed, key=lambda ph: timed[ph]["ms"])
    d = timed[dom]
    avg_us = d["ms"] * 1e3 / d["launches"]
    bytes_launch = d["bytes"] / d["launches"] if dom != "step" else nbytes
    kgbs = bytes_launch / (avg_us * 1e-6) / 1e9
    kname = kernel_name(dom, p.specs[0], p.T, p.tokens_per_req)
    traffic = stored_traffic(kname, name)
    # weight-streaming time of the step: its distinct dense, router and
    # expert bytes at the HBM peak (the pages' denominator, without KV)
    stream_us = (parts["dense"] + parts["experts"]) / (HBM_PEAK_GBS * 1e3)

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
        "config": {"workload": name, "n_layers": n_layers, "n_req": p.n_req,
                   "tokens_per_req": p.tokens_per_req, "kv_len": p.kv_len,
                   "dense": p.specs[0]["dense_dtype"], "experts": p.specs[0]["expert_dtype"],
                   "kv": p.specs[0]["kv_dtype"]},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": nbytes,
        "bytes_breakdown": parts,
        "step_over_weight_streaming": round(ms_step * 1e3 / stream_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kname, "phase": dom,
                     "bytes_per_launch": int(bytes_launch), "avg_launch_us": round(avg_us, 3),
                     "launches": d["launches"]},
        "kernels": {ph: {"avg_us": round(r["ms"] * 1e3 / r["launches"], 3),
                         "launches": r["launches"],
                         "gbs": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1)
                         if ph != "step" else None}
                    for ph, r in timed.items()},
        "path": {"layer_step": "layer_step", "per_op": "per_op_calls",
                 "persistent": "persistent_kernel"}[args.path],
    }
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(p)
    del p, ws, x, step
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    help="one workload name, or 'all': every workload, each on a line of its "
                         f"own, the largest ({HEADLINE}) last")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["layer_step", "per_op", "persistent"],
                    default="layer_step",
                    help="layer_step: msk_layer_step (per-phase kernels); per_op: the "
                         "msk_attn_step -> msk_moe_route -> msk_expert_ffn calls per layer; "
                         "persistent: msk_layer_step_timeline, the persistent step kernel "
                         "where one exists")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer step runs on a single MI355X "
              "(no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        copy_calibration()
        return
    torch.cuda.set_device(0)
    names = ALL_WORKLOADS if args.workload == "all" else [args.workload]
    for name in names:
        if name in PREFILL:
            print(json.dumps(measure_prefill(name, args)), flush=True)
            continue
        # the CPU oracle is timed once, beside the headline workload
        with_cpu = not args.no_cpu_baseline and name == names[-1]
        print(json.dumps(measure(name, args, with_cpu)), flush=True)


if __name__ == "__main__":
    main()
