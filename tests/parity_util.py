"""Shared helpers of the parity tests: run the oracle on the same bytes the GPU
path consumed, and compare with the stated tolerances.

Tolerances (per checked tensor, against that tensor's oracle RMS):
* all-fp32 layers: max|err| <= 1e-5 * RMS(reference);
* layers with any bf16 / e4m3 / NVFP4 storage: max|err| <= 2e-2 * RMS(reference).
Routing indices are compared exactly wherever the oracle's gap between the
k-th and (k+1)-th logit exceeds a margin that fp32 rounding cannot cross.
"""
import numpy as np
import torch

import synth
import verify_step_amd as msk
from oracle import formats as fm
from oracle import layer as ol

FP32_TOL = 1e-5
LOWP_TOL = 2e-2


def tol_for(spec):
    return FP32_TOL if (spec["dense_dtype"], spec["expert_dtype"], spec["kv_dtype"]) == \
        ("f32", "f32", "f32") else LOWP_TOL


def rel_err(gpu, ref, floor=None):
    """max over elements of |gpu - ref| / RMS(ref), after subtracting an
    element-wise allowance `floor` (clipped at zero)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "GPU result has non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(gpu - ref)
    if floor is not None:
        err = np.maximum(err - floor, 0.0)
    return float(np.max(err)) / max(rms, 1e-30)


def assert_close(name, gpu, ref, tol, floor=None):
    e = rel_err(gpu, ref, floor)
    print(f"[err] {name}: max|err|/RMS = {e:.3e} (tolerance {tol:.1e})", flush=True)
    assert e <= tol, f"{name}: max|err|/RMS = {e:.3e} > {tol:.1e}"
    return e


def fp32_store_floor(out):
    """Allowance for a difference of fp32 values: the stored fp32 output
    carries up to half an ulp of its own magnitude (<= 2^-24 |out|), which
    a delta out - h inherits in full; 2^-23 |out| covers it with margin."""
    return np.abs(np.asarray(out, dtype=np.float64)) * 2.0 ** -23


def fill_shift(p):
    """Softmax shift 0 in every layer: the library (and the oracle) take the
    score bound from the QK-norm gains."""
    for spec in p.specs:
        spec["softmax_shift"] = 0.0


def snapshot_kv(p):
    """Host copies of the cache slots the step appends to (for restoring and
    for checking the untouched slots)."""
    snaps = []
    for c in p.kv:
        s = {}
        for name in ("k", "v"):
            s[name] = [c[name][b, :, L:L + p.tokens_per_req].clone() for b, L in enumerate(p.kv_len)]
        snaps.append(s)
    return snaps


def restore_kv(p, snaps):
    for c, s in zip(p.kv, snaps):
        for name in ("k", "v"):
            for b, L in enumerate(p.kv_len):
                c[name][b, :, L:L + p.tokens_per_req].copy_(s[name][b])


def oracle_inputs(p, layer):
    return (p.specs[layer], synth.host_weights(p.weights[layer]), synth.host_kv(p.kv[layer]))


def code_distance(a, b, dtype):
    """|a - b| in units of the format's codes (sign-magnitude order)."""
    a = np.asarray(a)
    b = np.asarray(b)
    if dtype == "f32":
        raise ValueError
    bits = 16 if dtype == "bf16" else 8
    a = a.astype(np.int64)
    b = b.astype(np.int64)
    sign = 1 << (bits - 1)

    def ordered(x):
        return np.where(x & sign, -(x & (sign - 1)), x)

    return np.abs(ordered(a) - ordered(b))


def check_appended(p, layer, ref, tol, tokens=None, in_err=0.0):
    """K/V written at [L_b, L_b + Tr) equal the oracle's cast values, up to one
    code of the format where the fp32 and fp64 values straddle a rounding
    boundary.  tokens: optional mask over the T tokens to compare.  in_err:
    the layer's measured relative input difference in a free-running stack
    (see StackDrift.input_error); a value may then differ by more than one
    code as long as it stays within 10 x in_err x RMS of the oracle's
    values (small keys sit on the fine subnormal grid of the format)."""
    from oracle import formats as fm
    spec = p.specs[layer]
    kd = spec["kv_dtype"]
    Tr = p.tokens_per_req
    for name, bits_key in (("k", "k_new_bits"), ("v", "v_new_bits")):
        cache = p.kv[layer][name]
        for b, L in enumerate(p.kv_len):
            sel = np.ones(Tr, bool) if tokens is None else np.asarray(tokens)[b * Tr:(b + 1) * Tr]
            if not sel.any():
                continue
            got = synth.to_numpy(cache[b, :, L:L + Tr])[:, sel]         # [Hkv][Tr][D]
            want = np.asarray(ref[bits_key])[b * Tr:(b + 1) * Tr][sel]  # [Tr][Hkv][D]
            want = np.transpose(want, (1, 0, 2))
            if kd == "f32":
                np.testing.assert_allclose(got, want, rtol=2e-6, atol=2e-6 * np.abs(want).max())
                continue
            d = code_distance(got, want, kd)
            if in_err > 0:
                gv, wv = fm.decode(got, kd), fm.decode(want, kd)
                slack = 10.0 * in_err * float(np.sqrt(np.mean(wv * wv)))
                d = np.where(np.abs(gv - wv) <= slack, 0, d)
            assert d.max() <= 1, f"{name} append: {int((d > 0).sum())} codes differ, max {d.max()}"


def routing_margin(logits_ref, k, scale=1e-4):
    """Per token: gap between the k-th and (k+1)-th largest oracle logits."""
    s = -np.sort(-np.asarray(logits_ref), axis=1)
    if s.shape[1] == k:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


class StackDrift:
    """Free-running comparison of a layer stack: the oracle runs every layer
    from the same x, never from a GPU output.  Layer 0 sees identical inputs
    on both sides, and its routing is compared bit for bit wherever the
    oracle's top-k boundary gap exceeds `margin0` x RMS(logits).  A later
    layer sees inputs that differ by the earlier layers' rounding, and the
    layer's discontinuities (the top-k choice; the cast of appended keys and
    values to the cache format, where a value at a rounding boundary moves by
    a whole code) can turn such a difference into a different routing after
    enough layers.  So at a layer past the first, a token the GPU routes
    differently has left the oracle's trajectory: it is dropped from this
    layer's comparisons, and it and the later tokens of its request (which
    attend to its keys) from every later layer's.  At most `max_moved`
    tokens over the whole stack may leave this way; a systematic error moves
    many.  Each layer's own correctness is checked apart from the chaining,
    with the GPU layer fed the oracle's layer input (teacher-forced by the
    oracle), where routing is bit exact.  The report counts the tokens whose
    top-k gap lies within max(`drift`, 10 x in_err) x RMS(logits), in_err
    being the layer's measured max|GPU input - oracle input| / RMS(oracle
    input)."""

    def __init__(self, n_req, Tr, margin0, drift, max_moved=1):
        self.Tr = Tr
        self.alive = np.ones(n_req * Tr, bool)
        self.margin0, self.drift, self.max_moved = margin0, drift, max_moved
        self.moved = 0

    def input_error(self, gpu_in, ref_in):
        """max|gpu_in - ref_in| / RMS(ref_in) over the tokens still compared."""
        a = np.asarray(gpu_in, dtype=np.float64)[self.alive]
        b = np.asarray(ref_in, dtype=np.float64)[self.alive]
        if a.size == 0:
            return 0.0
        return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-30))

    def routing(self, layer, idx_gpu, logits_ref, idx_ref, k, in_err=0.0):
        """Checks the layer's routing; returns the mask of tokens to compare
        at this layer.  in_err: the layer's measured relative input
        difference (see input_error)."""
        idx_gpu = np.asarray(idx_gpu)
        idx_ref = np.asarray(idx_ref)
        rms = float(np.sqrt(np.mean(np.asarray(logits_ref) ** 2)))
        delta = (self.margin0 if layer == 0 else max(self.drift, 10.0 * in_err)) * rms
        near = near_mask(logits_ref, k, delta)
        differs = (idx_gpu != idx_ref).any(1)
        if layer == 0:
            cmp = self.alive & ~near
            assert not (differs & cmp).any(), \
                f"layer 0: routing differs on {int((differs & cmp).sum())} tokens"
        moved = self.alive & differs
        here = self.alive & ~moved
        for t in np.nonzero(moved)[0]:
            b = t // self.Tr
            self.alive[t:(b + 1) * self.Tr] = False
        self.moved += int(moved.sum())
        lost = 1.0 - self.alive.mean()
        print(f"[gpu-parity] layer {layer}: {int((here & near).sum())} tokens inside the "
              f"routing margin, {int(moved.sum())} routed differently "
              f"({int((moved & ~near).sum())} of them outside it), {lost:.0%} dropped",
              flush=True)
        assert self.moved <= self.max_moved, \
            f"{self.moved} tokens left the oracle's trajectory (at most {self.max_moved})"
        return here


def near_mask(logits_ref, k, delta):
    """Tokens whose top-k boundary gap is at most delta."""
    return routing_margin(logits_ref, k) <= delta


def check_routing(idx_gpu, logits_ref, idx_ref, k, delta):
    """Bit-exact indices for every token whose top-k boundary gap exceeds
    delta; returns the number of tokens inside the margin (not compared)."""
    idx_gpu = np.asarray(idx_gpu)
    gap = routing_margin(logits_ref, k)
    near = gap <= delta
    far = ~near
    assert np.array_equal(idx_gpu[far], np.asarray(idx_ref)[far]), \
        f"routing differs on {int((idx_gpu[far] != np.asarray(idx_ref)[far]).any(1).sum())} tokens"
    return int(near.sum())


def check_topk_of_gpu_logits(idx_gpu, logits_gpu, k):
    """The GPU's selection is exactly the top-k of its own fp32 logits under
    (value descending, index ascending): the integer decision is taken in the
    same precision on both sides."""
    want = ol.topk_desc_index_asc(np.asarray(logits_gpu, dtype=np.float32).astype(np.float64), k)
    assert np.array_equal(np.asarray(idx_gpu), want)
