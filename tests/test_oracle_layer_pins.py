"""Whole-layer pins of the CPU oracle: a layer worked by hand, and an
explicit-loop layer written without any of the oracle's helpers.

These pin the parts of the layer that only show in composition: the key
QK-norm (with its own gain), the cast of the appended key and value to the
cache format before they are attended, the router's input (the FFN RMSNorm
of h, with the FFN gain) and the residual the experts add to (h, not x).
Each of these plausible slips in the oracle fails at least one test here:

* the router normalising with attn_norm instead of ffn_norm;
* the router multiplying h instead of u;
* the key QK-norm dropped;
* the key QK-norm taking the q_norm gain;
* the appended key not cast to the cache format;
* the experts' residual starting from x instead of h.

Sources: QK-norm on queries and keys and the fixed-bound softmax (brifing.si
page, "Removing Attention Bottlenecks"); the fp8 KV cache (aitop.news page,
opening paragraphs); 8-of-256 routing (ainewsbites page, "One program
replaces many kernel boundaries"); the remaining steps are the readings the
oracle's module docstring lists.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as fm
from oracle import layer as ol

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _golden(golden_dir, name):
    rows = {}
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                rows[k] = v
    return rows


def _silu(z):
    return z / (1.0 + math.exp(-z))


# -------------------------------------------------------- the hand-worked layer

def _hand_problem():
    spec = dict(hidden=2, n_q_heads=2, n_kv_heads=1, head_dim=2, n_experts=3, top_k=2,
                ffn_dim=1, window=0, rms_eps=0.0, softmax_shift=2.0,
                dense_dtype="f32", expert_dtype="f32", kv_dtype="e4m3")
    f32 = lambda v: np.array(v, dtype=np.float32)  # noqa: E731
    w = dict(attn_norm=f32([2, 1]), q_norm=f32([1, 1]), k_norm=f32([1, 1.25]),
             ffn_norm=f32([1, 3]),
             wq=f32([[0.5, 0], [0, -1], [0.5, 0], [0, 1]]),
             wk=f32([[0.5, 0], [0, -7]]), wv=f32([[0.5, 0], [0, 2]]),
             wo=f32([[1, 0, 0, 0], [0, 0, -1, 0]]),
             w_router=f32([[1, 0], [0, -1], [1, 1]]),
             w_gate=f32([[[1, 0]], [[0, -1]], [[1, 1]]]),
             w_up=f32([[[0, 1]], [[1, 0]], [[1, 1]]]),
             w_down=f32([[[0], [1]], [[1], [0]], [[1], [1]]]))
    k = np.full((1, 1, 2, 2), 0x7F, dtype=np.uint8)      # NaN in the append slot
    v = np.full((1, 1, 2, 2), 0x7F, dtype=np.uint8)
    k[0, 0, 0] = [0x38, 0x00]                            # K = [1, 0]
    v[0, 0, 0] = [0x38, 0x48]                            # V = [1, 4]
    return spec, w, dict(k=k, v=v, cap=2), np.array([[1.0, -1.0]])


def test_hand_worked_layer(golden_dir):
    g = _golden(golden_dir, "hand_layer.txt")
    num = lambda key: np.array([float(v) for v in g[key]])  # noqa: E731
    hexes = lambda key: np.array([int(v, 16) for v in g[key]])  # noqa: E731
    spec, w, kv, x = _hand_problem()
    r = ol.layer_step(spec, w, kv, [1], 1, x)

    np.testing.assert_array_equal(r["q_hat"].reshape(-1), num("q_hat"))
    np.testing.assert_array_equal(r["k_new"].reshape(-1), num("k_new"))
    np.testing.assert_array_equal(r["k_new_bits"].reshape(-1), hexes("k_new_bits"))
    np.testing.assert_array_equal(r["v_new"].reshape(-1), num("v_new"))
    np.testing.assert_array_equal(r["v_new_bits"].reshape(-1), hexes("v_new_bits"))
    np.testing.assert_array_equal(r["win"].reshape(-1), num("win"))
    # the exact key before the cast differs from what is stored
    assert not np.array_equal(num("k_hat"), num("k_new"))

    s = num("scores_times_sqrt2")
    p = [1.0 / (1.0 + math.exp((s[2 * hd] - s[2 * hd + 1]) / math.sqrt(2))) for hd in (0, 1)]
    attn_o = [1.0, 4.0 - 6.0 * p[0], 1.0, 4.0 - 6.0 * p[1]]
    np.testing.assert_allclose(r["attn_o"].reshape(-1), attn_o, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["h"].reshape(-1), num("h"), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["u"].reshape(-1), num("u"), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["logits"].reshape(-1), num("logits"), rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(r["idx"].reshape(-1), num("idx"))

    w1, w0 = 1.0 / (1.0 + math.exp(-2.0)), 1.0 / (1.0 + math.exp(2.0))
    np.testing.assert_allclose(r["weights"].reshape(-1), [w1, w0], rtol=1e-14)
    out = [2.0 + w1 * _silu(3.0), -2.0 - 3.0 * w0 * _silu(1.0)]
    np.testing.assert_allclose(r["out"].reshape(-1), out, rtol=1e-14)


def test_route_alone_matches_hand_values(golden_dir):
    """route() by itself: u from h with the FFN gain, logits of u."""
    g = _golden(golden_dir, "hand_layer.txt")
    spec, w, _, _ = _hand_problem()
    r = ol.route(spec, w, np.array([[float(v) for v in g["h"]]]))
    np.testing.assert_allclose(r["u"][0], [float(v) for v in g["u"]], rtol=1e-14)
    np.testing.assert_allclose(r["logits"][0], [float(v) for v in g["logits"]], rtol=1e-14)
    assert r["idx"][0].tolist() == [int(float(v)) for v in g["idx"]]


# --------------------------------------------- explicit-loop reference layer

def _cast(val, dtype):
    """Stored value of one float in the cache format, by torch's own
    conversion (an implementation independent of the oracle's encoder)."""
    t = torch.tensor([val], dtype=torch.float64)
    if dtype == "e4m3":
        return float(t.clamp(-448.0, 448.0).to(torch.float32).to(torch.float8_e4m3fn)
                     .to(torch.float64)[0])
    if dtype == "bf16":
        return float(t.to(torch.float32).to(torch.bfloat16).to(torch.float64)[0])
    return float(t.to(torch.float32).to(torch.float64)[0])


def _cache_value(raw, dtype):
    t = torch.from_numpy(np.array([raw]))
    if dtype == "e4m3":
        return float(t.view(torch.float8_e4m3fn).to(torch.float64)[0])
    if dtype == "bf16":
        return float(t.view(torch.bfloat16).to(torch.float64)[0])
    return float(raw)


def _loop_layer(spec, w, kv, kv_len, Tr, x):
    """One layer in plain Python loops over lists, written from the layer's
    definition; none of the oracle's functions or formats are used."""
    H, Hq, Hkv, D = spec["hidden"], spec["n_q_heads"], spec["n_kv_heads"], spec["head_dim"]
    E, K, F, Wn = spec["n_experts"], spec["top_k"], spec["ffn_dim"], spec["window"]
    eps, kd = spec["rms_eps"], spec["kv_dtype"]
    G = Hq // Hkv
    T = len(kv_len) * Tr
    fl = lambda a: [float(v) for v in np.asarray(a, dtype=np.float64).reshape(-1)]  # noqa: E731

    def norm(vec, gain):
        ms = sum(v * v for v in vec) / len(vec)
        r = 1.0 / math.sqrt(ms + eps)
        return [v * r * gg for v, gg in zip(vec, gain)]

    def matvec(m, rows, cols, vec):
        return [sum(m[o * cols + i] * vec[i] for i in range(cols)) for o in range(rows)]

    wq, wk, wv, wo = fl(w["wq"]), fl(w["wk"]), fl(w["wv"]), fl(w["wo"])
    ga, gq, gk, gf = fl(w["attn_norm"]), fl(w["q_norm"]), fl(w["k_norm"]), fl(w["ffn_norm"])
    wr = fl(w["w_router"])
    res = dict(q_hat=[], k_new=[], v_new=[], win=[], attn_o=[], h=[], u=[], logits=[], idx=[],
               weights=[], out=[])
    # projections and the appended rows of every token first: a draft token
    # attends to the earlier drafts of its request
    qh_all, kn_all, vn_all = [], [], []
    for t in range(T):
        xt = fl(x[t])
        a = norm(xt, ga)
        q = matvec(wq, Hq * D, H, a)
        k = matvec(wk, Hkv * D, H, a)
        v = matvec(wv, Hkv * D, H, a)
        qh_all.append([norm(q[hd * D:(hd + 1) * D], gq) for hd in range(Hq)])
        kn_all.append([[_cast(e, kd) for e in norm(k[j * D:(j + 1) * D], gk)] for j in range(Hkv)])
        vn_all.append([[_cast(e, kd) for e in v[j * D:(j + 1) * D]] for j in range(Hkv)])
    for b, L in enumerate(kv_len):
        for t in range(Tr):
            row = b * Tr + t
            p = L + t
            lo = max(0, p - Wn + 1) if Wn > 0 else 0
            res["win"].append([lo, p])
            o_all = []
            for hd in range(Hq):
                j = hd // G
                keys, vals = [], []
                for i in range(lo, p + 1):
                    if i < L:
                        keys.append([_cache_value(kv["k"][b, j, i, d], kd) for d in range(D)])
                        vals.append([_cache_value(kv["v"][b, j, i, d], kd) for d in range(D)])
                    else:
                        keys.append(kn_all[b * Tr + (i - L)][j])
                        vals.append(vn_all[b * Tr + (i - L)][j])
                s = [sum(qh_all[row][hd][d] * kk[d] for d in range(D)) / math.sqrt(D) for kk in keys]
                m = max(s)
                e = [math.exp(si - m) for si in s]
                z = sum(e)
                o_all += [sum(e[i] * vals[i][d] for i in range(len(e))) / z for d in range(D)]
            xt = fl(x[row])
            h = [xt[o] + sum(wo[o * Hq * D + i] * o_all[i] for i in range(Hq * D)) for o in range(H)]
            u = norm(h, gf)
            lg = matvec(wr, E, H, u)
            order = sorted(range(E), key=lambda ee: (-lg[ee], ee))[:K]
            ex = [math.exp(lg[ee] - lg[order[0]]) for ee in order]
            wts = [v / sum(ex) for v in ex]
            out = list(h)
            for slot, ee in enumerate(order):
                if spec["expert_dtype"] != "f32":
                    raise ValueError("the loop reference takes fp32 experts")
                Wg = fl(w["w_gate"][ee])
                Wu = fl(w["w_up"][ee])
                Wd = fl(w["w_down"][ee])
                gate = matvec(Wg, F, H, u)
                up = matvec(Wu, F, H, u)
                act = [gg / (1.0 + math.exp(-gg)) * uu for gg, uu in zip(gate, up)]
                y = matvec(Wd, H, F, act)
                out = [oo + wts[slot] * yy for oo, yy in zip(out, y)]
            res["q_hat"].append(qh_all[row])
            res["k_new"].append(kn_all[row])
            res["v_new"].append(vn_all[row])
            res["attn_o"].append(o_all)
            res["h"].append(h)
            res["u"].append(u)
            res["logits"].append(lg)
            res["idx"].append(order)
            res["weights"].append(wts)
            res["out"].append(out)
    return {k: np.array(v) for k, v in res.items()}


def _rand_problem(rng, kd, window):
    spec = dict(hidden=8, n_q_heads=4, n_kv_heads=2, head_dim=4, n_experts=5, top_k=2,
                ffn_dim=3, window=window, rms_eps=1e-6, softmax_shift=4.0,
                dense_dtype="f32", expert_dtype="f32", kv_dtype=kd)
    H, Hq, Hkv, D, E, F = 8, 4, 2, 4, 5, 3
    f = lambda *s: (rng.standard_normal(s) * 0.5).astype(np.float32)  # noqa: E731
    # distinct gains everywhere, so a swapped gain changes the result
    w = dict(attn_norm=1 + f(H), q_norm=1 + f(D), k_norm=2 + f(D), ffn_norm=1 + f(H),
             wq=f(Hq * D, H), wk=f(Hkv * D, H), wv=f(Hkv * D, H) * 3, wo=f(H, Hq * D) * 2,
             w_router=f(E, H) * 2, w_gate=f(E, F, H), w_up=f(E, F, H), w_down=f(E, H, F))
    n_req, cap = 2, 12
    shape = (n_req, Hkv, cap, D)
    raw = rng.standard_normal(shape) * 1.5
    if kd == "e4m3":
        k = torch.from_numpy(raw).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        v = torch.from_numpy(raw[::-1].copy()).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    else:
        k = torch.from_numpy(raw).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        v = torch.from_numpy(raw[::-1].copy()).float().to(torch.bfloat16).view(torch.int16).numpy() \
            .view(np.uint16)
    return spec, w, dict(k=k, v=v, cap=cap)


@pytest.mark.parametrize("kd", ["e4m3", "bf16"])
@pytest.mark.parametrize("window", [0, 3])
def test_layer_matches_explicit_loops(kd, window):
    rng = np.random.default_rng(31 + window)
    spec, w, kv = _rand_problem(rng, kd, window)
    kv_len, Tr = [6, 1], 3
    x = rng.standard_normal((len(kv_len) * Tr, spec["hidden"])) * 2
    want = _loop_layer(spec, w, kv, kv_len, Tr, x)
    got = ol.layer_step(spec, w, kv, kv_len, Tr, x)
    for key in ("q_hat", "k_new", "v_new", "attn_o", "h", "u", "logits", "weights", "out"):
        np.testing.assert_allclose(np.asarray(got[key]).reshape(want[key].shape), want[key],
                                   rtol=1e-11, atol=1e-12, err_msg=key)
    np.testing.assert_array_equal(got["win"], want["win"])
    np.testing.assert_array_equal(got["idx"], want["idx"])
    assert np.abs(got["h"] - x).max() > 0.1           # Wo moves h away from x


def test_moe_residual_is_h_through_whole_layer():
    """With nonzero Wo and down weights: out - h equals the expert term that
    expert_ffn adds, and h - x equals Wo attn_o."""
    rng = np.random.default_rng(41)
    spec, w, kv = _rand_problem(rng, "e4m3", 0)
    x = rng.standard_normal((2, spec["hidden"]))
    r = ol.layer_step(spec, w, kv, [4, 2], 1, x)
    zero = np.zeros_like(r["h"])
    term = ol.expert_ffn(spec, w, r["u"], r["idx"], r["weights"], zero)
    np.testing.assert_allclose(r["out"] - r["h"], term, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["h"] - x, r["attn_o"] @ w["wo"].astype(np.float64).T,
                               rtol=1e-12, atol=1e-14)
    assert np.abs(r["h"] - x).max() > 0.1 and np.abs(term).max() > 1e-3
