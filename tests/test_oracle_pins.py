"""Pins of the CPU oracle against facts fixed outside it: format tables,
closed forms, invariants, brute force on tiny inputs and library routines.

Each test is written so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, an off-by-one window) fails it.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as fm
from oracle import layer as ol

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _golden(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ------------------------------------------------------------------ formats

def test_e2m1_table_matches_spec(golden_dir):
    for code, val in _golden(golden_dir, "e2m1_table.txt"):
        got = fm.e2m1_codes_to_f64(np.array([int(code)]))[0]
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e4m3_anchors(golden_dir):
    for byte, val in _golden(golden_dir, "e4m3_anchors.txt"):
        got = fm.e4m3_bits_to_f64(np.array([int(byte, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val)


def test_e4m3_table_matches_torch_reinterpretation():
    # torch's float8_e4m3fn is an independent implementation of the same format
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fm.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert nan.sum() == 2 and np.nanmax(ours) == 448.0
    assert np.min(np.abs(ours[np.abs(ours) > 0])) == 2.0 ** -9


def test_nvfp4_decode_full_table():
    # all 16 codes x all 256 scale bytes = 4096 products, against the literal
    # e2m1 table times torch's e4m3 decode, with a non-trivial matrix scale
    codes = np.tile(np.arange(16, dtype=np.uint8), 256 * 16 // 16)   # 4096 codes
    rows = 256
    codes = codes.reshape(rows, 16)                                    # one block per row
    scales = np.arange(256, dtype=np.uint8).reshape(rows, 1)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    g = np.float32(0.0123)
    got = fm.nvfp4_to_f64(packed, scales, g)
    lit = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    s_ref = torch.from_numpy(scales.reshape(-1)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = lit[codes] * s_ref[:, None] * np.float64(g)
    both_nan = np.isnan(want) & np.isnan(got)
    assert np.array_equal(np.isnan(want), np.isnan(got))
    assert np.array_equal(got[~both_nan], want[~both_nan])


def test_nibble_order_even_element_low():
    packed = np.array([[0x21, 0xF7]], dtype=np.uint8)
    codes = fm.unpack_nibbles(packed)
    assert codes.tolist() == [[1, 2, 7, 15]]
    v = fm.nvfp4_to_f64(np.tile(packed, (1, 4)), np.array([[0x38]], dtype=np.uint8), 1.0)
    assert v[0, :4].tolist() == [0.5, 1.0, 6.0, -6.0]


def test_e4m3_encoder_round_trip_and_ties():
    finite = np.array([b for b in range(256) if not np.isnan(fm.E4M3_TABLE[b])], dtype=np.uint8)
    vals = fm.E4M3_TABLE[finite]
    enc = fm.f64_to_e4m3_bits(vals)
    assert np.array_equal(fm.E4M3_TABLE[enc], vals)
    # midpoint between 1.0 (0x38, even mantissa) and 1.125 (0x39) -> 1.0;
    # between 1.125 and 1.25 (0x3A) -> 1.25
    assert fm.f64_to_e4m3_bits(np.array([1.0625]))[0] == 0x38
    assert fm.f64_to_e4m3_bits(np.array([1.1875]))[0] == 0x3A
    # subnormal grid and saturation
    assert fm.f64_to_e4m3_bits(np.array([2.0 ** -10]))[0] == 0x00    # tie -> even (0)
    assert fm.f64_to_e4m3_bits(np.array([3 * 2.0 ** -10]))[0] == 0x02
    assert fm.f64_to_e4m3_bits(np.array([1000.0, -1e9]))[0] == 0x7E
    assert fm.f64_to_e4m3_bits(np.array([-1e9]))[0] == 0xFE


def test_e4m3_encoder_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 100,
                        rng.standard_normal(2000) * 1e-2])
    x = x.astype(np.float32).astype(np.float64)     # torch rounds from float32
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fm.f64_to_e4m3_bits(x), ref)


def test_bf16_encoder_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fm.f64_to_bf16_bits(x.astype(np.float64)), ref)
    assert np.array_equal(fm.bf16_bits_to_f64(ref),
                          torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# ------------------------------------------------------- norms and activation

def test_rmsnorm_and_silu_hand_cases(golden_dir):
    g = {r[0]: [float(v) for v in r[1:]] for r in _golden(golden_dir, "hand_cases.txt")}
    np.testing.assert_allclose(ol.rmsnorm(np.array([3.0, 4.0]), [1, 1], 0.0), g["rmsnorm_eps0"], rtol=1e-14)
    np.testing.assert_allclose(ol.rmsnorm(np.array([1.0, 1.0]), [2, -1], 1.0), g["rmsnorm_eps1"], rtol=1e-14)
    np.testing.assert_allclose(ol.silu(np.array([1.0, -2.0])), g["silu"], rtol=1e-14)
    np.testing.assert_allclose(ol.softmax_textbook(np.array([0.0, math.log(3)])), g["softmax"], rtol=1e-14)


def test_rmsnorm_unit_rms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64)) * 3
    y = ol.rmsnorm(x, np.ones(64), 1e-6)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + 1e-6)), rtol=1e-13)


# ------------------------------------------------------------------ softmax

def test_nomax_matches_textbook_and_is_shift_invariant():
    rng = np.random.default_rng(3)
    D, n = 16, 300
    V = rng.standard_normal((n, D))
    c_star = 19.0
    for s in (rng.uniform(-c_star, c_star, (4, n)),
              np.concatenate([np.full((1, n), c_star), np.full((1, n), -c_star)]),
              rng.standard_normal((3, n))):
        want = ol.softmax_textbook(s) @ V
        for c in (0.0, c_star, c_star - 10, c_star + 10):
            for chunk in (None, 1, 7, 64):
                got = ol.nomax_attention(s, V, c, chunk)
                np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(4)
    cases = [rng.standard_normal(16) for _ in range(20)]
    cases += [np.round(rng.standard_normal(16) * 2) / 2 for _ in range(20)]   # many ties
    cases += [np.zeros(16), np.array([1.0, 3, 3, 2, 3, 1, 0, 3, 2, 2, 1, 0, 3, 1, 2, 0])]
    for v in cases:
        for k in range(1, 17):
            idx = ol.topk_desc_index_asc(v[None], k)[0]
            # brute force over all k-subsets: the unique best set under the
            # (value desc, index asc) order has the largest sorted key tuple
            best = max(itertools.combinations(range(16), k),
                       key=lambda S: sorted(((v[i], -i) for i in S), reverse=True)) \
                if k <= 3 else None
            if best is not None:
                assert sorted(idx.tolist()) == sorted(best)
            # every chosen index beats every unchosen one
            rest = [j for j in range(16) if j not in idx]
            for i in idx:
                for j in rest:
                    assert v[i] > v[j] or (v[i] == v[j] and i < j)
            # order within the selection, checked against numpy's lexsort
            assert idx.tolist() == np.lexsort((np.arange(16), -v))[:k].tolist()


def test_gating_weights_sum_to_one_and_ratio():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((6, 256))
    idx = ol.topk_desc_index_asc(lg, 8)
    w = ol.gating_weights(lg, idx)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    sel = np.take_along_axis(lg, idx, 1)
    np.testing.assert_allclose(w[:, 1] / w[:, 0], np.exp(sel[:, 1] - sel[:, 0]), rtol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)       # ordered like the logits


# ------------------------------------------------------------------ windows

@pytest.mark.parametrize("W", [1, 2, 128, 2048, 0])
@pytest.mark.parametrize("Tr", [1, 4, 8])
def test_window_bounds_brute_force(W, Tr):
    for L in sorted({0, 1, 5, max(W - 1, 0), W, W + 1, 3000}):
        win = ol.window_bounds([L], Tr, W)
        for t in range(Tr):
            p = L + t
            mask = [i for i in range(p + 100)
                    if i <= p and (W == 0 or p - i < W)]    # last W positions incl. self
            assert (win[t, 0], win[t, 1]) == (mask[0], mask[-1])


# ------------------------------------------------------------ tiny problems

def _tiny_spec(**kw):
    s = dict(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, n_experts=6, top_k=2,
             ffn_dim=16, window=0, rms_eps=1e-6, softmax_shift=5.0,
             dense_dtype="f32", expert_dtype="f32", kv_dtype="f32")
    s.update(kw)
    return s


def _tiny_weights(spec, rng):
    H, Hq, Hkv, D, E, F = (spec[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                             "n_experts", "ffn_dim"))
    f = lambda *s: (rng.standard_normal(s) * 0.3).astype(np.float32)  # noqa: E731
    return dict(attn_norm=1 + f(H) / 3, q_norm=1 + f(D) / 3, k_norm=1 + f(D) / 3,
                ffn_norm=1 + f(H) / 3, wq=f(Hq * D, H), wk=f(Hkv * D, H), wv=f(Hkv * D, H),
                wo=f(H, Hq * D), w_router=f(E, H), w_gate=f(E, F, H), w_up=f(E, F, H),
                w_down=f(E, H, F))


def _tiny_kv(spec, n_req, cap, rng):
    s = (n_req, spec["n_kv_heads"], cap, spec["head_dim"])
    return dict(k=rng.standard_normal(s).astype(np.float32),
                v=rng.standard_normal(s).astype(np.float32), cap=cap)


def test_window_and_causal_chain_via_position_valued_V():
    """q = 0 gives uniform attention, and V_i = i gives the mean position:
    (lo + hi) / 2 exactly, for every token of a verify chain."""
    rng = np.random.default_rng(6)
    for W in (0, 1, 3, 7):
        spec = _tiny_spec(window=W)
        w = _tiny_weights(spec, rng)
        w["wq"][:] = 0                        # q = 0 -> q_hat = 0 -> uniform weights
        L, Tr, cap = 20, 4, 32
        kv = _tiny_kv(spec, 1, cap, rng)
        kv["v"][:] = np.arange(cap, dtype=np.float32)[None, None, :, None]
        # appended values: make v = 0 for new tokens via Wv = 0 and put the
        # position in through V of the cache only; new positions then hold 0
        w["wv"][:] = 0
        x = rng.standard_normal((Tr, spec["hidden"]))
        r = ol.attention_block(spec, w, kv, [L], Tr, x)
        for t in range(Tr):
            p = L + t
            lo = max(0, p - W + 1) if W else 0
            cached = [i for i in range(lo, p + 1) if i < L]
            want = sum(cached) / (p - lo + 1)           # new positions contribute 0
            np.testing.assert_allclose(r["attn_o"][t], want, rtol=1e-13)
            assert tuple(r["win"][t]) == (lo, p)


def test_gqa_mapping_and_self_window():
    """Window 1: each token sees only itself, so o_h = v_new of kv-head h // G,
    as stored in the cache format."""
    rng = np.random.default_rng(7)
    for kvd in ("f32", "bf16", "e4m3"):
        spec = _tiny_spec(window=1, kv_dtype=kvd)
        w = _tiny_weights(spec, rng)
        if kvd != "f32":
            kv = dict(k=np.zeros((1, 2, 16, 8), dtype=np.uint16 if kvd == "bf16" else np.uint8),
                      v=np.zeros((1, 2, 16, 8), dtype=np.uint16 if kvd == "bf16" else np.uint8), cap=16)
        else:
            kv = _tiny_kv(spec, 1, 16, rng)
        x = rng.standard_normal((3, spec["hidden"]))
        r = ol.attention_block(spec, w, kv, [5], 3, x)
        G = spec["n_q_heads"] // spec["n_kv_heads"]
        o = r["attn_o"].reshape(3, spec["n_q_heads"], spec["head_dim"])
        for h in range(spec["n_q_heads"]):
            np.testing.assert_allclose(o[:, h], r["v_new"][:, h // G], rtol=1e-13)
        # the stored value is the format's rounding of the exact v
        a = ol.rmsnorm(x, w["attn_norm"], spec["rms_eps"])
        v_exact = (a @ w["wv"].astype(np.float64).T).reshape(3, 2, 8)
        np.testing.assert_array_equal(r["v_new"], fm.round_to_dtype(v_exact, kvd))


def test_mha_special_case_and_distinct_kv_heads():
    """With Hq == Hkv every head uses its own kv-head; with kv-head j holding
    the constant value j, o_h = h // G exactly for any scores."""
    rng = np.random.default_rng(8)
    for Hq, Hkv in ((2, 2), (4, 2), (6, 3), (8, 1)):
        spec = _tiny_spec(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=8, hidden=32)
        w = _tiny_weights(spec, rng)
        w["wv"][:] = 0
        kv = _tiny_kv(spec, 1, 16, rng)
        # the step's own v is 0, so give it weight ~0 by putting it in a
        # 1-position window? No: use full context with 12 cached positions and
        # compare with the closed form including the new (zero) position.
        kv["v"][:] = np.arange(Hkv, dtype=np.float32)[None, :, None, None]
        x = rng.standard_normal((1, 32))
        r = ol.attention_block(spec, w, kv, [12], 1, x)
        G = Hq // Hkv
        o = r["attn_o"].reshape(1, Hq, 8)
        q = r["q_hat"][0]
        for h in range(Hq):
            j = h // G
            K = np.concatenate([kv["k"][0, j, :12].astype(np.float64), r["k_new"][0, j][None]])
            p = ol.softmax_textbook(K @ q[h] / math.sqrt(8))
            np.testing.assert_allclose(o[0, h], j * p[:12].sum(), rtol=1e-12)


def test_attention_matches_textbook_softmax_full_layer():
    """The oracle's attention (no-max, block-streamed, appended positions
    handled apart) equals plain textbook softmax over the concatenated cache."""
    rng = np.random.default_rng(9)
    spec = _tiny_spec(window=9)
    w = _tiny_weights(spec, rng)
    kv = _tiny_kv(spec, 2, 40, rng)
    Tr = 3
    x = rng.standard_normal((2 * Tr, spec["hidden"]))
    for blk in (1, 5, 65536):
        r = ol.attention_block(spec, w, kv, [30, 4], Tr, x, kv_block=blk)
        o = r["attn_o"].reshape(2 * Tr, 4, 8)
        for b, L in enumerate((30, 4)):
            for j in range(2):
                K = np.concatenate([kv["k"][b, j, :L], r["k_new"][b * Tr:(b + 1) * Tr, j]])
                V = np.concatenate([kv["v"][b, j, :L], r["v_new"][b * Tr:(b + 1) * Tr, j]])
                for t in range(Tr):
                    p = L + t
                    lo = max(0, p - 9 + 1)
                    for h in (2 * j, 2 * j + 1):
                        s = K[lo:p + 1] @ r["q_hat"][b * Tr + t, h] / math.sqrt(8)
                        want = ol.softmax_textbook(s) @ V[lo:p + 1]
                        np.testing.assert_allclose(o[b * Tr + t, h], want, rtol=1e-12)


def test_score_bound_holds_for_normalised_keys():
    rng = np.random.default_rng(10)
    D = 32
    gq, gk = 1 + rng.standard_normal(D) * 0.1, 1 + rng.standard_normal(D) * 0.1
    c = ol.score_shift(gq, gk, D)
    q = ol.rmsnorm(rng.standard_normal((500, D)) * 7, gq, 1e-6)
    k = ol.rmsnorm(rng.standard_normal((500, D)) * 0.1, gk, 1e-6)
    s = q @ k.T / math.sqrt(D)
    assert np.max(np.abs(s)) <= c
    # the bound is tight for aligned one-hot-like vectors
    e = np.zeros(D)
    e[np.argmax(np.abs(gq))] = 1
    assert c >= abs(ol.rmsnorm(e, gq, 0) @ ol.rmsnorm(e, gk, 0)) / math.sqrt(D) - 1e-12


def test_projection_matches_explicit_loops():
    rng = np.random.default_rng(11)
    spec = _tiny_spec()
    w = _tiny_weights(spec, rng)
    kv = _tiny_kv(spec, 1, 8, rng)
    x = rng.standard_normal((1, 32))
    r = ol.attention_block(spec, w, kv, [3], 1, x)
    a = ol.rmsnorm(x, w["attn_norm"], spec["rms_eps"])[0]
    q = [sum(float(w["wq"][o, i]) * a[i] for i in range(32)) for o in range(32)]
    qh = ol.rmsnorm(np.array(q).reshape(4, 8), w["q_norm"], spec["rms_eps"])
    np.testing.assert_allclose(r["q_hat"][0], qh, rtol=1e-12)
    h = [x[0, o] + sum(float(w["wo"][o, i]) * r["attn_o"][0, i] for i in range(32)) for o in range(32)]
    np.testing.assert_allclose(r["h"][0], h, rtol=1e-12)


# ------------------------------------------------------------------- experts

def test_swiglu_scalar_closed_form():
    spec = _tiny_spec(hidden=1, ffn_dim=1, n_experts=1, top_k=1)
    # expert weights are stored as float32, so use float32-exact values
    a, b, c = (float(np.float32(v)) for v in (0.7, -1.3, 2.1))
    w = dict(w_gate=np.array([[[a]]]), w_up=np.array([[[b]]]), w_down=np.array([[[c]]]))
    u, h = np.array([[1.5]]), np.array([[0.25]])
    out = ol.expert_ffn(spec, w, u, np.array([[0]]), np.array([[1.0]]), h)
    z = a * 1.5
    want = 0.25 + c * (z / (1 + math.exp(-z))) * (b * 1.5)
    assert abs(out[0, 0] - want) < 1e-15


def test_moe_identities():
    rng = np.random.default_rng(12)
    spec = _tiny_spec()
    w = _tiny_weights(spec, rng)
    u = rng.standard_normal((5, 32))
    h = rng.standard_normal((5, 32))
    lg = rng.standard_normal((5, 6))
    idx = ol.topk_desc_index_asc(lg, 2)
    wt = ol.gating_weights(lg, idx)
    # zero gate -> silu(0) = 0 -> no change
    w0 = dict(w, w_gate=np.zeros_like(w["w_gate"]))
    np.testing.assert_array_equal(ol.expert_ffn(spec, w0, u, idx, wt, h), h)
    # identical experts -> output equals one expert's (weights sum to one)
    same = dict(w_gate=np.repeat(w["w_gate"][:1], 6, 0), w_up=np.repeat(w["w_up"][:1], 6, 0),
                w_down=np.repeat(w["w_down"][:1], 6, 0))
    one = ol.expert_ffn(spec, same, u, np.zeros((5, 1), dtype=np.int64), np.ones((5, 1)), h)
    np.testing.assert_allclose(ol.expert_ffn(spec, same, u, idx, wt, h), one, rtol=1e-12)
    # k = E: dense mixture over all experts, computed expert by expert
    idx_all = ol.topk_desc_index_asc(lg, 6)
    wt_all = ol.gating_weights(lg, idx_all)
    full = ol.expert_ffn(spec, w, u, idx_all, wt_all, h)
    p = ol.softmax_textbook(lg)
    want = h.copy()
    for e in range(6):
        g = u @ w["w_gate"][e].T
        ffn = (ol.silu(g) * (u @ w["w_up"][e].T)) @ w["w_down"][e].T
        want += p[:, e:e + 1] * ffn
    np.testing.assert_allclose(full, want, rtol=1e-12)


def test_expert_decoding_orientation():
    """gate/up are [F][H] (rows index the FFN dim), down is [H][F]; a
    non-square shape makes a transposed operand fail loudly."""
    spec = _tiny_spec(hidden=16, ffn_dim=32, n_experts=1, top_k=1, expert_dtype="nvfp4")
    rng = np.random.default_rng(13)
    mk = lambda r, c: (rng.integers(0, 256, (1, r, c // 2), dtype=np.uint8),  # noqa: E731
                       np.full((1, r, c // 16), 0x38, dtype=np.uint8))
    (wg, sg), (wu, su), (wd, sd) = mk(32, 16), mk(32, 16), mk(16, 32)
    w = dict(w_gate=wg, s_gate=sg, g_gate=np.array([0.5], np.float32), w_up=wu, s_up=su,
             g_up=np.array([0.25], np.float32), w_down=wd, s_down=sd, g_down=np.array([1.0], np.float32))
    u, h = rng.standard_normal((2, 16)), np.zeros((2, 16))
    out = ol.expert_ffn(spec, w, u, np.zeros((2, 1), dtype=np.int64), np.ones((2, 1)), h)
    G = fm.e2m1_codes_to_f64(fm.unpack_nibbles(wg[0])) * 0.5
    U = fm.e2m1_codes_to_f64(fm.unpack_nibbles(wu[0])) * 0.25
    Dn = fm.e2m1_codes_to_f64(fm.unpack_nibbles(wd[0]))
    want = (ol.silu(u @ G.T) * (u @ U.T)) @ Dn.T
    np.testing.assert_allclose(out, want, rtol=1e-13)


# -------------------------------------------------------------- whole layer

def test_layer_identity_when_outputs_zeroed():
    rng = np.random.default_rng(14)
    spec = _tiny_spec(window=4)
    w = _tiny_weights(spec, rng)
    w["wo"][:] = 0
    w["w_down"][:] = 0
    kv = _tiny_kv(spec, 2, 24, rng)
    x = rng.standard_normal((4, 32))
    r = ol.layer_step(spec, w, kv, [10, 17], 2, x)
    np.testing.assert_array_equal(r["out"], x)


def test_stack_feeds_each_layer_the_previous_output():
    rng = np.random.default_rng(15)
    specs = [_tiny_spec(window=3), _tiny_spec(window=0)]
    ws = [_tiny_weights(s, rng) for s in specs]
    kvs = [_tiny_kv(s, 1, 16, rng) for s in specs]
    x = rng.standard_normal((2, 32))
    rs = ol.stack_step(specs, ws, kvs, [9], 2, x)
    r1 = ol.layer_step(specs[1], ws[1], kvs[1], [9], 2, rs[0]["out"])
    np.testing.assert_array_equal(rs[1]["out"], r1["out"])
