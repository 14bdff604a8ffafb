"""Plain float64 reference of one decode/verify step of a Muse-Spark-style
mixture-of-experts decoder layer (and of a short stack of such layers).

Test infrastructure: this is the CPU oracle.  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it; it shares no code with the
GPU library and never imports it.

What the pages fix (sources are the five pages on "Optimizing Muse Spark Open
on TPU v7 with SGLang-TorchTPU"):

* every decoder layer is a mixture-of-experts layer and routes each token to
  8 of 256 experts (ainewsbites page, "One program replaces many kernel
  boundaries"; brifing.si page, "Model Architecture Details");
* attention is hybrid: sliding-window over the last 2,048 tokens in some
  layers, full context up to 1M tokens in the others (same two sections);
* QK-norm bounds the attention scores, so softmax needs no running maximum
  and chunks of the context reduce independently (brifing.si page, "Removing
  Attention Bottlenecks");
* the KV cache is fp8 (aitop.news page, opening paragraphs);
* expert weights are NVFP4 with one scale per 16 values (brifing.si page,
  "Expert Weight Quantization");
* a verify step checks draft tokens in one forward pass (brifing.si page,
  "Speculative Decoding Integration");
* the step maps hidden states in to hidden states out: embedding, LM head and
  sampling stay outside (ainewsbites page, "One program replaces many kernel
  boundaries").

Everything else (pre-norm residual block, RMSNorm with eps inside the root and
a plain multiplicative gain, QK-norm per head with shared gains, no positional
encoding, 1/sqrt(D) score scale, contiguous GQA groups, window including the
token itself, causal chain of draft tokens, cast of appended K/V to the cache
format before it is read, bias-free router, softmax over the k selected logits,
SwiGLU experts without biases) is a reading of the pages made where they are
silent; the list with reasons lives in the design notes.

Conventions: T = n_req * tokens_per_req tokens, request-major; token t of
request b sits at cache position p = L_b + t.  All arithmetic is float64 on
exactly decoded inputs.
"""
import math

import numpy as np

from . import formats as fm


# ------------------------------------------------------------------ helpers

def rmsnorm(x, gain, eps):
    """RMS normalisation over the last axis: x / sqrt(mean(x^2) + eps) * gain."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def silu(z):
    """silu(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def window_bounds(kv_len, tokens_per_req, window):
    """Visible cache positions [lo, hi] (inclusive) of each draft token.

    Token t of a request with L cached positions sits at p = L + t.  A sliding
    window of W positions includes the token itself, so lo = max(0, p - W + 1);
    full context (W == 0) starts at 0.  hi = p: drafts form a causal chain, each
    seeing the earlier ones and itself.  Returns int64 [n_req * Tr][2]."""
    out = []
    for L in kv_len:
        for t in range(tokens_per_req):
            p = int(L) + t
            lo = max(0, p - window + 1) if window > 0 else 0
            out.append((lo, p))
    return np.array(out, dtype=np.int64).reshape(-1, 2)


def softmax_textbook(s):
    """Softmax with the maximum subtracted first (the usual safe form)."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def nomax_partial(s, values, shift):
    """One chunk of the no-running-max softmax.

    With QK-norm every score obeys |s| <= shift, so exp(s - shift) neither
    overflows nor needs a per-chunk maximum; a chunk contributes the plain sums
    (l, o) = (sum_i e_i, sum_i e_i * v_i) with e_i = exp(s_i - shift)."""
    e = np.exp(np.asarray(s, dtype=np.float64) - shift)
    return np.sum(e, axis=-1), e @ values


def nomax_attention(s, values, shift, chunk=None):
    """Attention output sum_i softmax(s)_i v_i via independent chunks.

    s: scores [..., n]; values [n][D].  The chunks' (l, o) pairs add plainly;
    the result is o / l.  `chunk` is the number of positions per chunk (None:
    one chunk)."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[-1]
    step = n if chunk is None else max(1, int(chunk))
    l_tot = np.zeros(s.shape[:-1])
    o_tot = np.zeros(s.shape[:-1] + (values.shape[-1],))
    for a in range(0, n, step):
        l, o = nomax_partial(s[..., a:a + step], values[a:a + step], shift)
        l_tot = l_tot + l
        o_tot = o_tot + o
    return o_tot / l_tot[..., None]


def topk_desc_index_asc(logits, k):
    """Indices of the k largest values, ordered by value descending and, on
    equal values, by index ascending (the lower expert index wins a tie)."""
    logits = np.asarray(logits)
    out = np.empty(logits.shape[:-1] + (k,), dtype=np.int64)
    for r in np.ndindex(*logits.shape[:-1]):
        row = logits[r]
        order = sorted(range(row.shape[0]), key=lambda i: (-row[i], i))
        out[r] = order[:k]
    return out


def gating_weights(logits, idx):
    """Softmax over the k selected logits of each token."""
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), idx, axis=-1)
    return softmax_textbook(sel)


# ---------------------------------------------------------- weight decoding

def dense_matrix(w, name, dtype):
    """Decode a dense weight ([out][in]) to float64."""
    return fm.decode(w[name], dtype)


def expert_matrix(w, which, e, dtype):
    """Decode expert e's gate/up ([F][H]) or down ([H][F]) matrix to float64."""
    if dtype == "nvfp4":
        return fm.nvfp4_to_f64(np.asarray(w["w_" + which][e]),
                               np.asarray(w["s_" + which][e]),
                               np.asarray(w["g_" + which])[e])
    return fm.decode(np.asarray(w["w_" + which][e]), dtype)


# --------------------------------------------------------------- the step

def attention_block(spec, w, kv, kv_len, tokens_per_req, x, kv_block=65536):
    """RMSNorm, QKV, QK-norm, KV append, windowed attention, Wo + residual.

    Returns a dict with q_hat [T][Hq][D], k_new / v_new (appended values as
    stored, float64 [T][Hkv][D]), k_new_bits / v_new_bits (their encodings),
    win [T][2], attn_o [T][Hq*D] (pre-Wo) and h [T][H] = x + Wo attn_o.
    The cache itself is not modified."""
    H, Hq, Hkv, D = spec["hidden"], spec["n_q_heads"], spec["n_kv_heads"], spec["head_dim"]
    G = Hq // Hkv
    eps = spec["rms_eps"]
    # a given shift of 0 stands for the score bound taken from the gains
    shift = spec["softmax_shift"] or score_shift(w["q_norm"], w["k_norm"], D)
    dd, kd = spec["dense_dtype"], spec["kv_dtype"]
    Tr = tokens_per_req
    n_req = len(kv_len)
    T = n_req * Tr
    x = np.asarray(x, dtype=np.float64).reshape(T, H)

    a = rmsnorm(x, w["attn_norm"], eps)                                   # [T][H]
    q = a @ dense_matrix(w, "wq", dd).T                                   # [T][Hq*D]
    k = a @ dense_matrix(w, "wk", dd).T                                   # [T][Hkv*D]
    v = a @ dense_matrix(w, "wv", dd).T
    q_hat = rmsnorm(q.reshape(T, Hq, D), w["q_norm"], eps)
    k_hat = rmsnorm(k.reshape(T, Hkv, D), w["k_norm"], eps)
    v = v.reshape(T, Hkv, D)
    # the new keys and values enter the cache in its own format, and are
    # attended as stored
    k_new = fm.round_to_dtype(k_hat, kd)
    v_new = fm.round_to_dtype(v, kd)

    win = window_bounds(kv_len, Tr, spec["window"])
    inv_sqrt_d = 1.0 / math.sqrt(D)
    attn_o = np.zeros((T, Hq, D))
    for b in range(n_req):
        L = int(kv_len[b])
        rows = slice(b * Tr, (b + 1) * Tr)
        wb = win[rows]
        for j in range(Hkv):
            heads = slice(j * G, (j + 1) * G)
            qh = q_hat[rows, heads]                                       # [Tr][G][D]
            l_tot = np.zeros((Tr, G))
            o_tot = np.zeros((Tr, G, D))
            # cached positions, streamed in blocks; each token keeps the part
            # of a block that lies in its window
            for a0 in range(int(wb[:, 0].min()), min(int(wb[:, 1].max()) + 1, L), kv_block):
                a1 = min(a0 + kv_block, L)
                Kb = fm.decode(np.asarray(kv["k"][b, j, a0:a1]), kd)
                Vb = fm.decode(np.asarray(kv["v"][b, j, a0:a1]), kd)
                for t in range(Tr):
                    lo, hi = max(int(wb[t, 0]), a0), min(int(wb[t, 1]), a1 - 1)
                    if lo > hi:
                        continue
                    s = (qh[t] @ Kb[lo - a0:hi - a0 + 1].T) * inv_sqrt_d  # [G][n]
                    l, o = nomax_partial(s, Vb[lo - a0:hi - a0 + 1], shift)
                    l_tot[t] += l
                    o_tot[t] += o
            # appended draft positions L + t0 .. p of each token
            for t in range(Tr):
                t0 = max(int(wb[t, 0]), L) - L
                if t0 > t:
                    continue
                Kn = k_new[rows][t0:t + 1, j]
                Vn = v_new[rows][t0:t + 1, j]
                s = (qh[t] @ Kn.T) * inv_sqrt_d
                l, o = nomax_partial(s, Vn, shift)
                l_tot[t] += l
                o_tot[t] += o
            attn_o[rows, heads] = o_tot / l_tot[..., None]
    attn_o = attn_o.reshape(T, Hq * D)
    h = x + attn_o @ dense_matrix(w, "wo", dd).T
    return dict(q_hat=q_hat, k_new=k_new, v_new=v_new,
                k_new_bits=fm.encode(k_new, kd), v_new_bits=fm.encode(v_new, kd),
                win=win, attn_o=attn_o, h=h)


def route(spec, w, h):
    """FFN RMSNorm, router logits, top-k selection and gating weights.

    Returns u [T][H], logits [T][E], idx [T][k] (value desc, index asc) and
    weights [T][k] (softmax over the selected logits)."""
    h = np.asarray(h, dtype=np.float64)
    u = rmsnorm(h, w["ffn_norm"], spec["rms_eps"])
    logits = u @ dense_matrix(w, "w_router", spec["dense_dtype"]).T
    idx = topk_desc_index_asc(logits, spec["top_k"])
    return dict(u=u, logits=logits, idx=idx, weights=gating_weights(logits, idx))


def expert_ffn(spec, w, u, idx, weights, h):
    """out[t] = h[t] + sum_j weights[t][j] * down_e(silu(gate_e u) * up_e u),
    e = idx[t][j], summed in slot order j = 0..k-1.  Each distinct selected
    expert is decoded once and applied to every token routed to it."""
    u = np.asarray(u, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    idx = np.asarray(idx)
    T, k = idx.shape
    ed = spec["expert_dtype"]
    y = np.zeros((T, k, spec["hidden"]))
    for e in np.unique(idx):
        slots = np.argwhere(idx == e)                     # rows (t, j)
        ue = u[slots[:, 0]]
        g = ue @ expert_matrix(w, "gate", e, ed).T
        up = ue @ expert_matrix(w, "up", e, ed).T
        act = silu(g) * up
        y[slots[:, 0], slots[:, 1]] = act @ expert_matrix(w, "down", e, ed).T
    out = h.copy()
    for j in range(k):
        out += np.asarray(weights, dtype=np.float64)[:, j:j + 1] * y[:, j]
    return out


def layer_step(spec, w, kv, kv_len, tokens_per_req, x):
    """One decode/verify step of one MoE decoder layer (pre-norm residual)."""
    att = attention_block(spec, w, kv, kv_len, tokens_per_req, x)
    r = route(spec, w, att["h"])
    out = expert_ffn(spec, w, r["u"], r["idx"], r["weights"], att["h"])
    res = dict(att)
    res.update(u=r["u"], logits=r["logits"], idx=r["idx"], weights=r["weights"], out=out)
    return res


def stack_step(specs, ws, kvs, kv_len, tokens_per_req, x):
    """A decode/verify step through a stack of layers; layer l's output is
    layer l+1's input.  Returns the list of per-layer result dicts."""
    results = []
    cur = np.asarray(x, dtype=np.float64)
    for spec, w, kv in zip(specs, ws, kvs):
        r = layer_step(spec, w, kv, kv_len, tokens_per_req, cur)
        results.append(r)
        cur = r["out"]
    return results


def score_shift(q_norm, k_norm, head_dim):
    """Fixed softmax shift c from the QK-norm gains.

    After QK-norm, ||q_hat|| <= sqrt(D) max|g_q| and a normalised key obeys
    ||k_hat|| <= sqrt(D) max|g_k|, so the scaled score q_hat.k_hat / sqrt(D)
    is bounded by sqrt(D) max|g_q| max|g_k|.  Softmax is unchanged by the
    shift; the bound only keeps exp(s - c) at or below 1 for normalised keys."""
    return float(math.sqrt(head_dim) * np.max(np.abs(np.asarray(q_norm, dtype=np.float64)))
                 * np.max(np.abs(np.asarray(k_norm, dtype=np.float64))))
