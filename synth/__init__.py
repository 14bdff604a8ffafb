"""Seeded synthetic inputs for the MoE decode/verify layer step.

This module only draws random numbers and stores them in the formats the
layer consumes (fp32, bf16, e4m3 bytes, NVFP4-style packed bytes).  It holds
none of the layer's arithmetic, and both the GPU path and the CPU oracle read
the same bytes from it.

Recipe (the pages give no hidden size and no weights; these shapes and
distributions stand in for them):

* weights ~ N(0, 0.02) drawn in fp32, then rounded to the storage format
  (bf16: round to nearest even; NVFP4: the block quantiser below);
* router weights ~ N(0, 0.02), or N(0, 1/H) where the workload asks for
  router logits of unit scale;
* RMSNorm and QK-norm gains ~ N(1, 0.1), fp32;
* hidden input x ~ N(0, 1), fp32;
* cached K and V ~ N(0, 1) at positions [0, L_b), rounded to the cache format
  (e4m3: clamped to +-448 first, then round to nearest even); every other
  cache slot holds NaN, so a read outside the step's windows shows up;
* every tensor has its own generator seeded with seed * 2**20 + tensor_id.

NVFP4-style quantiser (input preparation only; the layer consumes the packed
bytes and never re-quantises): per matrix g = amax / (6 * 448); per block of 16
consecutive elements along the reduction dimension s = e4m3(amax16 / (6 g));
code = e2m1(clamp(w / (s g), -6, 6)) with round to nearest even; even element
in the low nibble.
"""
import dataclasses
import math

import torch

# ----------------------------------------------------------------- workloads

_BIG = dict(hidden=6144, n_q_heads=48, n_kv_heads=8, head_dim=128,
            n_experts=256, top_k=8, ffn_dim=2048)

WORKLOADS = {
    # hidden 256, 8 q / 2 kv heads, head_dim 32, 16 experts top-2, FFN 128;
    # one token; 512 cached positions; sliding window 128; all fp32
    "tiny-fp32": dict(
        dims=dict(hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=32,
                  n_experts=16, top_k=2, ffn_dim=128),
        n_req=1, tokens_per_req=1, kv_len=[512], windows=[128],
        dense="f32", expert="f32", kv="f32", router_sigma=0.02, seed=0),
    # one decode token; sliding window 2048 over 2048 bf16 cached positions
    "decode-bf16": dict(
        dims=_BIG, n_req=1, tokens_per_req=1, kv_len=[2048], windows=[2048],
        dense="bf16", expert="bf16", kv="bf16", router_sigma=0.02, seed=1),
    # verify: 2 requests x 8 draft tokens, full attention over 131072 e4m3
    # cached positions per request, bf16 experts
    "verify-bf16-128k": dict(
        dims=_BIG, n_req=2, tokens_per_req=8, kv_len=[131072, 131072], windows=[0],
        dense="bf16", expert="bf16", kv="e4m3", router_sigma="unit", seed=2),
    # 4-layer stack, 1 request x 8 draft tokens, layers alternate sliding
    # window 2048 and full context over 65536 e4m3 cached positions
    "stack4-nvfp4": dict(
        dims=_BIG, n_req=1, tokens_per_req=8, kv_len=[65536],
        windows=[2048, 0, 2048, 0],
        dense="bf16", expert="nvfp4", kv="e4m3", router_sigma="unit", seed=3),
    # 8 requests x 4 draft tokens, full attention, e4m3 cache lengths 2^20..2^13
    "longctx-nvfp4": dict(
        dims=_BIG, n_req=8, tokens_per_req=4,
        kv_len=[1 << 20, 1 << 19, 1 << 18, 1 << 17, 1 << 16, 1 << 15, 1 << 14, 1 << 13],
        windows=[0], dense="bf16", expert="nvfp4", kv="e4m3", router_sigma="unit", seed=4),
    # a deep hybrid stack: 32 layers, every fourth full context and the others
    # sliding-window 2048 (24 : 8, against the model's 46 : 16), all with a
    # 65536-position e4m3 cache; 1 request x 8 verify tokens; NVFP4 experts.
    # 32 layers of this shape (5.9 GB each) fill about 190 GB of HBM.
    "deep32-nvfp4": dict(
        dims=_BIG, n_req=1, tokens_per_req=8, kv_len=[65536],
        windows=[2048, 2048, 2048, 0] * 8,
        dense="bf16", expert="nvfp4", kv="e4m3", router_sigma="unit", seed=5),
}

RMS_EPS = 1e-6


@dataclasses.dataclass
class Problem:
    name: str
    specs: list          # per-layer dicts (dims, window, eps, dtypes, softmax_shift)
    weights: list        # per-layer dicts of torch tensors
    kv: list             # per-layer dicts: k, v [n_req][Hkv][cap][D], cap
    kv_len: list
    tokens_per_req: int
    x: torch.Tensor      # [T][H] float32

    @property
    def n_req(self):
        return len(self.kv_len)

    @property
    def T(self):
        return self.n_req * self.tokens_per_req


# ------------------------------------------------------------- primitives

def _gen(seed, tid, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * (1 << 20) + int(tid))
    return g


def _randn(shape, seed, tid, device, std=1.0, mean=0.0):
    x = torch.randn(shape, generator=_gen(seed, tid, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x


def store(x, dtype):
    """fp32 tensor -> storage tensor (float32, bfloat16 or uint8 e4m3 bits)."""
    if dtype == "f32":
        return x.contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "e4m3":
        return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    raise ValueError(dtype)


def nan_fill(t):
    """Fill a storage tensor with its format's NaN pattern."""
    if t.dtype == torch.uint8:
        t.fill_(0x7F)
    else:
        t.fill_(float("nan"))
    return t


_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_codes(y):
    """Round to the nearest e2m1 value (ties to even code); y already in [-6, 6]."""
    m = y.abs()
    b = torch.tensor(_E2M1_MID, device=y.device, dtype=y.dtype)
    code = torch.bucketize(m, b, right=False)            # ties -> lower code
    tie_up = (m == 0.75) | (m == 1.75) | (m == 3.5)      # lower code odd there
    code = code + tie_up.to(code.dtype)
    sign = (y < 0) & (code > 0)
    return (code | (sign.to(code.dtype) << 3)).to(torch.uint8)


def quantize_nvfp4(w):
    """fp32 [rows][cols] -> (packed uint8 [rows][cols/2], e4m3 scales
    [rows][cols/16], fp32 matrix scale)."""
    rows, cols = w.shape
    amax = w.abs().max().item()
    g = float(torch.tensor(amax / (6.0 * 448.0), dtype=torch.float32)) if amax > 0 else 1.0
    blocks = w.reshape(rows, cols // 16, 16)
    bmax = blocks.abs().amax(dim=-1)
    s8 = (bmax / (6.0 * g)).clamp(max=448.0).to(torch.float8_e4m3fn)
    s = s8.to(torch.float32)
    denom = (s * g).unsqueeze(-1)
    y = torch.where(denom > 0, blocks / torch.where(denom > 0, denom, torch.ones_like(denom)),
                    torch.zeros_like(blocks)).clamp(-6.0, 6.0)
    codes = _e2m1_codes(y).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    return packed, s8.view(torch.uint8).contiguous(), g


def quantize_nvfp4_batch(w):
    """quantize_nvfp4 over a batch of matrices fp32 [n][rows][cols] at once
    (the same arithmetic, without a host round trip per matrix): returns
    packed [n][rows][cols/2], scales [n][rows][cols/16] and the matrix
    scales as an fp32 tensor [n]."""
    n, rows, cols = w.shape
    amax = w.abs().amax(dim=(1, 2))
    # float32(amax / (6 * 448)) rounded once from the exact double quotient
    g = torch.where(amax > 0, (amax.double() / (6.0 * 448.0)).float(), torch.ones_like(amax))
    blocks = w.reshape(n, rows, cols // 16, 16)
    bmax = blocks.abs().amax(dim=-1)
    gv = g.view(n, 1, 1)
    s8 = (bmax / (6.0 * gv)).clamp(max=448.0).to(torch.float8_e4m3fn)
    s = s8.to(torch.float32)
    denom = (s * gv).unsqueeze(-1)
    y = torch.where(denom > 0, blocks / torch.where(denom > 0, denom, torch.ones_like(denom)),
                    torch.zeros_like(blocks)).clamp(-6.0, 6.0)
    codes = _e2m1_codes(y).reshape(n, rows, cols)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).contiguous()
    return packed, s8.view(torch.uint8).contiguous(), g


# --------------------------------------------------------------- generator

def _tid(layer, name, sub=0):
    names = ["attn_norm", "q_norm", "k_norm", "ffn_norm", "wq", "wk", "wv", "wo",
             "w_router", "w_gate", "w_up", "w_down", "k", "v", "x"]
    return (layer * 16 + names.index(name)) * 4096 + sub


def make_layer(dims, window, dense, expert, kv, router_sigma, seed, layer, device,
               kv_len, tokens_per_req):
    H, Hq, Hkv, D = dims["hidden"], dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    E, F = dims["n_experts"], dims["ffn_dim"]
    spec = dict(dims, window=int(window), rms_eps=RMS_EPS, softmax_shift=None,
                dense_dtype=dense, expert_dtype=expert, kv_dtype=kv)
    w = {}
    w["attn_norm"] = _randn((H,), seed, _tid(layer, "attn_norm"), device, 0.1, 1.0)
    w["q_norm"] = _randn((D,), seed, _tid(layer, "q_norm"), device, 0.1, 1.0)
    w["k_norm"] = _randn((D,), seed, _tid(layer, "k_norm"), device, 0.1, 1.0)
    w["ffn_norm"] = _randn((H,), seed, _tid(layer, "ffn_norm"), device, 0.1, 1.0)
    w["wq"] = store(_randn((Hq * D, H), seed, _tid(layer, "wq"), device, 0.02), dense)
    w["wk"] = store(_randn((Hkv * D, H), seed, _tid(layer, "wk"), device, 0.02), dense)
    w["wv"] = store(_randn((Hkv * D, H), seed, _tid(layer, "wv"), device, 0.02), dense)
    w["wo"] = store(_randn((H, Hq * D), seed, _tid(layer, "wo"), device, 0.02), dense)
    rs = 1.0 / math.sqrt(H) if router_sigma == "unit" else float(router_sigma)
    w["w_router"] = store(_randn((E, H), seed, _tid(layer, "w_router"), device, rs), dense)
    for which, shape in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        if expert == "nvfp4":
            packed = torch.empty((E, shape[0], shape[1] // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((E, shape[0], shape[1] // 16), dtype=torch.uint8, device=device)
            gs = torch.empty((E,), dtype=torch.float32, device=device)
            nb = 16   # experts quantised together
            for e0 in range(0, E, nb):
                e1 = min(E, e0 + nb)
                m = torch.stack([_randn(shape, seed, _tid(layer, "w_" + which, e), device, 0.02)
                                 for e in range(e0, e1)])
                p, s, g = quantize_nvfp4_batch(m)
                packed[e0:e1].copy_(p)
                scales[e0:e1].copy_(s)
                gs[e0:e1].copy_(g)
                del m
            w["w_" + which] = packed
            w["s_" + which] = scales
            w["g_" + which] = gs
        else:
            tdt = torch.float32 if expert == "f32" else torch.bfloat16
            t = torch.empty((E,) + shape, dtype=tdt, device=device)
            for e in range(E):
                t[e].copy_(store(_randn(shape, seed, _tid(layer, "w_" + which, e), device, 0.02),
                                 expert))
            w["w_" + which] = t
    n_req = len(kv_len)
    cap = ((max(kv_len) + tokens_per_req + 63) // 64) * 64
    sdt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}[kv]
    cache = {}
    for name in ("k", "v"):
        c = nan_fill(torch.empty((n_req, Hkv, cap, D), dtype=sdt, device=device))
        for b in range(n_req):
            L = int(kv_len[b])
            for j in range(Hkv):
                if L > 0:
                    c[b, j, :L].copy_(store(_randn((L, D), seed, _tid(layer, name, b * 64 + j),
                                                   device), kv))
        cache[name] = c
    cache["cap"] = cap
    return spec, w, cache


def make_problem(name, device="cpu", overrides=None):
    """Build the named workload (optionally with dimension/length overrides
    for small test variants) on `device`."""
    r = dict(WORKLOADS[name])
    if overrides:
        r = dict(r, **overrides)
        if "dims" in overrides:
            r["dims"] = dict(WORKLOADS[name]["dims"], **overrides["dims"])
    specs, weights, kvs = [], [], []
    for layer, win in enumerate(r["windows"]):
        s, w, c = make_layer(r["dims"], win, r["dense"], r["expert"], r["kv"],
                             r["router_sigma"], r["seed"], layer, device,
                             r["kv_len"], r["tokens_per_req"])
        specs.append(s)
        weights.append(w)
        kvs.append(c)
    T = len(r["kv_len"]) * r["tokens_per_req"]
    x = _randn((T, r["dims"]["hidden"]), r["seed"], _tid(0, "x"), device)
    return Problem(name=name, specs=specs, weights=weights, kv=kvs,
                   kv_len=[int(v) for v in r["kv_len"]],
                   tokens_per_req=int(r["tokens_per_req"]), x=x)


# -------------------------------------------------- host views for the oracle

def to_numpy(t):
    """Storage tensor -> numpy array of the same bits (bf16 -> uint16)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view("uint16")
    return t.cpu().numpy()


class HostView:
    """Array-like over a (possibly device-resident) tensor: indexing copies
    just the requested slice to host memory as numpy."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        return to_numpy(self.t[idx])

    def __array__(self, dtype=None, copy=None):
        a = to_numpy(self.t)
        return a if dtype is None else a.astype(dtype)


def host_weights(w, lazy_experts=True):
    """Per-layer weight dict for the oracle: small tensors copied, expert
    stacks wrapped so one expert at a time is copied."""
    out = {}
    for k, v in w.items():
        if lazy_experts and k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            out[k] = HostView(v)
        else:
            out[k] = to_numpy(v)
    return out


def host_kv(c):
    return dict(k=HostView(c["k"]), v=HostView(c["v"]), cap=c["cap"])
