"""Python binding of libmsk.so, the MI355X MoE decode/verify layer-step library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the stream.  The library must have
been built (``python -m verify_step_amd.build``); without it every entry point
raises instead of computing anything elsewhere.

Layer specs are dicts with the keys hidden, n_q_heads, n_kv_heads, head_dim,
n_experts, top_k, ffn_dim, window, rms_eps, softmax_shift, dense_dtype,
expert_dtype, kv_dtype (dtype strings 'f32', 'bf16', 'e4m3', 'nvfp4');
softmax_shift 0 (or None) lets the library derive the score bound from the
QK-norm gains on the device.
Weights are dicts of device tensors named as in the C header; a KV cache is a
dict with tensors 'k', 'v' of shape [n_req][Hkv][cap][D].
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsk.so")

DTYPE = {"f32": 0, "bf16": 1, "e4m3": 2, "nvfp4": 3}
MAX_REQ = 64
MAX_TOKENS = 64
MAX_STACK = 64

STATUS = {0: "MSK_OK", 1: "MSK_ERR_INVALID_ARG", 2: "MSK_ERR_UNSUPPORTED",
          3: "MSK_ERR_WORKSPACE", 4: "MSK_ERR_DEVICE", 5: "MSK_ERR_TIMEOUT"}


class MskError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("ffn_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("softmax_shift", ctypes.c_float),
                ("dense_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


_WEIGHT_FIELDS = ["attn_norm", "q_norm", "k_norm", "ffn_norm", "wq", "wk", "wv", "wo",
                  "w_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                  "g_gate", "g_up", "g_down"]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("cap", ctypes.c_int64)]


class Batch(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("tokens_per_req", ctypes.c_int32),
                ("kv_len_host", ctypes.POINTER(ctypes.c_int32))]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m verify_step_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        P = ctypes.POINTER
        L.msk_abi_version.restype = i32
        L.msk_last_error.restype = ctypes.c_char_p
        L.msk_workspace_size.restype = sz
        L.msk_workspace_size.argtypes = [P(LayerCfg), i32, P(Batch)]
        L.msk_workspace_status.restype = i32
        L.msk_workspace_status.argtypes = [vp, sz, vp]
        L.msk_attn_step.restype = i32
        L.msk_attn_step.argtypes = [P(LayerCfg), P(LayerWeights), P(KV), P(Batch), vp, vp, vp,
                                    vp, vp, sz, vp]
        L.msk_moe_route.restype = i32
        L.msk_moe_route.argtypes = [P(LayerCfg), P(LayerWeights), i32, vp, vp, vp, vp, vp, vp,
                                    sz, vp]
        L.msk_expert_ffn.restype = i32
        L.msk_expert_ffn.argtypes = [P(LayerCfg), P(LayerWeights), i32, vp, vp, vp, vp, vp, vp,
                                     sz, vp]
        L.msk_layer_step.restype = i32
        L.msk_layer_step.argtypes = [P(LayerCfg), P(LayerWeights), P(KV), i32, P(Batch), vp, vp,
                                     vp, vp, vp, sz, vp]
        L.msk_layer_step_noalloc.restype = i32
        L.msk_layer_step_noalloc.argtypes = [P(LayerCfg), P(LayerWeights), P(KV), i32, P(Batch),
                                             vp, vp, vp, vp, vp]
        L.msk_noalloc_scratch_bytes.restype = sz
        L.msk_noalloc_scratch_bytes.argtypes = []
        L.msk_moe_prefill.restype = i32
        L.msk_moe_prefill.argtypes = [P(LayerCfg), P(LayerWeights), i32, vp, vp, vp, vp, vp, vp,
                                      sz, vp]
        L.msk_moe_prefill_workspace_size.restype = sz
        L.msk_moe_prefill_workspace_size.argtypes = [P(LayerCfg), i32]
        L.msk_set_spin_limit.restype = i32
        L.msk_set_spin_limit.argtypes = [ctypes.c_uint32]
        L.msk_timer_start.restype = i32
        L.msk_timer_start.argtypes = [ctypes.c_uint32]
        L.msk_timer_read.restype = i32
        L.msk_timer_read.argtypes = [i32, P(ctypes.c_double), P(ctypes.c_int64)]
        L.msk_layer_step_timeline.restype = i32
        L.msk_layer_step_timeline.argtypes = [P(LayerCfg), P(LayerWeights), P(KV), i32, P(Batch),
                                              vp, vp, vp, vp, vp, vp, sz, vp]
        if L.msk_abi_version() != 1:
            raise RuntimeError("libmsk.so ABI version mismatch")
        _lib = L
    return _lib


def last_error():
    return lib().msk_last_error().decode()


def _check(status):
    if status != 0:
        raise MskError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------- marshalling

def make_cfg(spec):
    return LayerCfg(spec["hidden"], spec["n_q_heads"], spec["n_kv_heads"], spec["head_dim"],
                    spec["n_experts"], spec["top_k"], spec["ffn_dim"], spec["window"],
                    spec["rms_eps"], spec["softmax_shift"] or 0.0, DTYPE[spec["dense_dtype"]],
                    DTYPE[spec["expert_dtype"]], DTYPE[spec["kv_dtype"]])


def make_weights(w):
    return LayerWeights(*[(w[n].data_ptr() if n in w and w[n] is not None else None)
                          for n in _WEIGHT_FIELDS])


def make_kv(kv):
    return KV(kv["k"].data_ptr(), kv["v"].data_ptr(), int(kv["k"].shape[2]))


def make_batch(kv_len, tokens_per_req):
    arr = (ctypes.c_int32 * len(kv_len))(*[int(v) for v in kv_len])
    b = Batch(len(kv_len), int(tokens_per_req), arr)
    b._keep = arr
    return b


def _array(cls, items):
    arr = (cls * len(items))(*items)
    return arr


def workspace_size(specs, kv_len, tokens_per_req):
    if isinstance(specs, dict):
        specs = [specs]
    cfgs = _array(LayerCfg, [make_cfg(s) for s in specs])
    n = lib().msk_workspace_size(cfgs, len(specs), ctypes.byref(make_batch(kv_len, tokens_per_req)))
    if n == 0:
        raise MskError(1, last_error())
    return n


def new_workspace(specs, kv_len, tokens_per_req, device="cuda"):
    """A zero-filled workspace big enough for every entry point on these
    layers and this batch (zeroed once; calls leave it reusable)."""
    n = workspace_size(specs, kv_len, tokens_per_req)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def workspace_status(ws, stream=None):
    _check(lib().msk_workspace_status(_ptr(ws), ws.numel(), _stream(stream)))


# ------------------------------------------------------------ entry points

def attn_step(spec, w, kv, kv_len, tokens_per_req, x, ws, h=None, attn_o=None, win=None,
              stream=None):
    """Attention half of one layer; returns (h, attn_o, win)."""
    T, H = x.shape
    h = torch.empty_like(x) if h is None else h
    cfg, wt, kvs = make_cfg(spec), make_weights(w), make_kv(kv)
    b = make_batch(kv_len, tokens_per_req)
    _check(lib().msk_attn_step(ctypes.byref(cfg), ctypes.byref(wt), ctypes.byref(kvs),
                               ctypes.byref(b), _ptr(x), _ptr(h), _ptr(attn_o), _ptr(win),
                               _ptr(ws), ws.numel(), _stream(stream)))
    return h, attn_o, win


def moe_route(spec, w, h, ws, logits=None, stream=None):
    """Router: returns (u, topk_idx int32, topk_w, logits)."""
    T, H = h.shape
    u = torch.empty_like(h)
    idx = torch.empty((T, spec["top_k"]), dtype=torch.int32, device=h.device)
    wts = torch.empty((T, spec["top_k"]), dtype=torch.float32, device=h.device)
    cfg, wt = make_cfg(spec), make_weights(w)
    _check(lib().msk_moe_route(ctypes.byref(cfg), ctypes.byref(wt), T, _ptr(h), _ptr(u),
                               _ptr(idx), _ptr(wts), _ptr(logits), _ptr(ws), ws.numel(),
                               _stream(stream)))
    return u, idx, wts, logits


def expert_ffn(spec, w, u, idx, wts, h, ws, out=None, stream=None):
    """Experts: returns out = h + MoE(u)."""
    T, H = h.shape
    out = torch.empty_like(h) if out is None else out
    cfg, wt = make_cfg(spec), make_weights(w)
    _check(lib().msk_expert_ffn(ctypes.byref(cfg), ctypes.byref(wt), T, _ptr(u), _ptr(idx),
                                _ptr(wts), _ptr(h), _ptr(out), _ptr(ws), ws.numel(),
                                _stream(stream)))
    return out


def layer_step(specs, weights, kvs, kv_len, tokens_per_req, x, ws, layer_out=None,
               topk_idx=None, win=None, stream=None):
    """A whole step through len(specs) layers; x is updated in place."""
    n = len(specs)
    cfgs = _array(LayerCfg, [make_cfg(s) for s in specs])
    wts = _array(LayerWeights, [make_weights(w) for w in weights])
    kva = _array(KV, [make_kv(k) for k in kvs])
    b = make_batch(kv_len, tokens_per_req)
    _check(lib().msk_layer_step(cfgs, wts, kva, n, ctypes.byref(b), _ptr(x), _ptr(layer_out),
                                _ptr(topk_idx), _ptr(win), _ptr(ws), ws.numel(),
                                _stream(stream)))
    return x


def layer_step_noalloc(specs, weights, kvs, kv_len, tokens_per_req, x, layer_out=None,
                       topk_idx=None, win=None, stream=None):
    """layer_step without a workspace: the library's per-GPU scratch array is
    used (msk_layer_step_noalloc); x is updated in place."""
    n = len(specs)
    cfgs = _array(LayerCfg, [make_cfg(s) for s in specs])
    wts = _array(LayerWeights, [make_weights(w) for w in weights])
    kva = _array(KV, [make_kv(k) for k in kvs])
    b = make_batch(kv_len, tokens_per_req)
    _check(lib().msk_layer_step_noalloc(cfgs, wts, kva, n, ctypes.byref(b), _ptr(x),
                                        _ptr(layer_out), _ptr(topk_idx), _ptr(win),
                                        _stream(stream)))
    return x


def noalloc_scratch_bytes():
    return lib().msk_noalloc_scratch_bytes()


def prefill_workspace(spec, n_tokens, device="cuda"):
    """A workspace for msk_moe_prefill of n_tokens tokens."""
    cfg = make_cfg(spec)
    n = lib().msk_moe_prefill_workspace_size(ctypes.byref(cfg), n_tokens)
    if n == 0:
        raise MskError(1, last_error())
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_prefill(spec, w, u, idx, wts, h, ws, out=None, stream=None):
    """Experts of a prefill batch: returns out = h + MoE(u)."""
    T, H = h.shape
    out = torch.empty_like(h) if out is None else out
    cfg, wt = make_cfg(spec), make_weights(w)
    _check(lib().msk_moe_prefill(ctypes.byref(cfg), ctypes.byref(wt), T, _ptr(u), _ptr(idx),
                                 _ptr(wts), _ptr(h), _ptr(out), _ptr(ws), ws.numel(),
                                 _stream(stream)))
    return out


def set_spin_limit(polls):
    """Polls before a barrier wait of the timeline call gives up (0: the
    default)."""
    _check(lib().msk_set_spin_limit(polls))


PHASES = ("qkv", "attn", "combine", "wo", "router", "topk", "gateup", "down", "step", "union",
          "moe_sum", "prep", "dense_sum")


def timer_start(phases=PHASES):
    """Time every later launch of the named phases' kernels with HIP events
    stamped by the dispatch (msk_timer_start); an empty list stops timing."""
    mask = 0
    for ph in phases:
        mask |= 1 << PHASES.index(ph)
    _check(lib().msk_timer_start(mask))


def timer_read(phase):
    """(summed milliseconds, launches) of one phase since timer_start."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().msk_timer_read(PHASES.index(phase), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def layer_step_timeline(specs, weights, kvs, kv_len, tokens_per_req, x, ws, stamps,
                        layer_out=None, topk_idx=None, win=None, stream=None):
    """layer_step run as the persistent step kernel where one exists, recording
    per-workgroup phase timestamps into `stamps` (int64 device tensor
    [4 * CUs][32], zero-filled)."""
    n = len(specs)
    cfgs = _array(LayerCfg, [make_cfg(s) for s in specs])
    wts = _array(LayerWeights, [make_weights(w) for w in weights])
    kva = _array(KV, [make_kv(k) for k in kvs])
    b = make_batch(kv_len, tokens_per_req)
    _check(lib().msk_layer_step_timeline(cfgs, wts, kva, n, ctypes.byref(b), _ptr(x),
                                         _ptr(layer_out), _ptr(topk_idx), _ptr(win), _ptr(stamps),
                                         _ptr(ws), ws.numel(), _stream(stream)))
    return x


class Step:
    """Pre-marshalled arguments of one whole-step call, for repeated launches
    (timing loops): building ctypes structs once keeps Python overhead out of
    the launch path.  With `stamps` the call is msk_layer_step_timeline (the
    persistent step kernel where one exists)."""

    def __init__(self, specs, weights, kvs, kv_len, tokens_per_req, x, ws, layer_out=None,
                 topk_idx=None, win=None, stamps=None):
        self.n = len(specs)
        self.cfgs = _array(LayerCfg, [make_cfg(s) for s in specs])
        self.wts = _array(LayerWeights, [make_weights(w) for w in weights])
        self.kva = _array(KV, [make_kv(k) for k in kvs])
        self.batch = make_batch(kv_len, tokens_per_req)
        head = (self.cfgs, self.wts, self.kva, self.n, ctypes.byref(self.batch), _ptr(x),
                _ptr(layer_out), _ptr(topk_idx), _ptr(win))
        if stamps is None:
            self.args = head + (_ptr(ws), ws.numel())
            self.fn = lib().msk_layer_step
        else:
            self.args = head + (_ptr(stamps), _ptr(ws), ws.numel())
            self.fn = lib().msk_layer_step_timeline

    def __call__(self, stream=None):
        _check(self.fn(*self.args, _stream(stream)))
