// C ABI of libmsk.so: argument checks, workspace layout, attention planning
// and the calls into the kernel launchers.  Every check runs before any HIP
// call, so invalid arguments return with nothing enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/msk.h"
#include "launch.h"
#include "params.h"

namespace {

// The last error text of this thread, in a fixed buffer: no entry point
// allocates host memory, on its error paths either.
thread_local char g_err[512];

msk_status fail(msk_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

msk_status ok() {
  g_err[0] = '\0';
  return MSK_OK;
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Target number of attention work items (one wave each) per layer: about
// two rounds of the waves that fit on the chip at once.
constexpr long long kTargetItems = 2048;
// Rounds of resident workgroups the matrix-core attention items fill.
constexpr long long kAttnRounds = 1;

struct AttnSplit {
  int chunk, n_items, nrg, rows, nw, nph;
};

// Query rows of one (request, kv head) pair, G * Tr, go to the matrix cores
// when they fill more than one row group of the vector path and the cache
// values are exact in bf16 (bf16 or e4m3 caches); each wave then takes 16
// rows (or half the positions of 16 rows), at most 64 rows per item.
AttnSplit plan_attention(const msk_layer_cfg& c, const msk_batch& b) {
  const int G = c.n_q_heads / c.n_kv_heads;
  const int M = G * b.tokens_per_req;
  const bool mfma = (c.kv_dtype == MSK_BF16 || c.kv_dtype == MSK_E4M3) && M > msk::kRowGroup;
  const int m1 = M < 64 ? M : 64;
  int nw = mfma ? cdiv(m1, 16) : 0;
  // head_dim 128: a one-wave item over a bf16 cache would prefetch a whole
  // 32-KB tile into one wave's registers, so two waves at least; e4m3 items
  // take four waves, whose smaller per-thread share of the tile lets three
  // waves per SIMD stay resident
  if (mfma && c.head_dim == 128 && c.kv_dtype == MSK_BF16 && nw < 2) nw = 2;
  int nph = 1;
  if (mfma && c.head_dim == 128 && c.kv_dtype == MSK_E4M3) {
    // up to two row tiles: pairs of waves split each tile's positions
    nph = nw <= 2 ? 2 : 1;
    nw = 4;
  }
  const int rows = mfma ? 16 * nw / nph : msk::kRowGroup;
  const int nrg = cdiv(M, rows);
  long long total = 0;
  for (int r = 0; r < b.n_req; ++r) {
    int base, end;
    msk::req_span(b.kv_len_host[r], b.tokens_per_req, c.window, mfma, base, end);
    total += (long long)(end - base) * c.n_kv_heads * nrg;
  }
  // matrix-core items: at most kAttnRounds rounds of the 768 workgroups
  // (three per CU on 256 CUs) that its e4m3 head_dim-128 form keeps resident.
  // Fewer, longer items mean fewer partials for the combine and less start-up
  // per item; the chunk grows until every request's partial last chunk still
  // fits, so no round is left with a handful of full-length items.  (The
  // e4m3 head_dim-128 items take their head's 64-position tiles round-robin
  // rather than as one range; the count of items is the same.)
  const long long target = mfma ? kAttnRounds * 768LL : kTargetItems;
  auto count = [&](long long ch) {
    long long n = 0;
    for (int r = 0; r < b.n_req; ++r) {
      int base, end;
      msk::req_span(b.kv_len_host[r], b.tokens_per_req, c.window, mfma, base, end);
      n += (long long)cdiv(end - base, ch) * c.n_kv_heads * nrg;
    }
    return n;
  };
  long long chunk = (total + target - 1) / target;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 64) chunk = 64;
  while (chunk < (1 << 20) && count(chunk) > target) chunk += 64;
  if (chunk > (1 << 20)) chunk = 1 << 20;
  return AttnSplit{(int)chunk, (int)count(chunk), nrg, rows, nw, nph};
}

struct Layout {
  size_t sync, qkv, part, attn_o, h, u, logits, idx, wts, act, xa, xb, uni, ybuf, a3, dpart, total;
};

// with_attention = false: the router and expert entry points, which take a
// flat token count and use no attention partials (nor more workspace than a
// layer step of the same tokens).
Layout layout(const msk_layer_cfg* cfg, int n_layers, const msk_batch& b,
              bool with_attention = true) {
  const msk_layer_cfg& c = cfg[0];
  const size_t T = (size_t)b.n_req * b.tokens_per_req;
  const size_t H = c.hidden, D = c.head_dim;
  const size_t NR = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * D;
  size_t max_rows = 0;
  for (int l = 0; l < n_layers && with_attention; ++l) {
    const AttnSplit a = plan_attention(cfg[l], b);
    const size_t rows_total = (size_t)a.n_items * a.rows;
    if (rows_total > max_rows) max_rows = rows_total;
  }
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up(bytes);
    return at;
  };
  L.sync = take(msk::kSyncBytes);
  L.qkv = take(T * NR * 4);
  L.part = take(max_rows * (D + 1) * 4);  // item rows of every layer
  L.attn_o = take(T * c.n_q_heads * D * 4);
  L.h = take(T * H * 4);
  L.u = take(T * H * 4);
  L.logits = take(T * c.n_experts * 4);
  L.idx = take(T * c.top_k * 4);
  L.wts = take(T * c.top_k * 4);
  L.act = take(T * c.top_k * (size_t)c.ffn_dim * 4);
  L.xa = take(T * H * 4);
  L.xb = take(T * H * 4);
  L.uni = take(sizeof(msk::Union));
  L.ybuf = take(T * c.top_k * H * 4);
  const size_t HQD = (size_t)c.n_q_heads * D;
  L.a3 = take(3 * T * (H > HQD ? H : HQD) * 2);
  size_t dp = 0;
  const int dense_n[3] = {(int)NR, (int)H, c.n_experts};
  const int dense_k[3] = {(int)H, (int)HQD, (int)H};
  for (int i = 0; i < 3; ++i) {
    const size_t need = (size_t)(dense_n[i] + 63) / 64 * 64 *
                        msk::dense_slices(dense_n[i], dense_k[i]) * T;
    dp = dp > need ? dp : need;
  }
  L.dpart = take(dp * 4);
  L.total = o;
  return L;
}

bool dtype_in(int v, std::initializer_list<int> set) {
  for (int s : set)
    if (v == s) return true;
  return false;
}

msk_status check_cfg(const msk_layer_cfg* c, int l) {
  if (!c) return fail(MSK_ERR_INVALID_ARG, "layer %d: cfg is null", l);
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->n_experts <= 0 || c->top_k <= 0 || c->ffn_dim <= 0)
    return fail(MSK_ERR_INVALID_ARG, "layer %d: every dimension must be positive", l);
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(MSK_ERR_INVALID_ARG, "layer %d: n_q_heads %d is not a multiple of n_kv_heads %d", l,
                c->n_q_heads, c->n_kv_heads);
  if (c->top_k > c->n_experts)
    return fail(MSK_ERR_INVALID_ARG, "layer %d: top_k %d > n_experts %d", l, c->top_k, c->n_experts);
  if (c->window < 0) return fail(MSK_ERR_INVALID_ARG, "layer %d: window %d < 0", l, c->window);
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: rms_eps must be positive and finite", l);
  if (!std::isfinite(c->softmax_shift))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: softmax_shift must be finite", l);
  if (!dtype_in(c->dense_dtype, {MSK_F32, MSK_BF16}))
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: dense_dtype %d unsupported (F32, BF16)", l,
                c->dense_dtype);
  if (!dtype_in(c->expert_dtype, {MSK_F32, MSK_BF16, MSK_NVFP4}))
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: expert_dtype %d unsupported (F32, BF16, NVFP4)", l,
                c->expert_dtype);
  if (!dtype_in(c->kv_dtype, {MSK_F32, MSK_BF16, MSK_E4M3}))
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: kv_dtype %d unsupported (F32, BF16, E4M3)", l,
                c->kv_dtype);
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: head_dim %d unsupported (32, 64, 128)", l, c->head_dim);
  if (c->kv_dtype == MSK_F32 && c->head_dim == 128)
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: fp32 KV cache needs head_dim <= 64", l);
  if (c->hidden % 32 != 0 || c->ffn_dim % 32 != 0)
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: hidden and ffn_dim must be multiples of 32", l);
  if (c->n_experts > msk::kMaxExperts)
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: n_experts %d > %d", l, c->n_experts, msk::kMaxExperts);
  if (c->top_k > msk::kMaxTopK)
    return fail(MSK_ERR_UNSUPPORTED, "layer %d: top_k %d > %d", l, c->top_k, msk::kMaxTopK);
  return ok();
}

msk_status check_same_shape(const msk_layer_cfg* a, const msk_layer_cfg* b, int l) {
  if (a->hidden != b->hidden || a->n_q_heads != b->n_q_heads || a->n_kv_heads != b->n_kv_heads ||
      a->head_dim != b->head_dim || a->n_experts != b->n_experts || a->top_k != b->top_k ||
      a->ffn_dim != b->ffn_dim)
    return fail(MSK_ERR_INVALID_ARG, "layer %d: shape differs from layer 0", l);
  return ok();
}

msk_status check_batch(const msk_batch* b) {
  if (!b) return fail(MSK_ERR_INVALID_ARG, "batch is null");
  if (b->n_req < 1 || b->n_req > MSK_MAX_REQ)
    return fail(MSK_ERR_INVALID_ARG, "n_req %d outside [1, %d]", b->n_req, MSK_MAX_REQ);
  if (b->tokens_per_req < 1)
    return fail(MSK_ERR_INVALID_ARG, "tokens_per_req %d < 1", b->tokens_per_req);
  if ((long long)b->n_req * b->tokens_per_req > MSK_MAX_TOKENS)
    return fail(MSK_ERR_UNSUPPORTED, "n_req * tokens_per_req = %lld > %d",
                (long long)b->n_req * b->tokens_per_req, MSK_MAX_TOKENS);
  if (!b->kv_len_host) return fail(MSK_ERR_INVALID_ARG, "kv_len_host is null");
  for (int r = 0; r < b->n_req; ++r) {
    if (b->kv_len_host[r] < 0)
      return fail(MSK_ERR_INVALID_ARG, "kv_len[%d] = %d < 0", r, b->kv_len_host[r]);
    if ((long long)b->kv_len_host[r] + b->tokens_per_req > (1LL << 30))
      return fail(MSK_ERR_UNSUPPORTED, "kv_len[%d] + tokens_per_req exceeds 2^30", r);
  }
  return ok();
}

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

msk_status check_kv(const msk_kv* kv, const msk_batch* b, int l) {
  if (!kv || !kv->k || !kv->v) return fail(MSK_ERR_INVALID_ARG, "layer %d: kv cache pointer is null", l);
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: kv cache is not 16-byte aligned", l);
  for (int r = 0; r < b->n_req; ++r)
    if ((long long)b->kv_len_host[r] + b->tokens_per_req > kv->cap)
      return fail(MSK_ERR_INVALID_ARG, "layer %d: kv_len[%d] + tokens_per_req = %lld > cap %lld", l, r,
                  (long long)b->kv_len_host[r] + b->tokens_per_req, (long long)kv->cap);
  return ok();
}

msk_status check_attn_weights(const msk_layer_weights* w, int l) {
  if (!w) return fail(MSK_ERR_INVALID_ARG, "layer %d: weights are null", l);
  if (!w->attn_norm || !w->q_norm || !w->k_norm || !w->wq || !w->wk || !w->wv || !w->wo)
    return fail(MSK_ERR_INVALID_ARG, "layer %d: an attention weight pointer is null", l);
  if (!aligned(w->wq, 16) || !aligned(w->wk, 16) || !aligned(w->wv, 16) || !aligned(w->wo, 16))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: an attention weight is not 16-byte aligned", l);
  return ok();
}

msk_status check_route_weights(const msk_layer_weights* w, int l) {
  if (!w) return fail(MSK_ERR_INVALID_ARG, "layer %d: weights are null", l);
  if (!w->ffn_norm || !w->w_router)
    return fail(MSK_ERR_INVALID_ARG, "layer %d: ffn_norm or w_router is null", l);
  if (!aligned(w->w_router, 16))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: w_router is not 16-byte aligned", l);
  return ok();
}

msk_status check_expert_weights(const msk_layer_cfg* c, const msk_layer_weights* w, int l) {
  if (!w) return fail(MSK_ERR_INVALID_ARG, "layer %d: weights are null", l);
  if (!w->w_gate || !w->w_up || !w->w_down)
    return fail(MSK_ERR_INVALID_ARG, "layer %d: an expert weight pointer is null", l);
  if (c->expert_dtype == MSK_NVFP4 &&
      (!w->s_gate || !w->s_up || !w->s_down || !w->g_gate || !w->g_up || !w->g_down))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: NVFP4 experts need block and matrix scales", l);
  if (!aligned(w->w_gate, 16) || !aligned(w->w_up, 16) || !aligned(w->w_down, 16))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: an expert weight is not 16-byte aligned", l);
  if (c->expert_dtype == MSK_NVFP4 &&
      (!aligned(w->s_gate, 4) || !aligned(w->s_up, 4) || !aligned(w->s_down, 4)))
    return fail(MSK_ERR_INVALID_ARG, "layer %d: an NVFP4 scale array is not 4-byte aligned", l);
  return ok();
}

#define CHECK(x)                       \
  do {                                 \
    msk_status s_ = (x);               \
    if (s_ != MSK_OK) return s_;       \
  } while (0)

msk::LayerArgs make_layer(const msk_layer_cfg& c, const msk_layer_weights* w, const msk_kv* kv,
                          const msk_batch* b) {
  msk::LayerArgs L{};
  L.H = c.hidden;
  L.Hq = c.n_q_heads;
  L.Hkv = c.n_kv_heads;
  L.D = c.head_dim;
  L.E = c.n_experts;
  L.K = c.top_k;
  L.F = c.ffn_dim;
  L.window = c.window;
  L.eps = c.rms_eps;
  L.shift = c.softmax_shift;
  L.qscale = (float)(1.0 / std::sqrt((double)c.head_dim));
  L.ddt = c.dense_dtype;
  L.edt = c.expert_dtype;
  L.kdt = c.kv_dtype;
  if (w) {
    L.attn_norm = w->attn_norm;
    L.q_norm = w->q_norm;
    L.k_norm = w->k_norm;
    L.ffn_norm = w->ffn_norm;
    L.wq = static_cast<const uint8_t*>(w->wq);
    L.wk = static_cast<const uint8_t*>(w->wk);
    L.wv = static_cast<const uint8_t*>(w->wv);
    L.wo = static_cast<const uint8_t*>(w->wo);
    L.wr = static_cast<const uint8_t*>(w->w_router);
    L.wg = static_cast<const uint8_t*>(w->w_gate);
    L.wu = static_cast<const uint8_t*>(w->w_up);
    L.wd = static_cast<const uint8_t*>(w->w_down);
    L.sg = w->s_gate;
    L.su = w->s_up;
    L.sd = w->s_down;
    L.gg = w->g_gate;
    L.gu = w->g_up;
    L.gd = w->g_down;
  }
  if (kv) {
    L.kc = static_cast<uint8_t*>(kv->k);
    L.vc = static_cast<uint8_t*>(kv->v);
    L.cap = kv->cap;
  }
  if (b) {
    const AttnSplit a = plan_attention(c, *b);
    L.chunk = a.chunk;
    L.n_items = a.n_items;
    L.nrg = a.nrg;
    L.rg_rows = a.rows;
    L.attn_nw = a.nw;
    L.attn_nph = a.nph;
  }
  return L;
}

msk::StepArgs make_step(const Layout& lay, void* ws, int n_req, int Tr, const int32_t* kv_len) {
  msk::StepArgs S{};
  S.n_req = n_req;
  S.Tr = Tr;
  S.T = n_req * Tr;
  for (int r = 0; r < n_req && kv_len; ++r) S.kv_len[r] = kv_len[r];
  uint8_t* base = static_cast<uint8_t*>(ws);
  S.sync = reinterpret_cast<unsigned*>(base + lay.sync);
  S.qkv = reinterpret_cast<float*>(base + lay.qkv);
  S.part = reinterpret_cast<float*>(base + lay.part);
  S.attn_o = reinterpret_cast<float*>(base + lay.attn_o);
  S.h = reinterpret_cast<float*>(base + lay.h);
  S.u = reinterpret_cast<float*>(base + lay.u);
  S.logits = reinterpret_cast<float*>(base + lay.logits);
  S.idx = reinterpret_cast<int*>(base + lay.idx);
  S.wts = reinterpret_cast<float*>(base + lay.wts);
  S.act = reinterpret_cast<float*>(base + lay.act);
  S.xa = reinterpret_cast<float*>(base + lay.xa);
  S.xb = reinterpret_cast<float*>(base + lay.xb);
  S.uni = reinterpret_cast<msk::Union*>(base + lay.uni);
  S.ybuf = reinterpret_cast<float*>(base + lay.ybuf);
  S.a3 = reinterpret_cast<unsigned short*>(base + lay.a3);
  S.dpart = reinterpret_cast<float*>(base + lay.dpart);
  return S;
}

msk_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MSK_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Polls before a device-side wait gives up (msk_set_spin_limit).
std::atomic<unsigned> g_spin_limit{msk::kSpinLimit};

// Reads the workspace's error word once the device is idle; a set word is
// reported as MSK_ERR_TIMEOUT and the synchronisation words are reset, so
// the next call starts clean.
#define MSK_TRY_HOST(x)                \
  do {                                 \
    const hipError_t e_ = (x);         \
    if (e_ != hipSuccess) return e_;   \
  } while (0)
msk_status read_watchdog(void* ws) {
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return device_status(e, "hipDeviceSynchronize");
  unsigned words[2] = {0, 0};
  e = hipMemcpy(words, ws, sizeof(words), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return device_status(e, "hipMemcpy");
  if (words[1] == 0) return ok();
  e = hipMemset(ws, 0, msk::kSyncBytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return device_status(e, "hipMemset");
  return fail(MSK_ERR_TIMEOUT, "a device-side wait of an earlier call on this workspace gave up "
                               "(barrier watchdog)");
}

// Workspaces whose latest launch was the persistent step kernel, the one
// kernel with device-side waits.  Behind such a launch the library copies the
// workspace's error word to pinned host memory on the launch's stream and
// records an event.  Every later call on the workspace looks at the event
// without waiting: once it has completed, the call reads the copied word
// before it enqueues anything and reports a wait that gave up.  So the first
// call that starts after the launch has finished reports its trip (a call
// made while it still runs cannot know), and msk_workspace_status, which
// synchronises, always does.  At most kWatched workspaces are tracked; past
// that the oldest is dropped, and a trip of its launch stays in the workspace
// for msk_workspace_status to report.
struct Watch {
  void* ws;       // nullptr: free
  hipEvent_t ev;  // created on first use, on device `dev`
  int dev;
};
constexpr int kWatched = 64;
std::mutex g_watch_mu;
Watch g_watch[kWatched];
int g_watch_next = 0;            // the slot a full table gives up next
unsigned* g_flag = nullptr;      // pinned host copies of the error words [kWatched]

hipError_t watch(void* ws, hipStream_t st) {
  std::lock_guard<std::mutex> g(g_watch_mu);
  if (!g_flag) {
    MSK_TRY_HOST(hipHostMalloc(reinterpret_cast<void**>(&g_flag), kWatched * sizeof(unsigned),
                               hipHostMallocDefault));
    for (int i = 0; i < kWatched; ++i) g_flag[i] = 0;
  }
  int i = -1;
  for (int k = 0; k < kWatched && i < 0; ++k)
    if (g_watch[k].ws == ws) i = k;
  for (int k = 0; k < kWatched && i < 0; ++k)
    if (g_watch[k].ws == nullptr) i = k;
  if (i < 0) {
    i = g_watch_next;
    g_watch_next = (g_watch_next + 1) % kWatched;
  }
  int dev = 0;
  MSK_TRY_HOST(hipGetDevice(&dev));
  Watch& w = g_watch[i];
  if (w.ev == nullptr || w.dev != dev) {
    if (w.ev != nullptr) MSK_TRY_HOST(hipEventDestroy(w.ev));
    w.ev = nullptr;
    MSK_TRY_HOST(hipEventCreateWithFlags(&w.ev, hipEventDisableTiming));
    w.dev = dev;
  }
  w.ws = ws;
  MSK_TRY_HOST(hipMemcpyAsync(&g_flag[i], static_cast<uint8_t*>(ws) + sizeof(unsigned),
                              sizeof(unsigned), hipMemcpyDeviceToHost, st));
  return hipEventRecord(w.ev, st);
}

// Forgets the workspace (msk_workspace_status reads its word itself).
void unwatch(void* ws) {
  std::lock_guard<std::mutex> g(g_watch_mu);
  for (int k = 0; k < kWatched; ++k)
    if (g_watch[k].ws == ws) g_watch[k].ws = nullptr;
}

// The watchdog check every call on a workspace makes after its argument
// checks (see Watch).
msk_status watchdog(void* ws) {
  unsigned flag = 0;
  {
    std::lock_guard<std::mutex> g(g_watch_mu);
    int i = -1;
    for (int k = 0; k < kWatched && i < 0; ++k)
      if (g_watch[k].ws == ws) i = k;
    if (i < 0) return MSK_OK;
    const hipError_t e = hipEventQuery(g_watch[i].ev);
    if (e == hipErrorNotReady) return MSK_OK;  // still running: a later call looks again
    if (e != hipSuccess) return device_status(e, "hipEventQuery");
    flag = *static_cast<volatile unsigned*>(&g_flag[i]);
    g_watch[i].ws = nullptr;
  }
  return flag == 0 ? MSK_OK : read_watchdog(ws);
}

// Workspace of the prefill expert FFN for n tokens (see msk::PfArgs).
struct PfLayout {
  size_t off, nchunk, chunk, cur, perm, pos, pe, ue, ae, a, gu, act, y, total;
};
PfLayout pf_layout(const msk_layer_cfg& c, int n) {
  const size_t S = (size_t)n * c.top_k, E = c.n_experts, H = c.hidden, F = c.ffn_dim;
  PfLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up(bytes);
    return at;
  };
  L.off = take((E + 1) * sizeof(int));
  L.nchunk = take(sizeof(int));
  L.chunk = take((S / msk::kPfChunk + E + 1) * sizeof(msk::PfChunk));
  L.cur = take(E * sizeof(int));
  L.perm = take(S * sizeof(int));
  L.pos = take(S * sizeof(int));
  L.pe = take(S * sizeof(int));
  L.ue = take(S * sizeof(int));
  L.ae = take(S * sizeof(int));
  L.a = take(2 * (size_t)n * H * 2);  // by token: fp16, or two bf16 term planes
  L.gu = take(S * 2 * F * sizeof(float));
  L.act = take(2 * S * F * 2);
  L.y = take(S * H * sizeof(float));
  L.total = o;
  return L;
}

msk_status check_prefill(const msk_layer_cfg* cfg, const msk_layer_weights* w, int32_t n) {
  CHECK(check_cfg(cfg, 0));
  if (n < 1 || n > MSK_MAX_PREFILL_TOKENS)
    return fail(MSK_ERR_INVALID_ARG, "n_tokens %d outside [1, %d]", n, MSK_MAX_PREFILL_TOKENS);
  if (cfg->expert_dtype != MSK_BF16 && cfg->expert_dtype != MSK_NVFP4)
    return fail(MSK_ERR_UNSUPPORTED, "prefill experts are bf16 or NVFP4");
  if (cfg->hidden % 128 || cfg->ffn_dim % 128)
    return fail(MSK_ERR_UNSUPPORTED, "prefill needs hidden and ffn_dim multiples of 128");
  if (w) CHECK(check_expert_weights(cfg, w, 0));
  return ok();
}

// A one-token batch description for the calls that take only a token count.
struct FlatBatch {
  int32_t zero[MSK_MAX_TOKENS] = {};
  msk_batch b{};
  explicit FlatBatch(int T) {
    b.n_req = T;
    b.tokens_per_req = 1;
    b.kv_len_host = zero;
  }
};

}  // namespace

extern "C" {

int32_t msk_abi_version(void) { return MSK_ABI_VERSION; }

const char* msk_last_error(void) { return g_err; }

size_t msk_workspace_size(const msk_layer_cfg* cfg, int32_t n_layers, const msk_batch* batch) {
  if (!cfg || n_layers < 1 || n_layers > MSK_MAX_STACK) {
    fail(MSK_ERR_INVALID_ARG, "n_layers %d outside [1, %d] or cfg null", n_layers, MSK_MAX_STACK);
    return 0;
  }
  for (int l = 0; l < n_layers; ++l) {
    if (check_cfg(&cfg[l], l) != MSK_OK) return 0;
    if (l > 0 && check_same_shape(&cfg[0], &cfg[l], l) != MSK_OK) return 0;
  }
  if (check_batch(batch) != MSK_OK) return 0;
  ok();
  return layout(cfg, n_layers, *batch).total;
}

msk_status msk_workspace_status(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < (size_t)msk::kSyncBytes)
    return fail(MSK_ERR_WORKSPACE, "workspace missing or too small");
  const hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_status(e, "hipStreamSynchronize");
  unwatch(ws);
  return read_watchdog(ws);
}

msk_status msk_attn_step(const msk_layer_cfg* cfg, const msk_layer_weights* w, const msk_kv* kv,
                         const msk_batch* batch, const float* x, float* h, float* attn_o,
                         int32_t* win, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg, 0));
  CHECK(check_batch(batch));
  CHECK(check_kv(kv, batch, 0));
  CHECK(check_attn_weights(w, 0));
  if (!x || !h) return fail(MSK_ERR_INVALID_ARG, "x or h is null");
  if (x == h) return fail(MSK_ERR_INVALID_ARG, "x and h must not overlap");
  const Layout lay = layout(cfg, 1, *batch);
  if (!ws || ws_bytes < lay.total)
    return fail(MSK_ERR_WORKSPACE, "workspace %zu B < required %zu B", ws_bytes, lay.total);
  CHECK(watchdog(ws));
  msk::LayerArgs L = make_layer(*cfg, w, kv, batch);
  msk::StepArgs S = make_step(lay, ws, batch->n_req, batch->tokens_per_req, batch->kv_len_host);
  S.n_layers = 1;
  if (attn_o) S.attn_o = attn_o;
  S.win_out = win;
  return device_status(msk::launch_attn(L, S, x, h, static_cast<hipStream_t>(stream)),
                       "attention launch");
}

msk_status msk_moe_route(const msk_layer_cfg* cfg, const msk_layer_weights* w, int32_t n_tokens,
                         const float* h, float* u, int32_t* topk_idx, float* topk_w, float* logits,
                         void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg, 0));
  CHECK(check_route_weights(w, 0));
  if (n_tokens < 1 || n_tokens > MSK_MAX_TOKENS)
    return fail(MSK_ERR_INVALID_ARG, "n_tokens %d outside [1, %d]", n_tokens, MSK_MAX_TOKENS);
  if (!h || !u || !topk_idx || !topk_w) return fail(MSK_ERR_INVALID_ARG, "an output or h is null");
  FlatBatch fb(n_tokens);
  const Layout lay = layout(cfg, 1, fb.b, false);
  if (!ws || ws_bytes < lay.total)
    return fail(MSK_ERR_WORKSPACE, "workspace %zu B < required %zu B", ws_bytes, lay.total);
  CHECK(watchdog(ws));
  msk::LayerArgs L = make_layer(*cfg, w, nullptr, nullptr);
  msk::StepArgs S = make_step(lay, ws, n_tokens, 1, nullptr);
  S.u = u;
  S.idx = topk_idx;
  S.wts = topk_w;
  if (logits) S.logits = logits;
  return device_status(msk::launch_route(L, S, h, nullptr, static_cast<hipStream_t>(stream)),
                       "router launch");
}

msk_status msk_expert_ffn(const msk_layer_cfg* cfg, const msk_layer_weights* w, int32_t n_tokens,
                          const float* u, const int32_t* topk_idx, const float* topk_w,
                          const float* h, float* out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg, 0));
  CHECK(check_expert_weights(cfg, w, 0));
  if (n_tokens < 1 || n_tokens > MSK_MAX_TOKENS)
    return fail(MSK_ERR_INVALID_ARG, "n_tokens %d outside [1, %d]", n_tokens, MSK_MAX_TOKENS);
  if (!u || !topk_idx || !topk_w || !h || !out)
    return fail(MSK_ERR_INVALID_ARG, "an input or output pointer is null");
  FlatBatch fb(n_tokens);
  const Layout lay = layout(cfg, 1, fb.b, false);
  if (!ws || ws_bytes < lay.total)
    return fail(MSK_ERR_WORKSPACE, "workspace %zu B < required %zu B", ws_bytes, lay.total);
  CHECK(watchdog(ws));
  msk::LayerArgs L = make_layer(*cfg, w, nullptr, nullptr);
  msk::StepArgs S = make_step(lay, ws, n_tokens, 1, nullptr);
  S.u = const_cast<float*>(u);
  S.idx = const_cast<int*>(topk_idx);
  S.wts = const_cast<float*>(topk_w);
  return device_status(msk::launch_ffn(L, S, h, out, static_cast<hipStream_t>(stream)),
                       "expert launch");
}

// noalloc: the workspace is the library's per-GPU scratch array (ws and
// ws_bytes unused), and the call allocates nothing.
static msk_status layer_step_impl(const msk_layer_cfg* cfg, const msk_layer_weights* w,
                                  const msk_kv* kv, int32_t n_layers, const msk_batch* batch,
                                  float* x, float* layer_out, int32_t* topk_idx, int32_t* win,
                                  int64_t* stamps, void* ws, size_t ws_bytes, void* stream,
                                  bool noalloc = false) {
  if (!cfg || !w || !kv) return fail(MSK_ERR_INVALID_ARG, "cfg, w or kv is null");
  if (n_layers < 1 || n_layers > MSK_MAX_STACK)
    return fail(MSK_ERR_INVALID_ARG, "n_layers %d outside [1, %d]", n_layers, MSK_MAX_STACK);
  CHECK(check_batch(batch));
  for (int l = 0; l < n_layers; ++l) {
    CHECK(check_cfg(&cfg[l], l));
    if (l > 0) CHECK(check_same_shape(&cfg[0], &cfg[l], l));
    CHECK(check_kv(&kv[l], batch, l));
    CHECK(check_attn_weights(&w[l], l));
    CHECK(check_route_weights(&w[l], l));
    CHECK(check_expert_weights(&cfg[l], &w[l], l));
  }
  if (!x) return fail(MSK_ERR_INVALID_ARG, "x is null");
  const Layout lay = layout(cfg, n_layers, *batch);
  if (noalloc) {
    if (lay.total > msk::kScratchBytes)
      return fail(MSK_ERR_WORKSPACE,
                  "this step needs %zu B of scratch; the allocation-free entry point holds "
                  "%zu B per GPU",
                  lay.total, msk::kScratchBytes);
    const hipError_t e = msk::scratch_address(&ws);
    if (e != hipSuccess) return device_status(e, "scratch address");
    ws_bytes = msk::kScratchBytes;
  }
  if (!ws || ws_bytes < lay.total)
    return fail(MSK_ERR_WORKSPACE, "workspace %zu B < required %zu B", ws_bytes, lay.total);
  if (!noalloc) CHECK(watchdog(ws));
  msk::LayerArgs Ls[msk::kMaxLayers];
  for (int l = 0; l < n_layers; ++l) Ls[l] = make_layer(cfg[l], &w[l], &kv[l], batch);
  msk::StepArgs S = make_step(lay, ws, batch->n_req, batch->tokens_per_req, batch->kv_len_host);
  S.n_layers = n_layers;
  S.x_in = x;
  S.x_out = x;
  S.layer_out = layer_out;
  S.topk_out = topk_idx;
  S.win_out = win;
  S.stamps = reinterpret_cast<long long*>(stamps);
  S.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  // Per-phase kernels measure faster than the persistent kernel on this part
  // (its grid barriers cost more than the kernel boundaries they replace),
  // so only the timeline call, whose in-kernel stamps need it, runs the
  // persistent kernel.
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (noalloc) return device_status(msk::launch_step_noalloc(Ls, S, st), "layer-step launch");
  if (!stamps) return device_status(msk::launch_step_unfused(Ls, S, st), "layer-step launch");
  bool persistent = false;
  hipError_t e = msk::launch_step_fused(Ls, S, st, &persistent);
  if (e == hipSuccess && persistent) e = watch(ws, st);
  return device_status(e, "layer-step launch");
}

msk_status msk_layer_step(const msk_layer_cfg* cfg, const msk_layer_weights* w, const msk_kv* kv,
                          int32_t n_layers, const msk_batch* batch, float* x, float* layer_out,
                          int32_t* topk_idx, int32_t* win, void* ws, size_t ws_bytes,
                          void* stream) {
  return layer_step_impl(cfg, w, kv, n_layers, batch, x, layer_out, topk_idx, win, nullptr, ws,
                         ws_bytes, stream);
}

msk_status msk_layer_step_noalloc(const msk_layer_cfg* cfg, const msk_layer_weights* w,
                                  const msk_kv* kv, int32_t n_layers, const msk_batch* batch,
                                  float* x, float* layer_out, int32_t* topk_idx, int32_t* win,
                                  void* stream) {
  return layer_step_impl(cfg, w, kv, n_layers, batch, x, layer_out, topk_idx, win, nullptr,
                         nullptr, 0, stream, /*noalloc=*/true);
}

size_t msk_noalloc_scratch_bytes(void) { return msk::kScratchBytes; }

size_t msk_moe_prefill_workspace_size(const msk_layer_cfg* cfg, int32_t n_tokens) {
  if (!cfg) {
    fail(MSK_ERR_INVALID_ARG, "cfg is null");
    return 0;
  }
  if (check_prefill(cfg, nullptr, n_tokens) != MSK_OK) return 0;
  ok();
  return pf_layout(*cfg, n_tokens).total;
}

msk_status msk_moe_prefill(const msk_layer_cfg* cfg, const msk_layer_weights* w, int32_t n_tokens,
                           const float* u, const int32_t* topk_idx, const float* topk_w,
                           const float* h, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!cfg || !w) return fail(MSK_ERR_INVALID_ARG, "cfg or w is null");
  CHECK(check_prefill(cfg, w, n_tokens));
  if (!u || !topk_idx || !topk_w || !h || !out)
    return fail(MSK_ERR_INVALID_ARG, "an input or output pointer is null");
  if (!aligned(u, 16) || !aligned(h, 16) || !aligned(out, 16))
    return fail(MSK_ERR_INVALID_ARG, "u, h and out must be 16-byte aligned");
  const PfLayout lay = pf_layout(*cfg, n_tokens);
  if (!ws || ws_bytes < lay.total)
    return fail(MSK_ERR_WORKSPACE, "workspace %zu B < required %zu B", ws_bytes, lay.total);
  CHECK(watchdog(ws));
  msk::LayerArgs L = make_layer(*cfg, w, nullptr, nullptr);
  uint8_t* base = static_cast<uint8_t*>(ws);
  msk::PfArgs P{};
  P.T = n_tokens;
  P.idx = topk_idx;
  P.u = u;
  P.off = reinterpret_cast<int*>(base + lay.off);
  P.nchunk = reinterpret_cast<int*>(base + lay.nchunk);
  P.chunk = reinterpret_cast<msk::PfChunk*>(base + lay.chunk);
  P.cur = reinterpret_cast<int*>(base + lay.cur);
  P.perm = reinterpret_cast<int*>(base + lay.perm);
  P.pos = reinterpret_cast<int*>(base + lay.pos);
  P.pe = reinterpret_cast<int*>(base + lay.pe);
  P.ue = reinterpret_cast<int*>(base + lay.ue);
  P.ae = reinterpret_cast<int*>(base + lay.ae);
  P.a = reinterpret_cast<unsigned short*>(base + lay.a);
  P.gu = reinterpret_cast<float*>(base + lay.gu);
  P.act = reinterpret_cast<unsigned short*>(base + lay.act);
  P.y = reinterpret_cast<float*>(base + lay.y);
  return device_status(msk::launch_prefill(L, P, topk_w, h, out, static_cast<hipStream_t>(stream)),
                       "prefill launch");
}

msk_status msk_set_spin_limit(uint32_t polls) {
  g_spin_limit.store(polls ? polls : msk::kSpinLimit, std::memory_order_relaxed);
  return ok();
}

msk_status msk_layer_step_timeline(const msk_layer_cfg* cfg, const msk_layer_weights* w,
                                   const msk_kv* kv, int32_t n_layers, const msk_batch* batch,
                                   float* x, float* layer_out, int32_t* topk_idx, int32_t* win,
                                   int64_t* stamps, void* ws, size_t ws_bytes, void* stream) {
  if (!stamps) return fail(MSK_ERR_INVALID_ARG, "stamps is null");
  return layer_step_impl(cfg, w, kv, n_layers, batch, x, layer_out, topk_idx, win, stamps, ws,
                         ws_bytes, stream);
}

static_assert(MSK_N_PHASES == msk::kNumPhases && MSK_PH_STEP == msk::kPhStep &&
                  MSK_PH_UNION == msk::kPhUnion && MSK_PH_MOE_SUM == msk::kPhMoeSum &&
                  MSK_PH_PREP == msk::kPhPrep && MSK_PH_DENSE_SUM == msk::kPhDenseSum &&
                  MSK_PH_GATEUP == msk::kPhGateUp && MSK_PH_ATTN == msk::kPhAttn,
              "phase numbering of the header and the launchers must agree");

msk_status msk_timer_start(uint32_t mask) {
  if (mask >> msk::kNumPhases) return fail(MSK_ERR_INVALID_ARG, "timer mask names no phase");
  return device_status(msk::timer_start(mask), "timer start");
}

msk_status msk_timer_read(int32_t phase, double* total_ms, int64_t* launches) {
  if (phase < 0 || phase >= msk::kNumPhases) return fail(MSK_ERR_INVALID_ARG, "no such phase");
  if (!total_ms || !launches) return fail(MSK_ERR_INVALID_ARG, "null output");
  long long n = 0;
  const msk_status st = device_status(msk::timer_read(phase, total_ms, &n), "timer read");
  *launches = n;
  return st;
}

}  // extern "C"
