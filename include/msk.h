/*
 * msk.h -- C ABI of libmsk.so: one decode/verify step of a mixture-of-experts
 * decoder layer (or a short stack of them) on an AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the pages on "Optimizing Muse Spark Open on TPU v7
 * with SGLang-TorchTPU" describe: every decoder layer is a mixture-of-experts
 * layer that routes each token to 8 of 256 experts and mixes sliding-window
 * (2,048 tokens) with full-context attention (ainewsbites page, section "One
 * program replaces many kernel boundaries"); QK-norm lets softmax run without
 * a running maximum, so context chunks reduce independently (brifing.si page,
 * section "Removing Attention Bottlenecks"); the KV cache is fp8 (aitop.news
 * page, opening paragraphs); expert weights are NVFP4 with one scale per 16
 * values (brifing.si page, "Expert Weight Quantization"); a verify step checks
 * the draft tokens of each request in one pass (brifing.si page, "Speculative
 * Decoding Integration").  The serving stack keeps embedding, draft model, LM
 * head and sampling (ainewsbites page, "One program replaces many kernel
 * boundaries"), so the step maps hidden states in to hidden states out.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *   allocates no device memory and keeps no state between calls; scratch space
 *   comes from the caller's workspace (see msk_workspace_size).
 * - Weight matrices and KV caches are 16-byte aligned, NVFP4 scale arrays
 *   4-byte aligned; a misaligned pointer is an argument error.
 * - Row-major, innermost dimension last.  T = n_req * tokens_per_req tokens,
 *   request-major: token t of request b is row b * tokens_per_req + t and sits
 *   at cache position p = kv_len[b] + t.
 * - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream) and
 *   return without waiting.  Nothing is synchronised implicitly.
 * - Argument errors return before anything is enqueued; msk_last_error()
 *   then describes them.  A failed launch returns MSK_ERR_DEVICE.
 * - A workspace must not be used by two calls that may run at the same time.
 *   It must be zero-filled before its first use; afterwards calls keep its
 *   synchronisation words consistent themselves (never clear it again, except
 *   through msk_workspace_status after a timeout).
 * - The KV cache is written at positions [kv_len[b], kv_len[b] + tokens_per_req)
 *   only; lengths are never changed by the library (accepting or rejecting
 *   drafts is the caller's business).
 */
#ifndef MSK_H
#define MSK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSK_ABI_VERSION 1
#define MSK_MAX_REQ 64       /* requests per call                          */
#define MSK_MAX_TOKENS 64    /* T = n_req * tokens_per_req per call         */
#define MSK_MAX_PREFILL_TOKENS 8192 /* tokens per msk_moe_prefill call        */
#define MSK_MAX_STACK 64     /* layers per msk_layer_step call             */

typedef enum {
  MSK_OK = 0,
  MSK_ERR_INVALID_ARG = 1, /* null pointer, inconsistent shape, bad length   */
  MSK_ERR_UNSUPPORTED = 2, /* valid but outside what this library handles   */
  MSK_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  MSK_ERR_DEVICE = 4,      /* a HIP call or launch failed                   */
  MSK_ERR_TIMEOUT = 5      /* a device-side wait of an earlier call on the same
                              workspace gave up (see msk_workspace_status) */
} msk_status;

typedef enum {
  MSK_F32 = 0,   /* IEEE binary32                                              */
  MSK_BF16 = 1,  /* bfloat16 bit patterns (uint16)                             */
  MSK_E4M3 = 2,  /* OCP FP8 E4M3FN bytes, no scale (KV cache only)             */
  MSK_NVFP4 = 3  /* e2m1 codes, 2 per byte (even element in the low nibble),
                    one e4m3 scale per 16 consecutive elements along the
                    reduction dimension, one fp32 scale per matrix (experts only) */
} msk_dtype;

/* Shape and numeric configuration of one layer. */
typedef struct {
  int32_t hidden;      /* H: hidden size; multiple of 32                        */
  int32_t n_q_heads;   /* Hq: query heads; multiple of n_kv_heads                */
  int32_t n_kv_heads;  /* Hkv: key/value heads; query head h uses kv head
                          h / (Hq / Hkv) (contiguous groups)                      */
  int32_t head_dim;    /* D: 32, 64 or 128                                       */
  int32_t n_experts;   /* E: 1..256                                              */
  int32_t top_k;       /* k: experts per token, 1..min(E, 16)                   */
  int32_t ffn_dim;     /* F: expert FFN width; multiple of 32                    */
  int32_t window;      /* 0 = full context; W > 0 = sliding window of the W
                          positions ending at the token itself: [p-W+1, p]       */
  float rms_eps;       /* eps of all RMSNorms: x / sqrt(mean(x^2) + eps) * g     */
  float softmax_shift; /* c: fixed score bound; attention weights are
                          exp(s - c) summed without a running maximum.  Any c
                          with s - c < 88 for every score gives the same result
                          up to rounding.  0: the library takes the bound of
                          QK-normalised scores from the gains on the device,
                          c = sqrt(D) * max|q_norm| * max|k_norm|             */
  int32_t dense_dtype;  /* MSK_F32 | MSK_BF16: wq, wk, wv, wo, w_router          */
  int32_t expert_dtype; /* MSK_F32 | MSK_BF16 | MSK_NVFP4: w_gate, w_up, w_down  */
  int32_t kv_dtype;     /* MSK_F32 (head_dim <= 64) | MSK_BF16 | MSK_E4M3        */
} msk_layer_cfg;

/* Weights of one layer (device pointers, caller-owned, read only). */
typedef struct {
  const float *attn_norm;  /* [H]  gain of the attention RMSNorm                 */
  const float *q_norm;     /* [D]  QK-norm gain for queries (shared by heads)    */
  const float *k_norm;     /* [D]  QK-norm gain for keys                         */
  const float *ffn_norm;   /* [H]  gain of the FFN RMSNorm                       */
  const void *wq;          /* [Hq*D][H]  row h*D+d produces query head h, dim d  */
  const void *wk;          /* [Hkv*D][H]                                         */
  const void *wv;          /* [Hkv*D][H]                                         */
  const void *wo;          /* [H][Hq*D]                                          */
  const void *w_router;    /* [E][H]  logits = w_router . u, no bias             */
  const void *w_gate;      /* [E][F][H]  (NVFP4: uint8 [E][F][H/2])              */
  const void *w_up;        /* [E][F][H]  (NVFP4: uint8 [E][F][H/2])              */
  const void *w_down;      /* [E][H][F]  (NVFP4: uint8 [E][H][F/2])              */
  const uint8_t *s_gate;   /* NVFP4 only: e4m3 [E][F][H/16]                      */
  const uint8_t *s_up;     /* NVFP4 only: e4m3 [E][F][H/16]                      */
  const uint8_t *s_down;   /* NVFP4 only: e4m3 [E][H][F/16]                      */
  const float *g_gate;     /* NVFP4 only: fp32 per-matrix scale [E]              */
  const float *g_up;       /* NVFP4 only: [E]                                    */
  const float *g_down;     /* NVFP4 only: [E]                                    */
} msk_layer_weights;

/* KV cache of one layer: k, v are [n_req][Hkv][cap][D] in kv_dtype.  Positions
 * [0, kv_len[b]) hold request b's cached keys (already QK-normalised) and
 * values; the step appends at [kv_len[b], kv_len[b] + tokens_per_req). */
typedef struct {
  void *k;
  void *v;
  int64_t cap;
} msk_kv;

/* Batch description.  kv_len_host is a HOST array [n_req]: positions cached
 * per request before this step. */
typedef struct {
  int32_t n_req;           /* 1..MSK_MAX_REQ                                     */
  int32_t tokens_per_req;  /* Tr: 1 for decode, the draft length for verify      */
  const int32_t *kv_len_host;
} msk_batch;

/* ABI version of the loaded library (MSK_ABI_VERSION). */
int32_t msk_abi_version(void);

/* Text of the last error returned on this thread; valid until the next call. */
const char *msk_last_error(void);

/* Bytes of workspace the calls below need for these layers and this batch
 * (the largest need over the entry points, so one workspace serves all of
 * them).  Returns 0 and sets msk_last_error() on invalid arguments. */
size_t msk_workspace_size(const msk_layer_cfg *cfg, int32_t n_layers,
                          const msk_batch *batch);

/* Synchronises `stream` and the device, then reports whether a device-side
 * wait in a call that used `ws` gave up (MSK_ERR_TIMEOUT; the workspace's
 * synchronisation words are then reset so the next call starts clean) or
 * MSK_OK.  MSK_ERR_DEVICE if the stream reports an error.  Without this call
 * a later call on `ws` reports such a wait the same way, after its argument
 * checks and before it enqueues anything (see msk_layer_step_timeline). */
msk_status msk_workspace_status(void *ws, size_t ws_bytes, void *stream);

/* Attention half of a layer (steps: attention RMSNorm, QKV projection,
 * QK-norm, KV append, windowed no-max split-KV attention, output projection
 * with residual).  Defined by: QK-norm and softmax without a running maximum,
 * chunks reduced independently (brifing.si page, "Removing Attention
 * Bottlenecks"); sliding-window 2,048 or full-context attention (ainewsbites
 * page, "One program replaces many kernel boundaries"; brifing.si page, "Model
 * Architecture Details"); the fp8 cache (aitop.news page, opening paragraphs).
 *   x      [T][H] fp32 in
 *   h      [T][H] fp32 out: x + wo . attn
 *   attn_o [T][Hq*D] fp32 out, nullable: attention output before wo
 *   win    [T][2] int32 out, nullable: visible cache positions [lo, hi] of each
 *          token (hi = its own position)
 * Writes the appended K/V into kv (in kv_dtype, round to nearest even; e4m3
 * saturates to +-448).  x and h must not overlap. */
msk_status msk_attn_step(const msk_layer_cfg *cfg, const msk_layer_weights *w,
                         const msk_kv *kv, const msk_batch *batch, const float *x,
                         float *h, float *attn_o, int32_t *win, void *ws,
                         size_t ws_bytes, void *stream);

/* Router: u = RMSNorm(h) * ffn_norm; logits = w_router . u (fp32); per token the
 * top_k experts by logit (descending; the lower index wins a tie) and their
 * weights (softmax over the selected logits).  Defined by: every layer routes
 * each token to 8 of 256 experts (ainewsbites page, "One program replaces many
 * kernel boundaries"; brifing.si page, "Model Architecture Details").
 *   h [T][H] in; u [T][H] out; topk_idx [T][k] int32 out; topk_w [T][k] out;
 *   logits [T][E] out, nullable. */
msk_status msk_moe_route(const msk_layer_cfg *cfg, const msk_layer_weights *w,
                         int32_t n_tokens, const float *h, float *u,
                         int32_t *topk_idx, float *topk_w, float *logits,
                         void *ws, size_t ws_bytes, void *stream);

/* Experts: out[t] = h[t] + sum_j topk_w[t][j] * down_e(silu(gate_e u[t]) * up_e u[t])
 * with e = topk_idx[t][j], summed in slot order j = 0..k-1.  Only the distinct
 * selected experts are read, each once for all tokens routed to it.  Defined
 * by: the selected experts' weights are fetched once routing is known, and a
 * verify step streams the step's distinct experts (ainewsbites page, "One
 * program replaces many kernel boundaries" and "Reported decode and
 * verification gains"); NVFP4 experts with one scale per 16 values (brifing.si
 * page, "Expert Weight Quantization").
 *   u, h [T][H] in; topk_idx, topk_w [T][k] in; out [T][H] out (may equal h). */
msk_status msk_expert_ffn(const msk_layer_cfg *cfg, const msk_layer_weights *w,
                          int32_t n_tokens, const float *u, const int32_t *topk_idx,
                          const float *topk_w, const float *h, float *out, void *ws,
                          size_t ws_bytes, void *stream);

/* A whole decode/verify step through n_layers (1..MSK_MAX_STACK) layers.
 * Defined by: one program runs every layer of a decode or verify step
 * (ainewsbites page, "One program replaces many kernel boundaries"; brifing.si
 * page, "Megakernel Architecture Benefits"), and a verify step checks all
 * draft tokens of a request in one pass (brifing.si page, "Speculative
 * Decoding Integration").  The step is enqueued on one stream as the
 * per-phase kernels of every layer in order: layer l's output is layer l+1's
 * input.  cfg, w and kv are
 * arrays of n_layers entries (shapes must agree; window and dtypes may differ).
 *   x         [T][H] fp32 in/out: the step's input, replaced by its output
 *   layer_out [n_layers][T][H] out, nullable: each layer's output
 *   topk_idx  [n_layers][T][k] out, nullable
 *   win       [n_layers][T][2] out, nullable */
msk_status msk_layer_step(const msk_layer_cfg *cfg, const msk_layer_weights *w,
                          const msk_kv *kv, int32_t n_layers, const msk_batch *batch,
                          float *x, float *layer_out, int32_t *topk_idx, int32_t *win,
                          void *ws, size_t ws_bytes, void *stream);

/* msk_layer_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step and outputs, with its scratch in an array the library keeps
 * on every GPU it runs on (msk_noalloc_scratch_bytes() bytes per GPU, 64 MiB,
 * held until the process ends) instead of a caller workspace.  It calls no
 * hipMalloc, hipFree or other allocating routine (no host allocation either).
 * Arguments as msk_layer_step, minus the workspace.  Errors: as
 * msk_layer_step; MSK_ERR_WORKSPACE if the step needs more scratch than the
 * array holds (msk_workspace_size above msk_noalloc_scratch_bytes()).  Every
 * call on one GPU shares that GPU's array: calls that may overlap on one GPU
 * (several streams or threads) race and must not be issued.  The array keeps
 * the previous call's contents; each call zeroes the words it needs zeroed.
 * Kernel timing (msk_timer_start) does not record these calls. */
msk_status msk_layer_step_noalloc(const msk_layer_cfg *cfg, const msk_layer_weights *w,
                                  const msk_kv *kv, int32_t n_layers, const msk_batch *batch,
                                  float *x, float *layer_out, int32_t *topk_idx, int32_t *win,
                                  void *stream);
/* Bytes of the per-GPU scratch array of msk_layer_step_noalloc. */
size_t msk_noalloc_scratch_bytes(void);

/* Profiling aid: msk_layer_step run as the persistent
 * step kernel where one exists for the stack (one token per step; bf16 dense
 * and experts over a bf16 cache, bf16 dense with NVFP4 experts over an e4m3
 * cache, or all fp32; head_dim 128, 128 and 32): every phase of up to four
 * layers in one launch, its workgroups meeting at device-wide barriers
 * where a phase needs the whole result of the one before.  Other stacks run
 * as per-phase kernels and leave stamps untouched.  It records, for every
 * workgroup of the persistent kernel, the GPU's constant 100 MHz real-time
 * counter at the start and after each phase:
 *   stamps  DEVICE int64 [4 * CUs][32], caller-owned and zero-filled; slot 0
 *           = start, then per layer: QKV, attention, combine, Wo, router,
 *           gate/up, down (the first four layers).  Rows of workgroups that
 *           did not run stay zero.
 * Every barrier wait is bounded (msk_set_spin_limit): one that gives up sets
 * the workspace's error flag.  Behind the launch the library copies the flag
 * to pinned host memory and records an event on `stream`; the first call on
 * the workspace (any entry point that takes it) that starts after the launch
 * has finished finds the flag without waiting, resets the workspace's
 * synchronisation words and returns MSK_ERR_TIMEOUT before it enqueues
 * anything.  A call made while the launch still runs cannot know yet and
 * leaves the check to a later one; msk_workspace_status, which synchronises,
 * always reports it.  The library tracks the last 64 workspaces this call ran
 * the persistent kernel on; the flag of an older one is reported by
 * msk_workspace_status alone.  The outputs of a call whose wait gave up are
 * undefined.  The first persistent launch allocates the pinned words and
 * each tracked workspace one event. */
msk_status msk_layer_step_timeline(const msk_layer_cfg *cfg, const msk_layer_weights *w,
                                   const msk_kv *kv, int32_t n_layers, const msk_batch *batch,
                                   float *x, float *layer_out, int32_t *topk_idx, int32_t *win,
                                   int64_t *stamps, void *ws, size_t ws_bytes, void *stream);

/* Test aid: the number of polls after which a device-side barrier wait of
 * msk_layer_step_timeline gives up (0 restores the default, 2^22 polls, of
 * seconds).  Process-wide; read by each call when it launches.  A small
 * bound makes waits give up on purpose, so that the error path can be
 * exercised with every kernel still running to its end. */
msk_status msk_set_spin_limit(uint32_t polls);

/* Experts of a prefill batch: the same result as msk_expert_ffn, for up to
 * MSK_MAX_PREFILL_TOKENS tokens.  With many tokens per expert the gate/up and
 * down products are matrix products on the matrix cores: the slots (t, j) are
 * grouped by expert, and each chunk of an expert's slots (up to 160 for NVFP4
 * experts, 128 for bf16 experts) meets that expert's weights in one product
 * with fp32 accumulation.  NVFP4 weights
 * are decoded exactly to fp16 and meet fp16 inputs (u and the SwiGLU
 * activations, each slot's row scaled by a power of two: 11 significant
 * bits); bf16 weights meet two bf16 terms of each input (exact to about
 * 2^-17).  Defined by: a fused MoE kernel among the
 * prefill optimisations
 * (ainewsbites page, "Agentic coding benchmark and serving tradeoffs");
 * NVFP4 experts with one scale per 16 values (brifing.si page, "Expert Weight
 * Quantization").
 *   u, h [T][H] in (16-byte aligned); topk_idx, topk_w [T][k] in (an index
 *   outside [0, E) makes its slot add nothing); out [T][H] out (may equal h).
 *   Experts bf16 or NVFP4, hidden and ffn_dim multiples of 128, else
 *   MSK_ERR_UNSUPPORTED.  ws: msk_moe_prefill_workspace_size() bytes.
 *   Results do not depend on the order the slots of an expert are grouped in. */
msk_status msk_moe_prefill(const msk_layer_cfg *cfg, const msk_layer_weights *w,
                           int32_t n_tokens, const float *u, const int32_t *topk_idx,
                           const float *topk_w, const float *h, float *out, void *ws,
                           size_t ws_bytes, void *stream);

/* Workspace bytes of msk_moe_prefill for n_tokens tokens (grouped inputs,
 * products and per-slot outputs: about n_tokens * (k * (4 H + 12 F) + 4 H)
 * bytes);
 * 0 and msk_last_error() on invalid or unsupported arguments. */
size_t msk_moe_prefill_workspace_size(const msk_layer_cfg *cfg, int32_t n_tokens);

/* Kernel timing for measurement harnesses.  The step's kernels fall into
 * phases:
 *   MSK_PH_QKV      RMSNorm + QKV projection + QK-norm + KV append
 *   MSK_PH_ATTN     split-KV no-max attention partials (and their sums and
 *                   the window bounds, with no combine launch, where the
 *                   vector kernel runs, the output projection does not run
 *                   on the matrix cores, and every group spans at most
 *                   eight chunks)
 *   MSK_PH_COMBINE  sum of the partials, window bounds
 *   MSK_PH_WO       output projection + residual
 *   MSK_PH_ROUTER   FFN RMSNorm + router logits (one token; with several,
 *                   the router's product on the matrix cores)
 *   MSK_PH_TOPK     top-k and gating weights (one token: msk_moe_route
 *                   alone; within msk_layer_step the gate/up kernel selects
 *                   itself).  Several tokens: the router's K-slice sums,
 *                   the top-k and the expert union in one kernel
 *   MSK_PH_GATEUP   expert gate/up + SwiGLU
 *   MSK_PH_DOWN     expert down + weighted combine + residual
 *   MSK_PH_STEP     the persistent whole-step kernel, where it runs
 *   MSK_PH_UNION    distinct selected experts and their slots (more than
 *                   one token, msk_expert_ffn alone)
 *   MSK_PH_MOE_SUM  weighted sum of the per-slot expert outputs + residual
 *                   (more than one token; between layers of a stack it also
 *                   writes the next layer's QKV input terms)
 *   MSK_PH_PREP     RMSNorm of a projection's input into bf16 terms for the
 *                   matrix cores (more than one token, bf16 dense weights);
 *                   before the router it also forms h from Wo's K-slice sums
 *   MSK_PH_DENSE_SUM  sum of a matrix-core projection's K-slice partials
 *                   (+ residual; the QKV product within msk_layer_step)
 * msk_timer_start(mask) forgets earlier records and, from then on, brackets
 * every launch of each phase whose bit (1 << phase) is set in mask with a
 * pair of HIP events that the dispatch itself stamps (hipExtLaunchKernel),
 * so a pair measures that kernel alone, on the stream it runs on.  mask 0
 * stops timing.  msk_timer_read(phase, &ms, &n) waits for the phase's last
 * recorded launch and returns the summed duration in milliseconds and the
 * number of launches recorded since the last msk_timer_start.  The library
 * keeps one process-wide timer: calls on several threads or streams at once
 * are recorded together.  Errors: MSK_ERR_INVALID_ARG for a phase outside
 * the list or null outputs, MSK_ERR_DEVICE when an event call fails. */
enum {
  MSK_PH_QKV = 0, MSK_PH_ATTN = 1, MSK_PH_COMBINE = 2, MSK_PH_WO = 3, MSK_PH_ROUTER = 4,
  MSK_PH_TOPK = 5, MSK_PH_GATEUP = 6, MSK_PH_DOWN = 7, MSK_PH_STEP = 8, MSK_PH_UNION = 9,
  MSK_PH_MOE_SUM = 10, MSK_PH_PREP = 11, MSK_PH_DENSE_SUM = 12, MSK_N_PHASES = 13
};
msk_status msk_timer_start(uint32_t mask);
msk_status msk_timer_read(int32_t phase, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* MSK_H */
