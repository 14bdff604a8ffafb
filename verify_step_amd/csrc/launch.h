// Internal interface between the C ABI (argument checks, planning) and the
// kernel launchers.
#pragma once
#include <hip/hip_runtime.h>

#include "params.h"

namespace msk {

// Attention half: QKV, attention partials, combine, Wo (+ residual).
// wo_parts: a Wo product split over K leaves its partial tiles for the
// router launch to sum (launch_route with wo_resid = x).
// a3_ready: the QKV product's input terms are in S.a3 already (written by
// the previous layer's expert sum, launch_ffn with next_norm).
hipError_t launch_attn(const LayerArgs& L, const StepArgs& S, const float* x, float* h,
                       hipStream_t st, bool wo_parts = false, bool a3_ready = false);
// Router: u, logits, top-k indices and weights.  wo_resid: h = wo_resid +
// the Wo partial tiles left by launch_attn(wo_parts) is formed here first.
hipError_t launch_route(const LayerArgs& L, const StepArgs& S, const float* h, int* topk_out,
                        hipStream_t st, bool defer_topk = false,
                        const float* wo_resid = nullptr);
// Several tokens with bf16 Wo and router products on the matrix cores: the
// Wo partial sums can go to the router's input preparation.
bool wo_sum_in_route(const LayerArgs& L, const StepArgs& S);
// Experts: out = h + MoE(u).  next_norm (several tokens only): also write
// the next layer's QKV input terms of out (RMSNorm with gain next_norm and
// next_eps) into S.a3.
hipError_t launch_ffn(const LayerArgs& L, const StepArgs& S, const float* h, float* out,
                      hipStream_t st, bool union_ready = false, bool own_topk = false,
                      int* topk_out = nullptr, const float* next_norm = nullptr,
                      float next_eps = 0.f);
// Several tokens with a bf16 QKV product on the matrix cores.
bool qkv_on_mfma(const LayerArgs& L, const StepArgs& S);
// The expert phase of S's tokens runs the one-token kernels.
bool ffn_one_token(const LayerArgs& L, const StepArgs& S);
// Whole step over S.n_layers layers as the persistent step kernel (one launch
// per kMaxFusedLayers layers) where an instantiation covers the shape, else
// as launch_step_unfused; *persistent says which ran.
hipError_t launch_step_fused(const LayerArgs* Ls, const StepArgs& S, hipStream_t st,
                             bool* persistent);
// Expert FFN of a prefill batch (see phases_prefill.h): route, gather,
// gate/up, SwiGLU, down, weighted sum, on `st`.
hipError_t launch_prefill(const LayerArgs& L, const PfArgs& P, const float* wts, const float* h,
                          float* out, hipStream_t st);
// Whole step as a sequence of per-phase kernels.
hipError_t launch_step_unfused(const LayerArgs* Ls, const StepArgs& S, hipStream_t st);

// Scratch of the allocation-free entry point: kScratchBytes per GPU, at the
// address scratch_address gives for the current device (looked up once per
// device).  launch_step_noalloc runs the per-phase step on S, whose
// workspace pointers lie in that scratch, after zeroing its barrier and
// counter words; it creates and records no timing events.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_address(void** out);
hipError_t launch_step_noalloc(const LayerArgs* Ls, const StepArgs& S, hipStream_t st);

// Kernel timing (msk_timer_start / msk_timer_read): arm the phases in
// `mask`, forget earlier records; read the summed milliseconds and launch
// count of one phase, waiting for its last recorded launch.
hipError_t timer_start(uint32_t mask);
hipError_t timer_read(int phase, double* total_ms, long long* launches);

// LDS bytes a launch needs, for the planner's checks.
size_t attn_lds_bytes(int kdt, int D);

}  // namespace msk
