// Internal interface between the C ABI (argument checks, planning) and the
// kernel launchers.
#pragma once
#include <hip/hip_runtime.h>

#include "params.h"

namespace msk {

// Attention half: QKV, attention partials, combine, Wo (+ residual).
hipError_t launch_attn(const LayerArgs& L, const StepArgs& S, const float* x, float* h,
                       hipStream_t st);
// Router: u, logits, top-k indices and weights.
hipError_t launch_route(const LayerArgs& L, const StepArgs& S, const float* h, int* topk_out,
                        hipStream_t st, bool defer_topk = false);
// Experts: out = h + MoE(u).
hipError_t launch_ffn(const LayerArgs& L, const StepArgs& S, const float* h, float* out,
                      hipStream_t st, bool union_ready = false, bool own_topk = false,
                      int* topk_out = nullptr);
// The expert phase of S's tokens runs the one-token kernels.
bool ffn_one_token(const LayerArgs& L, const StepArgs& S);
// Whole step over S.n_layers layers as one persistent cooperative kernel.
hipError_t launch_step_fused(const LayerArgs* Ls, const StepArgs& S, hipStream_t st);
// Whole step as a sequence of per-phase kernels (the unfused comparison path).
hipError_t launch_step_unfused(const LayerArgs* Ls, const StepArgs& S, hipStream_t st);

// Kernel timing (msk_timer_start / msk_timer_read): arm the phases in
// `mask`, forget earlier records; read the summed milliseconds and launch
// count of one phase, waiting for its last recorded launch.
hipError_t timer_start(uint32_t mask);
hipError_t timer_read(int phase, double* total_ms, long long* launches);

// LDS bytes a launch needs, for the planner's checks.
size_t attn_lds_bytes(int kdt, int D);

}  // namespace msk
