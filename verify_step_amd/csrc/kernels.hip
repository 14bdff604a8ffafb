// Kernels of the MoE decode/verify layer step for gfx950, and their host
// launchers.  Each phase of the step is also a kernel of its own (the
// unfused path); the fused path runs every phase of every layer in one
// persistent cooperative launch with grid barriers between dependent phases.
#include "launch.h"
#include "phases.h"

namespace msk {

extern __shared__ __align__(16) uint8_t msk_smem[];

constexpr int kMaxGrid = 1024;

__host__ __device__ constexpr size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------ kernels
template <int DT, int NV>
__global__ __launch_bounds__(kBlockThreads) void k_qkv(LayerArgs L, StepArgs S, const float* x) {
  float* rs = reinterpret_cast<float*>(msk_smem);
  block_rstd(x, S.T, L.H, L.eps, rs);
  phase_qkv<DT, NV>(L, S, x, rs, blockIdx.x, gridDim.x);
}

template <int KDT, int D>
__global__ __launch_bounds__(kBlockThreads) void k_attn(LayerArgs L, StepArgs S) {
  AttnPlan* P = reinterpret_cast<AttnPlan*>(msk_smem);
  build_plan(L, S, P);
  phase_attn<KDT, D>(L, S, P, msk_smem + align_up(sizeof(AttnPlan), 16), blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(kBlockThreads) void k_combine(LayerArgs L, StepArgs S) {
  AttnPlan* P = reinterpret_cast<AttnPlan*>(msk_smem);
  build_plan(L, S, P);
  phase_combine(L, S, P, blockIdx.x, gridDim.x);
}

template <int DT, int NV>
__global__ __launch_bounds__(kBlockThreads) void k_wo(LayerArgs L, StepArgs S, const float* x,
                                                      float* h) {
  phase_wo<DT, NV>(L, S, x, h, blockIdx.x, gridDim.x);
}

template <int DT, int NV>
__global__ __launch_bounds__(kBlockThreads) void k_router(LayerArgs L, StepArgs S, const float* h) {
  float* rs = reinterpret_cast<float*>(msk_smem);
  block_rstd(h, S.T, L.H, L.eps, rs);
  phase_router<DT, NV>(L, S, h, rs, blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(kBlockThreads) void k_topk(LayerArgs L, StepArgs S, int* topk_out) {
  phase_topk(L, S, topk_out, blockIdx.x, gridDim.x);
}

template <int DT, int NVMAX>
__global__ __launch_bounds__(kBlockThreads) void k_gateup(LayerArgs L, StepArgs S) {
  Union* U = reinterpret_cast<Union*>(msk_smem);
  build_union(S.idx, S.T, L.K, L.E, U);
  phase_gateup<DT, NVMAX>(L, S, U, blockIdx.x, gridDim.x);
}

template <int DT, int NVMAX>
__global__ __launch_bounds__(kBlockThreads) void k_down(LayerArgs L, StepArgs S, const float* h,
                                                        float* out) {
  Union* U = reinterpret_cast<Union*>(msk_smem);
  build_union(S.idx, S.T, L.K, L.E, U);
  float* ybuf = reinterpret_cast<float*>(msk_smem + align_up(sizeof(Union), 16));
  phase_down<DT, NVMAX>(L, S, U, h, out, ybuf, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------- LDS budgets
size_t attn_lds_bytes(int kdt, int D) {
  size_t w = 0;
#define MSK_GEOM(K, DD) \
  if (kdt == K && D == DD) w = AttnGeom<K, DD>::LDS_WAVE;
  MSK_GEOM(kF32, 32) MSK_GEOM(kF32, 64) MSK_GEOM(kF32, 128)
  MSK_GEOM(kBF16, 32) MSK_GEOM(kBF16, 64) MSK_GEOM(kBF16, 128)
  MSK_GEOM(kE4M3, 32) MSK_GEOM(kE4M3, 64) MSK_GEOM(kE4M3, 128)
#undef MSK_GEOM
  return align_up(sizeof(AttnPlan), 16) + kWaves * w;
}

static size_t down_lds_bytes(const LayerArgs& L, const StepArgs& S) {
  return align_up(sizeof(Union), 16) + (size_t)kWaves * S.T * L.K * 4 * sizeof(float);
}

static int DenseRowsHost(int nv) { return nv >= 16 ? 2 : 4; }

static int grid_for_waves(long long waves) {
  long long b = (waves + kWaves - 1) / kWaves;
  if (b < 1) b = 1;
  return (int)(b < kMaxGrid ? b : kMaxGrid);
}

template <class K>
static hipError_t launch(K kernel, int grid, size_t lds, hipStream_t st, const LayerArgs& L,
                         const StepArgs& S) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlockThreads), lds, st, L, S);
  return hipGetLastError();
}

template <class K, class... A>
static hipError_t launch_x(K kernel, int grid, size_t lds, hipStream_t st, A... args) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlockThreads), lds, st, args...);
  return hipGetLastError();
}

static hipError_t set_lds_limit(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

#define MSK_TRY(x)                          \
  do {                                      \
    hipError_t e_ = (x);                    \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

// ------------------------------------------------------ launchers
// Token-group width of the dense projections: the smallest power of two
// covering T, at most 32 (more tokens are processed in groups).
static int dense_nv(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : T <= 8 ? 8 : T <= 16 ? 16 : 32; }
// Largest token count an expert handles in one pass over its rows.
static int expert_nv(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8; }

#define MSK_NV_CASES(NVVAL, BODY)   \
  switch (NVVAL) {                  \
    case 1: { constexpr int NV = 1; BODY; } break;   \
    case 2: { constexpr int NV = 2; BODY; } break;   \
    case 4: { constexpr int NV = 4; BODY; } break;   \
    case 8: { constexpr int NV = 8; BODY; } break;   \
    case 16: { constexpr int NV = 16; BODY; } break; \
    default: { constexpr int NV = 32; BODY; } break; \
  }
#define MSK_ENV_CASES(NVVAL, BODY)  \
  switch (NVVAL) {                  \
    case 1: { constexpr int NV = 1; BODY; } break;   \
    case 2: { constexpr int NV = 2; BODY; } break;   \
    case 4: { constexpr int NV = 4; BODY; } break;   \
    default: { constexpr int NV = 8; BODY; } break;  \
  }

hipError_t launch_attn(const LayerArgs& L, const StepArgs& S, const float* x, float* h,
                       hipStream_t st) {
  const int NR = (L.Hq + 2 * L.Hkv) * L.D;
  const size_t rs_lds = (size_t)S.T * sizeof(float);
  const int nv = dense_nv(S.T);
  const int qgrid = grid_for_waves(NR / DenseRowsHost(nv));
  if (L.ddt == kBF16) {
    MSK_NV_CASES(nv, MSK_TRY(launch_x(k_qkv<kBF16, NV>, qgrid, rs_lds, st, L, S, x)))
  } else {
    MSK_NV_CASES(nv, MSK_TRY(launch_x(k_qkv<kF32, NV>, qgrid, rs_lds, st, L, S, x)))
  }

  const size_t alds = attn_lds_bytes(L.kdt, L.D);
  const int agrid = grid_for_waves(L.n_items);
#define MSK_ATTN(K, DD)                                                             \
  if (L.kdt == K && L.D == DD) {                                                    \
    MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_attn<K, DD>), alds));   \
    MSK_TRY(launch(k_attn<K, DD>, agrid, alds, st, L, S));                          \
  }
  MSK_ATTN(kF32, 32) MSK_ATTN(kF32, 64) MSK_ATTN(kF32, 128)
  MSK_ATTN(kBF16, 32) MSK_ATTN(kBF16, 64) MSK_ATTN(kBF16, 128)
  MSK_ATTN(kE4M3, 32) MSK_ATTN(kE4M3, 64) MSK_ATTN(kE4M3, 128)
#undef MSK_ATTN
  MSK_TRY(launch(k_combine, grid_for_waves((long long)S.T * L.Hq), sizeof(AttnPlan), st, L, S));
  const int wgrid = grid_for_waves(L.H / DenseRowsHost(nv));
  if (L.ddt == kBF16) {
    MSK_NV_CASES(nv, MSK_TRY(launch_x(k_wo<kBF16, NV>, wgrid, 0, st, L, S, x, h)))
  } else {
    MSK_NV_CASES(nv, MSK_TRY(launch_x(k_wo<kF32, NV>, wgrid, 0, st, L, S, x, h)))
  }
  return hipSuccess;
}

hipError_t launch_route(const LayerArgs& L, const StepArgs& S, const float* h, int* topk_out,
                        hipStream_t st) {
  const size_t rs_lds = (size_t)S.T * sizeof(float);
  const int nv = dense_nv(S.T);
  const int rows = (L.E + DenseRowsHost(nv) - 1) / DenseRowsHost(nv);
  const int grid = grid_for_waves(rows > 64 ? rows : 64);
  if (L.ddt == kBF16) {
    MSK_NV_CASES(nv, MSK_TRY(launch_x(k_router<kBF16, NV>, grid, rs_lds, st, L, S, h)))
  } else {
    MSK_NV_CASES(nv, MSK_TRY(launch_x(k_router<kF32, NV>, grid, rs_lds, st, L, S, h)))
  }
  MSK_TRY(launch_x(k_topk, grid_for_waves(S.T), 0, st, L, S, topk_out));
  return hipSuccess;
}

template <int DT, int NV>
static hipError_t launch_ffn_t(const LayerArgs& L, const StepArgs& S, const float* h, float* out,
                               hipStream_t st) {
  const size_t ulds = sizeof(Union);
  const size_t dlds = down_lds_bytes(L, S);
  // the number of distinct experts is known only on the device: size the
  // gate/up grid for the largest possible union, capped
  const long long gu_items = (long long)(S.T * L.K < L.E ? S.T * L.K : L.E) * (L.F / 4);
  MSK_TRY(launch(k_gateup<DT, NV>, grid_for_waves(gu_items), ulds, st, L, S));
  MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_down<DT, NV>), dlds));
  MSK_TRY(launch_x(k_down<DT, NV>, grid_for_waves(L.H / 4), dlds, st, L, S, h, out));
  return hipSuccess;
}

hipError_t launch_ffn(const LayerArgs& L, const StepArgs& S, const float* h, float* out,
                      hipStream_t st) {
  const int nv = expert_nv(S.T);
  switch (L.edt) {
    case kF32: MSK_ENV_CASES(nv, return (launch_ffn_t<kF32, NV>(L, S, h, out, st))) break;
    case kBF16: MSK_ENV_CASES(nv, return (launch_ffn_t<kBF16, NV>(L, S, h, out, st))) break;
    default: MSK_ENV_CASES(nv, return (launch_ffn_t<kNVFP4, NV>(L, S, h, out, st))) break;
  }
  return hipSuccess;
}

// Layer l reads `cur` and writes the next buffer; the last layer writes x_out.
hipError_t launch_step_unfused(const LayerArgs* Ls, const StepArgs& S0, hipStream_t st) {
  StepArgs S = S0;
  const float* cur = S.x_in;
  for (int l = 0; l < S.n_layers; ++l) {
    const LayerArgs& L = Ls[l];
    float* nxt = (l == S.n_layers - 1) ? S.x_out : ((l & 1) ? S.xb : S.xa);
    S.win_out = S0.win_out ? S0.win_out + (size_t)l * S.T * 2 : nullptr;
    MSK_TRY(launch_attn(L, S, cur, S.h, st));
    MSK_TRY(launch_route(L, S, S.h, S0.topk_out ? S0.topk_out + (size_t)l * S.T * L.K : nullptr,
                         st));
    MSK_TRY(launch_ffn(L, S, S.h, nxt, st));
    if (S.layer_out)
      MSK_TRY(hipMemcpyAsync(S.layer_out + (size_t)l * S.T * L.H, nxt,
                             (size_t)S.T * L.H * sizeof(float), hipMemcpyDeviceToDevice, st));
    cur = nxt;
  }
  return hipSuccess;
}

hipError_t launch_step_fused(const LayerArgs* Ls, const StepArgs& S, hipStream_t st) {
  // the persistent kernel is not built yet: run the per-phase kernels
  return launch_step_unfused(Ls, S, st);
}

}  // namespace msk
