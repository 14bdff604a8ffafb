// Kernels of the MoE decode/verify layer step for gfx950, and their host
// launchers.  Each phase of the step is a kernel of its own, launched in
// order on one stream; the persistent kernel k_step_p runs every phase of up
// to four layers in one launch of resident workgroups, with tree barriers
// between dependent phases (the timeline call).
#include <hip/hip_ext.h>

#include <mutex>
#include <utility>
#include <vector>

#include "launch.h"
#include "phases_dense.h"
#include "phases_mfma.h"
#include "phases_t1.h"
#include "phases_tn.h"
#include "phases_prefill.h"

namespace msk {

extern __shared__ __align__(16) uint8_t msk_smem[];

constexpr int kMaxGrid = 1024;
constexpr size_t kMaxLds = 160 * 1024;

__host__ __device__ constexpr size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------ kernels
// Device-coherent (agent-scope) word operations for counters and barriers.
__device__ __forceinline__ unsigned a_ld(unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void a_st(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned a_add(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Vector attention items whose group's last arrival also sums the group's
// partials into attn_o (no combine launch); workgroup 0 writes the windows.
template <int KDT, int D>
__global__ __launch_bounds__(kBlockThreads) void k_attn_c(LayerArgs L, StepArgs S) {
  static_assert(CombineLds<D>::BYTES <= AttnGeom<KDT, D>::LDS_ITEM, "combine LDS");
  AttnPlan* P = reinterpret_cast<AttnPlan*>(msk_smem);
  build_plan(L, S, P);
  uint8_t* lds = msk_smem + align_up(sizeof(AttnPlan), 16);
  const int n_items = P->item0[S.n_req];
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    attn_item<KDT, D, CohSt>(L, S, P, item, lds);
    combine_if_last<D>(L, S, P, item, S.sync + kAttnCountWord, lds);
    __syncthreads();
  }
  if (blockIdx.x == 0 && S.win_out != nullptr) write_windows(L, S, S.win_out);
}

// The tile fetch is one tile deep per workgroup, so the bytes in flight come
// from resident workgroups: e4m3 caches (16 KB tiles) run three waves per
// SIMD; bf16 tiles are twice the registers and keep the compiler's choice.
template <int KDT> struct AttnWaves { static constexpr int N = KDT == kE4M3 ? 3 : 1; };

template <int KDT, int D, int NW, int NPH>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(AttnWaves<KDT>::N)))
void k_attn_mfma(LayerArgs L, StepArgs S) {
  AttnPlan* P = reinterpret_cast<AttnPlan*>(msk_smem);
  build_plan(L, S, P);
  phase_attn_mfma<KDT, D, NW, NPH>(L, S, P, msk_smem + align_up(sizeof(AttnPlan), 16),
                                   blockIdx.x, gridDim.x);
}

// Several tokens: the expert union once, then gate/up and down over it,
// then the weighted sum over each token's slots.
__global__ __launch_bounds__(kBlockThreads) void k_union(LayerArgs L, StepArgs S) {
  union_to_global(S.idx, S.T, L.K, L.E, reinterpret_cast<Union*>(msk_smem), S.uni);
}

template <int DT, int NVMAX, int NWV>
__global__ __launch_bounds__(NWV * 64) void k_gateup_tn(LayerArgs L, StepArgs S) {
  float* act = reinterpret_cast<float*>(msk_smem);
  gateup_tn<DT, NVMAX, NWV>(L, S, S.uni, act, act + NVMAX * tn_vec_floats<DT>(L.H));
}

template <int DT, int NVMAX, int NWV>
__global__ __launch_bounds__(NWV * 64) void k_down_tn(LayerArgs L, StepArgs S) {
  float* act = reinterpret_cast<float*>(msk_smem);
  down_tn<DT, NVMAX, NWV>(L, S, S.uni, act, act + NVMAX * tn_vec_floats<DT>(L.F), S.ybuf);
}

__global__ __launch_bounds__(kBlockThreads) void k_moe_sum(LayerArgs L, StepArgs S, const float* h,
                                                           float* out) {
  down_combine(L, S, h, S.ybuf, out);
}

__global__ __launch_bounds__(kBlockThreads) void k_combine(LayerArgs L, StepArgs S, int* win,
                                                           unsigned short* a3) {
  AttnPlan* P = reinterpret_cast<AttnPlan*>(msk_smem);
  build_plan(L, S, P);
  phase_combine(L, S, P, win, blockIdx.x, gridDim.x,
                reinterpret_cast<float*>(msk_smem + align_up(sizeof(AttnPlan), 16)), a3);
}

// Matrix-core dense projections of several tokens and their input terms.

constexpr int kSumPrepThreads = 1024;
__global__ __launch_bounds__(kSumPrepThreads) void k_sum_prep(const float* part, int ks,
                                                              const float* resid, float* h,
                                                              const float* g, int T, int H,
                                                              float eps, float* a32,
                                                              unsigned short* a3) {
  float* red = reinterpret_cast<float*>(msk_smem);
  sum_prep_act(part, ks, resid, h, g, T, H, eps, a32, a3, red + 16, red);
}

__global__ __launch_bounds__(kSumPrepThreads) void k_moe_sum_prep(LayerArgs L, StepArgs S,
                                                                  const float* h, float* out,
                                                                  const float* g, float eps) {
  float* red = reinterpret_cast<float*>(msk_smem);
  down_combine_prep(L, S, h, S.ybuf, out, g, eps, S.a3, red + 16, red);
}

template <int CT, int NT>
__global__ __launch_bounds__(kBlockThreads) void k_dense_mfma(DenseArgs A) {
  dense_mfma<CT, NT>(A, msk_smem);
}

__global__ __launch_bounds__(kBlockThreads) void k_dense_sum(const float* part, int N, int T,
                                                             int ks, const float* resid,
                                                             float* out) {
  dense_sum(part, N, T, ks, resid, out);
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

// Several tokens' routing: one wave per token sums the router logits (in
// slice order, from the dense product's split-K partial tiles when ks > 1)
// and writes them out, then takes the token's top-k (a selection is a chain of
// dependent wave reductions, so the tokens go to waves of kTopkWaves-wave
// workgroups, all at once).  The workgroup that arrives last, counted on a
// word of the workspace, reads every token's selection and builds the expert
// union (what k_topk and k_union do, in one launch).  The selections travel
// between workgroups through device-coherent stores and loads, written and
// waited for before the arrival is counted: no cache flush is needed.
constexpr int kTopkWaves = 4;
__global__ __launch_bounds__(kTopkWaves * 64) void k_topk_union(LayerArgs L, StepArgs S,
                                                                int* topk_out, const float* part,
                                                                int ks) {
  Union* U = reinterpret_cast<Union*>(msk_smem);
  int* sel = reinterpret_cast<int*>(U + 1);  // [T][K]
  __shared__ int last;
  const int ln = lane_id();
  const int t = blockIdx.x * kTopkWaves + wave_id();
  if (t < S.T) {
    // lane: experts e_i = ln + 64 i; every load is issued before any sum
    // (addresses clamped into range, results past E unused)
    float x[4];
    float* lg = S.logits + (size_t)t * L.E;
    if (ks > 1) {
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      for (int q0 = 0; q0 < ks; q0 += 16) {
        float v[4][16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = ln + 64 * i < L.E ? ln + 64 * i : L.E - 1;
          // partial tile of row block e / 64, slice q: [q][T][64] within the block
          const float* src = part + ((size_t)(e >> 6) * ks * S.T + t) * 64 + (e & 63);
#pragma unroll
          for (int q = 0; q < 16; ++q)
            v[i][q] = src[(size_t)(q0 + q < ks ? q0 + q : ks - 1) * S.T * 64];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (q0 + q < ks) a[i] += v[i][q];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = ln + 64 * i;
        if (e < L.E) lg[e] = a[i];
        x[i] = e < L.E ? a[i] : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = ln + 64 * i;
        const float v = lg[e < L.E ? e : L.E - 1];
        x[i] = e < L.E ? v : -INFINITY;
      }
    }
    int bis[kMaxTopK];
    float exs[kMaxTopK], den;
    topk_vals(x, L.E, L.K, bis, exs, den);
    if (ln == 0) {
      const float inv = 1.0f / den;
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k)
        if (k < L.K) {
          const size_t o = (size_t)t * L.K + k;
          __hip_atomic_store(&S.idx[o], bis[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          S.wts[o] = exs[k] * inv;
          if (topk_out) topk_out[o] = bis[k];
        }
    }
  }
  // this workgroup's selections have landed before its arrival is counted
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = S.sync + kTopkCountWord;
    last = a_add(cnt, 1u) == gridDim.x - 1;
    if (last) a_st(cnt, 0u);  // zero again for the next launch
  }
  __syncthreads();
  if (!last) return;
  for (int i = threadIdx.x; i < S.T * L.K; i += blockDim.x)
    sel[i] = __hip_atomic_load(&S.idx[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  union_to_global(sel, S.T, L.K, L.E, U, S.uni);
}


// ------------------------------------------------- one-token kernels
// LDS of the one-token kernels: a reduction scratch, the top-k of the token,
// one hidden-size input vector (act0) and the K expert activations (act1);
// the attention phase of the persistent kernel reuses the same space.

struct T1Lds {
  size_t red, tki, tkw, act0, act1, end_act, attn;
};
__host__ __device__ inline T1Lds t1_lds(int H, int HqD, int K, int F) {
  T1Lds o;
  o.red = 0;
  o.tki = 64;
  o.tkw = 128;
  o.act0 = 256;
  o.act1 = o.act0 + align_up((size_t)4 * (H > HqD ? H : HqD), 256);
  o.end_act = o.act1 + (size_t)4 * K * F;
  o.attn = 256;
  return o;
}

// The input vector of a one-token GEMV is loaded into registers before the
// weight stream's first loads are issued (up to kT1Regs four-float pieces
// per thread): loaded after them, it would wait for them on the in-order
// load counter before the staging could start.  The staging meets the other
// waves at an LDS-only barrier, which leaves the weight loads in flight.
// Longer vectors take the plain staging.
constexpr int kT1Regs = 8;
struct T1Vec {
  v4f v[kT1Regs], g[kT1Regs];
};
__device__ __forceinline__ void t1_load(const float* x, const float* g, int n, T1Vec& r) {
#pragma unroll
  for (int i = 0; i < kT1Regs; ++i) {
    const int c = (int)threadIdx.x * 4 + i * kBlockThreads * 4;
    const int cl = c < n ? c : 0;
    r.v[i] = *reinterpret_cast<const v4f*>(x + cl);
    if (g) r.g[i] = *reinterpret_cast<const v4f*>(g + cl);
  }
  __builtin_amdgcn_sched_barrier(0);
}
// act = v * g / sqrt(mean(v^2) + eps) (g given) or act = v, from registers.
__device__ __forceinline__ void t1_stage(const T1Vec& r, bool norm, int n, float eps, float* act,
                                         float* red) {
  float rr = 1.f;
  if (norm) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kT1Regs; ++i) {
      const int c = (int)threadIdx.x * 4 + i * kBlockThreads * 4;
      if (c < n) s += r.v[i].x * r.v[i].x + r.v[i].y * r.v[i].y + r.v[i].z * r.v[i].z + r.v[i].w * r.v[i].w;
    }
    rr = 1.0f / sqrtf(block_sum(s, red) / (float)n + eps);
  }
#pragma unroll
  for (int i = 0; i < kT1Regs; ++i) {
    const int c = (int)threadIdx.x * 4 + i * kBlockThreads * 4;
    if (c < n) {
      const v4f a = r.v[i];
      *reinterpret_cast<v4f*>(act + c) =
          norm ? v4f{a.x * rr * r.g[i].x, a.y * rr * r.g[i].y, a.z * rr * r.g[i].z, a.w * rr * r.g[i].w}
               : a;
    }
  }
  lds_barrier();
}

template <int DT>
__global__ __launch_bounds__(kBlockThreads) void k_qkv_t1(LayerArgs L, StepArgs S, const float* x) {
  const T1Lds o = t1_lds(L.H, L.Hq * L.D, L.K, L.F);
  float* act = reinterpret_cast<float*>(msk_smem + o.act0);
  float* red = reinterpret_cast<float*>(msk_smem + o.red);
  const bool regs = L.H <= kT1Regs * kBlockThreads * 4;
  T1Vec r;
  if (regs) t1_load(x, L.attn_norm, L.H, r);
  qkv_t1<DT>(L, S, act, blockIdx.x, gridDim.x, [&]() {
    if (regs) t1_stage(r, true, L.H, L.eps, act, red);
    else stage_norm_t1(x, L.attn_norm, L.H, L.eps, act, red);
  });
}

template <int DT>
__global__ __launch_bounds__(kBlockThreads) void k_wo_t1(LayerArgs L, StepArgs S, const float* x,
                                                         float* h) {
  const T1Lds o = t1_lds(L.H, L.Hq * L.D, L.K, L.F);
  float* act = reinterpret_cast<float*>(msk_smem + o.act0);
  const int n = L.Hq * L.D;
  const bool regs = n <= kT1Regs * kBlockThreads * 4;
  T1Vec r;
  if (regs) t1_load(S.attn_o, nullptr, n, r);
  wo_t1<DT>(L, S, x, h, act, blockIdx.x, gridDim.x, [&]() {
    if (regs) t1_stage(r, false, n, 0.f, act, nullptr);
    else stage_copy(S.attn_o, n, act);
  });
}

// Router logits of one token (the top-k is taken by the kernel that reads
// them: k_topk, or every wave of k_gateup_t1 within a layer step).
template <int DT>
__global__ __launch_bounds__(kBlockThreads) void k_router_t1(LayerArgs L, StepArgs S,
                                                             const float* h) {
  const T1Lds o = t1_lds(L.H, L.Hq * L.D, L.K, L.F);
  float* act = reinterpret_cast<float*>(msk_smem + o.act0);
  float* red = reinterpret_cast<float*>(msk_smem + o.red);
  const bool regs = L.H <= kT1Regs * kBlockThreads * 4;
  T1Vec r;
  if (regs) t1_load(h, L.ffn_norm, L.H, r);
  router_t1<DT>(L, S, act, reinterpret_cast<float*>(msk_smem + o.act1), blockIdx.x, gridDim.x,
                [&]() {
                  if (regs) t1_stage(r, true, L.H, L.eps, act, red);
                  else stage_norm_t1(h, L.ffn_norm, L.H, L.eps, act, red);
                });
}

template <int DT>
__global__ __launch_bounds__(kBlockThreads) void k_gateup_t1(LayerArgs L, StepArgs S,
                                                             int* topk_out, int own_topk) {
  const T1Lds o = t1_lds(L.H, L.Hq * L.D, L.K, L.F);
  float* u = reinterpret_cast<float*>(msk_smem + o.act0);
  // u into registers first: its loads then overlap the selection and never
  // wait behind the expert rows' loads
  const bool regs = L.H <= kT1Regs * kBlockThreads * 4;
  T1Vec ur;
  if (regs) t1_load(S.u, nullptr, L.H, ur);
  auto stage_u = [&]() {
    if (regs) t1_stage(ur, false, L.H, 0.f, u, nullptr);
    else stage_copy(S.u, L.H, u);
  };
  if (own_topk) {
    // every wave selects the experts itself from the router logits (into
    // scalar registers: no launch, no barrier); workgroup 0 records them
    int sel[kMaxTopK];
    float ex[kMaxTopK], den;
    topk_regs(S.logits, L.E, L.K, sel, ex, den);
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) sel[k] = __builtin_amdgcn_readfirstlane(sel[k]);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      const float inv = 1.0f / den;
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k)
        if (k < L.K) {
          S.idx[k] = sel[k];
          S.wts[k] = ex[k] * inv;
          if (topk_out) topk_out[k] = sel[k];
        }
    }
    // lane k of one vector register holds the k-th id; a wave-uniform slot
    // index then reads it back with one cross-lane read (no private array)
    const int lane = threadIdx.x & 63;
    int selv = sel[0];
#pragma unroll
    for (int k = 1; k < kMaxTopK; ++k) selv = lane == k ? sel[k] : selv;
    auto pick = [selv](int j) { return __builtin_amdgcn_readlane(selv, j); };
    gateup_t1<DT>(L, S, pick, u, blockIdx.x, gridDim.x, stage_u);
  } else {
    const int selv = (threadIdx.x & 63) < L.K ? S.idx[threadIdx.x & 63] : 0;
    gateup_t1<DT>(L, S, [selv](int j) { return __builtin_amdgcn_readlane(selv, j); }, u,
                  blockIdx.x, gridDim.x, stage_u);
  }
}

template <int DT>
__global__ __launch_bounds__(kBlockThreads) void k_down_t1(LayerArgs L, StepArgs S, const float* h,
                                                           float* out) {
  // only the expert activations are staged here: [K][F] after the scratch words
  float* act = reinterpret_cast<float*>(msk_smem + 256);
  const int n = L.K * L.F;
  constexpr int kPart = kT1Regs * kBlockThreads * 4;
  const bool regs = n <= 2 * kPart;
  T1Vec r0, r1;
  if (regs) {
    t1_load(S.act, nullptr, n, r0);
    if (n > kPart) t1_load(S.act + kPart, nullptr, n - kPart, r1);
  }
  down_t1<DT>(L, S, S.idx, S.wts, act, h, out, nullptr, blockIdx.x, gridDim.x, [&]() {
    if (regs) {
      t1_stage(r0, false, n, 0.f, act, nullptr);
      if (n > kPart) t1_stage(r1, false, n - kPart, 0.f, act + kPart, nullptr);
    } else {
      stage_copy(S.act, n, act);
    }
  });
}

// ------------------------------------------- persistent one-token step
// Tree barrier of the persistent step kernel, in the workspace's barrier
// words (zero before a workspace's first use):
//   words[0]          generation: barriers completed so far (only grows)
//   words[1]          error flag: a wait gave up
//   words[32]         arrivals of group leaders at the current barrier
//   words[64 + 32 g]  arrivals of group g (the workgroups b with b % 8 == g)
// The last arrival of a group returns the group's counter to zero and
// arrives at the top counter; the last arrival there returns it to zero and
// publishes the new generation, which every workgroup waits for.  A launch
// starts from the generation the previous one left.  A workgroup arrives
// after its __syncthreads, whose wait for outstanding memory operations
// completes its stores first.  Counters and generation are relaxed
// agent-scope atomics, and the data a barrier hands over moves with Coh
// loads and stores, so no barrier needs an L2 writeback or invalidate
// (measured here: 2.1 us per barrier over 256 workgroups and 2.6 us over
// 512, against 5.6-9.3 us with agent-scope fences, and 3.9-6.8 us with one
// counter for all workgroups).  Every wait is bounded (StepArgs::spin_limit
// polls): a missing arrival sets the workspace's error flag instead of
// hanging, and the next call on that workspace reports it.  A workgroup whose
// wait gave up runs on with whatever its inputs hold: every index it derives
// from data is clamped to its range, so its accesses stay in bounds, and its
// later waits are bounded the same way.
constexpr int kTreeGroups = 8;
struct TreeSync {
  unsigned* w;
  unsigned epoch;
  unsigned limit;  // polls before a wait gives up
};


__device__ __forceinline__ TreeSync tree_begin(unsigned* w, unsigned limit) {
  // every workgroup reads the same generation: it cannot advance before all
  // of this launch's workgroups have arrived at its first barrier
  return TreeSync{w, a_ld(&w[0]), limit};
}

__device__ __forceinline__ void tree_sync(TreeSync& ts) {
  __syncthreads();
  ++ts.epoch;
  if (threadIdx.x == 0) {
    unsigned* w = ts.w;
    const unsigned g = blockIdx.x % kTreeGroups;
    const unsigned ng = (gridDim.x - g + kTreeGroups - 1) / kTreeGroups;
    const unsigned ngroups = gridDim.x < (unsigned)kTreeGroups ? gridDim.x : (unsigned)kTreeGroups;
    if (a_add(&w[64 + 32 * g], 1u) == ng - 1) {
      a_st(&w[64 + 32 * g], 0u);
      __builtin_amdgcn_s_waitcnt(0);  // the reset lands before the next barrier can begin
      if (a_add(&w[32], 1u) == ngroups - 1) {
        a_st(&w[32], 0u);
        __builtin_amdgcn_s_waitcnt(0);
        a_st(&w[0], ts.epoch);
      }
    }
    unsigned spins = 0;
    while ((int)(a_ld(&w[0]) - ts.epoch) < 0) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > ts.limit) {
        a_st(&w[1], 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Kernel arguments of the persistent step: the step's buffers and up to
// kMaxFusedLayers layers (l0: the stack index of the first).
struct StepLayers {
  StepArgs S;
  LayerArgs L[kMaxFusedLayers];
  int l0, nl;
};

// LDS of the persistent step: reduction scratch, the top-k of the token,
// the router's per-wave partial sums, then one region shared by the staged
// input vector of each GEMV phase and by the attention plan and tiles.
struct PLds {
  static constexpr size_t red = 0, tki = 64, tkw = 128, rpart = 256, act = 512;
};
__host__ __device__ inline size_t p_lds_bytes(int H, int HqD, int K, int F, size_t attn) {
  const size_t v = (size_t)4 * (H > HqD ? H : HqD);
  const size_t a = (size_t)4 * K * F;
  const size_t m = v > a ? v : a;
  return PLds::act + (m > attn ? m : attn);
}

// The whole one-token step through nl layers in one launch.  Phases follow
// each other as in the per-phase kernels; where a phase needs every
// workgroup's result of the one before, the workgroups meet at a tree
// barrier.  A GEMV phase's first weight rows are issued before its barrier
// (its staging, which waits for the barrier, is the stream's prologue), so
// the weight fetch overlaps the wait: the one-program pipelining of
// "Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU" (brifing.si
// page, "Pipelining Data Movement"), where loads are issued ahead of the
// compute that needs them, also across layer boundaries.  Each workgroup
// takes the top-k from the router logits itself.  stamps (optional): the
// GPU's 100 MHz real-time counter per workgroup at the start and after each
// phase.
template <int DDT, int EDT, int KDT, int D>
__global__ __launch_bounds__(kBlockThreads) void k_step_p(StepLayers PK) {
  // layers are indexed at run time: each is copied out of the kernel
  // argument segment (scalar loads) into a local
  typedef __attribute__((address_space(4))) const StepLayers KStepLayers;
  KStepLayers* PP = (KStepLayers*)__builtin_amdgcn_kernarg_segment_ptr();
  const StepArgs& S = PK.S;
  const int vb = blockIdx.x, nvb = gridDim.x;
  // slot 0: start of the step; slot 1 + 7 lg + ph: end of phase ph of layer lg
  auto stamp = [&](int slot) {
    if (S.stamps != nullptr && threadIdx.x == 0 && slot < kStamps)
      S.stamps[(size_t)vb * kStamps + slot] = (long long)__builtin_amdgcn_s_memrealtime();
  };
  if (PK.l0 == 0) stamp(0);
  TreeSync ts = tree_begin(S.sync, S.spin_limit);
  float* red = reinterpret_cast<float*>(msk_smem + PLds::red);
  int* tki = reinterpret_cast<int*>(msk_smem + PLds::tki);
  float* tkw = reinterpret_cast<float*>(msk_smem + PLds::tkw);
  float* rpart = reinterpret_cast<float*>(msk_smem + PLds::rpart);
  float* act = reinterpret_cast<float*>(msk_smem + PLds::act);
  const int n_all = S.n_layers;
  for (int l = 0; l < PK.nl; ++l) {
    const LayerArgs L = *(const LayerArgs*)(&PP->L[l]);
    const int lg = PK.l0 + l;
    const int s0 = 1 + 7 * lg;
    const float* xin = lg == 0 ? S.x_in : (((lg - 1) & 1) ? S.xb : S.xa);
    float* xout = lg == n_all - 1 ? S.x_out : ((lg & 1) ? S.xb : S.xa);

    // QKV (the input comes from the previous layer's expert phase)
    qkv_t1<DDT, Coh>(L, S, act, vb, nvb, [&]() {
      if (l > 0) tree_sync(ts);
      stage_norm_t1<Coh>(xin, L.attn_norm, L.H, L.eps, act, red);
    });
    stamp(s0 + 0);
    tree_sync(ts);
    // attention partials, then their sums
    AttnPlan* P = reinterpret_cast<AttnPlan*>(msk_smem + PLds::act);
    build_plan(L, S, P);
    phase_attn<KDT, D, Coh>(L, S, P, msk_smem + PLds::act + align_up(sizeof(AttnPlan), 16), vb,
                            nvb);
    stamp(s0 + 1);
    tree_sync(ts);
    phase_combine<Coh>(L, S, P, S.win_out ? S.win_out + (size_t)lg * 2 * S.T : nullptr, vb, nvb,
                       reinterpret_cast<float*>(msk_smem + PLds::act + align_up(sizeof(AttnPlan), 16)));
    stamp(s0 + 2);
    // output projection + residual
    wo_t1<DDT, Coh>(L, S, xin, S.h, act, vb, nvb, [&]() {
      tree_sync(ts);
      stage_copy<Coh>(S.attn_o, L.Hq * L.D, act);
    });
    stamp(s0 + 3);
    // router logits
    router_t1<DDT, Coh>(L, S, act, rpart, vb, nvb, [&]() {
      tree_sync(ts);
      stage_norm_t1<Coh>(S.h, L.ffn_norm, L.H, L.eps, act, red);
    });
    stamp(s0 + 4);
    tree_sync(ts);
    // every wave selects the experts from the logits; workgroup 0 records them
    {
      int sel[kMaxTopK];
      float ex[kMaxTopK], den;
      topk_regs<Coh>(S.logits, L.E, L.K, sel, ex, den);
      const int ln = lane_id();
      const float inv = 1.0f / den;
      if (wave_id() == 0 && ln == 0) {
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k)
          if (k < L.K) {
            tki[k] = sel[k];
            tkw[k] = ex[k] * inv;
            if (vb == 0) {
              S.idx[k] = sel[k];
              S.wts[k] = ex[k] * inv;
              if (S.topk_out) S.topk_out[(size_t)lg * L.K + k] = sel[k];
            }
          }
      }
      int selv = sel[0];
#pragma unroll
      for (int k = 1; k < kMaxTopK; ++k) selv = ln == k ? sel[k] : selv;
      gateup_t1<EDT, Coh>(L, S, [selv](int j) { return __builtin_amdgcn_readlane(selv, j); }, act,
                          vb, nvb, [&]() { stage_copy<Coh>(S.u, L.H, act); });
    }
    stamp(s0 + 5);
    down_t1<EDT, Coh>(L, S, tki, tkw, act, S.h, xout,
                      S.layer_out ? S.layer_out + (size_t)lg * L.H : nullptr, vb, nvb, [&]() {
                        tree_sync(ts);
                        stage_copy<Coh>(S.act, L.K * L.F, act);
                      });
    stamp(s0 + 6);
  }
}

// ------------------------------------------------------- LDS budgets
size_t attn_lds_bytes(int kdt, int D) {
  size_t w = 0;
#define MSK_GEOM(K, DD) \
  if (kdt == K && D == DD) w = AttnGeom<K, DD>::LDS_ITEM;
  MSK_GEOM(kF32, 32) MSK_GEOM(kF32, 64) MSK_GEOM(kF32, 128)
  MSK_GEOM(kBF16, 32) MSK_GEOM(kBF16, 64) MSK_GEOM(kBF16, 128)
  MSK_GEOM(kE4M3, 32) MSK_GEOM(kE4M3, 64) MSK_GEOM(kE4M3, 128)
#undef MSK_GEOM
  return align_up(sizeof(AttnPlan), 16) + w;
}


static int DenseRowsHost(int nv) { return nv >= 16 ? 2 : 4; }

static int grid_for_waves(long long waves) {
  long long b = (waves + kWaves - 1) / kWaves;
  if (b < 1) b = 1;
  return (int)(b < kMaxGrid ? b : kMaxGrid);
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

static size_t t1_act_lds(const LayerArgs& L) { return t1_lds(L.H, L.Hq * L.D, L.K, L.F).end_act; }
// LDS of the one-token kernels that stage only the hidden-size vector.
static size_t t1_vec_lds(const LayerArgs& L) { return t1_lds(L.H, L.Hq * L.D, L.K, L.F).act1; }

// Workgroups for `tasks` one-wave tasks: every wave gets the same number of
// tasks, at most four workgroups per CU.
static int t1_grid(long long tasks) {
  const long long cap = 4LL * cu_count();
  const long long per_wave = (tasks + cap * kWaves - 1) / (cap * kWaves);
  long long g = (tasks + per_wave * kWaves - 1) / (per_wave * kWaves);
  if (g < 1) g = 1;
  return (int)g;
}

#define MSK_TRY(x)                          \
  do {                                      \
    hipError_t e_ = (x);                    \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

// ------------------------------------------------------ kernel timing
// While a phase's bit is armed, each launch of that phase's kernel takes a
// pair of HIP events stamped by the dispatch itself (hipExtLaunchKernel), so
// the pair brackets the kernel and nothing else.  Events are created on
// first use and reused after msk_timer_start re-arms.
struct PhaseTimer {
  std::mutex mu;
  uint32_t mask = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[kNumPhases];
  size_t used[kNumPhases] = {};
};
static PhaseTimer g_timer;
// Set for the duration of an allocation-free call: no event is created or
// recorded then (event creation allocates).
static thread_local bool g_timer_off = false;

static hipError_t timer_pair(int ph, hipEvent_t* a, hipEvent_t* b) {
  *a = *b = nullptr;
  if (g_timer_off) return hipSuccess;
  std::lock_guard<std::mutex> g(g_timer.mu);
  if (!(g_timer.mask >> ph & 1u)) return hipSuccess;
  auto& v = g_timer.ev[ph];
  if (g_timer.used[ph] == v.size()) {
    hipEvent_t e0, e1;
    MSK_TRY(hipEventCreate(&e0));
    MSK_TRY(hipEventCreate(&e1));
    v.emplace_back(e0, e1);
  }
  *a = v[g_timer.used[ph]].first;
  *b = v[g_timer.used[ph]].second;
  ++g_timer.used[ph];
  return hipSuccess;
}

hipError_t timer_start(uint32_t mask) {
  std::lock_guard<std::mutex> g(g_timer.mu);
  g_timer.mask = mask;
  for (int p = 0; p < kNumPhases; ++p) g_timer.used[p] = 0;
  return hipSuccess;
}

hipError_t timer_read(int ph, double* total_ms, long long* launches) {
  std::lock_guard<std::mutex> g(g_timer.mu);
  double sum = 0;
  for (size_t i = 0; i < g_timer.used[ph]; ++i) {
    float ms = 0;
    MSK_TRY(hipEventSynchronize(g_timer.ev[ph][i].second));
    MSK_TRY(hipEventElapsedTime(&ms, g_timer.ev[ph][i].first, g_timer.ev[ph][i].second));
    sum += ms;
  }
  *total_ms = sum;
  *launches = (long long)g_timer.used[ph];
  return hipSuccess;
}

template <class K, class... A>
static hipError_t launch_b(int ph, K kernel, int grid, int block, size_t lds, hipStream_t st,
                           A... args) {
  hipEvent_t e0, e1;
  MSK_TRY(timer_pair(ph, &e0, &e1));
  if (e0)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), (uint32_t)lds, st, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), lds, st, args...);
  return hipGetLastError();
}

template <class K, class... A>
static hipError_t launch_x(int ph, K kernel, int grid, size_t lds, hipStream_t st, A... args) {
  return launch_b(ph, kernel, grid, kBlockThreads, lds, st, args...);
}

template <class K>
static hipError_t launch(int ph, K kernel, int grid, size_t lds, hipStream_t st,
                         const LayerArgs& L, const StepArgs& S) {
  return launch_x(ph, kernel, grid, lds, st, L, S);
}

static hipError_t set_lds_limit(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}


// ------------------------------------------------------ launchers
// Token-group width of the dense projections: the smallest power of two
// covering T, at most 32 (more tokens are processed in groups).
static int dense_nv(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : T <= 8 ? 8 : T <= 16 ? 16 : 32; }

#define MSK_NV_CASES(NVVAL, BODY)   \
  switch (NVVAL) {                  \
    case 1: { constexpr int NV = 1; BODY; } break;   \
    case 2: { constexpr int NV = 2; BODY; } break;   \
    case 4: { constexpr int NV = 4; BODY; } break;   \
    case 8: { constexpr int NV = 8; BODY; } break;   \
    case 16: { constexpr int NV = 16; BODY; } break; \
    default: { constexpr int NV = 32; BODY; } break; \
  }

// The matrix-core dense path takes bf16 weights, several tokens, whole
// 16-row tiles and whole 128-column k-tiles.
static bool dense_on_mfma(const LayerArgs& L, const StepArgs& S, int N, int K) {
  return S.T > 1 && L.ddt == kBF16 && N % 16 == 0 && K % 128 == 0;
}

template <int CT, int NT>
static hipError_t launch_dense_t(const DenseArgs& A, int ph, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&k_dense_mfma<CT, NT>);
  const size_t lds = DenseLds<CT, NT>::BYTES;
  MSK_TRY(set_lds_limit(fn, lds));
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    MSK_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kBlockThreads, lds));
    per_cu = n > 0 ? n : 1;
  }
  const long long items = (long long)((A.N + 63) / 64) * A.ks;
  const long long cap = (long long)per_cu * cu_count();
  return launch_x(ph, k_dense_mfma<CT, NT>, (int)(items < cap ? items : cap), lds, st, A);
}

// out = resid + W a for the three (QKV) or one weight segments.
// a = RMSNorm(x) * g of T rows as bf16 terms (and as fp32 when a32 is
// given): one 1024-thread workgroup per row, the row loaded once.
static hipError_t launch_prep(const float* x, const float* g, int T, int H, float eps, float* a32,
                              unsigned short* a3, hipStream_t st) {
  const size_t lds = (16 + (size_t)H) * sizeof(float);
  MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_sum_prep), lds));
  return launch_b(kPhPrep, k_sum_prep, T, kSumPrepThreads, lds, st, (const float*)nullptr, 0,
                  (const float*)nullptr, const_cast<float*>(x), g, T, H, eps, a32, a3);
}

// keep_parts: with K split into several slices the partial tiles are left
// in S.dpart for the consumer to sum (dense_slices(N, K) of them).  terms:
// how many of the input's bf16 terms the product takes (2 or 3).
static hipError_t launch_dense(const StepArgs& S, const uint8_t* w0, const uint8_t* w1,
                               const uint8_t* w2, int seg1, int seg2, int N, int K,
                               const float* resid, float* out, int ph, hipStream_t st,
                               bool keep_parts = false, int terms = 3) {
  DenseArgs A;
  A.w[0] = w0; A.w[1] = w1 ? w1 : w0; A.w[2] = w2 ? w2 : w0;
  A.seg[0] = 0; A.seg[1] = seg1; A.seg[2] = seg2;
  A.N = N; A.K = K; A.T = S.T;
  A.ks = dense_slices(N, K);
  A.a3 = S.a3; A.resid = resid; A.out = out; A.part = S.dpart;
  if (terms == 2) {
    switch ((S.T + 15) / 16) {
      case 1: MSK_TRY((launch_dense_t<1, 2>(A, ph, st))); break;
      case 2: MSK_TRY((launch_dense_t<2, 2>(A, ph, st))); break;
      case 3: MSK_TRY((launch_dense_t<3, 2>(A, ph, st))); break;
      default: MSK_TRY((launch_dense_t<4, 2>(A, ph, st))); break;
    }
  } else {
    switch ((S.T + 15) / 16) {
      case 1: MSK_TRY((launch_dense_t<1, 3>(A, ph, st))); break;
      case 2: MSK_TRY((launch_dense_t<2, 3>(A, ph, st))); break;
      case 3: MSK_TRY((launch_dense_t<3, 3>(A, ph, st))); break;
      default: MSK_TRY((launch_dense_t<4, 3>(A, ph, st))); break;
    }
  }
  if (A.ks == 1 || keep_parts) return hipSuccess;
  const long long n = (long long)S.T * N;
  return launch_x(kPhDenseSum, k_dense_sum, (int)((n + kBlockThreads - 1) / kBlockThreads), 0,
                  st, (const float*)S.dpart, N, S.T, A.ks, resid, out);
}

// Matrix-core attention: as many resident workgroups as the CUs hold, each
// looping over items.
template <int KDT, int D, int NW, int NPH = 1>
static hipError_t launch_attn_mfma_t(const LayerArgs& L, const StepArgs& S, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&k_attn_mfma<KDT, D, NW, NPH>);
  constexpr size_t item_lds = KDT == kE4M3 && D == 128 && NW == 4 ? (size_t)F8Geom<NPH>::LDS
                                                                    : (size_t)MfmaGeom<KDT, D, NW, NPH>::LDS;
  const size_t lds = align_up(sizeof(AttnPlan), 16) + item_lds;
  MSK_TRY(set_lds_limit(fn, lds));
  static int per_cu = 0;  // one value per instantiation
  if (per_cu == 0) {
    int n = 0;
    MSK_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, NW * 64, lds));
    per_cu = n > 0 ? n : 1;
  }
  const long long cap = (long long)per_cu * cu_count();
  const int grid = (int)(L.n_items < cap ? L.n_items : cap);
  return launch_b(kPhAttn, k_attn_mfma<KDT, D, NW, NPH>, grid, NW * 64, lds, st, L, S);
}

template <int KDT, int D>
static hipError_t launch_attn_mfma_d(const LayerArgs& L, const StepArgs& S, hipStream_t st) {
  switch (L.attn_nw) {
    // the planner gives bf16 caches of head_dim 128 at least two waves and
    // e4m3 caches of head_dim 128 four (register budget)
    case 1:
      if constexpr (D == 128) return hipErrorInvalidValue;
      else return launch_attn_mfma_t<KDT, D, 1>(L, S, st);
    case 2:
      if constexpr (D == 128 && KDT == kE4M3) return hipErrorInvalidValue;
      else return launch_attn_mfma_t<KDT, D, 2>(L, S, st);
    case 3:
      if constexpr (D == 128 && KDT == kE4M3) return hipErrorInvalidValue;
      else return launch_attn_mfma_t<KDT, D, 3>(L, S, st);
    default:
      if constexpr (D == 128 && KDT == kE4M3)
        if (L.attn_nph == 2) return launch_attn_mfma_t<KDT, D, 4, 2>(L, S, st);
      return launch_attn_mfma_t<KDT, D, 4>(L, S, st);
  }
}

static hipError_t launch_attn_mfma(const LayerArgs& L, const StepArgs& S, hipStream_t st) {
  if (L.kdt == kBF16) {
    if (L.D == 32) return launch_attn_mfma_d<kBF16, 32>(L, S, st);
    if (L.D == 64) return launch_attn_mfma_d<kBF16, 64>(L, S, st);
    return launch_attn_mfma_d<kBF16, 128>(L, S, st);
  }
  if (L.D == 32) return launch_attn_mfma_d<kE4M3, 32>(L, S, st);
  if (L.D == 64) return launch_attn_mfma_d<kE4M3, 64>(L, S, st);
  return launch_attn_mfma_d<kE4M3, 128>(L, S, st);
}

// Most chunks per group for which the vector attention items sum their own
// partials.
constexpr int kFuseChunks = 8;

// The attention partials (matrix-core or vector kernel); with `fused` the
// vector kernel also sums them (k_attn_c).
static hipError_t launch_attn_kernel(const LayerArgs& L, const StepArgs& S, hipStream_t st,
                                     bool fused) {
  if (L.attn_nw > 0) return launch_attn_mfma(L, S, st);
  const size_t alds = attn_lds_bytes(L.kdt, L.D);
  const int agrid = L.n_items < 8 * cu_count() ? L.n_items : 8 * cu_count();
#define MSK_ATTN(K, DD)                                                             \
  if (L.kdt == K && L.D == DD) {                                                    \
    if (fused) {                                                                    \
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_attn_c<K, DD>), alds)); \
      return launch(kPhAttn, k_attn_c<K, DD>, agrid, alds, st, L, S);                \
    }                                                                               \
    MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_attn<K, DD>), alds));   \
    return launch(kPhAttn, k_attn<K, DD>, agrid, alds, st, L, S);                  \
  }
  MSK_ATTN(kF32, 32) MSK_ATTN(kF32, 64) MSK_ATTN(kF32, 128)
  MSK_ATTN(kBF16, 32) MSK_ATTN(kBF16, 64) MSK_ATTN(kBF16, 128)
  MSK_ATTN(kE4M3, 32) MSK_ATTN(kE4M3, 64) MSK_ATTN(kE4M3, 128)
#undef MSK_ATTN
  return hipErrorInvalidValue;
}

bool wo_sum_in_route(const LayerArgs& L, const StepArgs& S) {
  return dense_on_mfma(L, S, L.H, L.Hq * L.D) && dense_on_mfma(L, S, L.E, L.H);
}

bool qkv_on_mfma(const LayerArgs& L, const StepArgs& S) {
  return dense_on_mfma(L, S, (L.Hq + 2 * L.Hkv) * L.D, L.H);
}

hipError_t launch_attn(const LayerArgs& L, const StepArgs& S, const float* x, float* h,
                       hipStream_t st, bool wo_parts, bool a3_ready) {
  const int NR = (L.Hq + 2 * L.Hkv) * L.D;
  const size_t rs_lds = (size_t)S.T * sizeof(float);
  const int nv = dense_nv(S.T);
  const int qgrid = grid_for_waves(NR / DenseRowsHost(nv));
  const bool one = S.T == 1;
  if (one) {
    const size_t lds = t1_vec_lds(L);
    const int g = t1_grid(NR / 4);
    if (L.ddt == kBF16) {
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_qkv_t1<kBF16>), lds));
      MSK_TRY(launch_x(kPhQkv, k_qkv_t1<kBF16>, g, lds, st, L, S, x));
    } else {
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_qkv_t1<kF32>), lds));
      MSK_TRY(launch_x(kPhQkv, k_qkv_t1<kF32>, g, lds, st, L, S, x));
    }
  } else if (dense_on_mfma(L, S, NR, L.H)) {
    if (!a3_ready)
      MSK_TRY(launch_prep(x, L.attn_norm, S.T, L.H, L.eps, nullptr, S.a3, st));
    const int NQ = L.Hq * L.D, NK = L.Hkv * L.D;
    MSK_TRY(launch_dense(S, L.wq, L.wk, L.wv, NQ, NQ + NK, NR, L.H, nullptr, S.qkv, kPhQkv, st));
  } else {
    if (L.ddt == kBF16)
      MSK_NV_CASES(nv, MSK_TRY(launch_x(kPhQkv, k_qkv<kBF16, NV>, qgrid, rs_lds, st, L, S, x)))
    else
      MSK_NV_CASES(nv, MSK_TRY(launch_x(kPhQkv, k_qkv<kF32, NV>, qgrid, rs_lds, st, L, S, x)))
  }

  const bool mm = dense_on_mfma(L, S, L.H, L.Hq * L.D);
  // Vector items (a group holds at most kRowGroup rows) over a few chunks per
  // group: the last item of a group sums its partials.  Its tail (waiting
  // for the partial stores, the counter's round trip, then reading every
  // chunk back) grows with the chunks: over 32 chunks of six rows (a
  // 2048-position window at head_dim 128) it added 6.2 us to the attention
  // kernel, against 4.2 us for a combine launch.  Matrix-core items, whose
  // groups hold up to 64 rows, groups of more chunks, and steps whose output
  // projection runs on the matrix cores (it reads attn_o as bf16 terms,
  // which the combine launch writes) leave the sums to a combine launch
  // spread over every (token, q head).
  int most = 0;
  for (int b = 0; b < S.n_req; ++b) {
    int base, end;
    req_span(S.kv_len[b], S.Tr, L.window, L.attn_nw != 0, base, end);
    const int n = ceil_div(end - base, L.chunk);
    most = n > most ? n : most;
  }
  const bool fused = L.attn_nw == 0 && !mm && most <= kFuseChunks &&
                     S.n_req * L.Hkv * L.nrg <= kAttnCountMax;
  MSK_TRY(launch_attn_kernel(L, S, st, fused));
  if (!fused) {
    const size_t lds = align_up(sizeof(AttnPlan), 16) + (size_t)kWaves * (L.D + 1) * sizeof(float);
    const int rows = S.T * L.Hq;  // one workgroup per (token, q head)
    MSK_TRY(launch_x(kPhCombine, k_combine, rows < 8192 ? rows : 8192, lds, st, L, S, S.win_out,
                     mm ? S.a3 : nullptr));
  }
  const int wgrid = grid_for_waves(L.H / DenseRowsHost(nv));
  if (one) {
    const size_t lds = t1_vec_lds(L);
    const int g = t1_grid((L.H + 1) / 2);
    if (L.ddt == kBF16) {
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_wo_t1<kBF16>), lds));
      MSK_TRY(launch_x(kPhWo, k_wo_t1<kBF16>, g, lds, st, L, S, x, h));
    } else {
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_wo_t1<kF32>), lds));
      MSK_TRY(launch_x(kPhWo, k_wo_t1<kF32>, g, lds, st, L, S, x, h));
    }
  } else if (mm) {
    MSK_TRY(launch_dense(S, L.wo, nullptr, nullptr, 0, 0, L.H, L.Hq * L.D, x, h, kPhWo, st,
                         wo_parts && wo_sum_in_route(L, S), /*terms=*/2));
  } else {
    if (L.ddt == kBF16)
      MSK_NV_CASES(nv, MSK_TRY(launch_x(kPhWo, k_wo<kBF16, NV>, wgrid, 0, st, L, S, x, h)))
    else
      MSK_NV_CASES(nv, MSK_TRY(launch_x(kPhWo, k_wo<kF32, NV>, wgrid, 0, st, L, S, x, h)))
  }
  return hipSuccess;
}

hipError_t launch_route(const LayerArgs& L, const StepArgs& S, const float* h, int* topk_out,
                        hipStream_t st, bool defer_topk, const float* wo_resid) {
  const size_t rs_lds = (size_t)S.T * sizeof(float);
  const int nv = dense_nv(S.T);
  const int rows = (L.E + DenseRowsHost(nv) - 1) / DenseRowsHost(nv);
  const int grid = grid_for_waves(rows > 64 ? rows : 64);
  int ks = 1;  // split-K slices of the logits left for the top-k kernel to sum
  if (S.T == 1) {
    const size_t lds = t1_vec_lds(L) + (size_t)kWaves * kRouterRows * sizeof(float);
    const int g = L.E < cu_count() ? L.E : cu_count();
    if (L.ddt == kBF16) {
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_router_t1<kBF16>), lds));
      MSK_TRY(launch_x(kPhRouter, k_router_t1<kBF16>, g, lds, st, L, S, h));
    } else {
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_router_t1<kF32>), lds));
      MSK_TRY(launch_x(kPhRouter, k_router_t1<kF32>, g, lds, st, L, S, h));
    }
    // top-k outside the router kernel: finding the last router workgroup
    // costs every workgroup an agent-scope acquire and release, which here
    // means L2 writeback and invalidate.  Within a layer step the one-token
    // gate/up kernel selects the experts itself (defer_topk).
    if (defer_topk) return hipSuccess;
    return launch_x(kPhTopk, k_topk, 1, 0, st, L, S, topk_out);
  } else if (dense_on_mfma(L, S, L.E, L.H)) {
    if (wo_resid != nullptr && wo_sum_in_route(L, S)) {
      // h = x + the Wo partial tiles, then the router's input, in one pass
      const size_t lds = (16 + (size_t)L.H) * sizeof(float);
      MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_sum_prep), lds));
      MSK_TRY(launch_b(kPhPrep, k_sum_prep, S.T, kSumPrepThreads, lds, st, (const float*)S.dpart,
                       dense_slices(L.H, L.Hq * L.D), wo_resid, S.h, L.ffn_norm, S.T, L.H, L.eps,
                       S.u, S.a3));
    } else {
      MSK_TRY(launch_prep(h, L.ffn_norm, S.T, L.H, L.eps, S.u, S.a3, st));
    }
    MSK_TRY(launch_dense(S, L.wr, nullptr, nullptr, 0, 0, L.E, L.H, nullptr, S.logits, kPhRouter,
                         st, /*keep_parts=*/true));
    ks = dense_slices(L.E, L.H);
  } else {
    if (L.ddt == kBF16)
      MSK_NV_CASES(nv, MSK_TRY(launch_x(kPhRouter, k_router<kBF16, NV>, grid, rs_lds, st, L, S, h)))
    else
      MSK_NV_CASES(nv, MSK_TRY(launch_x(kPhRouter, k_router<kF32, NV>, grid, rs_lds, st, L, S, h)))
  }
  // the expert union comes with the selection: the multi-token expert
  // kernels read it (launch_ffn with union_ready)
  return launch_b(kPhTopk, k_topk_union, (S.T + kTopkWaves - 1) / kTopkWaves, kTopkWaves * 64,
                  kUnionLds, st, L, S, topk_out, (const float*)S.dpart, ks);
}

template <int DT>
static hipError_t launch_ffn_t1(const LayerArgs& L, const StepArgs& S, const float* h, float* out,
                                hipStream_t st, bool own_topk, int* topk_out) {
  const size_t vlds = t1_vec_lds(L), alds = 256 + (size_t)4 * L.K * L.F;
  MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_gateup_t1<DT>), vlds));
  MSK_TRY(launch_x(kPhGateUp, k_gateup_t1<DT>, t1_grid((long long)L.K * (L.F / 2)), vlds, st, L, S,
                   topk_out, (int)own_topk));
  MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_down_t1<DT>), alds));
  MSK_TRY(launch_x(kPhDown, k_down_t1<DT>, t1_grid((L.H + 2) / 3), alds, st, L, S, h, out));
  return hipSuccess;
}


// Resident workgroups of a kernel at `lds` bytes, times the CU count,
// remembered per (kernel, LDS size): the expert kernels' LDS depends on the
// hidden and FFN sizes of the call.
static int resident_grid(const void* fn, size_t lds, int threads = kBlockThreads) {
  struct Entry { const void* fn; size_t lds; int threads, grid, dev; };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> g(mu);
  for (int i = 0; i < used; ++i) {
    const Entry& e = cache[i];
    if (e.fn == fn && e.lds == lds && e.threads == threads && e.dev == dev) return e.grid;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess ||
      n < 1)
    n = 1;
  const int grid = n * cu_count();
  if (used < 64) cache[used++] = Entry{fn, lds, threads, grid, dev};
  return grid;
}

// token vectors staged per gate/up pass: four fp32 vectors (96 KB at
// H = 6144, one workgroup per CU) for fp32 and bf16 experts, three fp16 ones
// for NVFP4 (register pressure of its decode).  Measured: bf16 four per
// pass 10% faster than two on verify-bf16-128k (two with one workgroup per
// CU much slower than either); NVFP4 three 3% faster than two on
// stack4-nvfp4, four slower.
template <int DT> constexpr int kGateUpTokens = DT == kNVFP4 ? 3 : 4;
// waves per gate/up workgroup (sharing its staged inputs): eight for the
// one-per-CU fp32 and bf16 workgroups (4% faster than four on
// verify-bf16-128k)
template <int DT> constexpr int kGateUpWaves = DT == kNVFP4 ? 4 : 8;
// slot vectors staged per down pass (NVFP4 three: 4% faster than two on
// longctx-nvfp4, four slower)
template <int DT> constexpr int kDownTokens = DT == kNVFP4 ? 3 : 4;
// waves per down workgroup
template <int DT> constexpr int kDownWaves = 4;

template <int DT>
static hipError_t launch_experts_tn(const LayerArgs& L, const StepArgs& S, hipStream_t st) {
  {
    constexpr int nwv = kGateUpWaves<DT>;
    auto fn = k_gateup_tn<DT, kGateUpTokens<DT>, nwv>;
    const size_t lds = ((size_t)kGateUpTokens<DT> * tn_vec_floats<DT>(L.H) + nwv) * sizeof(float);
    MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(fn), lds));
    const int grid = resident_grid(reinterpret_cast<const void*>(fn), lds, nwv * 64);
    MSK_TRY(launch_b(kPhGateUp, fn, grid, nwv * 64, lds, st, L, S));
  }
  {
    constexpr int nwv = kDownWaves<DT>;
    auto fn = k_down_tn<DT, kDownTokens<DT>, nwv>;
    const size_t lds = ((size_t)kDownTokens<DT> * tn_vec_floats<DT>(L.F) + nwv) * sizeof(float);
    MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(fn), lds));
    const int grid = resident_grid(reinterpret_cast<const void*>(fn), lds, nwv * 64);
    MSK_TRY(launch_b(kPhDown, fn, grid, nwv * 64, lds, st, L, S));
  }
  return hipSuccess;
}

template <int DT>
static hipError_t launch_ffn_tn(const LayerArgs& L, const StepArgs& S, const float* h, float* out,
                                hipStream_t st, bool union_ready, const float* next_norm,
                                float next_eps) {
  if (!union_ready) MSK_TRY(launch_x(kPhUnion, k_union, 1, kUnionLds, st, L, S));
  MSK_TRY(launch_experts_tn<DT>(L, S, st));
  if (next_norm != nullptr) {
    // the sum and the next layer's QKV input terms in one pass per token
    const size_t lds = (16 + (size_t)L.H) * sizeof(float);
    MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(&k_moe_sum_prep), lds));
    return launch_b(kPhMoeSum, k_moe_sum_prep, S.T, kSumPrepThreads, lds, st, L, S, h, out,
                    next_norm, next_eps);
  }
  const long long n4 = (long long)S.T * L.H / 4;
  return launch_x(kPhMoeSum, k_moe_sum, (int)((n4 + kBlockThreads - 1) / kBlockThreads), 0, st,
                  L, S, h, out);
}

// ------------------------------------------------- prefill expert FFN
__global__ __launch_bounds__(1024) void k_pf_route(LayerArgs L, PfArgs P, int cmax) {
  pf_route(L, P, cmax, reinterpret_cast<int*>(msk_smem));
}
template <bool FP4>
__global__ __launch_bounds__(kBlockThreads) void k_pf_gather(LayerArgs L, PfArgs P) {
  pf_gather<FP4>(L, P);
}
template <bool FP4>
__global__ __launch_bounds__(kBlockThreads) void k_pf_swiglu(LayerArgs L, PfArgs P) {
  pf_swiglu<FP4>(L, P);
}
template <bool FP4, bool GU>
__global__ __launch_bounds__(kBlockThreads) void k_pf_gemm(LayerArgs L, PfArgs P) {
  pf_gemm<FP4, GU>(L, P, msk_smem);
}

template <bool FP4>
static hipError_t launch_pf(const LayerArgs& L, const PfArgs& P, hipStream_t st) {
  const int slots = P.T * L.K;
  // one wave per token, then per grouped position
  MSK_TRY(launch_x(kPhPrep, k_pf_gather<FP4>, (P.T + kWaves - 1) / kWaves, 0, st, L, P));
  auto gemm = [&](auto fn, int ph) -> hipError_t {
    constexpr size_t lds = pf_lds<FP4>();
    MSK_TRY(set_lds_limit(reinterpret_cast<const void*>(fn), lds));
    // a multiple of 8 workgroups: the items are split by XCD
    int grid = resident_grid(reinterpret_cast<const void*>(fn), lds) & ~7;
    if (grid < 8) grid = 8;
    return launch_x(ph, fn, grid, lds, st, L, P);
  };
  MSK_TRY(gemm(k_pf_gemm<FP4, true>, kPhGateUp));
  MSK_TRY(launch_x(kPhPrep, k_pf_swiglu<FP4>, (slots + kWaves - 1) / kWaves, 0, st, L, P));
  return gemm(k_pf_gemm<FP4, false>, kPhDown);
}

hipError_t launch_prefill(const LayerArgs& L, const PfArgs& P, const float* wts, const float* h,
                          float* out, hipStream_t st) {
  const size_t rl = (3 * kMaxExperts + 8) * sizeof(int);
  const int cmax = L.edt == kNVFP4 ? PfFmt<true>::CHUNK : PfFmt<false>::CHUNK;
  MSK_TRY(launch_b(kPhUnion, k_pf_route, 1, 1024, rl, st, L, P, cmax));
  if (L.edt == kNVFP4)
    MSK_TRY(launch_pf<true>(L, P, st));
  else
    MSK_TRY(launch_pf<false>(L, P, st));
  // out[t] = h[t] + sum_j w[t][j] y[t K + j], the decode path's weighted combine
  StepArgs S{};
  S.T = P.T;
  S.idx = const_cast<int*>(P.idx);
  S.wts = const_cast<float*>(wts);
  S.ybuf = P.y;
  const long long n4 = (long long)P.T * L.H / 4;
  return launch_x(kPhMoeSum, k_moe_sum, (int)((n4 + kBlockThreads - 1) / kBlockThreads), 0, st,
                  L, S, h, out);
}

bool ffn_one_token(const LayerArgs& L, const StepArgs& S) {
  return S.T == 1 && t1_act_lds(L) <= kMaxLds;
}

hipError_t launch_ffn(const LayerArgs& L, const StepArgs& S, const float* h, float* out,
                      hipStream_t st, bool union_ready, bool own_topk, int* topk_out,
                      const float* next_norm, float next_eps) {
  if (ffn_one_token(L, S)) {
    switch (L.edt) {
      case kF32: return launch_ffn_t1<kF32>(L, S, h, out, st, own_topk, topk_out);
      case kBF16: return launch_ffn_t1<kBF16>(L, S, h, out, st, own_topk, topk_out);
      default: return launch_ffn_t1<kNVFP4>(L, S, h, out, st, own_topk, topk_out);
    }
  }
  switch (L.edt) {
    case kF32: return launch_ffn_tn<kF32>(L, S, h, out, st, union_ready, next_norm, next_eps);
    case kBF16: return launch_ffn_tn<kBF16>(L, S, h, out, st, union_ready, next_norm, next_eps);
    default: return launch_ffn_tn<kNVFP4>(L, S, h, out, st, union_ready, next_norm, next_eps);
  }
}

// Layer l reads `cur` and writes the next buffer; the last layer writes x_out.
hipError_t launch_step_unfused(const LayerArgs* Ls, const StepArgs& S0, hipStream_t st) {
  StepArgs S = S0;
  const float* cur = S.x_in;
  bool a3_ready = false;  // this layer's QKV input terms came with the previous layer's sum
  for (int l = 0; l < S.n_layers; ++l) {
    const LayerArgs& L = Ls[l];
    float* nxt = (l == S.n_layers - 1) ? S.x_out : ((l & 1) ? S.xb : S.xa);
    int* topk = S0.topk_out ? S0.topk_out + (size_t)l * S.T * L.K : nullptr;
    S.win_out = S0.win_out ? S0.win_out + (size_t)l * S.T * 2 : nullptr;
    // one token: the gate/up kernel takes the top-k; several: the router's
    // top-k kernel also builds the expert union
    const bool own = ffn_one_token(L, S);
    // several tokens: the Wo partial sums join the router's input pass
    const bool wsr = wo_sum_in_route(L, S);
    MSK_TRY(launch_attn(L, S, cur, S.h, st, /*wo_parts=*/wsr, a3_ready));
    MSK_TRY(launch_route(L, S, S.h, topk, st, /*defer_topk=*/own, wsr ? cur : nullptr));
    // several tokens: the expert sum also prepares the next layer's QKV input
    const bool pre = l + 1 < S.n_layers && !own && qkv_on_mfma(Ls[l + 1], S);
    MSK_TRY(launch_ffn(L, S, S.h, nxt, st, /*union_ready=*/S.T > 1, own, topk,
                       pre ? Ls[l + 1].attn_norm : nullptr, pre ? Ls[l + 1].eps : 0.f));
    a3_ready = pre;
    if (S.layer_out)
      MSK_TRY(hipMemcpyAsync(S.layer_out + (size_t)l * S.T * L.H, nxt,
                             (size_t)S.T * L.H * sizeof(float), hipMemcpyDeviceToDevice, st));
    cur = nxt;
  }
  return hipSuccess;
}

// The persistent step kernel over the stack, kMaxFusedLayers layers per
// launch.  *launched is false (nothing enqueued) when this instantiation
// cannot hold its workgroups resident at this LDS size.
template <int DDT, int EDT, int KDT, int D>
static hipError_t launch_persistent(const LayerArgs* Ls, const StepArgs& S, hipStream_t st,
                                    bool* launched) {
  *launched = false;
  auto fn = k_step_p<DDT, EDT, KDT, D>;
  const void* fp = reinterpret_cast<const void*>(fn);
  size_t lds = 0;
  for (int l = 0; l < S.n_layers; ++l) {
    const size_t attn = align_up(sizeof(AttnPlan), 16) + AttnGeom<KDT, D>::LDS_ITEM;
    const size_t need = p_lds_bytes(Ls[l].H, Ls[l].Hq * Ls[l].D, Ls[l].K, Ls[l].F, attn);
    lds = lds > need ? lds : need;
  }
  if (lds > kMaxLds) return hipSuccess;
  MSK_TRY(set_lds_limit(fp, lds));
  // every workgroup must be resident at once (the barriers wait for all of
  // them): at most the occupancy at this LDS size, and at most two per CU
  // (a barrier over more workgroups costs more)
  int per_cu = 0;
  MSK_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fp, kBlockThreads, lds));
  if (per_cu < 1) return hipSuccess;
  const int grid = (per_cu < 2 ? per_cu : 2) * cu_count();
  for (int l0 = 0; l0 < S.n_layers; l0 += kMaxFusedLayers) {
    StepLayers P;
    P.S = S;
    P.l0 = l0;
    P.nl = S.n_layers - l0 < kMaxFusedLayers ? S.n_layers - l0 : kMaxFusedLayers;
    for (int l = 0; l < kMaxFusedLayers; ++l) P.L[l] = Ls[l0 + (l < P.nl ? l : 0)];
    if (l0 > 0) P.S.x_in = ((l0 - 1) & 1) ? S.xb : S.xa;  // the previous launch's output
    MSK_TRY(launch_b(kPhStep, fn, grid, kBlockThreads, lds, st, P));
  }
  *launched = true;
  return hipSuccess;
}

bool persistent_supported(const LayerArgs* Ls, const StepArgs& S) {
  if (S.T != 1) return false;
  // its attention phase runs the vector items
  for (int l = 0; l < S.n_layers; ++l)
    if (Ls[l].attn_nw != 0) return false;
  for (int l = 1; l < S.n_layers; ++l)
    if (Ls[l].ddt != Ls[0].ddt || Ls[l].edt != Ls[0].edt || Ls[l].kdt != Ls[0].kdt ||
        Ls[l].D != Ls[0].D)
      return false;
  const LayerArgs& L = Ls[0];
  if (L.ddt == kBF16 && L.edt == kBF16 && L.kdt == kBF16 && L.D == 128) return true;
  if (L.ddt == kBF16 && L.edt == kNVFP4 && L.kdt == kE4M3 && L.D == 128) return true;
  if (L.ddt == kF32 && L.edt == kF32 && L.kdt == kF32 && L.D == 32) return true;
  return false;
}

// The whole one-token step as the persistent kernel where an instantiation
// exists and its workgroups fit; otherwise the per-phase kernels.
hipError_t launch_step_fused(const LayerArgs* Ls, const StepArgs& S, hipStream_t st,
                             bool* persistent) {
  bool launched = false;
  *persistent = false;
  if (persistent_supported(Ls, S)) {
    const LayerArgs& L = Ls[0];
    if (L.ddt == kBF16 && L.edt == kBF16)
      MSK_TRY((launch_persistent<kBF16, kBF16, kBF16, 128>(Ls, S, st, &launched)));
    else if (L.ddt == kBF16)
      MSK_TRY((launch_persistent<kBF16, kNVFP4, kE4M3, 128>(Ls, S, st, &launched)));
    else
      MSK_TRY((launch_persistent<kF32, kF32, kF32, 32>(Ls, S, st, &launched)));
  }
  *persistent = launched;
  if (launched) return hipSuccess;
  return launch_step_unfused(Ls, S, st);
}

// ------------------------------------------- allocation-free scratch
// Scratch of the allocation-free entry point: one array per GPU, allocated
// by the code object loader with the library and held until the process
// ends.  Host code never uses this name as an address (in host code it is a
// stand-in, not the device address): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  *out = nullptr;
  int dev = 0;
  MSK_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> g(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    MSK_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// Zero n words with a plain kernel (no memset node, so the call can sit in a
// captured graph).
__global__ __launch_bounds__(kBlockThreads) void k_clear_words(unsigned* w, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0u;
}

hipError_t launch_step_noalloc(const LayerArgs* Ls, const StepArgs& S, hipStream_t st) {
  struct Off {
    Off() { g_timer_off = true; }
    ~Off() { g_timer_off = false; }
  } off;
  // the array keeps the previous call's contents: the barrier and counter
  // words must start at zero
  const int n = kSyncBytes / 4;
  hipLaunchKernelGGL(k_clear_words, dim3((n + kBlockThreads - 1) / kBlockThreads),
                     dim3(kBlockThreads), 0, st, S.sync, n);
  MSK_TRY(hipGetLastError());
  return launch_step_unfused(Ls, S, st);
}

}  // namespace msk
