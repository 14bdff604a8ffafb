// One-token (decode) phases.  With a single token every phase's input vector
// fits in LDS, so each workgroup stages it once (RMSNorm and gain applied on
// the way in) and the weight rows stream through registers two buffers deep
// (stream_t1).  Work is dealt out wave-major over the workgroups so that a
// phase with fewer tasks than waves still spreads over every CU.
#pragma once
#include "phases.h"

namespace msk {

// Tasks of wave gw out of ntask dealt round-robin over nw waves.
__device__ __forceinline__ int my_count(int gw, int nw, int ntask) {
  return gw < ntask ? (ntask - 1 - gw) / nw + 1 : 0;
}

// act[c] = x[c] * g[c] / sqrt(mean(x^2) + eps) into LDS (g may be null).
template <class M = Plain>
__device__ inline void stage_norm_t1(const float* x, const float* g, int H, float eps, float* act,
                                     float* red) {
  float s = 0.f;
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    v4f a = M::ld4(x + c);
    s += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  }
  const float r = 1.0f / sqrtf(block_sum(s, red) / (float)H + eps);
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    v4f a = M::ld4(x + c);
    v4f gg = *reinterpret_cast<const v4f*>(g + c);
    *reinterpret_cast<v4f*>(act + c) = v4f{a.x * r * gg.x, a.y * r * gg.y, a.z * r * gg.z, a.w * r * gg.w};
  }
  __syncthreads();
}

// Plain copy of n floats (n % 4 == 0) into LDS.
template <class M = Plain>
__device__ inline void stage_copy(const float* src, int n, float* dst) {
  for (int c = threadIdx.x * 4; c < n; c += blockDim.x * 4)
    *reinterpret_cast<v4f*>(dst + c) = M::ld4(src + c);
  __syncthreads();
}

// Lane r < R stores acc[r] through st(r, value).
template <int R, class F>
__device__ __forceinline__ void lane_store(const float (&acc)[R], F&& st) {
  const int ln = lane_id();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (ln == r) st(r, acc[r]);
}

// qkv[r] = sum_c W[r][c] act[c] over the stacked rows of wq, wk, wv.
template <int DT, class M = Plain, class Pre>
__device__ void qkv_t1(const LayerArgs& L, const StepArgs& S, const float* act, int vb, int nvb,
                       Pre&& pre) {
  constexpr int R = 4, U = 2;
  const int NQ = L.Hq * L.D, NK = L.Hkv * L.D, NR = NQ + 2 * NK;
  const size_t rb = dense_row_bytes(DT, L.H);
  const int gw = gwave(vb, nvb), nw = nvb * kWaves;
  const int n = my_count(gw, nw, NR / R);
  stream_t1<DT, R, U>(
      n, L.H, [&](int) { return act; },
      [&](int k, auto& wr, auto& sr) {
        const int r0 = (gw + k * nw) * R;
        const uint8_t* base;
        int rr;
        if (r0 < NQ) { base = L.wq; rr = r0; }
        else if (r0 < NQ + NK) { base = L.wk; rr = r0 - NQ; }
        else { base = L.wv; rr = r0 - NQ - NK; }
#pragma unroll
        for (int r = 0; r < R; ++r) { wr[r] = base + (size_t)(rr + r) * rb; sr[r] = nullptr; }
      },
      [&](int k, auto& acc) {
        const int r0 = (gw + k * nw) * R;
        lane_store<R>(acc, [&](int r, float v) { M::st(&S.qkv[r0 + r], v); });
      },
      pre);
}

// h[r] = x[r] + sum_c wo[r][c] act[c]  (act = staged attention output)
template <int DT, class M = Plain, class Pre>
__device__ void wo_t1(const LayerArgs& L, const StepArgs& S, const float* x, float* h,
                      const float* act, int vb, int nvb, Pre&& pre) {
  // two rows per task: at hidden 6144 one task per wave then gives twice the
  // waves of four-row tasks, and with them twice the rows in flight (Wo went
  // from 15.3 to 13.6 us; QKV, which has 2048 four-row tasks, did not gain)
  constexpr int R = 2, U = 2;
  const int NI = L.Hq * L.D;
  const size_t rb = dense_row_bytes(DT, NI);
  const int gw = gwave(vb, nvb), nw = nvb * kWaves;
  const int n = my_count(gw, nw, (L.H + R - 1) / R);
  stream_t1<DT, R, U>(
      n, NI, [&](int) { return act; },
      [&](int k, auto& wr, auto& sr) {
        const int r0 = (gw + k * nw) * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = r0 + r < L.H ? r0 + r : L.H - 1;
          wr[r] = L.wo + (size_t)row * rb;
          sr[r] = nullptr;
        }
      },
      [&](int k, auto& acc) {
        const int r0 = (gw + k * nw) * R;
        lane_store<R>(acc, [&](int r, float v) {
          if (r0 + r < L.H) M::st(&h[r0 + r], M::ld(&x[r0 + r]) + v);
        });
      },
      pre);
}

// u = RMSNorm(h) * ffn_norm into LDS by stage() (workgroup vb then writes its
// slice of u to global memory); logits[e] = w_router[e] . u.  Workgroup vb owns rows
// vb, vb + nvb, ...; each of its waves streams one quarter of every row and
// the quarters are added in fixed order.  part: LDS [kWaves][kRouterRows].
constexpr int kRouterRows = 16;

template <int DT, class M = Plain, class Stage>
__device__ void router_t1(const LayerArgs& L, const StepArgs& S, float* act, float* part, int vb,
                          int nvb, Stage stage) {
  constexpr int R = 1, U = 2;
  const int w = wave_id();
  const int cols = L.H / kWaves;
  const size_t rb = dense_row_bytes(DT, L.H);
  const size_t coff = dense_row_bytes(DT, w * cols);
  const int n = my_count(vb, nvb, L.E);
  stream_t1<DT, R, U>(
      n, cols, [&](int) { return act + w * cols; },
      [&](int k, auto& wr, auto& sr) {
        wr[0] = L.wr + (size_t)(vb + k * nvb) * rb + coff;
        sr[0] = nullptr;
      },
      [&](int k, auto& acc) {
        if (lane_id() == 0) part[w * kRouterRows + k] = acc[0];
      },
      [&]() {
        stage();
        const int per = ((L.H / 4 + nvb - 1) / nvb) * 4;
        const int c0 = vb * per, c1 = c0 + per < L.H ? c0 + per : L.H;
        for (int c = c0 + threadIdx.x * 4; c < c1; c += blockDim.x * 4)
          M::st4(S.u + c, *reinterpret_cast<const v4f*>(act + c));
      });
  __syncthreads();
  for (int k = threadIdx.x; k < n; k += blockDim.x) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) v += part[q * kRouterRows + k];
    M::st(&S.logits[vb + k * nvb], v);
  }
}

// Order key of a logit: a larger value gives a larger key (NaN counts as
// -inf, -0 as +0).  Every logit's key is nonzero; 0 marks no expert.
__device__ __forceinline__ unsigned topk_key(float x) {
  float v = (x == x) ? x : -INFINITY;
  if (v == 0.f) v = 0.f;
  const unsigned b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float topk_key_value(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave-wide maximum of an unsigned key (DPP within rows of 16 lanes, then
// four lane reads); every lane gets it.
__device__ __forceinline__ unsigned wave_max_u(unsigned v) {
  v = max(v, (unsigned)dpp_i<kDppXor1>((int)v));
  v = max(v, (unsigned)dpp_i<kDppXor2>((int)v));
  v = max(v, (unsigned)dpp_i<kDppRor4>((int)v));
  v = max(v, (unsigned)dpp_i<kDppRor8>((int)v));
  const unsigned a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const unsigned c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Top-k of one token's logits by one wave (value descending, index ascending
// on ties) into registers (uniform over the wave): bis[k] the experts,
// exs[k] / den their softmax weights.  Lane l holds the logits of experts
// l + 64 i in x[i] (i < 4; entries at E or beyond are never selected; E <=
// 256).  Each lane sorts its four (key, expert) pairs once; a round takes the
// wave-wide maximum of the lanes' first keys, and the lane holding it (among
// equal keys the one whose expert index is lowest) moves to its next.
__device__ __forceinline__ void topk_vals(const float (&x)[4], int E, int K,
                                          int (&bis)[kMaxTopK], float (&exs)[kMaxTopK],
                                          float& den) {
  const int ln = lane_id();
  unsigned kv[4];
  int ke[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = ln + 64 * i;
    kv[i] = e < E ? topk_key(x[i]) : 0u;
    ke[i] = e;
  }
  auto cs = [](unsigned& ka, int& ea, unsigned& kb, int& eb) {  // (ka, ea) ranks first afterwards
    const bool sw = kb > ka || (kb == ka && eb < ea);
    const unsigned k0 = sw ? kb : ka, k1 = sw ? ka : kb;
    const int e0 = sw ? eb : ea, e1 = sw ? ea : eb;
    ka = k0; kb = k1; ea = e0; eb = e1;
  };
  cs(kv[0], ke[0], kv[1], ke[1]);
  cs(kv[2], ke[2], kv[3], ke[3]);
  cs(kv[0], ke[0], kv[2], ke[2]);
  cs(kv[1], ke[1], kv[3], ke[3]);
  cs(kv[1], ke[1], kv[2], ke[2]);
  float v0 = 0.f;
  den = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    exs[r] = 0.f;
    bis[r] = 0;
    if (r >= K) continue;
    const unsigned m = wave_max_u(kv[0]);
    if (m == 0u) continue;  // fewer selectable logits than k: expert 0, weight 0
    // the lane holding the maximum: the only one, or among lanes whose first
    // keys are equal, the one whose first expert index is lowest
    const unsigned long long tied = __ballot(kv[0] == m);
    int wl;
    if (__popcll(tied) == 1)
      wl = __ffsll((long long)tied) - 1;
    else
      wl = wave_min_i(kv[0] == m ? ke[0] : 0x7fffffff) & 63;
    const int ew = __builtin_amdgcn_readlane(ke[0], wl);
    const bool win = ln == wl;
    kv[0] = win ? kv[1] : kv[0];
    kv[1] = win ? kv[2] : kv[1];
    kv[2] = win ? kv[3] : kv[2];
    kv[3] = win ? 0u : kv[3];
    ke[0] = win ? ke[1] : ke[0];
    ke[1] = win ? ke[2] : ke[1];
    ke[2] = win ? ke[3] : ke[2];
    const float val = topk_key_value(m);
    if (r == 0) v0 = val;
    const float ex = __expf(val - v0);
    den += ex;
    exs[r] = ex;
    bis[r] = ew;
  }
}

// The same with the logits read from memory.
template <class M = Plain>
__device__ __forceinline__ void topk_regs(const float* logits, int E, int K,
                                          int (&bis)[kMaxTopK], float (&exs)[kMaxTopK],
                                          float& den) {
  const int ln = lane_id();
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = ln + 64 * i;
    x[i] = e < E ? M::ld(&logits[e]) : -INFINITY;
  }
  topk_vals(x, E, K, bis, exs, den);
}

// The same, written out by lane 0: idx, w = softmax over the selected, and
// the caller's copy idx2 when given.
__device__ __forceinline__ void topk_row(const float* logits, int E, int K, int* idx, float* w,
                                int* idx2 = nullptr) {
  int bis[kMaxTopK];
  float exs[kMaxTopK], den;
  topk_regs(logits, E, K, bis, exs, den);
  if (lane_id() == 0) {
    const float inv = 1.0f / den;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      if (k < K) {
        idx[k] = bis[k];
        w[k] = exs[k] * inv;
        if (idx2) idx2[k] = bis[k];
      }
    }
  }
}

// One wave per token: top-k and gating weights into S.idx / S.wts.
__device__ void phase_topk(const LayerArgs& L, const StepArgs& S, int* topk_out, int vb, int nvb) {
  for (int t = gwave(vb, nvb); t < S.T; t += nvb * kWaves) {
    topk_row(S.logits + (size_t)t * L.E, L.E, L.K, S.idx + (size_t)t * L.K, S.wts + (size_t)t * L.K,
             topk_out ? topk_out + (size_t)t * L.K : nullptr);
  }
}

// act[j][f] = silu(gate_e[f] . u) * (up_e[f] . u), e = idx[j]; u staged in LDS.
template <int DT, class M = Plain, class Sel, class Pre>
__device__ void gateup_t1(const LayerArgs& L, const StepArgs& S, Sel&& idx, const float* u,
                          int vb, int nvb, Pre&& pre) {
  constexpr int R = 2, U = 2;
  const int nrb = L.F / R;
  const size_t rb = expert_row_bytes(DT, L.H);
  const size_t sb = (size_t)L.H / 16;
  const int gw = gwave(vb, nvb), nw = nvb * kWaves;
  const int n = my_count(gw, nw, L.K * nrb);
  stream_t1<DT, 2 * R, U>(
      n, L.H, [&](int) { return u; },
      [&](int k, auto& wr, auto& sr) {
        const int t = gw + k * nw, j = t / nrb, f0 = (t - j * nrb) * R;
        int e = idx(j);
        e = e >= 0 && e < L.E ? e : 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const size_t row = (size_t)e * L.F + f0 + r;
          wr[r] = L.wg + row * rb;
          wr[R + r] = L.wu + row * rb;
          sr[r] = DT == kNVFP4 ? L.sg + row * sb : nullptr;
          sr[R + r] = DT == kNVFP4 ? L.su + row * sb : nullptr;
        }
      },
      [&](int k, auto& acc) {
        const int t = gw + k * nw, j = t / nrb, f0 = (t - j * nrb) * R;
        int e = idx(j);
        e = e >= 0 && e < L.E ? e : 0;
        const float gs = DT == kNVFP4 ? L.gg[e] : 1.f, us = DT == kNVFP4 ? L.gu[e] : 1.f;
        float res[R];
#pragma unroll
        for (int r = 0; r < R; ++r) res[r] = silu(acc[r] * gs) * (acc[R + r] * us);
        lane_store<R>(res, [&](int r, float v) { M::st(&S.act[(size_t)j * L.F + f0 + r], v); });
      },
      pre);
}

// out[c] = h[c] + sum_j w[j] * (down_e[c] . act[j]), e = idx[j], in slot order;
// act staged in LDS as [K][F].  Entries of idx outside [0, E) add nothing.
// Each lane folds the weighted partial sums of the K experts of a row block
// together and the wave reduces once per row block.
template <int DT, class M = Plain, class Pre>
__device__ void down_t1(const LayerArgs& L, const StepArgs& S, const int* idx, const float* wts,
                        const float* act, const float* h, float* out, float* out2, int vb,
                        int nvb, Pre&& pre) {
  // three rows per task: at hidden 6144 that is 2048 row blocks, one per
  // wave of the 512 workgroups whose staged activations fit in LDS at once
  constexpr int R = 3, U = 2;
  const size_t rb = expert_row_bytes(DT, L.F);
  const size_t sb = (size_t)L.F / 16;
  const int gw = gwave(vb, nvb), nw = nvb * kWaves;
  const int K = L.K;
  const int nrb = my_count(gw, nw, (L.H + R - 1) / R);
  // lane j holds slot j's expert; a wave-uniform slot reads it back with one
  // cross-lane read
  const int ev = lane_id() < K ? idx[lane_id()] : -1;
  // and slot j's weight (times the expert's global scale for NVFP4), complete
  // before the first weight row is issued, so the loop waits for nothing but
  // the weight rows
  const float wv = lane_id() < K ? wts[lane_id()] : 0.f;
  const bool okv = ev >= 0 && ev < L.E;
  float sv = okv ? wv : 0.f;
  if (DT == kNVFP4) sv *= okv ? L.gd[ev] : 0.f;
  asm volatile("" ::"v"(sv));
  // task k = (row block b, slot j): b = k / K by a multiply-high, exact for
  // k < 2^32 / K (K = 1 would need the multiplier 2^32)
  const unsigned mK = 0xffffffffu / (unsigned)K + 1u;
  auto split = [&](int k, int& b, int& j) {
    b = K == 1 ? k : (int)__umulhi((unsigned)k, mK);
    j = k - b * K;
  };
  float o[R];
#pragma unroll
  for (int r = 0; r < R; ++r) o[r] = 0.f;
  stream_t1<DT, R, U, true>(
      nrb * K, L.F,
      [&](int k) {
        int b, j;
        split(k, b, j);
        return act + (size_t)j * L.F;
      },
      [&](int k, auto& wr, auto& sr) {
        int b, j;
        split(k, b, j);
        const int r0 = (gw + b * nw) * R;
        int e = __builtin_amdgcn_readlane(ev, j);
        e = e >= 0 && e < L.E ? e : 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = r0 + r < L.H ? r0 + r : L.H - 1;
          const size_t row = (size_t)e * L.H + c;
          wr[r] = L.wd + row * rb;
          sr[r] = DT == kNVFP4 ? L.sd + row * sb : nullptr;
        }
      },
      [&](int k, auto& acc) {
        int b, j;
        split(k, b, j);
        const int r0 = (gw + b * nw) * R;
        const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), j));
#pragma unroll
        for (int r = 0; r < R; ++r) o[r] = fmaf(s, acc[r], o[r]);
        if (j == K - 1) {
#pragma unroll
          for (int r = 0; r < R; ++r) o[r] = wave_sum(o[r]);
          lane_store<R>(o, [&](int r, float v) {
            const int c = r0 + r;
            if (c < L.H) {
              const float y = M::ld(&h[c]) + v;
              M::st(&out[c], y);
              if (out2) out2[c] = y;
            }
          });
#pragma unroll
          for (int r = 0; r < R; ++r) o[r] = 0.f;
        }
      },
      pre);
}

}  // namespace msk
