// Expert FFN of a prefill batch: many tokens, each routed to k experts.
//
// Where a decode or verify step streams each selected expert once for a few
// tokens (a GEMV), a prefill batch gives every expert tens to hundreds of
// tokens, and its gate/up and down products become matrix products that run
// on the matrix cores: the fused MoE kernel the ainewsbites page lists among
// the prefill optimisations ("Agentic coding benchmark and serving
// tradeoffs"), over NVFP4 or bf16 experts (brifing.si page, "Expert Weight
// Quantization").  The slots (token t,
// choice j) are grouped by expert; each expert's slots form blocks of up to
// 64, and a block times 64 weight rows is one work item of the dense
// matrix-core loop (dense_item / dense_item_fp4):
//   route    count the slots per expert, place them grouped by expert (the
//            order within an expert does not change any result), list blocks;
//   gather   each position's token input u as two bf16 terms (hi, then the
//            rest, together exact to about 2^-17 of u);
//   gate/up  gu[pos] = [W_g; W_u]_e u  (fp32), e the position's expert;
//   swiglu   act[pos] = silu(g_g gu_gate) * (g_u gu_up) as two bf16 terms
//            (g: NVFP4 matrix scales, else 1);
//   down     y[slot] = g_d W_d,e act[pos];
//   sum      out[t] = h[t] + sum_j w[t][j] y[t k + j], j ascending (the
//            decode path's weighted combine, k_moe_sum).
#pragma once
#include "phases_dense.h"

namespace msk {

// One workgroup: counts per expert (LDS atomics), offsets, placement, blocks.
// lds: 3 * kMaxExperts + 1 ints.
__device__ inline void pf_route(const LayerArgs& L, const PfArgs& P, int* lds) {
  int* cnt = lds;
  int* cur = lds + kMaxExperts;
  int* bo = lds + 2 * kMaxExperts;  // [E + 1] first block of each expert
  const int S = P.T * L.K;
  for (int e = threadIdx.x; e < L.E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = P.idx[s];
    if (e >= 0 && e < L.E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 0, b = 0;
    for (int e = 0; e < L.E; ++e) {
      cur[e] = o;
      bo[e] = b;
      P.off[e] = o;
      o += cnt[e];
      b += (cnt[e] + 63) / 64;
    }
    bo[L.E] = b;
    P.off[L.E] = o;
    *P.nblk = b;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < L.E; e += blockDim.x)
    for (int b = 0; 64 * b < cnt[e]; ++b) {
      const int n = cnt[e] - 64 * b;
      P.blk[bo[e] + b] = PfBlock{e, cur[e] + 64 * b, n < 64 ? n : 64};
    }
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = P.idx[s];
    if (e < 0 || e >= L.E) continue;
    const int p = atomicAdd(&cur[e], 1);
    P.perm[p] = s;
    P.pe[p] = e;
  }
}

// Eight fp32 values as two bf16 terms: hi = bf16(x), lo = bf16(x - hi), at
// element off of the two planes that are `plane` elements apart.
__device__ __forceinline__ void store_split2(unsigned short* dst, size_t plane, size_t off,
                                             const float (&v)[8]) {
  unsigned hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = cvt_pk_bf16(v[2 * i], v[2 * i + 1]);
    lo[i] = cvt_pk_bf16(v[2 * i] - bf16_lo(hi[i]), v[2 * i + 1] - bf16_hi(hi[i]));
  }
  *reinterpret_cast<v4u*>(dst + off) = v4u{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<v4u*>(dst + plane + off) = v4u{lo[0], lo[1], lo[2], lo[3]};
}

// a[pos] = u[token of pos] as two bf16 terms, eight inputs per thread and step.
__device__ inline void pf_gather(const LayerArgs& L, const PfArgs& P) {
  const int n = P.off[L.E];
  const int per = L.H / 8;
  const size_t plane = (size_t)P.T * L.K * L.H;
  const long long total = (long long)n * per;
  for (long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (long long)gridDim.x * blockDim.x) {
    const int pos = (int)(q / per), c = (int)(q - (long long)pos * per) * 8;
    const int t = P.perm[pos] / L.K;
    const float* src = P.u + (size_t)t * L.H + c;
    const v4f x0 = *reinterpret_cast<const v4f*>(src);
    const v4f x1 = *reinterpret_cast<const v4f*>(src + 4);
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    store_split2(P.a, plane, (size_t)pos * L.H + c, v);
  }
}

// act[pos][f] = silu(g_g gu[pos][f]) * (g_u gu[pos][F + f]) as two bf16 terms.
__device__ inline void pf_swiglu(const LayerArgs& L, const PfArgs& P) {
  const int n = P.off[L.E];
  const int per = L.F / 8;
  const size_t plane = (size_t)P.T * L.K * L.F;
  const long long total = (long long)n * per;
  for (long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (long long)gridDim.x * blockDim.x) {
    const int pos = (int)(q / per), c = (int)(q - (long long)pos * per) * 8;
    const int e = P.pe[pos];
    const float gs = L.edt == kNVFP4 ? L.gg[e] : 1.f;
    const float us = L.edt == kNVFP4 ? L.gu[e] : 1.f;
    const float* g = P.gu + (size_t)pos * 2 * L.F + c;
    const float* up = g + L.F;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
      const v4f a = *reinterpret_cast<const v4f*>(g + i);
      const v4f b = *reinterpret_cast<const v4f*>(up + i);
      v[i] = silu(gs * a.x) * (us * b.x);
      v[i + 1] = silu(gs * a.y) * (us * b.y);
      v[i + 2] = silu(gs * a.z) * (us * b.z);
      v[i + 3] = silu(gs * a.w) * (us * b.w);
    }
    store_split2(P.act, plane, (size_t)pos * L.F + c, v);
  }
}

// The gate/up (GU) or down product of every block: item = (block, 64-row
// block of the expert's rows).
template <bool FP4, bool GU>
__device__ void pf_dense(const LayerArgs& L, const PfArgs& P, uint8_t* lds) {
  const int N = GU ? 2 * L.F : L.H, K = GU ? L.H : L.F;
  const int n_rb = N / 64;
  const long long items = (long long)(*P.nblk) * n_rb;
  const size_t rbytes = FP4 ? (size_t)K / 2 : (size_t)K * 2;  // weight bytes per row
  const size_t sbytes = (size_t)K / 16;                         // NVFP4 scale bytes per row
  for (long long item = blockIdx.x; item < items; item += gridDim.x) {
    const PfBlock b = P.blk[item / n_rb];
    const int rb = (int)(item - (item / n_rb) * n_rb);
    DenseArgs D{};
    D.K = K;
    D.N = N;
    D.T = b.n;
    D.ks = 1;
    D.oscale = 1.f;
    D.a3_plane = (size_t)P.T * L.K * K;  // the two terms' planes span every slot
    if constexpr (GU) {
      const size_t r0 = (size_t)b.e * L.F;
      D.w[0] = L.wg + r0 * rbytes;
      D.w[1] = L.wu + r0 * rbytes;
      D.w[2] = D.w[0];
      D.s[0] = FP4 ? L.sg + r0 * sbytes : nullptr;
      D.s[1] = FP4 ? L.su + r0 * sbytes : nullptr;
      D.s[2] = D.s[0];
      D.seg[1] = L.F;
      D.a3 = P.a + (size_t)b.pos0 * K;
      D.out = P.gu + (size_t)b.pos0 * N;
    } else {
      const size_t r0 = (size_t)b.e * L.H;
      D.w[0] = D.w[1] = D.w[2] = L.wd + r0 * rbytes;
      D.s[0] = D.s[1] = D.s[2] = FP4 ? L.sd + r0 * sbytes : nullptr;
      D.a3 = P.act + (size_t)b.pos0 * K;
      D.out = P.y;
      D.tmap = P.perm + b.pos0;
      D.oscale = FP4 ? L.gd[b.e] : 1.f;
    }
    if constexpr (FP4)
      dense_item_fp4<4, 2>(D, rb, lds);
    else
      dense_item<4, 2>(D, rb, lds);
  }
}

}  // namespace msk
