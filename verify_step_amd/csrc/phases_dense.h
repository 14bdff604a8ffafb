// Dense projections (QKV, Wo, router) of steps with several tokens, on the
// matrix cores: out[t][r] = resid[t][r] + sum_k W[r][k] * a[t][k] for bf16
// weights W [N][K] and fp32 activations a [T][K].
//
// v_mfma_f32_16x16x32_bf16 takes the weight rows as the A operand (16 rows,
// eight consecutive k per lane) and the activations as the B operand (16
// tokens), both read from LDS tiles (below).  Each
// activation is written as three bf16 terms a = hi + mid + lo (each the
// round-to-nearest-even of what the previous terms leave), [3][T][K], once
// per call by the kernel that produces the activations.  A product takes the
// first NT of them: QKV and the router all three (products as exact as fp32
// ones: the new K and V rows are rounded to the cache format, where a
// difference at a rounding boundary moves a value by a whole fp8 step, and
// routing is compared bit for bit), Wo two (hi + mid leaves at most 2^-17
// of each input out).  The sums stay in fp32.
//
// Work item: (block of 64 output rows, one of KS slices of K); each of the
// four waves owns 16 of the rows.  With KS > 1 each item writes a partial
// tile and a second kernel sums the KS partials in slice order (a kernel
// boundary makes them visible without cache maintenance inside the kernel,
// which on this part costs far more than the sum).
#pragma once
#include "phases_mfma.h"

namespace msk {

struct DenseArgs {
  const uint8_t* w[3];   // row segments (QKV: wq, wk, wv; otherwise one)
  int seg[3];            // first global row of segments 1 and 2 (seg[0] = 0)
  int N, K, T;
  int ks;                // K slices
  const unsigned short* a3;  // [3][T][K] bf16 terms
  const float* resid;    // [T][N] or null
  float* out;            // [T][N]
  float* part;           // [n_rb][ks][T][64] partial tiles (ks > 1)
};

// a3[p][t][k] for eight consecutive k of one token from fp32 values.
__device__ __forceinline__ void store_split8(unsigned short* a3, size_t plane, size_t off,
                                             const float* v) {
  unsigned h[8], m[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split3_bf16(v[e], h[e], m[e], l[e]);
  *reinterpret_cast<v4u*>(a3 + off) =
      v4u{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
  *reinterpret_cast<v4u*>(a3 + plane + off) =
      v4u{m[0] | m[1] << 16, m[2] | m[3] << 16, m[4] | m[5] << 16, m[6] | m[7] << 16};
  *reinterpret_cast<v4u*>(a3 + 2 * plane + off) =
      v4u{l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16};
}

// src[0] + src[stride] + ... + src[(n - 1) stride] (four consecutive
// floats each), added in that order, with up to 8 loads in flight at once (a
// plain loop would wait for each load before issuing the next).
__device__ __forceinline__ v4f sum_slices4(const float* src, size_t stride, int n) {
  v4f a = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < n; q0 += 8) {
    v4f v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      v[q] = *reinterpret_cast<const v4f*>(src + (size_t)(q0 + q < n ? q0 + q : n - 1) * stride);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < n) {
        a.x += v[q].x; a.y += v[q].y; a.z += v[q].z; a.w += v[q].w;
      }
  }
  return a;
}

// Sum over every wave of the workgroup (any size up to 16 waves); every
// thread gets the total.  red: 16 floats of LDS.
__device__ __forceinline__ float wg_sum(float v, float* red) {
  v = wave_sum(v);
  const int nw = blockDim.x / 64;
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

// One workgroup per token t: h[t] = resid[t] + (the partial tiles of a
// split-K dense product summed in slice order, as dense_sum does), written
// out, then a = h[t] * g / sqrt(mean(h[t]^2) + eps) as bf16 terms
// (store_split8) and, when a32 is given, as fp32.  ks <= 1: h is complete
// already and is only read (the plain RMSNorm of an input row).  hl: H
// floats of LDS, red: 16 floats of LDS.
__device__ inline void sum_prep_act(const float* part, int ks, const float* resid, float* h,
                                    const float* g, int T, int H, float eps, float* a32,
                                    unsigned short* a3, float* hl, float* red) {
  const int t = blockIdx.x;
  float* hr = h + (size_t)t * H;
  float s = 0.f;
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    v4f v;
    if (ks > 1) {
      // four consecutive rows of one 64-row block
      const v4f a = sum_slices4(part + ((size_t)(c >> 6) * ks * T + t) * 64 + (c & 63),
                                (size_t)T * 64, ks);
      const v4f r0 = resid ? *reinterpret_cast<const v4f*>(resid + (size_t)t * H + c)
                           : v4f{0.f, 0.f, 0.f, 0.f};
      v = v4f{r0.x + a.x, r0.y + a.y, r0.z + a.z, r0.w + a.w};
      *reinterpret_cast<v4f*>(hr + c) = v;
    } else {
      v = *reinterpret_cast<const v4f*>(hr + c);
    }
    *reinterpret_cast<v4f*>(hl + c) = v;
    s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  const float r = 1.0f / sqrtf(wg_sum(s, red) / (float)H + eps);  // also orders hl
  const size_t plane = (size_t)T * H;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = hl[c + e] * r * g[c + e];
    if (a32) {
      *reinterpret_cast<v4f*>(a32 + (size_t)t * H + c) = v4f{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<v4f*>(a32 + (size_t)t * H + c + 4) = v4f{v[4], v[5], v[6], v[7]};
    }
    store_split8(a3, plane, (size_t)t * H + c, v);
  }
}

// One workgroup per token t: out[t] as down_combine forms it, then the next
// layer's QKV input terms from it: a3 = bf16 terms of out[t] * g /
// sqrt(mean(out[t]^2) + eps) (store_split8, as sum_prep_act writes them).
// ol: H floats of LDS, red: 16 floats of LDS.
__device__ inline void down_combine_prep(const LayerArgs& L, const StepArgs& S, const float* h,
                                         const float* y, float* out, const float* g, float eps,
                                         unsigned short* a3, float* ol, float* red) {
  const int t = blockIdx.x, H = L.H;
  float s2 = 0.f;
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    v4f acc = *reinterpret_cast<const v4f*>(h + (size_t)t * H + c);
    // eight slots' loads in flight at once; a slot whose expert id is out of
    // range adds nothing (its y is not used)
    for (int j0 = 0; j0 < L.K; j0 += 8) {
      v4f yy[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q < L.K ? j0 + q : L.K - 1;
        yy[q] = *reinterpret_cast<const v4f*>(y + ((size_t)t * L.K + j) * H + c);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int s = t * L.K + j0 + q;
        if (j0 + q >= L.K) break;
        const int e = S.idx[s];
        if (e < 0 || e >= L.E) continue;
        const float w = S.wts[s];
        acc.x = fmaf(w, yy[q].x, acc.x);
        acc.y = fmaf(w, yy[q].y, acc.y);
        acc.z = fmaf(w, yy[q].z, acc.z);
        acc.w = fmaf(w, yy[q].w, acc.w);
      }
    }
    *reinterpret_cast<v4f*>(out + (size_t)t * H + c) = acc;
    *reinterpret_cast<v4f*>(ol + c) = acc;
    s2 += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
  }
  const float r = 1.0f / sqrtf(wg_sum(s2, red) / (float)H + eps);  // also orders ol
  const size_t plane = (size_t)S.T * H;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ol[c + e] * r * g[c + e];
    store_split8(a3, plane, (size_t)t * H + c, v);
  }
}

// Per 128-column k-tile the weights of a wave's 16 rows (16 x 256 B) and the
// workgroup's activation terms (NT planes x 16 CT tokens x 256 B) are fetched
// with direct global->LDS loads, double buffered.  A load instruction moves
// 1 KB: four rows x 256 B, each row's 16-B pieces stored at piece ^ (row &
// 15), so the MFMA operand reads (16 rows, one piece each) hit 16 distinct
// bank groups.
constexpr int kDenseKT = 128;       // columns per k-tile
constexpr int kDenseATile = 16 * 256;  // one wave's weight tile, bytes

template <int CT, int NT>
struct DenseLds {
  static constexpr int BT = NT * 16 * CT * 256;  // activation tile, bytes
  static constexpr int A0 = 0;
  static constexpr int B0 = A0 + 2 * kWaves * kDenseATile;
  static constexpr int BYTES = B0 + 2 * BT;  // weight tiles [2][4 waves], term tiles [2]
};

// vmcnt <= N (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int CT, int NT>
__device__ void dense_mfma(const DenseArgs& A, uint8_t* lds) {
  using G = DenseLds<CT, NT>;
  const int ln = lane_id(), wv = wave_id();
  const int r = ln & 15, g = ln >> 4;
  const int n_rb = (A.N + 63) / 64;
  const int tiles = A.K / kDenseKT;
  const size_t plane = (size_t)A.T * A.K;
  const int n_items = n_rb * A.ks;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int rb = item / A.ks, sl = item - (item / A.ks) * A.ks;
    const int t0 = (int)((long long)tiles * sl / A.ks);
    const int t1 = (int)((long long)tiles * (sl + 1) / A.ks);
    const int r0 = rb * 64 + 16 * wv;    // this wave's first row
    const bool active = r0 < A.N;
    // global row of local row lr, and its base address
    auto wrow = [&](int lr) -> const uint8_t* {
      const int row = r0 + lr;
      const int sg = row >= A.seg[2] && A.seg[2] > 0 ? 2 : (row >= A.seg[1] && A.seg[1] > 0 ? 1 : 0);
      return A.w[sg] + (size_t)(row - (sg ? A.seg[sg] : 0)) * A.K * 2;
    };
    const uint8_t* wr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[i] = active ? wrow(4 * i + g) : A.w[0];
    auto issue = [&](int tau, int buf) {
      uint8_t* at = lds + G::A0 + (buf * kWaves + wv) * kDenseATile;
      if (active) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lr = 4 * i + g;          // local row this lane fetches for
          const int p = r ^ lr;              // global piece stored at slot r
          __builtin_amdgcn_global_load_lds(wr[i] + (size_t)tau * 256 + p * 16, at + i * 1024, 16,
                                           0, 0);
        }
      }
      uint8_t* bt = lds + G::B0 + buf * G::BT;
#pragma unroll
      for (int k = 0; k < NT * CT; ++k) {
        const int i = wv + kWaves * k;       // instruction of the 4 NT CT in the B tile
        const int brow = 4 * i + g;          // plane-major row: p3 * 16 CT + t
        const int p3 = brow / (16 * CT), t = brow - p3 * 16 * CT;
        const int tt = t < A.T ? t : 0;
        const int p = r ^ (t & 15);
        __builtin_amdgcn_global_load_lds(
            A.a3 + p3 * plane + (size_t)tt * A.K + (size_t)tau * kDenseKT + p * 8, bt + i * 1024,
            16, 0, 0);
      }
    };
    f32x4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t0 < t1) issue(t0, 0);
    for (int tau = t0; tau < t1; ++tau) {
      const int buf = (tau - t0) & 1;
      if (tau + 1 < t1) {
        issue(tau + 1, buf ^ 1);
        // this tile's loads are the older ones: 4 (weights) + NT CT (terms) per lane remain
        if (active) wait_vm<4 + NT * CT>();
        else wait_vm<NT * CT>();
      } else {
        wait_vm<0>();
      }
      lds_barrier();
      if (active) {
        const uint8_t* at = lds + G::A0 + (buf * kWaves + wv) * kDenseATile;
        const uint8_t* bt = lds + G::B0 + buf * G::BT;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = (4 * q + g) ^ r;
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const v4u*>(at + r * 256 + slot * 16));
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int p3 = 0; p3 < NT; ++p3) {
              const bf16x8 bb = as_bf16x8(*reinterpret_cast<const v4u*>(
                  bt + (p3 * 16 * CT + 16 * ct + r) * 256 + slot * 16));
              acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, acc[ct], 0, 0, 0);
            }
        }
      }
      lds_barrier();  // the buffer is refilled two tiles on
    }
    // lane: token 16 ct + r, rows r0 + 4 g + i
    float* dst = A.part + (size_t)item * A.T * 64;
    if (active) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int t = 16 * ct + r;
        if (t < A.T) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = r0 + 4 * g + i;
            if (A.ks == 1) {
              const size_t o = (size_t)t * A.N + row;
              A.out[o] = (A.resid ? A.resid[o] : 0.f) + acc[ct][i];
            } else {
              dst[t * 64 + 16 * wv + 4 * g + i] = acc[ct][i];
            }
          }
        }
      }
    }
  }
}

// out[t][r] = resid[t][r] + sum over slices s (ascending) of the partial
// tiles of r's row block.
__device__ inline void dense_sum(const float* part, int N, int T, int ks, const float* resid,
                                 float* out) {
  const int n = T * N;
  for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < n; q += gridDim.x * blockDim.x) {
    const int t = q / N, row = q - (q / N) * N;
    const int rb = row >> 6, rr = row & 63;
    const float* src = part + (size_t)rb * ks * T * 64 + t * 64 + rr;
    // the slices' loads issued together, eight at a time, then added in order
    float v = 0.f;
    for (int s0 = 0; s0 < ks; s0 += 8) {
      float pv[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) pv[s] = src[(size_t)(s0 + s < ks ? s0 + s : ks - 1) * T * 64];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s0 + s < ks) v += pv[s];
    }
    out[q] = (resid ? resid[q] : 0.f) + v;
  }
}

}  // namespace msk
