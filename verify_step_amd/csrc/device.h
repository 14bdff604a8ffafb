// Device building blocks for the MoE layer step on gfx950 (wave64):
// number-format decode/encode, wave reductions, and the streaming GEMV core.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.h"

namespace msk {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Sum over the 64 lanes; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Orders LDS traffic of one wave: its earlier LDS writes are complete before
// its later LDS reads (used for wave-private tiles, no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------ formats
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ unsigned f2bf16(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Four e4m3 bytes -> four floats (byte i -> f[i]).
__device__ __forceinline__ void e4m3x4(unsigned w, float* f) {
  v2f a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  v2f b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
}

// Two floats -> two e4m3 bytes in the low half, round to nearest even.  The
// hardware convert turns values past the largest finite into NaN, so clamp
// first: the cache format saturates at +-448.
__device__ __forceinline__ unsigned f2e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Eight e2m1 codes (one 32-bit word; element 2i in the low nibble of byte i)
// -> eight floats, unscaled.  The convert's scale operand only contributes
// its exponent, so it is 1 here and block scales are applied separately.
__device__ __forceinline__ void e2m1x8(unsigned w, float* f) {
  v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  v2f c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  v2f d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// ----------------------------------------------------- weight streaming
// A lane reads 16 B of a weight row per step: 4 fp32, 8 bf16 or 32 e2m1.
template <int DT> struct WT;
template <> struct WT<kF32> { enum { EPL = 4, SUB = 4, NSUB = 1 }; };
template <> struct WT<kBF16> { enum { EPL = 8, SUB = 8, NSUB = 1 }; };
template <> struct WT<kNVFP4> { enum { EPL = 32, SUB = 8, NSUB = 4 }; };

template <int DT>
__device__ __forceinline__ void decode_sub(const v4u& w, int s, float* f) {
  if constexpr (DT == kF32) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  } else if constexpr (DT == kBF16) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  } else {
    const unsigned word = s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w;
    e2m1x8(word, f);
  }
}

__device__ __forceinline__ void load_act(const float* p, float* a, int n) {
  if (n == 4) {
    v4f x = *reinterpret_cast<const v4f*>(p);
    a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
  } else {
    v4f x = *reinterpret_cast<const v4f*>(p);
    v4f y = *reinterpret_cast<const v4f*>(p + 4);
    a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
    a[4] = y.x; a[5] = y.y; a[6] = y.z; a[7] = y.w;
  }
}

// One wave computes acc[r][v] = sum_c W_r[c] * in_v[c] * gain[c] for R weight
// rows (any row pointers) and up to NV fp32 input vectors (nv valid).  The
// rows are streamed once, 16 B per lane per step with two steps in flight;
// the inputs come through the caches.  For NVFP4 rows, srow holds the e4m3
// block scales (one per 16 elements); the matrix scale is left to the caller.
// On return every lane holds the full sums.
template <int DT, int R, int NV>
__device__ __forceinline__ void wave_gemv(const uint8_t* const (&wrow)[R],
                                          const uint8_t* const (&srow)[R], int ncols,
                                          const float* const (&vin)[NV], int nv,
                                          const float* __restrict__ gain, float (&acc)[R][NV]) {
  using W = WT<DT>;
  constexpr int U = 2;
  const int ln = lane_id();
  const int nch = ncols / W::EPL;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[r][v] = 0.f;

  for (int ch0 = ln; ch0 < nch; ch0 += 64 * U) {
    v4u w[U][R];
    v2f sc[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = ch0 + 64 * u;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (ch < nch) {
          w[u][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wrow[r]) + ch);
          if constexpr (DT == kNVFP4) {
            unsigned s2 = *reinterpret_cast<const unsigned short*>(srow[r] + 2 * ch);
            sc[u][r] = __builtin_amdgcn_cvt_pk_f32_fp8(s2, false);
          }
        } else {
          w[u][r] = v4u{0u, 0u, 0u, 0u};
          sc[u][r] = v2f{0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = ch0 + 64 * u;
      if (ch >= nch) break;
#pragma unroll
      for (int s = 0; s < W::NSUB; ++s) {
        float f[R][W::SUB];
#pragma unroll
        for (int r = 0; r < R; ++r) decode_sub<DT>(w[u][r], s, f[r]);
        const int c0 = ch * W::EPL + s * W::SUB;
        float g[W::SUB];
        if (gain) load_act(gain + c0, g, W::SUB);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          if (v < nv) {
            float a[W::SUB];
            load_act(vin[v] + c0, a, W::SUB);
            if (gain) {
#pragma unroll
              for (int i = 0; i < W::SUB; ++i) a[i] *= g[i];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
              float d = 0.f;
#pragma unroll
              for (int i = 0; i < W::SUB; ++i) d = fmaf(f[r][i], a[i], d);
              if constexpr (DT == kNVFP4)
                acc[r][v] = fmaf((s >> 1) ? sc[u][r].y : sc[u][r].x, d, acc[r][v]);
              else
                acc[r][v] += d;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[r][v] = wave_sum(acc[r][v]);
}

// ---------------------------------------------------- grid-wide barrier
// All workgroups of a cooperative launch meet here.  Counter words live in
// the caller's workspace: sync[0] counts arrivals (monotone within a launch),
// sync[2] is the error flag.  A bounded spin turns a missing arrival into an
// error flag instead of a hang.
__device__ __forceinline__ void grid_barrier(unsigned* sync, unsigned& epoch) {
  __syncthreads();
  epoch += gridDim.x;
  if (threadIdx.x == 0) {
    __threadfence();
    __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    while (__hip_atomic_load(&sync[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < epoch) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > (1u << 22)) {
        __hip_atomic_store(&sync[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __threadfence();
  }
  __syncthreads();
}

}  // namespace msk
