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

template <int N> struct IC { static constexpr int value = N; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// Wave index within the workgroup, marked wave-uniform so that values
// derived from it (task and row indices) live in scalar registers and the
// loads they address are scalar loads, which never queue behind the vector
// loads of a streaming pipeline.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// A wave-uniform float moved to a scalar register where it is read: the load
// that produced it is waited for here, not inside a later streaming loop.
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Wave-wide max / min through DPP row rotations (within rows of 16 lanes)
// and four lane reads (across rows): no LDS round trips.  Every lane gets
// the result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRor2 = 0x122;   // row_ror:2
constexpr int kDppRor4 = 0x124;   // row_ror:4
constexpr int kDppRor8 = 0x128;   // row_ror:8
constexpr int kDppMirror = 0x140;      // row_mirror: lane j of a row <- 15 - j
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane j of 8 <- 7 - j

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppRor4>(v));
  v = fmaxf(v, dpp_f<kDppRor8>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppRor4>(v));
  v = min(v, dpp_i<kDppRor8>(v));
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// Sum over the 64 lanes; every lane gets the total (fixed order, so the
// result is reproducible bit for bit).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppRor4>(v);
  v += dpp_f<kDppRor8>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// v[l] + v[l ^ 16] and v[l] + v[l ^ 32] through the gfx950 lane swaps.
__device__ __forceinline__ float add_xor16(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Wave sums of P per-lane values (P = 1, 2, 4, 8 or 16) with fewer
// cross-lane steps than P separate sums: each of the first log2 P steps
// trades half of a lane's values with the lane at distance 32, 16, 8, 4
// (lane swaps, a DPP rotation, a swizzle) and adds the other half, so
// afterwards every lane holds one value; the remaining lane bits are summed
// as in wave_sum.  Lane l returns the total of value l >> (6 - log2 P) (of
// value 0 for P = 1).
template <int P>
__device__ __forceinline__ float reduce_scatter(const float (&a)[P]) {
  static_assert(P == 1 || P == 2 || P == 4 || P == 8 || P == 16, "P is a power of two <= 16");
  constexpr int L = P == 1 ? 0 : P == 2 ? 1 : P == 4 ? 2 : P == 8 ? 3 : 4;
  const int ln = lane_id();
  float b[P];
#pragma unroll
  for (int j = 0; j < P; ++j) b[j] = a[j];
  auto halve = [&](auto n_c, int d, auto partner) {
    constexpr int N = decltype(n_c)::value;
    const bool up = (ln & d) != 0;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      const float keep = up ? b[j + N / 2] : b[j];
      const float give = up ? b[j] : b[j + N / 2];
      b[j] = keep + partner(give);
    }
  };
  auto p32 = [&](float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(ln < 32 ? p[1] : p[0]);
  };
  auto p16 = [&](float x) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((ln & 16) ? p[0] : p[1]);
  };
  auto p8 = [&](float x) { return dpp_f<kDppRor8>(x); };  // lane j <-> j ^ 8 in a row
  auto p4 = [&](float x) {  // xor 4 within 32 lanes (swizzle bit mode)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
  };
  if constexpr (L >= 1) halve(IC<P>{}, 32, p32);
  if constexpr (L >= 2) halve(IC<P / 2>{}, 16, p16);
  if constexpr (L >= 3) halve(IC<P / 4>{}, 8, p8);
  if constexpr (L >= 4) halve(IC<P / 8>{}, 4, p4);
  float v = b[0];
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  if constexpr (L < 4) v += dpp_f<kDppHalfMirror>(v);  // quads uniform: the other quad of 8
  if constexpr (L < 3) v += dpp_f<kDppMirror>(v);      // halves uniform: the other 8 of 16
  if constexpr (L < 2) v = add_xor16(v);
  if constexpr (L < 1) v = add_xor32(v);
  return v;
}

// Sum of v over the lanes congruent to this one modulo LPP (LPP = 2, 4, 8,
// 16 or 32): the lanes that hold the same slice for different positions.
template <int LPP>
__device__ __forceinline__ float sum_groups(float v) {
  if constexpr (LPP <= 2) v += dpp_f<kDppRor2>(v);
  if constexpr (LPP <= 4) v += dpp_f<kDppRor4>(v);
  if constexpr (LPP <= 8) v += dpp_f<kDppRor8>(v);
  if constexpr (LPP <= 16) v = add_xor16(v);
  v = add_xor32(v);
  return v;
}



// Sum of v over the aligned group of N consecutive lanes holding this one
// (N = 1, 2, 4, 8, 16 or 32); every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float sum_within(float v) {
  if constexpr (N >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (N >= 32) v = add_xor16(v);
  return v;
}

// Orders LDS traffic of one wave: its earlier LDS writes are complete before
// its later LDS reads (used for wave-private tiles, no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier for hand-offs through LDS only: waits for this wave's LDS
// operations and meets the other waves, but leaves its global loads in
// flight.  (__syncthreads() carries a workgroup fence that also waits for
// every outstanding global load, which would drain any prefetch.)  Data that
// direct global->LDS loads bring in must be waited for with vmcnt before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8(const v4u& v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats -> two bf16 (round to nearest even), packed a | b << 16.
__device__ __forceinline__ unsigned cvt_pk_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f2){a, b}, bf16x2));
}

// Two floats -> two fp16 (round to nearest even), packed a | b << 16.
__device__ __forceinline__ unsigned cvt_pk_f16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f2){a, b}, f16x2));
}

// NVFP4 block scales of 16-B chunk c of a row: the two e4m3 bytes at
// srow + 2c, read as the aligned dword holding them (scale arrays are 4-byte
// aligned and a whole number of dwords long, so the dword never leaves the
// array), then picked out of it.
__device__ __forceinline__ unsigned scale_dword(const uint8_t* srow, unsigned c) {
  const unsigned mis = (unsigned)(uintptr_t)srow & 2u;  // rows start on even bytes
  return *reinterpret_cast<const unsigned*>(srow - mis + ((c * 2u + mis) & ~3u));
}
__device__ __forceinline__ unsigned scale_pair(unsigned dw, const uint8_t* srow, int c) {
  return dw >> ((((unsigned)(uintptr_t)srow + (unsigned)c * 2u) & 2u) * 8u);
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

// ------------------------------------------- one-token streaming GEMV
// One wave works through its own list of tasks k = 0..ntask-1; task k is R
// weight rows (rowfn(k, wr, sr) gives their row and NVFP4 scale pointers)
// dotted with one fp32 vector in LDS (actfn(k)).  The weight stream is
// software-pipelined two buffers deep across row ends and task ends, and the
// input vector comes from LDS, so no cache load ever waits behind a weight
// load.  out(k, acc) receives the sums (in every lane), or with LANE each
// lane's partial sum, for a caller that combines tasks linearly before one
// wave reduction; pre() runs once, in every wave, after the first loads are
// issued.
template <int DT, int R, int U, bool LANE = false, class ActFn, class RowFn, class OutFn,
          class PreFn>
__device__ __forceinline__ void stream_t1(int ntask, int ncols, ActFn&& actfn, RowFn&& rowfn,
                                          OutFn&& out, PreFn&& pre) {
  using W = WT<DT>;
  const int ln = lane_id();
  const int nch = ncols / W::EPL;
  const int NI = (nch + 64 * U - 1) / (64 * U);
  const int total = ntask * NI;
  v4u A[U][R], B[U][R];
  unsigned sA[U][R], sB[U][R];
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;

  // Loads are issued on every path (a chunk past the row end is clamped to
  // the last one and compute adds nothing for it), nothing touches a loaded
  // value before compute needs it, and compute has no branch on the chunk:
  // otherwise the compiler's waits for the loads in flight become
  // conservative and drain the second buffer at every step.
  // step f of the stream is (task k, chunk group i); cursors move step by
  // step with scalar adds (no division per step)
  struct At { int k, i; };
  auto next = [&](At a) -> At {
    if (++a.i == NI) { a.i = 0; ++a.k; }
    return a;
  };
  auto issue = [&](v4u(&w)[U][R], unsigned(&s)[U][R], At at) {
    const int k = at.k, i = at.i;
    const uint8_t* wr[R];
    const uint8_t* sr[R];
    rowfn(k, wr, sr);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a scalar row base plus one 32-bit lane offset shared by the rows
      const int ch = (i * U + u) * 64 + ln;
      const unsigned cc = (unsigned)(ch < nch ? ch : nch - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        w[u][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wr[r] + cc * 16u));
        if constexpr (DT == kNVFP4)
          s[u][r] = scale_dword(sr[r], cc);
        else
          s[u][r] = 0u;
      }
    }
  };
  auto compute = [&](const v4u(&w)[U][R], const unsigned(&s)[U][R], At at) {
    const int k = at.k, i = at.i;
    const float* act = actfn(k);
    const uint8_t* sr[R];  // NVFP4: the scale rows again, for their alignment
    if constexpr (DT == kNVFP4) {
      const uint8_t* wr[R];
      rowfn(k, wr, sr);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = (i * U + u) * 64 + ln;
      const bool in = ch < nch;
      const int cl = in ? ch : nch - 1;
      v2f sc[R];
      if constexpr (DT == kNVFP4) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          sc[r] = __builtin_amdgcn_cvt_pk_f32_fp8(scale_pair(s[u][r], sr[r], cl), false);
          sc[r].x = in ? sc[r].x : 0.f;
          sc[r].y = in ? sc[r].y : 0.f;
        }
      }
#pragma unroll
      for (int sub = 0; sub < W::NSUB; ++sub) {
        float a[W::SUB];
        load_act(act + cl * W::EPL + sub * W::SUB, a, W::SUB);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float fw[W::SUB];
          decode_sub<DT>(w[u][r], sub, fw);
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < W::SUB; ++e) d = fmaf(fw[e], a[e], d);
          if constexpr (DT == kNVFP4)
            acc[r] = fmaf((sub >> 1) ? sc[r].y : sc[r].x, d, acc[r]);
          else  // one sub-block per chunk
            acc[r] += in ? d : 0.f;
        }
      }
    }
    if (i == NI - 1) {
      if constexpr (!LANE) {
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
      }
      out(k, acc);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
    }
  };
  // the first two buffers go out before the prologue (typically staging the
  // input vector into LDS, which every wave of the workgroup joins), so its
  // latency overlaps the first weight fetches; all of A's loads precede all
  // of B's, as inside the loop (a single-step task list loads its one step
  // twice).  The loop issues both refills on every iteration and the last
  // steps are peeled off, so the loop holds no conditional load.
  const int last = total - 1;
  At c0{0, 0}, c1 = next(c0);
  if (total > 0) {
    issue(A, sA, c0);
    __builtin_amdgcn_sched_barrier(0);
    issue(B, sB, 1 <= last ? c1 : c0);
    __builtin_amdgcn_sched_barrier(0);
  }
  pre();
  int f = 0;
  // steady state: both refills are real steps
  for (; f + 3 < total; f += 2) {
    const At c2 = next(c1), c3 = next(c2);
    compute(A, sA, c0);
    issue(A, sA, c2);
    compute(B, sB, c1);
    issue(B, sB, c3);
    c0 = c2;
    c1 = c3;
  }
  // the last one to three steps: A holds step f, B step f + 1
  if (f < total) {
    const At c2 = next(c1);
    compute(A, sA, c0);
    if (f + 2 < total) issue(A, sA, c2);
    if (f + 1 < total) compute(B, sB, c1);
    if (f + 2 < total) compute(A, sA, c2);
  }
}

// Maximum over the block (all waves, at most 16); every thread gets it.
// red is one float of LDS per wave.  NW: the number of waves, if known at
// compile time (0: read from blockDim).
template <int NW = 0>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  lds_barrier();
  if (lane_id() == 0) red[wave_id()] = v;
  lds_barrier();
  float t = red[0];
  const int nw = NW ? NW : (int)(blockDim.x >> 6);
  for (int w = 1; w < nw; ++w) t = fmaxf(t, red[w]);
  return t;
}

// Sum over the block (all waves); every thread gets the total.  red is
// kWaves floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  lds_barrier();
  if (lane_id() == 0) red[wave_id()] = v;
  lds_barrier();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  return t;
}

// How a phase reads data that another workgroup wrote, and writes data that
// another workgroup reads, within the step.  Plain: the producer ran in an
// earlier kernel, whose end made its stores visible everywhere.  Coh: the
// producer runs in the same (persistent) launch, possibly on another XCD,
// whose L2 is not kept coherent with this one's: relaxed agent-scope atomic
// loads and stores, which the hardware keeps coherent across the device
// without the cost of an L2 writeback or invalidate.  Together with a
// barrier whose arrival follows the stores' completion, a Coh load after the
// barrier sees the Coh stores made before it.
struct Plain {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ v4f ld4(const float* p) { return *reinterpret_cast<const v4f*>(p); }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ void st4(float* p, v4f v) { *reinterpret_cast<v4f*>(p) = v; }
};
struct Coh {
  static __device__ __forceinline__ float ld(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ __forceinline__ v4f ld4(const float* p) {
    return v4f{ld(p), ld(p + 1), ld(p + 2), ld(p + 3)};
  }
  static __device__ __forceinline__ void st(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ __forceinline__ void st4(float* p, v4f v) {
    st(p, v.x); st(p + 1, v.y); st(p + 2, v.z); st(p + 3, v.w);
  }
};

// Fixed softmax shift of a layer: the given value, or (given 0) the score
// bound sqrt(D) * max|q_norm| * max|k_norm| of a QK-normalised query against
// a QK-normalised key.  The softmax does not depend on it; it only keeps
// exp(s - c) in range.  The gains are read as two values per lane (D <= 128)
// by gain_pair, issued together with a kernel's other prologue loads, and
// reduced over the wave by layer_shift where the loads have landed anyway.
__device__ __forceinline__ v2f gain_pair(const float* g, int D) {
  const int ln = lane_id();
  return v2f{ln < D ? g[ln] : 0.f, ln + 64 < D ? g[ln + 64] : 0.f};
}
__device__ __forceinline__ float layer_shift(float given, v2f gq, v2f gk, int D) {
  if (given != 0.f) return given;
  const float mq = wave_max(fmaxf(fabsf(gq.x), fabsf(gq.y)));
  const float mk = wave_max(fmaxf(fabsf(gk.x), fabsf(gk.y)));
  return sqrtf((float)D) * mq * mk;
}

}  // namespace msk
