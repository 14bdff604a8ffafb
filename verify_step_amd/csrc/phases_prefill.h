// Expert FFN of a prefill batch: many tokens, each routed to k experts.
//
// Where a decode or verify step streams each selected expert once for a few
// tokens (a GEMV), a prefill batch gives every expert tens to hundreds of
// tokens, and its gate/up and down products become matrix products that run
// on the matrix cores: the fused MoE kernel the ainewsbites page lists among
// the prefill optimisations ("Agentic coding benchmark and serving
// tradeoffs"), over NVFP4 or bf16 experts (brifing.si page, "Expert Weight
// Quantization").  The slots (token t, choice j) are grouped by expert and
// each expert's slots split into near-equal chunks of at most 160 (NVFP4
// experts) or 128 (bf16 experts):
//   route    count the slots per expert, lay out their grouped positions by
//            expert, list the chunks;
//   gather   place each token's slots (a per-expert cursor: the order within
//            an expert does not change any result) and write the token's
//            input row u[t] in the matrix-product format, once (the gate/up
//            product reads it through the slot's token);
//   gate/up  gu[pos] = [W_g; W_u]_e u  (fp32), e the position's expert;
//   swiglu   act[pos] = silu(g_g gu_gate) * (g_u gu_up), in the same format
//            (g: NVFP4 matrix scales, else 1);
//   down     y[slot] = g_d W_d,e act[pos];
//   sum      out[t] = h[t] + sum_j w[t][j] y[t k + j], j ascending (the
//            decode path's weighted combine, k_moe_sum).
//
// Number formats.  An e2m1 code times its e4m3 block scale has at most six
// significant bits and lies in [2^-10, 2688], so NVFP4 weights are exact in
// fp16; their products run as v_mfma_f32_16x16x32_f16 with fp16 inputs, each
// input row multiplied by a power of two that puts its largest magnitude in
// [2^14, 2^15) (11 significant bits per input, no overflow; the power is
// undone on the fp32 result).  bf16 weights are not exact in fp16, so those
// products run as v_mfma_f32_16x16x32_bf16 with each input as two bf16 terms
// (hi = rne(x), lo = rne(x - hi): about 2^-17 relative left out).  The pages
// run the experts in FP8; both formats keep far more of each input.  Sums are
// fp32.
//
// Matrix product item: (chunk of expert e, 256 output rows); each of the
// four waves owns 64 rows x all the chunk's slots (4 x TF accumulator tiles
// of 16 x 16, TF 16-slot tiles: at most 10 for NVFP4, 8 for bf16, which is
// what the register file holds).  Per k-tile of 64 columns, in a ring of
// three tiles (two in flight while one is used; deeper rings measured
// slower, as more loads in flight per CU lower what each one gets):
//   - the chunk's input rows arrive in LDS by direct global->LDS loads, each
//     row's 16-B pieces stored at piece ^ (row & 7) so an operand read (16
//     rows, one piece each) meets no bank conflict; every wave reads all of
//     them;
//   - NVFP4 weight rows (codes and block scales) arrive in the same ring slot
//     by direct loads as well, each wave's own rows, and are decoded from LDS;
//     bf16 weight rows go straight to registers (a lane holds 16 consecutive
//     columns of one row, which serve both k-steps of the tile).  The k index
//     of step j, lane group g is numbered (KT / 4) g + 8 j + (0..7) on both
//     operands, which keeps every lane's part of a row one contiguous run.
// The weights are streamed from HBM once per chunk (once per expert when it
// has at most 160 slots: at 4096 tokens, top-8 of 256, nearly every expert).  The items of one chunk are consecutive and an XCD
// runs a contiguous range of items, so the chunk's inputs, which every row
// block of the chunk reads, are re-read from that XCD's L2.
#pragma once
#include <utility>

#include "phases_dense.h"

namespace msk {

// One workgroup: counts per expert (LDS atomics), offsets and chunk counts
// (prefix sums over the experts, one expert per thread of the first four
// waves), the chunk list, and each expert's placement cursor.
// cmax: most slots per chunk.  lds: 3 * kMaxExperts + 8 ints.
__device__ inline void pf_route(const LayerArgs& L, const PfArgs& P, int cmax, int* lds) {
  int* cnt = lds;
  int* cur = lds + kMaxExperts;
  int* co = lds + 2 * kMaxExperts;  // [E] first chunk of each expert
  const int S = P.T * L.K;
  for (int e = threadIdx.x; e < L.E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = P.idx[s];
    if (e >= 0 && e < L.E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  static_assert(kMaxExperts <= 256, "one expert per thread of four waves");
  int* wsum = lds + 3 * kMaxExperts;  // [4] slots, [4] chunks of each wave
  const int x = threadIdx.x, ln = lane_id(), w = threadIdx.x >> 6;
  int ps = 0, pc = 0;  // prefix sums of slots and of chunks
  if (x < kMaxExperts) {
    ps = x < L.E ? cnt[x] : 0;
    pc = (ps + cmax - 1) / cmax;
    // inclusive sums within the wave
    for (int d = 1; d < 64; d <<= 1) {
      const int a = __shfl_up(ps, d), b = __shfl_up(pc, d);
      if (ln >= d) {
        ps += a;
        pc += b;
      }
    }
    if (ln == 63) {
      wsum[w] = ps;
      wsum[4 + w] = pc;
    }
  }
  __syncthreads();
  if (x < kMaxExperts) {
    for (int v = 0; v < w; ++v) {
      ps += wsum[v];
      pc += wsum[4 + v];
    }
    if (x < L.E) {
      const int c0 = cnt[x];
      const int o = ps - c0;  // first grouped position of expert x
      cur[x] = o;
      co[x] = pc - (c0 + cmax - 1) / cmax;
      P.off[x] = o;
      P.cur[x] = o;
      if (x == L.E - 1) {
        P.off[L.E] = ps;
        *P.nchunk = pc;
      }
    }
  }
  __syncthreads();
  // an expert's slots in nc near-equal chunks (measured faster than chunks
  // of cmax and a last one with the rest)
  for (int e = threadIdx.x; e < L.E; e += blockDim.x) {
    const int n = cnt[e], nc = (n + cmax - 1) / cmax;
    for (int c = 0; c < nc; ++c) {
      const int lo = n * c / nc, hi = n * (c + 1) / nc;
      P.chunk[co[e] + c] = PfChunk{e, cur[e] + lo, hi - lo};
    }
  }
}

// Power of two s such that m * 2^-s lies in [2^14, 2^15) (0 when m is zero
// or not finite).
__device__ __forceinline__ int pf_shift(float m) {
  if (!(m > 0.f) || !isfinite(m)) return 0;
  int x;
  frexpf(m, &x);  // m = f 2^x, f in [0.5, 1)
  return x - 15;
}

// Eight values stored at element off of the input planes (plane elements
// apart): fp16 of v * 2^-sh (FP4), or the two bf16 terms of v.
template <bool FP4>
__device__ __forceinline__ void pf_store8(unsigned short* dst, size_t plane, size_t off,
                                          const float (&v)[8], int sh) {
  unsigned hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (FP4) {
      hi[i] = cvt_pk_f16(ldexpf(v[2 * i], -sh), ldexpf(v[2 * i + 1], -sh));
    } else {
      hi[i] = cvt_pk_bf16(v[2 * i], v[2 * i + 1]);
      lo[i] = cvt_pk_bf16(v[2 * i] - bf16_lo(hi[i]), v[2 * i + 1] - bf16_hi(hi[i]));
    }
  }
  *reinterpret_cast<v4u*>(dst + off) = v4u{hi[0], hi[1], hi[2], hi[3]};
  if constexpr (!FP4) *reinterpret_cast<v4u*>(dst + plane + off) = v4u{lo[0], lo[1], lo[2], lo[3]};
}

// A wave converts one row of n values (eight per lane per 512 columns) to the
// product format: for FP4 the power of two of its largest magnitude comes
// first (pf_shift), so the row is needed twice.  Rows of up to 512 NR values
// stay in registers in between (one read); longer rows are produced twice.
// produce8(c, v) forms columns c .. c + 7; store8(c, v, sh) writes them.
// Returns the power of two.
template <bool FP4, int NR, class Produce, class Store>
__device__ __forceinline__ int pf_convert_row(int n, Produce&& produce8, Store&& store8) {
  const int ln = lane_id();
  if (n <= 512 * NR) {
    float v[NR][8];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = 8 * ln + 512 * i;
      if (c < n) {
        produce8(c, v[i]);
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[i][k]));
      }
    }
    const int sh = FP4 ? pf_shift(wave_max(m)) : 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = 8 * ln + 512 * i;
      if (c < n) store8(c, v[i], sh);
    }
    return sh;
  }
  int sh = 0;
  if constexpr (FP4) {
    float m = 0.f;
    for (int c = 8 * ln; c < n; c += 512) {
      float v[8];
      produce8(c, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
    }
    sh = pf_shift(wave_max(m));
  }
  for (int c = 8 * ln; c < n; c += 512) {
    float v[8];
    produce8(c, v);
    store8(c, v, sh);
  }
  return sh;
}

// One wave per token t: its slots' grouped positions (lane j < k takes slot
// j's from its expert's cursor), its input row u[t] in the product format,
// and its power of two at each of those positions.
template <bool FP4>
__device__ inline void pf_gather(const LayerArgs& L, const PfArgs& P) {
  const int t = blockIdx.x * kWaves + wave_id();
  if (t >= P.T) return;
  const int ln = lane_id();
  const float* src = P.u + (size_t)t * L.H;
  const int sh = pf_convert_row<FP4, 12>(
      L.H,
      [&](int c, float (&v)[8]) {
        const v4f x0 = *reinterpret_cast<const v4f*>(src + c);
        const v4f x1 = *reinterpret_cast<const v4f*>(src + c + 4);
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      },
      [&](int c, const float (&v)[8], int sh) {
        pf_store8<FP4>(P.a, (size_t)P.T * L.H, (size_t)t * L.H + c, v, sh);
      });
  static_assert(kMaxTopK <= 64, "one lane per slot of a token");
  if (ln < L.K) {
    const int s = t * L.K + ln;
    const int e = P.idx[s];
    int p = -1;
    if (e >= 0 && e < L.E) {
      p = __hip_atomic_fetch_add(P.cur + e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      P.perm[p] = s;
      P.pe[p] = e;
      P.ue[p] = sh;
    }
    P.pos[s] = p;
  }
}

// One wave per grouped position: act = silu(g_g gate) * (g_u up) in the
// product format, with its power of two.
template <bool FP4>
__device__ inline void pf_swiglu(const LayerArgs& L, const PfArgs& P) {
  const int pos = blockIdx.x * kWaves + wave_id();
  if (pos >= P.off[L.E]) return;
  const int e = P.pe[pos];
  const float gs = FP4 ? L.gg[e] : 1.f;
  const float us = FP4 ? L.gu[e] : 1.f;
  const float* g = P.gu + (size_t)pos * 2 * L.F;
  const float* up = g + L.F;
  const int sh = pf_convert_row<FP4, 8>(
      L.F,
      [&](int c, float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 8; i += 4) {
          const v4f a = *reinterpret_cast<const v4f*>(g + c + i);
          const v4f b = *reinterpret_cast<const v4f*>(up + c + i);
          v[i] = silu(gs * a.x) * (us * b.x);
          v[i + 1] = silu(gs * a.y) * (us * b.y);
          v[i + 2] = silu(gs * a.z) * (us * b.z);
          v[i + 3] = silu(gs * a.w) * (us * b.w);
        }
      },
      [&](int c, const float (&v)[8], int sh) {
        pf_store8<FP4>(P.act, (size_t)P.T * L.K * L.F, (size_t)pos * L.F + c, v, sh);
      });
  if (lane_id() == 0) P.ae[pos] = sh;
}

constexpr int kPfRows = 4 * 64;             // output rows per item
// Per format: input terms, k columns per tile, ring slots, loads per tile of
// one wave besides its share of the input tile, bytes of one ring slot.
//   NVFP4: a wave's 64 weight rows of a tile (64 x 32 B of e2m1 codes and
//   64 x 4 B of e4m3 scales) come into the slot by direct global->LDS loads
//   too: two 1-KB loads of codes (32 rows each, row-major: an operand read of
//   16 rows x 8 B is one contiguous 512 B, free of bank conflicts) and one
//   256-B load of scales.
//   bf16: a lane's 16 columns of four rows (32 B each) go straight to
//   registers, two tiles ahead.
template <bool FP4>
struct PfFmt;
template <>
struct PfFmt<true> {
  static constexpr int CHUNK = kPfChunkFp4, NTERM = 1, KT = 64, STAGES = 3, LOADS = 3;
  static constexpr int IN = CHUNK * KT * 2 * NTERM;  // bytes of one k-tile of inputs
  static constexpr int CODES = IN, SCALES = CODES + 4 * 2048, STAGE = SCALES + 4 * 256;
};
template <>
struct PfFmt<false> {
  static constexpr int CHUNK = kPfChunk, NTERM = 2, KT = 64, STAGES = 3, LOADS = 8;
  static constexpr int IN = CHUNK * KT * 2 * NTERM, STAGE = IN;
};
template <bool FP4>
constexpr int pf_lds() { return PfFmt<FP4>::STAGES * PfFmt<FP4>::STAGE; }

// f(IC<0>{}), ..., f(IC<N - 1>{})
template <class F, int... I>
__device__ __forceinline__ void pf_unroll(F&& f, std::integer_sequence<int, I...>) {
  (f(IC<I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void pf_for(F&& f) {
  pf_unroll(f, std::make_integer_sequence<int, N>{});
}

// bf16 weight registers of one tile: lane (r, g) holds columns 16 g .. + 15
// of rows 16 rf + r.
struct PfWbf {
  v4u w[4][2];
};

// The NVFP4 weight operand of k-step j from a lane's 16 B of codes (32
// columns) and its block scale for those 8 columns.
__device__ __forceinline__ f16x8 pf_weights(unsigned d, f16x2 sc) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * sc;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * sc;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * sc;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * sc;
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  const f16x4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const f16x4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One item: rows rb * 256 .. + 255 of the product for chunk ch, in TF 16-slot
// tiles (ch.n <= 16 TF; slots past ch.n repeat its last one and are not
// written).  Ends with the LDS free.
template <bool FP4, bool GU, int TF>
__device__ void pf_item(const LayerArgs& L, const PfArgs& P, const PfChunk ch, int rb,
                        uint8_t* lds) {
  using Fm = PfFmt<FP4>;
  constexpr int KT = Fm::KT, NTERM = Fm::NTERM, J = KT / 32, NS = Fm::STAGES, LA = NS - 1;
  constexpr int RB = KT * 2, PR = RB / 16, RPI = 1024 / RB;  // row bytes, pieces, rows per 1 KB
  constexpr int LPP = 16 * TF * RB / 1024;                     // 1-KB loads per term plane
  constexpr int NL = NTERM * LPP, NLW = (NL + 3) / 4;          // 1-KB input loads: all, per wave
  constexpr int PLANE = Fm::CHUNK * RB;                        // LDS bytes per term plane
  const int N = GU ? 2 * L.F : L.H, K = GU ? L.H : L.F;
  const int ln = lane_id(), wv = wave_id(), r = ln & 15, g = ln >> 4;
  const int tiles = K / KT;
  const int r0 = rb * kPfRows + 64 * wv;  // this wave's first row (64 never straddle W_g / W_u)
  const bool active = r0 < N;
  // first byte of weight row `row` (global row index of the product) and of
  // its NVFP4 scales
  auto wrow = [&](int row, const uint8_t*& w, const uint8_t*& sc) {
    const uint8_t* m;
    const uint8_t* sm;
    size_t gr;
    if constexpr (GU) {
      const bool up = row >= L.F;
      m = up ? L.wu : L.wg;
      sm = up ? L.su : L.sg;
      gr = (size_t)ch.e * L.F + (up ? row - L.F : row);
    } else {
      m = L.wd;
      sm = L.sd;
      gr = (size_t)ch.e * L.H + row;
    }
    if constexpr (FP4) {
      w = m + gr * (K / 2);
      sc = sm + gr * (K / 16);
    } else {
      w = m + gr * K * 2;
      sc = nullptr;
    }
  };
  const int wr0 = active ? r0 : 0;  // idle waves fetch rows they never use
  // NVFP4: this lane's rows in the two code loads (32 i + ln / 2, 16-B
  // piece ln & 1) and in the scale load (ln); bf16: rows 16 rf + r
  const uint8_t* wp[4];
  const uint8_t* sp = nullptr;
  if constexpr (FP4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint8_t* sc;
      wrow(wr0 + 32 * i + (ln >> 1), wp[i], sc);
      wp[i] += 16 * (ln & 1);
    }
    const uint8_t* w;
    wrow(wr0 + ln, w, sp);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* sc;
      wrow(wr0 + 16 * i + r, wp[i], sc);
      wp[i] += 32 * g;
    }
  }
  auto load_w = [&](int tau, PfWbf& W) {
#pragma unroll
    for (int rf = 0; rf < 4; ++rf)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        W.w[rf][q] = *reinterpret_cast<const v4u*>(wp[rf] + (size_t)tau * 128 + 16 * q);
  };
  auto dma_w = [&](int tau, int buf) {
    if constexpr (FP4) {
      uint8_t* st = lds + buf * Fm::STAGE;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(wp[i] + (size_t)tau * (KT / 2),
                                         st + Fm::CODES + wv * 2048 + i * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(sp + (size_t)tau * (KT / 16), st + Fm::SCALES + wv * 256,
                                       4, 0, 0);
    }
  };
  // input rows: u by token (gate/up), act by grouped position (down)
  const unsigned short* in = GU ? P.a : P.act;
  const size_t in_plane = GU ? (size_t)P.T * L.H : (size_t)P.T * L.K * L.F;
  // 1-KB input load m of this wave is load (wv + 4 m) % NL of the tile
  // (with two loads, waves 2 and 3 repeat those of waves 0 and 1)
  const unsigned short* isrc[NLW];  // this lane's row and piece in its load m
#pragma unroll
  for (int m = 0; m < NLW; ++m) {
    const int q = (wv + 4 * m) % NL;
    const int pl = q / LPP, ql = q - pl * LPP;
    const int R = ql * RPI + ln / PR;  // chunk row this lane fills, slot ln % PR
    const int tk = R < ch.n ? R : ch.n - 1;
    const int p = (ln % PR) ^ (R & (PR - 1));  // the piece that belongs in that slot
    const int row = GU ? P.perm[ch.pos0 + tk] / L.K : ch.pos0 + tk;
    isrc[m] = in + pl * in_plane + (size_t)row * K + p * 8;
  }
  auto issue_in = [&](int tau, int buf) {
    uint8_t* bt = lds + buf * Fm::STAGE;
#pragma unroll
    for (int m = 0; m < NLW; ++m) {
      const int q = (wv + 4 * m) % NL;
      const int pl = q / LPP, ql = q - pl * LPP;
      __builtin_amdgcn_global_load_lds(isrc[m] + (size_t)tau * KT, bt + pl * PLANE + ql * 1024,
                                       16, 0, 0);
    }
  };
  f32x4 acc[4][TF];
#pragma unroll
  for (int rf = 0; rf < 4; ++rf)
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) acc[rf][tf] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const PfWbf& W, int buf) {
    const uint8_t* bt = lds + buf * Fm::STAGE;
    v2u cw[4];
    f16x2 sc[4];
    if constexpr (FP4) {
      // this wave's codes and scales of the tile: lane group g holds columns
      // 16 g .. 16 g + 15 of its row (8 B of codes, block scale g)
#pragma unroll
      for (int rf = 0; rf < 4; ++rf) {
        const int row = 16 * rf + r;
        cw[rf] = *reinterpret_cast<const v2u*>(bt + Fm::CODES + wv * 2048 + row * 32 + g * 8);
        const unsigned sv =
            *reinterpret_cast<const unsigned*>(bt + Fm::SCALES + wv * 256 + row * 4);
        const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)(sv >> (8 * g)), 0);
        sc[rf] = f16x2{s0, s0};
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      v4u b[NTERM][TF];
#pragma unroll
      for (int pl = 0; pl < NTERM; ++pl)
#pragma unroll
        for (int tf = 0; tf < TF; ++tf)
          b[pl][tf] = *reinterpret_cast<const v4u*>(
              bt + pl * PLANE + (16 * tf + r) * RB + (((J * g + j) ^ (r & (PR - 1))) * 16));
#pragma unroll
      for (int rf = 0; rf < 4; ++rf) {
        if constexpr (FP4) {
          const f16x8 a = pf_weights(cw[rf][j], sc[rf]);
#pragma unroll
          for (int tf = 0; tf < TF; ++tf)
            acc[rf][tf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a, __builtin_bit_cast(f16x8, b[0][tf]), acc[rf][tf], 0, 0, 0);
        } else {
          const bf16x8 a = as_bf16x8(W.w[rf][j]);
#pragma unroll
          for (int tf = 0; tf < TF; ++tf)
#pragma unroll
            for (int pl = 0; pl < NTERM; ++pl)
              acc[rf][tf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(b[pl][tf]),
                                                                    acc[rf][tf], 0, 0, 0);
        }
      }
    }
  };
  // Tile tau, ring slot S = tau % NS: wait for its loads (those of the
  // LA - 1 tiles after it may stay in flight), meet the other waves (so every
  // wave is done with tile tau - 1, whose slot is refilled), fetch tile
  // tau + LA and use tile tau.  Every wave issues the same loads at every
  // step (idle waves fetch rows they never use) and the loads are never
  // conditional inside the loop, so the compiler's own counter bookkeeping
  // stays exact and adds no wait that would drain the loads in flight.
  PfWbf W[NS];  // bf16 weight registers (unused for NVFP4)
  constexpr int PER = NLW + Fm::LOADS;  // loads per tile of every wave
  static_assert((LA - 1) * PER < 64, "loads in flight within the counter's range");
  auto fetch = [&](auto S_, int tau) {
    constexpr int S = decltype(S_)::value;
    issue_in(tau, S);
    if constexpr (FP4)
      dma_w(tau, S);
    else
      load_w(tau, W[S]);
  };
  // FETCH: whether this step fetches ahead; AFTER: tiles whose loads may
  // still be in flight after this one's
  auto step = [&](auto S_, auto FETCH_, auto AFTER_, int tau) {
    constexpr int S = decltype(S_)::value;
    wait_vm<decltype(AFTER_)::value * PER>();
    lds_barrier();
    if constexpr (decltype(FETCH_)::value) fetch(IC<(S + LA) % NS>{}, tau + LA);
    if (active) compute(W[S], S);
  };
  using T_ = IC<1>;
  using F_ = IC<0>;
  // The previous item's output stores are still counted: until a wait for
  // zero, the compiler treats the counter as out of order and turns every
  // wait it adds for a weight register into a wait for zero (a full drain
  // at a step of the loop below).  One drain here, before anything of this
  // item is in flight, costs only the stores' round trip.
  wait_vm<0>();
  // tiles 0 .. LA - 1 (fewer tiles: copies of the last, never used)
  pf_for<LA>([&](auto I) { fetch(I, decltype(I)::value < tiles ? decltype(I)::value : tiles - 1); });
  if (tiles >= LA) {
    const int nla = tiles - LA;  // steps that fetch ahead: 0 .. nla - 1
    int tau = 0;
    for (; tau + NS <= nla; tau += NS)
      pf_for<NS>([&](auto I) { step(I, T_{}, IC<LA - 1>{}, tau + decltype(I)::value); });
    // R more steps that fetch ahead, in slots 0 .. R - 1, then the last LA
    // tiles, in slots R .. R + LA - 1 (mod NS)
    const int rem = nla - tau;
    pf_for<NS>([&](auto R_) {
      constexpr int R = decltype(R_)::value;
      if (rem == R) {
        pf_for<R>([&](auto I) { step(I, T_{}, IC<LA - 1>{}, tau + decltype(I)::value); });
        pf_for<LA>([&](auto I) {
          constexpr int i = decltype(I)::value;
          step(IC<(R + i) % NS>{}, F_{}, IC<LA - 1 - i>{}, tau + R + i);
        });
      }
    });
  } else {
    pf_for<LA>([&](auto I) {
      if (decltype(I)::value < tiles) step(I, F_{}, IC<0>{}, decltype(I)::value);
    });
  }
  lds_barrier();  // every wave is done with the ring before the next item fills it
  if (!active) return;
  // lane (r, g): slot 16 tf + r, rows r0 + 16 rf + 4 g + i
#pragma unroll
  for (int tf = 0; tf < TF; ++tf) {
    const int tk = 16 * tf + r;
    if (tk >= ch.n) continue;
    const int pos = ch.pos0 + tk;
    float* o;
    int sh;
    float osc = 1.f;
    if constexpr (GU) {
      sh = P.ue[pos];
      o = P.gu + (size_t)pos * N + r0 + 4 * g;
    } else {
      sh = P.ae[pos];
      if constexpr (FP4) osc = L.gd[ch.e];
      o = P.y + (size_t)P.perm[pos] * N + r0 + 4 * g;
    }
#pragma unroll
    for (int rf = 0; rf < 4; ++rf) {
      const f32x4 a = acc[rf][tf];
      *reinterpret_cast<v4f*>(o + 16 * rf) =
          v4f{ldexpf(osc * a[0], sh), ldexpf(osc * a[1], sh), ldexpf(osc * a[2], sh),
              ldexpf(osc * a[3], sh)};
    }
  }
}

// Every item of the gate/up (GU) or down product: item = chunk * n_rb + row
// block.  Workgroup b runs on XCD b % 8 (gridDim.x is a multiple of 8); XCD
// x takes the contiguous items [x per, (x + 1) per) in order.
template <bool FP4, bool GU>
__device__ void pf_gemm(const LayerArgs& L, const PfArgs& P, uint8_t* lds) {
  const int N = GU ? 2 * L.F : L.H;
  const int n_rb = (N + kPfRows - 1) / kPfRows;
  const long long items = (long long)(*P.nchunk) * n_rb;
  const long long per = (items + 7) >> 3;
  const int x = blockIdx.x & 7, v = blockIdx.x >> 3, gx = gridDim.x >> 3;
  for (long long i = v; i < per; i += gx) {
    const long long item = x * per + i;
    if (item >= items) break;
    const long long c = item / n_rb;
    const PfChunk ch = P.chunk[c];
    const int rb = (int)(item - c * n_rb);
    const int ntf = (ch.n + 15) >> 4;
    if (FP4 && ntf > 8)
      pf_item<FP4, GU, FP4 ? 10 : 8>(L, P, ch, rb, lds);
    else if (ntf > 6)
      pf_item<FP4, GU, 8>(L, P, ch, rb, lds);
    else if (ntf > 4)
      pf_item<FP4, GU, 6>(L, P, ch, rb, lds);
    else if (ntf > 2)
      pf_item<FP4, GU, 4>(L, P, ch, rb, lds);
    else if (ntf > 1)
      pf_item<FP4, GU, 2>(L, P, ch, rb, lds);
    else
      pf_item<FP4, GU, 1>(L, P, ch, rb, lds);
  }
}

}  // namespace msk
