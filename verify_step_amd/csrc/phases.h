// The phases of one MoE layer step, written as grid-stride device functions
// so that the same code runs as separate kernels (one launch per phase) and
// inside the persistent whole-step kernel (phases separated by grid barriers).
//
// Every phase takes the "virtual block" index vb and count nvb it runs on.
#pragma once
#include "device.h"

namespace msk {


// Global index of this wave when waves are numbered across workgroups first,
// so that a phase with fewer tasks than waves still spreads over every CU.
__device__ __forceinline__ int gwave(int vb, int nvb) { return wave_id() * nvb + vb; }

// Calls f(IC<NV>) with the smallest power of two NV >= n, n <= NVMAX.
template <int NVMAX, class F>
__device__ __forceinline__ void nv_dispatch(int n, F&& f) {
  if (NVMAX <= 1 || n <= 1) f(IC<1>{});
  else if (NVMAX <= 2 || n <= 2) f(IC<(NVMAX < 2 ? NVMAX : 2)>{});
  else if (NVMAX <= 4 || n <= 4) f(IC<(NVMAX < 4 ? NVMAX : 4)>{});
  else if (NVMAX <= 8 || n <= 8) f(IC<(NVMAX < 8 ? NVMAX : 8)>{});
  else if (NVMAX <= 16 || n <= 16) f(IC<(NVMAX < 16 ? NVMAX : 16)>{});
  else f(IC<NVMAX>{});
}

// Rows per wave of the dense projections for NV token vectors: fewer rows
// when many tokens share them, so the accumulators stay in registers.
template <int NV> struct DenseRows { static constexpr int R = NV >= 16 ? 2 : 4; };

__host__ __device__ inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }


// Attention work split of one layer, kept in LDS by every workgroup.
struct AttnPlan {
  int item0[kMaxReq + 1];  // first item of request b; item0[n_req] = all items
  int nch[kMaxReq];        // chunks per (kv head, row group) of request b
  int base[kMaxReq];
  int end[kMaxReq];
};

__device__ inline void build_plan(const LayerArgs& L, const StepArgs& S, AttnPlan* P) {
  // lane b plans request b (at most 64 requests): one load for all of them,
  // item offsets by a prefix sum over the lanes
  if (threadIdx.x < 64) {
    const int b = threadIdx.x;
    int base = 0, end = 0, n = 0;
    if (b < S.n_req) {
      req_span(S.kv_len[b], S.Tr, L.window, L.attn_nw != 0, base, end);
      n = ceil_div(end - base, L.chunk);
    }
    const int cnt = n * L.Hkv * L.nrg;
    int inc = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int a = __shfl_up(inc, off, 64);
      if (b >= off) inc += a;
    }
    if (b < S.n_req) {
      P->base[b] = base;
      P->end[b] = end;
      P->nch[b] = n;
      P->item0[b] = inc - cnt;
    }
    if (b == (S.n_req > 0 ? S.n_req - 1 : 0)) P->item0[S.n_req] = S.n_req > 0 ? inc : 0;
  }
  __syncthreads();
}

// 1/sqrt(mean(x^2) + eps) of T rows of length H, into rs[0..T).
__device__ inline void block_rstd(const float* x, int T, int H, float eps, float* rs) {
  for (int t = wave_id(); t < T; t += kWaves) {
    const float* row = x + (size_t)t * H;
    float s = 0.f;
    for (int c = lane_id() * 4; c < H; c += 256) {
      v4f a = *reinterpret_cast<const v4f*>(row + c);
      s += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
    s = wave_sum(s);
    if (lane_id() == 0) rs[t] = 1.0f / sqrtf(s / (float)H + eps);
  }
  __syncthreads();
}

__device__ __forceinline__ size_t dense_row_bytes(int dt, int n) {
  return (size_t)n * (dt == kBF16 ? 2 : 4);
}
__device__ __forceinline__ size_t expert_row_bytes(int dt, int n) {
  return dt == kNVFP4 ? (size_t)n / 2 : (size_t)n * (dt == kBF16 ? 2 : 4);
}

// Lane (r * NV + v) % 64 stores value acc[r][v]; all lanes hold all values.
template <int R, int NV, class F>
__device__ __forceinline__ void store_results(const float (&acc)[R][NV], int nv, F&& st) {
  const int ln = lane_id();
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int v = 0; v < NV; ++v)
      if (v < nv && ln == ((r * NV + v) & 63)) st(r, v, acc[r][v]);
}

// x = hi + mid + lo to within 2^-24 |x|; bf16 bits, each term the
// round-to-nearest-even of what the previous terms leave.
__device__ __forceinline__ void split3_bf16(float x, unsigned& h, unsigned& m, unsigned& l) {
  h = f2bf16(x);
  float r = x - bf16_lo(h);
  m = f2bf16(r);
  r -= bf16_lo(m);
  l = f2bf16(r);
}

// ------------------------------------------------------------- QKV
// qkv[t][r] = rstd[t] * sum_c W[r][c] * attn_norm[c] * x[t][c] for the rows of
// wq, wk, wv stacked (r < Hq*D: wq; then wk; then wv).
template <int DT, int NV>
__device__ void phase_qkv(const LayerArgs& L, const StepArgs& S, const float* x,
                          const float* rs, int vb, int nvb) {
  constexpr int R = DenseRows<NV>::R;
  const int NQ = L.Hq * L.D, NK = L.Hkv * L.D, NR = NQ + 2 * NK;
  const size_t rb = dense_row_bytes(DT, L.H);
  const int gw = gwave(vb, nvb), nw = nvb * kWaves;
  for (int t0 = 0; t0 < S.T; t0 += NV) {
    const int nt = S.T - t0 < NV ? S.T - t0 : NV;
    const float* vin[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) vin[v] = x + (size_t)(t0 + (v < nt ? v : 0)) * L.H;
    const uint8_t* srow[R] = {};
    for (int blk = gw; blk * R < NR; blk += nw) {
      const int r0 = blk * R;
      const uint8_t* base;
      int rr;
      if (r0 < NQ) { base = L.wq; rr = r0; }
      else if (r0 < NQ + NK) { base = L.wk; rr = r0 - NQ; }
      else { base = L.wv; rr = r0 - NQ - NK; }
      const uint8_t* wrow[R];
#pragma unroll
      for (int r = 0; r < R; ++r) wrow[r] = base + (size_t)(rr + r) * rb;
      float acc[R][NV];
      wave_gemv<DT, R, NV>(wrow, srow, L.H, vin, nt, L.attn_norm, acc);
      store_results<R, NV>(acc, nt, [&](int r, int v, float val) {
        S.qkv[(size_t)(t0 + v) * NR + r0 + r] = val * rs[t0 + v];
      });
    }
  }
}

// ------------------------------------------------------- attention
// One workgroup per work item (request b, kv head j, query row group rg,
// chunk c).  Rows of a group are (draft token t, query head g of the group)
// pairs, m = t * G + g, eight at a time, two per wave.  For each 64-position
// block of the chunk:
//  - the K and V rows go straight from HBM into the workgroup's LDS tiles
//    (direct global->LDS loads, shared by the four waves; no registers are
//    held while they fly);
//  - a step of a wave covers whole rows: each lane takes one 16-byte chunk
//    of K and of V at one position, forms its part of the two rows' scores
//    against query values held in registers, and a sum over the position's
//    lanes gives the scores;
//  - e = exp(s - shift) inside the token's window, else 0 (no running max);
//  - the lane adds e times its V chunk to its own accumulators, which are
//    summed over the positions' lanes once, at the end of the item.
// Positions at or past kv_len[b] are the step's own draft tokens: their K/V
// are rebuilt from the QKV output (QK-norm on k, cast to the cache format),
// and the row-group-0 item also writes them into the cache.
// The item writes its plain partial sums (o[8][D], l[8]).
template <int KDT> struct KV;
template <> struct KV<kF32> { enum { ES = 4 }; };
template <> struct KV<kBF16> { enum { ES = 2 }; };
template <> struct KV<kE4M3> { enum { ES = 1 }; };

template <int KDT, int D>
struct AttnGeom {
  static constexpr int ES = KV<KDT>::ES;
  static constexpr int RB = D * ES;           // cache row bytes
  static constexpr int CPR = RB / 16;         // 16-B chunks per row
  static constexpr int EPC = 16 / ES;         // elements per 16-B chunk
  static constexpr int TILE = 64 * RB;        // one 64-position tile
  static constexpr int NLD = TILE / 1024;     // 1-KB wave loads per tile
  // per-workgroup LDS: q rows, K tile, V tile, windows
  static constexpr int LDS_Q = kRowGroup * D * 4;
  static constexpr int LDS_K = TILE;
  static constexpr int LDS_V = TILE;
  static constexpr int LDS_WIN = kRowGroup * 8;
  static constexpr int LDS_ITEM = LDS_Q + LDS_K + LDS_V + LDS_WIN;
  static constexpr int RPW = kRowGroup / kWaves;  // query rows per wave
};

template <int KDT>
__device__ __forceinline__ v4u encode16(const float* f);
template <>
__device__ __forceinline__ v4u encode16<kF32>(const float* f) {
  return v4u{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
             __float_as_uint(f[3])};
}
template <>
__device__ __forceinline__ v4u encode16<kBF16>(const float* f) {
  return v4u{f2bf16(f[0]) | (f2bf16(f[1]) << 16), f2bf16(f[2]) | (f2bf16(f[3]) << 16),
             f2bf16(f[4]) | (f2bf16(f[5]) << 16), f2bf16(f[6]) | (f2bf16(f[7]) << 16)};
}
template <>
__device__ __forceinline__ v4u encode16<kE4M3>(const float* f) {
  return v4u{f2e4m3x2(f[0], f[1]) | (f2e4m3x2(f[2], f[3]) << 16),
             f2e4m3x2(f[4], f[5]) | (f2e4m3x2(f[6], f[7]) << 16),
             f2e4m3x2(f[8], f[9]) | (f2e4m3x2(f[10], f[11]) << 16),
             f2e4m3x2(f[12], f[13]) | (f2e4m3x2(f[14], f[15]) << 16)};
}

// Decode the EPC elements of one 16-B chunk.
template <int KDT>
__device__ __forceinline__ void decode16(const v4u& w, float* f) {
  if constexpr (KDT == kF32) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  } else if constexpr (KDT == kBF16) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  } else {
    e4m3x4(w.x, f); e4m3x4(w.y, f + 4); e4m3x4(w.z, f + 8); e4m3x4(w.w, f + 12);
  }
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0); }

template <int KDT, int D, class MP = Plain>
__device__ void attn_item(const LayerArgs& L, const StepArgs& S, const AttnPlan* P, int item,
                          uint8_t* wl) {
  using Gm = AttnGeom<KDT, D>;
  constexpr int RB = Gm::RB, CPR = Gm::CPR, EPC = Gm::EPC, NLD = Gm::NLD, RPW = Gm::RPW;
  float* qs = reinterpret_cast<float*>(wl);
  uint8_t* kt = wl + Gm::LDS_Q;
  uint8_t* vt = kt + Gm::LDS_K;
  int* win = reinterpret_cast<int*>(vt + Gm::LDS_V);

  const int ln = lane_id(), wv = wave_id();
  int b = 0;
  while (b + 1 < S.n_req && P->item0[b + 1] <= item) ++b;
  const int nch = P->nch[b];
  int rem = item - P->item0[b];
  const int j = rem / (L.nrg * nch);
  rem -= j * L.nrg * nch;
  const int rg = rem / nch;
  const int c = rem - rg * nch;
  const int p0 = P->base[b] + c * L.chunk;
  const int p1 = p0 + L.chunk < P->end[b] ? p0 + L.chunk : P->end[b];
  const int Lb = S.kv_len[b];
  const int G = L.Hq / L.Hkv;
  const int M = G * S.Tr;
  const int m0 = rg * kRowGroup;
  const int NQ = L.Hq * L.D, NK = L.Hkv * L.D, NR = NQ + 2 * NK;
  const size_t head_off = ((size_t)b * L.Hkv + j) * (size_t)L.cap;  // in rows
  uint8_t* kc = L.kc + head_off * RB;
  uint8_t* vc = L.vc + head_off * RB;
  const bool writer = (rg == 0);

  // positions before the group's earliest window start (that of its first
  // row's token) are never visible
  const int lo_min = L.window > 0 ? (Lb + m0 / G - L.window + 1 > 0 ? Lb + m0 / G - L.window + 1 : 0)
                                  : 0;
  // cached rows of one 64-position block straight into the LDS tiles, the
  // 1-KB loads dealt over the waves.  Lane l of load i carries tile bytes
  // [i KB + 16 l, +16), i.e. row (1024 i + 16 l) / RB; only rows that are
  // visible and already cached are fetched.
  auto issue_tiles = [&](int pb, int npos) {
#pragma unroll
    for (int i0 = 0; i0 < NLD; i0 += kWaves) {
      const int i = i0 + wv;
      const int off = i * 1024 + ln * 16;
      const int pos = pb + off / RB;
      if (i < NLD && pos < pb + npos && pos >= lo_min && pos < Lb) {
        __builtin_amdgcn_global_load_lds(kc + (size_t)pb * RB + off, kt + i * 1024, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vc + (size_t)pb * RB + off, vt + i * 1024, 16, 0, 0);
      }
    }
  };

  // The step's own rows in block [pb, pb + npos) (positions >= kv_len),
  // rebuilt from the QKV output into the LDS tiles: k QK-normalised, both
  // cast to the cache format.  Wave w takes the tokens t = w mod kWaves, lane
  // l < CPR the row's 16-byte chunk l.  Their loads follow the block's tile
  // loads, so one wait covers both.
  auto own_rows = [&](int pb, int npos) {
    const int t0 = pb > Lb ? pb - Lb : 0;
    const int t1 = pb + npos - Lb < S.Tr ? pb + npos - Lb : S.Tr;
    const int d0 = ln * EPC;
    const bool act = ln < CPR;
    for (int t = t0 + wv; t < t1; t += kWaves) {
      const float* kq = S.qkv + (size_t)(b * S.Tr + t) * NR + NQ + (size_t)j * D + (act ? d0 : 0);
      const float* vq = kq + NK;
      float fk[EPC], fv[EPC], gk[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        fk[e] = act ? MP::ld(&kq[e]) : 0.f;
        fv[e] = act ? MP::ld(&vq[e]) : 0.f;
        gk[e] = act ? L.k_norm[d0 + e] : 0.f;
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) ss += fk[e] * fk[e];
      const float r = 1.0f / sqrtf(wave_sum(ss) / (float)D + L.eps);
      if (act) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) gk[e] = fk[e] * r * gk[e];
        const int row = Lb + t - pb;
        *reinterpret_cast<v4u*>(kt + row * RB + ln * 16) = encode16<KDT>(gk);
        *reinterpret_cast<v4u*>(vt + row * RB + ln * 16) = encode16<KDT>(fv);
      }
    }
  };
  // ... and, by the row-group-0 item, from the LDS tiles into the cache
  auto store_own_rows = [&](int pb, int npos) {
    const int t0 = pb > Lb ? pb - Lb : 0;
    const int t1 = pb + npos - Lb < S.Tr ? pb + npos - Lb : S.Tr;
    if (!writer || ln >= CPR) return;
    for (int t = t0 + wv; t < t1; t += kWaves) {
      const int row = Lb + t - pb;
      *reinterpret_cast<v4u*>(kc + (size_t)(Lb + t) * RB + ln * 16) =
          *reinterpret_cast<const v4u*>(kt + row * RB + ln * 16);
      *reinterpret_cast<v4u*>(vc + (size_t)(Lb + t) * RB + ln * 16) =
          *reinterpret_cast<const v4u*>(vt + row * RB + ln * 16);
    }
  };

  // this wave's query rows, normalised and pre-scaled, and their windows.
  // The first block's tiles and own rows are loaded right after the query
  // values, so the three arrive in one round trip.
  constexpr int QD = (D + 63) / 64;
  const v2f gq2 = gain_pair(L.q_norm, D), gk2 = gain_pair(L.k_norm, D);
  {
    float qv[RPW][QD];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int mm = wv * RPW + r;
      const int m = m0 + mm < M ? m0 + mm : M - 1;  // rows past M load a valid row, unused
      const int t = m / G, g = m - (m / G) * G;
      const float* q = S.qkv + (size_t)(b * S.Tr + t) * NR + (size_t)(j * G + g) * D;
#pragma unroll
      for (int i = 0; i < QD; ++i) {
        const int d = ln + 64 * i;
        qv[r][i] = (m0 + mm < M && d < D) ? MP::ld(&q[d]) : 0.f;
      }
    }
    if (p0 < p1) {
      issue_tiles(p0, p1 - p0 < 64 ? p1 - p0 : 64);
      own_rows(p0, p1 - p0 < 64 ? p1 - p0 : 64);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int mm = wv * RPW + r;
      const int m = m0 + mm;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < QD; ++i) ss += qv[r][i] * qv[r][i];
      ss = wave_sum(ss);
      const float rr = 1.0f / sqrtf(ss / (float)D + L.eps);
#pragma unroll
      for (int i = 0; i < QD; ++i) {
        const int d = ln + 64 * i;
        if (d < D) qs[mm * D + d] = m < M ? qv[r][i] * rr * (i == 0 ? gq2.x : gq2.y) * L.qscale : 0.f;
      }
      if (ln == 0) {
        const int t = m / G;
        const int p = Lb + t;
        win[2 * mm] = m < M ? (L.window > 0 ? (p - L.window + 1 > 0 ? p - L.window + 1 : 0) : 0) : 1;
        win[2 * mm + 1] = m < M ? p : 0;
      }
    }
  }
  lds_barrier();
  const float shift = layer_shift(L.shift, gq2, gk2, D);

  // Lane (g, c) = (ln / CPR, ln % CPR) takes 16-byte chunk c of position
  // PG i + g of the block at step i: a step's loads cover PG whole rows.  A
  // score is summed over the CPR lanes of its position, and the lane adds
  // its weighted V chunk to its own accumulators, so weights never pass
  // through LDS; the position groups are summed once at the end.  The
  // query values of this wave's rows stay in registers.
  constexpr int PG = 64 / CPR;
  const int cq = ln % CPR, gq = ln / CPR;
  const bool live = m0 + wv * RPW < M;  // a wave without live rows skips the products
  float qr[RPW][EPC];
  int wlo[RPW], whi[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int mm = wv * RPW + r;
#pragma unroll
    for (int e = 0; e < EPC; ++e) qr[r][e] = qs[mm * D + cq * EPC + e];
    wlo[r] = win[2 * mm];
    whi[r] = win[2 * mm + 1];
  }
  float lsum[RPW];
  float o[RPW][EPC];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    lsum[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[r][e] = 0.f;
  }

  for (int pb = p0; pb < p1; pb += 64) {
    const int npos = p1 - pb < 64 ? p1 - pb : 64;
    if (pb != p0) {
      issue_tiles(pb, npos);
      own_rows(pb, npos);
    }
    wait_vm_all();
    __syncthreads();
    if (live) {
      const int nit = (npos + PG - 1) / PG;  // steps holding positions of the block
#pragma unroll 4
      for (int i = 0; i < CPR; ++i) {
        if (i >= nit) break;
        const int pp = i * PG + gq;
        const int pos = pb + pp;
        float kf[EPC], vf[EPC];
        decode16<KDT>(*reinterpret_cast<const v4u*>(kt + pp * RB + cq * 16), kf);
        decode16<KDT>(*reinterpret_cast<const v4u*>(vt + pp * RB + cq * 16), vf);
        // rows that were not fetched hold stale bytes: their V is zeroed so
        // that a zero weight never meets a NaN
        const bool loaded = pp < npos && pos >= lo_min;
#pragma unroll
        for (int e = 0; e < EPC; ++e) vf[e] = loaded ? vf[e] : 0.f;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float sc = 0.f;
#pragma unroll
          for (int e = 0; e < EPC; ++e) sc = fmaf(qr[r][e], kf[e], sc);
          sc = sum_within<CPR>(sc);
          const bool ok = loaded && pos >= wlo[r] && pos <= whi[r];
          const float w = ok ? __expf(sc - shift) : 0.f;
          lsum[r] += w;
#pragma unroll
          for (int e = 0; e < EPC; ++e) o[r][e] = fmaf(w, vf[e], o[r][e]);
        }
      }
    }
    store_own_rows(pb, npos);
    __syncthreads();  // tiles are refilled by the next block
  }
  // sum over the position groups and write this wave's partial sums
  if (!live) return;
  float* part = S.part + (size_t)item * kRowGroup * (D + 1);
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int mm = wv * RPW + r;
    const float l = sum_groups<CPR>(lsum[r]);  // lanes of a position hold equal sums
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[r][e] = sum_groups<CPR>(o[r][e]);
    if (gq == 0) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) MP::st(&part[mm * (D + 1) + cq * EPC + e], o[r][e]);
    }
    if (ln == 0) MP::st(&part[mm * (D + 1) + D], l);
  }
}

template <int KDT, int D, class MP = Plain>
__device__ void phase_attn(const LayerArgs& L, const StepArgs& S, const AttnPlan* P,
                           uint8_t* lds, int vb, int nvb) {
  const int n_items = P->item0[S.n_req];
  for (int item = vb; item < n_items; item += nvb) {
    attn_item<KDT, D, MP>(L, S, P, item, lds);
    __syncthreads();
  }
}

// ------------------------------------------- combine by the last item
// Variant of the attention items for the per-phase kernel: each item writes
// its partial sums with agent-coherent stores (Coh) and waits for them to
// complete before counting itself in on its group's counter; the last of a
// group's items to arrive reads the group's partials back with agent-coherent
// loads, sums them in chunk order and writes attn_o.  This takes the separate
// combine launch off the path where a group holds few rows (the vector items).
struct CohSt {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { Coh::st(p, v); }
};

// Bytes of LDS combine_if_last uses at the start of the item area.
template <int D> struct CombineLds {
  static constexpr int RED = kRowGroup * (D + 1) * 4 + 16;
  static constexpr int BYTES = RED + 16;
};

// ctr: one zero-initialised word per (request, kv head, row group), left at
// zero again by the group's last item.
template <int D>
__device__ void combine_if_last(const LayerArgs& L, const StepArgs& S, const AttnPlan* P,
                                int item, unsigned* ctr, uint8_t* lds) {
  float* red = reinterpret_cast<float*>(lds);
  int* flag = reinterpret_cast<int*>(lds + CombineLds<D>::RED);
  wait_vm_all();  // this thread's partial stores have completed ...
  __syncthreads();  // ... and every other thread's
  int b = 0;
  while (b + 1 < S.n_req && P->item0[b + 1] <= item) ++b;
  const int nch = P->nch[b];
  const int gi = (item - P->item0[b]) / nch;  // j * nrg + rg
  const int grp = b * L.Hkv * L.nrg + gi;
  if (threadIdx.x == 0) {
    const unsigned seen = __hip_atomic_fetch_add(&ctr[grp], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const int last = seen + 1 == (unsigned)nch;
    if (last) __hip_atomic_store(&ctr[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  const int j = gi / L.nrg, rg = gi - (gi / L.nrg) * L.nrg;
  const int G = L.Hq / L.Hkv, M = G * S.Tr;
  const int rows = L.rg_rows, m0 = rg * rows;
  const int live = M - m0 < rows ? M - m0 : rows;
  const int nf4 = (live * (D + 1) + 3) / 4;
  const int stride = rows * (D + 1) * 4;  // bytes from one item's partials to the next
  const float* base = S.part + (size_t)(P->item0[b] + gi * nch) * rows * (D + 1);
  // raw buffer over the group's partials: loads past the last chunk return 0;
  // cache policy sc1, the agent-coherent policy of Coh's loads
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(base), 0, nch * stride, 0x00020000);
  constexpr int CB = 8;  // chunks in flight per thread (one round for the fused groups)
  for (int f = threadIdx.x; f < nf4; f += blockDim.x) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nch; c0 += CB) {
      v4f t[CB];
#pragma unroll
      for (int q = 0; q < CB; ++q)
        t[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, (c0 + q) * stride + f * 16, 0, 16);
#pragma unroll
      for (int q = 0; q < CB; ++q) acc += t[q];
    }
    *reinterpret_cast<v4f*>(red + 4 * f) = acc;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < live * D; v += blockDim.x) {
    const int mm = v / D, d = v - (v / D) * D;
    const int m = m0 + mm, t = m / G, g = m - (m / G) * G;
    S.attn_o[((size_t)(b * S.Tr + t) * L.Hq + j * G + g) * D + d] =
        red[mm * (D + 1) + d] / red[mm * (D + 1) + D];
  }
}

// Cache windows of the step's tokens, [T][2] (lo, hi).
__device__ inline void write_windows(const LayerArgs& L, const StepArgs& S, int* win_out) {
  for (int tok = threadIdx.x; tok < S.T; tok += blockDim.x) {
    const int b = tok / S.Tr, t = tok - (tok / S.Tr) * S.Tr;
    const int p = S.kv_len[b] + t;
    win_out[2 * tok] = L.window > 0 ? (p - L.window + 1 > 0 ? p - L.window + 1 : 0) : 0;
    win_out[2 * tok + 1] = p;
  }
}

// ---------------------------------------------------------- combine
// attn_o[t][h] = sum_chunks o / sum_chunks l.  One workgroup per row (token,
// q head): wave w adds the chunks w, w + kWaves, ... (sixteen chunks' loads
// in flight), then wave 0 adds the waves' sums in wave order.  red: LDS of
// kWaves * (D + 1) floats.
template <class MP = Plain>
__device__ void phase_combine(const LayerArgs& L, const StepArgs& S, const AttnPlan* P, int* win_out,
                              int vb, int nvb, float* red, unsigned short* a3 = nullptr) {
  const int D = L.D, G = L.Hq / L.Hkv;
  const int rows = S.T * L.Hq;
  const int ln = lane_id(), w = wave_id();
  // dims ln and ln + 64 (a lane past D loads dim 0 and never stores)
  const int d0 = ln < D ? ln : 0, d1 = ln + 64 < D ? ln + 64 : 0;
  for (int row = vb; row < rows; row += nvb) {
    const int tok = row / L.Hq, hh = row - (row / L.Hq) * L.Hq;
    const int b = tok / S.Tr, tt = tok - (tok / S.Tr) * S.Tr;
    const int j = hh / G, g = hh - (hh / G) * G;
    const int m = tt * G + g, rg = m / L.rg_rows, mm = m - rg * L.rg_rows;
    const int nch = P->nch[b];
    const int it0 = P->item0[b] + (j * L.nrg + rg) * nch;
    const float* base = S.part + (size_t)it0 * L.rg_rows * (D + 1) + mm * (D + 1);
    const size_t stride = (size_t)L.rg_rows * (D + 1);
    float l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int c0 = w; c0 < nch; c0 += 16 * kWaves) {
      float pl[16], p0[16], p1[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int c = c0 + q * kWaves;
        const float* p = base + (size_t)(c < nch ? c : c0) * stride;
        pl[q] = MP::ld(&p[D]);
        p0[q] = MP::ld(&p[d0]);
        p1[q] = MP::ld(&p[d1]);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (c0 + q * kWaves < nch) { l += pl[q]; o0 += p0[q]; o1 += p1[q]; }
    }
    float* rw = red + w * (D + 1);
    if (ln < D) rw[ln] = o0;
    if (ln + 64 < D) rw[ln + 64] = o1;
    if (ln == 0) rw[D] = l;
    __syncthreads();
    if (w == 0) {
      l = red[D];
      o0 = ln < D ? red[ln] : 0.f;
      o1 = ln + 64 < D ? red[ln + 64] : 0.f;
      for (int q = 1; q < kWaves; ++q) {
        const float* rq = red + q * (D + 1);
        l += rq[D];
        if (ln < D) o0 += rq[ln];
        if (ln + 64 < D) o1 += rq[ln + 64];
      }
      const size_t at = (size_t)tok * L.Hq * D + (size_t)hh * D;
      const float v0 = o0 / l, v1 = o1 / l;
      if (ln < D) MP::st(&S.attn_o[at + ln], v0);
      if (ln + 64 < D) MP::st(&S.attn_o[at + ln + 64], v1);
      if (a3 != nullptr) {  // bf16 terms of the output projection's input
        const size_t plane = (size_t)S.T * L.Hq * D;
        unsigned h, m, lo;
        if (ln < D) {
          split3_bf16(v0, h, m, lo);
          a3[at + ln] = (unsigned short)h;
          a3[plane + at + ln] = (unsigned short)m;
          a3[2 * plane + at + ln] = (unsigned short)lo;
        }
        if (ln + 64 < D) {
          split3_bf16(v1, h, m, lo);
          a3[at + ln + 64] = (unsigned short)h;
          a3[plane + at + ln + 64] = (unsigned short)m;
          a3[2 * plane + at + ln + 64] = (unsigned short)lo;
        }
      }
    }
    __syncthreads();  // red is reused by the next row
  }
  if (win_out != nullptr && vb == 0) write_windows(L, S, win_out);
}

// ------------------------------------------------------------- Wo
// h[t][r] = x[t][r] + sum_c wo[r][c] * attn_o[t][c]
template <int DT, int NV>
__device__ void phase_wo(const LayerArgs& L, const StepArgs& S, const float* x, float* h, int vb,
                         int nvb) {
  constexpr int R = DenseRows<NV>::R;
  const int NI = L.Hq * L.D;
  const size_t rb = dense_row_bytes(DT, NI);
  const int gw = gwave(vb, nvb), nw = nvb * kWaves;
  for (int t0 = 0; t0 < S.T; t0 += NV) {
    const int nt = S.T - t0 < NV ? S.T - t0 : NV;
    const float* vin[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) vin[v] = S.attn_o + (size_t)(t0 + (v < nt ? v : 0)) * NI;
    const uint8_t* srow[R] = {};
    for (int blk = gw; blk * R < L.H; blk += nw) {
      const int r0 = blk * R;
      const uint8_t* wrow[R];
#pragma unroll
      for (int r = 0; r < R; ++r) wrow[r] = L.wo + (size_t)(r0 + r) * rb;
      float acc[R][NV];
      wave_gemv<DT, R, NV>(wrow, srow, NI, vin, nt, nullptr, acc);
      store_results<R, NV>(acc, nt, [&](int r, int v, float val) {
        const size_t o = (size_t)(t0 + v) * L.H + r0 + r;
        h[o] = x[o] + val;
      });
    }
  }
}

// ----------------------------------------------------------- router
// u = h * rstd * ffn_norm (written), logits[t][e] = rstd[t] * sum_c wr[e][c] h[t][c] g[c]
template <int DT, int NV>
__device__ void phase_router(const LayerArgs& L, const StepArgs& S, const float* h, const float* rs,
                             int vb, int nvb) {
  constexpr int R = DenseRows<NV>::R;
  // u, split over blocks by float4 groups
  const int n4 = S.T * L.H / 4;
  for (int i = vb * blockDim.x + threadIdx.x; i < n4; i += nvb * blockDim.x) {
    const int t = (i * 4) / L.H, c = i * 4 - ((i * 4) / L.H) * L.H;
    v4f a = *reinterpret_cast<const v4f*>(h + (size_t)t * L.H + c);
    v4f g = *reinterpret_cast<const v4f*>(L.ffn_norm + c);
    const float r = rs[t];
    *reinterpret_cast<v4f*>(S.u + (size_t)t * L.H + c) =
        v4f{a.x * r * g.x, a.y * r * g.y, a.z * r * g.z, a.w * r * g.w};
  }
  const size_t rb = dense_row_bytes(DT, L.H);
  const int gw = gwave(vb, nvb), nw = nvb * kWaves;
  for (int t0 = 0; t0 < S.T; t0 += NV) {
    const int nt = S.T - t0 < NV ? S.T - t0 : NV;
    const float* vin[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) vin[v] = h + (size_t)(t0 + (v < nt ? v : 0)) * L.H;
    const uint8_t* srow[R] = {};
    for (int blk = gw; blk * R < L.E; blk += nw) {
      const int r0 = blk * R;
      const uint8_t* wrow[R];
#pragma unroll
      for (int r = 0; r < R; ++r) wrow[r] = L.wr + (size_t)(r0 + r < L.E ? r0 + r : r0) * rb;
      float acc[R][NV];
      wave_gemv<DT, R, NV>(wrow, srow, L.H, vin, nt, L.ffn_norm, acc);
      store_results<R, NV>(acc, nt, [&](int r, int v, float val) {
        if (r0 + r < L.E) S.logits[(size_t)(t0 + v) * L.E + r0 + r] = val * rs[t0 + v];
      });
    }
  }
}

// ------------------------------------------------------------- top-k
// One wave per token: k rounds of a wave-wide arg-max under the order
// (logit descending, expert index ascending); weights = softmax over the
// selected logits.
__device__ inline bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ void phase_topk(const LayerArgs& L, const StepArgs& S, int* topk_out, int vb, int nvb);

// ------------------------------------------------------ expert union
// Distinct selected experts in ascending order, and per expert the slots
// (t * K + j) routed to it in ascending order.  Built identically by every
// workgroup from idx.

// sidx: LDS for T * K + 16 ints followed by kMaxExperts + 1 64-bit words,
// 8-byte aligned.  A slot's place among its expert's slots is the number of
// earlier slots of that expert.  When no token lists an expert twice (the
// router's selections never do) that is the number of earlier tokens that
// selected it: a popcount of the expert's token mask.  Otherwise the earlier
// slots are counted one by one.
__device__ inline void build_union(const int* idx, int T, int K, int E, Union* U, int* sidx) {
  const int S = T * K;
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(sidx + kMaxTok * kMaxTopK + 16);
  unsigned long long* repeat = mask + kMaxExperts;  // nonzero: some token repeats an expert
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    U->start[e] = 0;
    mask[e] = 0ull;
  }
  if (threadIdx.x == 0) *repeat = 0ull;
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = idx[s];
    sidx[s] = e;
    if (e >= 0 && e < E) {
      atomicAdd(&U->start[e], 1);
      const unsigned long long bit = 1ull << (s / K);
      if (atomicOr(&mask[e], bit) & bit) atomicOr(repeat, 1ull);
    }
  }
  __syncthreads();
  if (wave_id() == 0) {
    const int ln = lane_id();
    int c[4], nz = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = ln * 4 + i;
      c[i] = e < E ? U->start[e] : 0;
      nz += c[i] > 0;
      tot += c[i];
    }
    // exclusive prefix sums over the lanes and wave totals, one ballot per
    // bit (nz <= 4, tot <= S <= 1024): no cross-lane data movement
    const unsigned long long below = (1ull << ln) - 1ull;
    int pnz = 0, ptot = 0, inz = 0, itot = 0;
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const unsigned long long m = __ballot((nz >> b) & 1);
      pnz += __popcll(m & below) << b;
      inz += __popcll(m) << b;
    }
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const unsigned long long m = __ballot((tot >> b) & 1);
      ptot += __popcll(m & below) << b;
      itot += __popcll(m) << b;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = ln * 4 + i;
      if (e < E) {
        if (c[i] > 0) {
          U->list[pnz] = e;
          U->off[pnz] = ptot;
          ++pnz;
        }
        U->start[e] = ptot;
        ptot += c[i];
      }
    }
    if (ln == 0) { U->n = inz; U->off[inz] = itot; }
  }
  __syncthreads();
  const bool repeats = *repeat != 0ull;
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = sidx[s];
    if (e < 0 || e >= E) continue;
    int rank = 0;
    if (!repeats) {
      rank = __popcll(mask[e] & ((1ull << (s / K)) - 1ull));
    } else {
      for (int q = 0; q < s; ++q) rank += sidx[q] == e ? 1 : 0;
    }
    U->slots[U->start[e] + rank] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace msk
