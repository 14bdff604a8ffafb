// Split-KV no-max attention partials on the matrix cores, for the verify
// step's many query rows per kv head.
//
// One work item is (request b, kv head j, row group, chunk of cache
// positions), as for the vector path, but a row group holds up to 64 query
// rows (rows m = t * G + g in token order) and each wave owns 16 of them.
// Per 64-position tile:
//   scores  S^T[pos][m] = sum_d K[pos][d] * qhat[m][d]        (MFMA, k = d)
//   weights e = exp(s - c) on the row's window, else 0         (VALU)
//   output  O^T[d][m]  += sum_pos V^T[d][pos] * e[pos][m]      (MFMA, k = pos)
// with v_mfma_f32_16x16x32_bf16.  Cached K and V are bf16 or e4m3, both
// exact in bf16.  qhat is fp32 and enters as a sum of two bf16 terms (hi =
// rne(x), lo = rne(x - hi)), so a score is exact to about 2^-16 relative of
// its terms; the weights e enter rounded to bf16 once (2^-9 relative each,
// averaged over many positions), and the normaliser sums those same rounded
// weights.  Sums stay in fp32.  The score accumulator's layout (lane
// = column m, four consecutive positions per lane) is used directly as the
// weight operand of the output product by numbering that product's k index
// so that a lane's eight k values are its own eight positions of the 32:
// no shuffle and no LDS round trip for the weights.
//
// The tile is fetched into registers one tile ahead (nontemporal 16-B
// loads) and converted once per workgroup into two bf16 LDS tiles: K
// row-major [pos][d] and V transposed [d][pos], both padded against bank
// conflicts.  Positions outside the visible range are zero in both tiles, so
// masked weights never meet a NaN.  The step's own positions (>= kv_len)
// are rebuilt from the QKV output as stored (QK-norm on k, cast to the cache
// format), and the row-group-0 item writes them into the cache.
//
// Cite: no-max softmax with a fixed score bound (brifing.si page, "Removing
// Attention Bottlenecks"), split-KV partials combined by plain sums.
#pragma once
#include "phases.h"

namespace msk {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int KDT, int D, int NW, int NPH = 1>
struct MfmaGeom {
  static constexpr int ES = KV<KDT>::ES;
  static constexpr int RB = D * ES;        // cache row bytes
  static constexpr int CPR = RB / 16;      // 16-B chunks per cache row
  static constexpr int EPC = 16 / ES;      // elements per chunk
  static constexpr int NT = NW * 64;       // threads per workgroup
  static constexpr int NKC = 64 * CPR;     // K chunks per tile
  static constexpr int KPT = (NKC + NT - 1) / NT;
  static constexpr int NVP = 32 * CPR;     // V (position pair pp = q % 32, chunk q / 32) tasks
  static constexpr int VPT = (NVP + NT - 1) / NT;
  static constexpr int KBS = D * 2 + 16;   // bf16 K tile row stride, bytes
  // bf16 V^T tile row stride, bytes: a V^T store instruction writes one row
  // (32 position pairs, 128 B) per half-wave, the halves EPC rows apart; the
  // stride puts them on opposite halves of the 64 banks (e4m3: 16 rows x 136
  // B; bf16: 8 rows x 144 B), and keeps the 16 rows of an operand read on
  // distinct banks
  static constexpr int VTS = KDT == kE4M3 ? 64 * 2 + 8 : 64 * 2 + 16;
  static constexpr int DS = D / 32;        // k steps of the score product
  static constexpr int NDT = D / 16;       // d tiles of the output product
  static constexpr int LDS_KB = 64 * KBS;
  static constexpr int LDS_VT = D * VTS;
  static constexpr int LDS = LDS_KB + LDS_VT + kMaxTok * 4;
  static constexpr int ROWS = 16 * NW / NPH;  // query rows per item
  static constexpr int NPT = 4 / NPH;      // 16-position tiles per wave
  static constexpr int NKS = 2 / NPH;      // 32-position k steps per wave
};

__device__ __forceinline__ unsigned pack_bf16_exact(float a, float b) {
  // a and b are exact in bf16: keep their upper halves
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// One 16-B chunk of cache-format data -> its EPC values as bf16, two per
// word (exact: every e4m3 value is a bf16 value; the convert's scale of 1
// leaves the values unchanged).
template <int KDT>
__device__ __forceinline__ void chunk_to_bf16(const v4u& w, unsigned* o) {
  if constexpr (KDT == kBF16) {
    o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
  } else {
    const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __builtin_bit_cast(unsigned,
                                    __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, false));
      o[2 * i + 1] = __builtin_bit_cast(unsigned,
                                        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, true));
    }
  }
}

// x = hi + lo (+ a residual of at most 2^-16 |x|), both bf16 bits.
__device__ __forceinline__ void split_bf16(float x, unsigned& hi, unsigned& lo) {
  hi = f2bf16(x);
  lo = f2bf16(x - bf16_lo(hi));
}

// The same for a pair, packed: hi = (hi_a | hi_b << 16), lo likewise.
__device__ __forceinline__ void split2_bf16(float a, float b, unsigned& hi, unsigned& lo) {
  hi = cvt_pk_bf16(a, b);
  lo = cvt_pk_bf16(a - bf16_lo(hi), b - bf16_hi(hi));
}

// NPH = 2: the waves pair up on the same 16 rows, each taking half of every
// tile's positions; the pair's sums are added at the end of the item.
template <int KDT, int D, int NW, int NPH>
__device__ void attn_item_mfma(const LayerArgs& L, const StepArgs& S, const AttnPlan* P, int item,
                               uint8_t* wl) {
  using Gm = MfmaGeom<KDT, D, NW, NPH>;
  constexpr int RB = Gm::RB, CPR = Gm::CPR, EPC = Gm::EPC, NT = Gm::NT;
  constexpr int KPT = Gm::KPT, VPT = Gm::VPT, KBS = Gm::KBS, VTS = Gm::VTS;
  constexpr int DS = Gm::DS, NDT = Gm::NDT, ROWS = Gm::ROWS, NPT = Gm::NPT, NKS = Gm::NKS;
  uint8_t* kb = wl;
  uint8_t* vt = wl + Gm::LDS_KB;
  float* rk = reinterpret_cast<float*>(vt + Gm::LDS_VT);

  const int tid = threadIdx.x, ln = lane_id(), wv = wave_id();
  const int rt = wv / NPH, ph = wv - (wv / NPH) * NPH;  // row tile, position half
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
  const int m0 = rg * ROWS;
  const int NQ = L.Hq * L.D, NK = L.Hkv * L.D, NR = NQ + 2 * NK;
  const size_t head_off = ((size_t)b * L.Hkv + j) * (size_t)L.cap;  // in rows
  uint8_t* kc = L.kc + head_off * RB;
  uint8_t* vc = L.vc + head_off * RB;
  const bool writer = (rg == 0);

  // this lane's query row (lanes l, l^16, l^32, l^48 share it) and its window
  const int mr = m0 + 16 * rt + (ln & 15);
  const bool live = mr < M;
  const int t_me = live ? mr / G : 0;
  const int g_me = live ? mr - t_me * G : 0;
  const int p_me = Lb + t_me;
  const int w_lo = live ? (L.window > 0 ? (p_me - L.window + 1 > 0 ? p_me - L.window + 1 : 0) : 0)
                        : 1;
  const int w_hi = live ? p_me : 0;
  // the group's earliest window start: its first row's token
  const int t_first = m0 / G;
  const int lo_min = L.window > 0 ? (Lb + t_first - L.window + 1 > 0 ? Lb + t_first - L.window + 1 : 0)
                                  : 0;

  // qhat as the B operand of the score product: lane holds row m, d = 32 ks + 8 (ln >> 4) + e
  bf16x8 qh[DS], ql[DS];
  const v2f gq2 = gain_pair(L.q_norm, D), gk2 = gain_pair(L.k_norm, D);
  {
    const float* q = S.qkv + (size_t)(b * S.Tr + t_me) * NR + (size_t)(j * G + g_me) * D;
    float qf[DS][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const int d0 = 32 * ks + 8 * (ln >> 4);
      const v4f a = live ? *reinterpret_cast<const v4f*>(q + d0) : v4f{0.f, 0.f, 0.f, 0.f};
      const v4f bq = live ? *reinterpret_cast<const v4f*>(q + d0 + 4) : v4f{0.f, 0.f, 0.f, 0.f};
      qf[ks][0] = a.x; qf[ks][1] = a.y; qf[ks][2] = a.z; qf[ks][3] = a.w;
      qf[ks][4] = bq.x; qf[ks][5] = bq.y; qf[ks][6] = bq.z; qf[ks][7] = bq.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += qf[ks][e] * qf[ks][e];
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    // scores come out in log2 units (times log2(e)), so the weights are
    // exp2(s - c log2(e)) = exp(s - c) up to rounding
    const float rr = 1.0f / sqrtf(ss / (float)D + L.eps) * L.qscale * 1.44269504088896341f;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      unsigned h[4], l[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int d = 32 * ks + 8 * (ln >> 4) + e;
        split2_bf16(qf[ks][e] * rr * L.q_norm[d], qf[ks][e + 1] * rr * L.q_norm[d + 1], h[e / 2],
                    l[e / 2]);
      }
      qh[ks] = as_bf16x8(v4u{h[0], h[1], h[2], h[3]});
      ql[ks] = as_bf16x8(v4u{l[0], l[1], l[2], l[3]});
    }
  }
  // tiles inside every live row's window of this wave need no mask
  int lo_all = live ? w_lo : 0, hi_all = live ? w_hi : 0x7fffffff;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    lo_all = max(lo_all, __shfl_xor(lo_all, o));
    hi_all = min(hi_all, __shfl_xor(hi_all, o));
  }
  const float shift2 = layer_shift(L.shift, gq2, gk2, D) * 1.44269504088896341f;
  // 1/rms of the step's new keys that fall in this chunk
  const int tn0 = p0 - Lb > 0 ? p0 - Lb : 0;
  const int tn1 = p1 - Lb < S.Tr ? p1 - Lb : S.Tr;
  for (int t = tn0 + wv; t < tn1; t += NW) {
    const float* k = S.qkv + (size_t)(b * S.Tr + t) * NR + NQ + (size_t)j * D;
    float ss = 0.f;
    for (int d = ln; d < D; d += 64) ss += k[d] * k[d];
    ss = wave_sum(ss);
    if (ln == 0) rk[t] = 1.0f / sqrtf(ss / (float)D + L.eps);
  }

  // cached rows of a tile into registers; rows outside [lo_min, Lb) are 0
  v4u kr[KPT], vr[VPT][2];
  auto fetch = [&](int pb) {
    const int vlo = pb > lo_min ? pb : lo_min;
    const int vhi = p1 < Lb ? p1 : Lb;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int q = tid + u * NT;
      const int pos = pb + q / CPR;
      kr[u] = v4u{0u, 0u, 0u, 0u};
      if (q < Gm::NKC && pos >= vlo && pos < vhi)
        kr[u] = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(kc + (size_t)pos * RB + (q % CPR) * 16));
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int q = tid + u * NT;
      const int pos = pb + 2 * (q & 31);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        vr[u][h] = v4u{0u, 0u, 0u, 0u};
        if (q < Gm::NVP && pos + h >= vlo && pos + h < vhi)
          vr[u][h] = __builtin_nontemporal_load(
              reinterpret_cast<const v4u*>(vc + (size_t)(pos + h) * RB + (q >> 5) * 16));
      }
    }
  };
  // chunk cc of the step's own row at position pos, as stored in the cache
  auto new_chunk = [&](int pos, int cc, bool value) -> v4u {
    const int t = pos - Lb;
    const int d0 = cc * EPC;
    const float* kq = S.qkv + (size_t)(b * S.Tr + t) * NR + NQ + (size_t)j * D + d0;
    float f[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      f[e] = e < EPC ? (value ? kq[NK + e] : kq[e] * rk[t] * L.k_norm[d0 + e]) : 0.f;
    const v4u enc = encode16<KDT>(f);
    if (writer) *reinterpret_cast<v4u*>((value ? vc : kc) + (size_t)pos * RB + cc * 16) = enc;
    return enc;
  };

  f32x4 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;

  fetch(p0);
  __syncthreads();  // rk is written
  for (int pb = p0; pb < p1; pb += 64) {
    lds_barrier();  // the previous tile's readers are done
    // K -> kb[pos][d] (bf16)
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int q = tid + u * NT;
      if (q < Gm::NKC) {
        const int row = q / CPR, cc = q % CPR;
        unsigned o[EPC / 2];
        chunk_to_bf16<KDT>(kr[u], o);
        uint8_t* dst = kb + row * KBS + cc * EPC * 2;
#pragma unroll
        for (int w = 0; w < EPC / 2; w += 4)
          *reinterpret_cast<v4u*>(dst + 4 * w) = v4u{o[w], o[w + 1], o[w + 2], o[w + 3]};
      }
    }
    // V -> vt[d][pos] (bf16), two positions per 32-bit store
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int q = tid + u * NT;
      if (q < Gm::NVP) {
        const int pp = q & 31, cc = q >> 5;
        unsigned o[2][EPC / 2];
#pragma unroll
        for (int h = 0; h < 2; ++h) chunk_to_bf16<KDT>(vr[u][h], o[h]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          // element e of positions 2pp (low half) and 2pp + 1 (high half)
          const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
          *reinterpret_cast<unsigned*>(vt + (cc * EPC + e) * VTS + 4 * pp) =
              __builtin_amdgcn_perm(o[1][e >> 1], o[0][e >> 1], sel);
        }
      }
    }
    if (pb + 64 < p1) fetch(pb + 64);
    // the step's own rows in this tile (zero above): rebuilt, stored, converted
    const int n0 = pb > Lb ? pb : Lb;
    const int n1 = pb + 64 < p1 ? pb + 64 : p1;
    if (n0 < n1) {
      lds_barrier();
      const int nn = (n1 - n0) * CPR;
      for (int q = tid; q < 2 * nn; q += NT) {
        const bool value = q >= nn;
        const int qq = value ? q - nn : q;
        const int pos = n0 + qq / CPR, cc = qq % CPR;
        unsigned o[EPC / 2];
        chunk_to_bf16<KDT>(new_chunk(pos, cc, value), o);
        const int row = pos - pb;
        if (!value) {
          uint8_t* dst = kb + row * KBS + cc * EPC * 2;
#pragma unroll
          for (int w = 0; w < EPC / 2; w += 4)
            *reinterpret_cast<v4u*>(dst + 4 * w) = v4u{o[w], o[w + 1], o[w + 2], o[w + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            *reinterpret_cast<unsigned short*>(vt + (cc * EPC + e) * VTS + 2 * row) =
                (unsigned short)((e & 1) ? o[e >> 1] >> 16 : o[e >> 1] & 0xffffu);
        }
      }
    }
    lds_barrier();

    if (m0 + 16 * rt >= M) continue;  // a wave without live rows only fetches
    // scores of this wave's 16 rows against its NPT 16-position tiles
    f32x4 sacc[NPT];
#pragma unroll
    for (int pq = 0; pq < NPT; ++pq) {
      const int pt = ph * NPT + pq;
      sacc[pq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const v4u*>(
            kb + (16 * pt + (ln & 15)) * KBS + (32 * ks + 8 * (ln >> 4)) * 2));
        sacc[pq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[ks], sacc[pq], 0, 0, 0);
        sacc[pq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[ks], sacc[pq], 0, 0, 0);
      }
    }
    // weights: lane holds row m, positions 16 pt + 4 (ln >> 4) + i
    const bool open = pb >= lo_all && pb + 63 <= hi_all && pb + 64 <= p1;
    unsigned wh[NKS][4];
#pragma unroll
    for (int pq = 0; pq < NPT; ++pq) {
      const int pt = ph * NPT + pq;
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = __builtin_amdgcn_exp2f(sacc[pq][i] - shift2);
        if (!open) {
          const int pos = pb + 16 * pt + 4 * (ln >> 4) + i;
          e[i] = (pos >= w_lo && pos <= w_hi && pos < p1) ? e[i] : 0.f;
        }
      }
      // k index 8 (ln >> 4) + 4 (pt & 1) + i of k step pt / 2; the sum of
      // weights takes the same rounded values the product does
      const unsigned h0 = cvt_pk_bf16(e[0], e[1]), h1 = cvt_pk_bf16(e[2], e[3]);
      wh[pq >> 1][2 * (pt & 1)] = h0;
      wh[pq >> 1][2 * (pt & 1) + 1] = h1;
      lsum += (bf16_lo(h0) + bf16_hi(h0)) + (bf16_lo(h1) + bf16_hi(h1));
    }
    // O^T[d][m] += V^T[d][pos] e[pos][m]; the A operand's k numbering matches
    // the weights': positions 32 ks + 4 (ln >> 4) + {0..3} and + 16 + {0..3}
#pragma unroll
    for (int kq = 0; kq < NKS; ++kq) {
      const int ks = ph * NKS + kq;
      const bf16x8 bh = as_bf16x8(v4u{wh[kq][0], wh[kq][1], wh[kq][2], wh[kq][3]});
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint8_t* src = vt + (16 * dt + (ln & 15)) * VTS + (32 * ks + 4 * (ln >> 4)) * 2;
        const v2u x0 = *reinterpret_cast<const v2u*>(src);
        const v2u x1 = *reinterpret_cast<const v2u*>(src + 32);
        const bf16x8 a = as_bf16x8(v4u{x0.x, x0.y, x1.x, x1.y});
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, oacc[dt], 0, 0, 0);
      }
    }
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if constexpr (NPH == 2) {
    // the second half's sums go through LDS (the K tile is free by now) to
    // the first, which adds them in that order
    float* xs = reinterpret_cast<float*>(kb) + rt * (NDT * 4 + 1) * 64;
    lds_barrier();
    if (ph == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[(dt * 4 + i) * 64 + ln] = oacc[dt][i];
      xs[NDT * 4 * 64 + ln] = lsum;
    }
    lds_barrier();
    if (ph == 1) return;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][i] += xs[(dt * 4 + i) * 64 + ln];
    lsum += xs[NDT * 4 * 64 + ln];
  }
  // partial sums of this wave's rows: part[item][row][d], part[item][row][D] = l
  if (m0 + 16 * rt >= M) return;
  float* part = S.part + ((size_t)item * ROWS + 16 * rt + (ln & 15)) * (D + 1);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[16 * dt + 4 * (ln >> 4) + i] = oacc[dt][i];
  if (ln < 16) part[D] = lsum;
}

// ------------------------------------------- e4m3 caches, head_dim 128
// The cache bytes are matrix-core operands as they are: the score product
// runs on v_mfma_scale_f32_16x16x128_f8f6f4 with K straight from a raw tile
// (A: 16 positions x 128 dims, e4m3) and qhat as three e4m3 terms (B: 128
// dims x 16 rows).  Each row of qhat is first multiplied by a power of two
// that puts its largest magnitude in [128, 256); the terms are t1 = rne(x),
// t2 = rne(x - t1), t3 = rne(x - t1 - t2), so a score carries about 2^-12
// of its terms' magnitude (the fp8 subnormal step bounds the last term), and
// the power of two comes back out with the exp2 argument.  The output
// product stays on bf16 (weights rounded once, as in attn_item_mfma), with
// its V^T operand read from the raw V tile by the gfx950 transpose load
// (ds_read_b64_tr_b8) and converted in registers: no converted copy of V.
//
// Raw tiles (64 positions x 128 B of K, then of V) land in an NSLOT-slot LDS
// ring through direct global->LDS loads, NSLOT - 1 tiles ahead, each issued
// as soon as the slot it overwrites is released, so no register holds a tile
// in flight.  A tile row's 16-B chunk c sits at chunk c ^ ((row >> 1) & 7) of
// the row: the 16 rows of a score operand read then hit 16 distinct bank
// groups, and so do the 16 lanes of a transpose load.
//
// Item shapes (waves per 16-row tile NPH): four row tiles (NPH 1), or up to
// two with wave pairs splitting each tile's positions (NPH 2); four waves,
// three workgroups per CU.  One tile ahead per workgroup (NSLOT 2) measures
// as fast as two or three on this part: with 48 KB in flight per CU the
// cache stream is as close to its ceiling as deeper rings bring it.
template <int NPH>
struct F8Geom {
  static constexpr int D = 128, NW = 4;
  static constexpr int RAW = 64 * D;                 // one raw K or V tile, bytes
  static constexpr int SLOT = 2 * RAW;               // K then V
  static constexpr int NSLOT = 2;
  static constexpr int LDS_RING = NSLOT * SLOT;
  static constexpr int LDS = 128 + LDS_RING + kMaxTok * 4;  // ring aligned to 128 B
  static constexpr int ROWS = 16 * NW / NPH, NPT = 4 / NPH, NKS = 2 / NPH, NDT = D / 16;
  static_assert(NSLOT >= 2 && NSLOT <= 4, "vmcnt waits cover up to two tiles ahead");
};

__device__ __forceinline__ int f8_slot(int row, int c) { return row * 8 + (c ^ ((row >> 1) & 7)); }

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Two e4m3 bytes of w (bytes 0, 1, or 2, 3 with HI) as a bf16 pair (exact).
template <bool HI>
__device__ __forceinline__ unsigned e4m3x2_bf16(unsigned w) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// The eight transpose reads of one k-step's V^T operands (one per 16-dim
// tile dt, at LDS byte (base ^ (dt << 4)) + OFF), issued together and waited
// for in the same asm block.  Written with the builtin, each read made the compiler
// wait for every global->LDS load in flight first (it cannot tell the slot
// being read from the slots being filled), which drained the tile prefetch
// once per tile.  The reads here only touch a slot whose loads the loop has
// already waited for.
template <int OFF>
__device__ __forceinline__ void v_tr_reads(unsigned base, v2i (&r)[8]) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  // the seven other addresses are formed inside the block, so that they are
  // not kept live across the tile loop
  unsigned t[7];
  asm volatile(
      "v_xor_b32 %8, 16, %15\n\t"
      "v_xor_b32 %9, 32, %15\n\t"
      "v_xor_b32 %10, 48, %15\n\t"
      "v_xor_b32 %11, 64, %15\n\t"
      "v_xor_b32 %12, 0x50, %15\n\t"
      "v_xor_b32 %13, 0x60, %15\n\t"
      "v_xor_b32 %14, 0x70, %15\n\t"
      "ds_read_b64_tr_b8 %0, %15 offset:%16\n\t"
      "ds_read_b64_tr_b8 %1, %8 offset:%16\n\t"
      "ds_read_b64_tr_b8 %2, %9 offset:%16\n\t"
      "ds_read_b64_tr_b8 %3, %10 offset:%16\n\t"
      "ds_read_b64_tr_b8 %4, %11 offset:%16\n\t"
      "ds_read_b64_tr_b8 %5, %12 offset:%16\n\t"
      "ds_read_b64_tr_b8 %6, %13 offset:%16\n\t"
      "ds_read_b64_tr_b8 %7, %14 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]),
        "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6])
      : "v"(base), "i"(OFF)
      : "memory");
}

// A ring slot index as a type (the tile loop is unrolled over the slots).
template <int N> struct F8Slot { static constexpr int v = N; };

template <int NPH>
__device__ void attn_item_f8(const LayerArgs& L, const StepArgs& S, const AttnPlan* P, int item,
                             uint8_t* wl) {
  using Gm = F8Geom<NPH>;
  constexpr int D = Gm::D, NW = Gm::NW, RB = D, CPR = D / 16, EPC = 16;
  constexpr int NDT = Gm::NDT, ROWS = Gm::ROWS, NPT = Gm::NPT, NKS = Gm::NKS;
  uint8_t* ring = wl + ((128 - ((unsigned)(size_t)(__attribute__((address_space(3))) uint8_t*)wl & 127)) & 127);
  float* rk = reinterpret_cast<float*>(ring + Gm::LDS_RING);

  const int tid = threadIdx.x, ln = lane_id(), wv = wave_id();
  const int rt = wv / NPH, ph = wv - (wv / NPH) * NPH;
  int b = 0;
  while (b + 1 < S.n_req && P->item0[b + 1] <= item) ++b;
  const int nch = P->nch[b];
  int rem = item - P->item0[b];
  const int j = rem / (L.nrg * nch);
  rem -= j * L.nrg * nch;
  const int rg = rem / nch;
  const int c = rem - rg * nch;
  // the head's 64-position tiles in [base, pe) go round-robin to its nch
  // items: item c takes tiles c, c + nch, ...  The items of a head then
  // stream neighbouring tiles at any one time, rather than nch regions far
  // apart.
  const int pe = P->end[b];
  const int ts = 64 * nch;               // positions between this item's tiles
  const int pb0 = P->base[b] + 64 * c;   // its first tile
  const int Lb = S.kv_len[b];
  const int G = L.Hq / L.Hkv;
  const int M = G * S.Tr;
  const int m0 = rg * ROWS;
  const int NQ = L.Hq * L.D, NK = L.Hkv * L.D, NR = NQ + 2 * NK;
  const size_t head_off = ((size_t)b * L.Hkv + j) * (size_t)L.cap;
  uint8_t* kc = L.kc + head_off * RB;
  uint8_t* vc = L.vc + head_off * RB;
  const bool writer = (rg == 0);

  const int mr = m0 + 16 * rt + (ln & 15);
  const bool live = mr < M;
  const int t_me = live ? mr / G : 0;
  const int g_me = live ? mr - t_me * G : 0;
  const int p_me = Lb + t_me;
  const int w_lo = live ? (L.window > 0 ? (p_me - L.window + 1 > 0 ? p_me - L.window + 1 : 0) : 0)
                        : 1;
  const int w_hi = live ? p_me : 0;
  const int t_first = m0 / G;
  const int lo_min = L.window > 0 ? (Lb + t_first - L.window + 1 > 0 ? Lb + t_first - L.window + 1 : 0)
                                  : 0;

  // raw tile at positions [pb, pb + 64) into a ring slot.  Every lane
  // loads, so each wave has exactly 4 loads per tile in flight; a row
  // outside [vlo, vhi) fetches the head's row 0 instead (the step's own rows
  // are rebuilt below, the other ones are masked)
  auto issue = [&](int pb, uint8_t* slot) {
    const int vlo = pb > lo_min ? pb : lo_min;
    const int vhi = Lb;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int blk = 2 * wv + u;               // 64-granule block of the tile
      const int row = 8 * blk + (ln >> 3);
      const int pos = pb + row;
      const int cg = (ln & 7) ^ ((row >> 1) & 7);  // global chunk that goes to this slot
      const size_t off = (size_t)(pos >= vlo && pos < vhi ? pos : 0) * RB + cg * 16;
      __builtin_amdgcn_global_load_lds(kc + off, slot + blk * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vc + off, slot + Gm::RAW + blk * 1024, 16, 0, 0);
    }
  };
  // this lane's query values and q-norm gains are loaded before the first
  // tiles are issued: issued after them, they would wait for the tiles on
  // the in-order load counter (a lane past M reads row 0 and zeroes it)
  const int d0 = 32 * (ln >> 4);
  v4f qa[8], qn[8];
  const v2f gq2 = gain_pair(L.q_norm, D), gk2 = gain_pair(L.k_norm, D);
  {
    const float* q = S.qkv + (size_t)(b * S.Tr + t_me) * NR + (size_t)(j * G + g_me) * D;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qa[e] = *reinterpret_cast<const v4f*>(q + d0 + 4 * e);
      qn[e] = *reinterpret_cast<const v4f*>(L.q_norm + d0 + 4 * e);
    }
  }
#pragma unroll
  for (int k = 0; k + 1 < Gm::NSLOT; ++k)
    if (pb0 + ts * k < pe) issue(pb0 + ts * k, ring + k * Gm::SLOT);

  // qhat as three e4m3 terms, lane: row m = ln & 15, dims 32 (ln >> 4) + e
  v8i qt[3];
  float qinv;
  {
    float qf[32];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 32; e += 4) {
      const v4f a = live ? qa[e >> 2] : v4f{0.f, 0.f, 0.f, 0.f};
      qf[e] = a.x; qf[e + 1] = a.y; qf[e + 2] = a.z; qf[e + 3] = a.w;
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float rr = 1.0f / sqrtf(ss / (float)D + L.eps) * L.qscale * 1.44269504088896341f;
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      qf[e] *= rr * qn[e >> 2][e & 3];
      mx = fmaxf(mx, fabsf(qf[e]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    int ex = 0;
    frexpf(mx, &ex);  // mx < 2^ex
    const float up = mx > 0.f ? ldexpf(1.f, 8 - ex) : 1.f;
    qinv = mx > 0.f ? ldexpf(1.f, ex - 8) : 1.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) qf[e] *= up;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
#pragma unroll
      for (int w4 = 0; w4 < 8; ++w4) {
        const float* x = qf + 4 * w4;
        const unsigned lo = f2e4m3x2(x[0], x[1]), hi = f2e4m3x2(x[2], x[3]);
        qt[k][w4] = (int)(lo | (hi << 16));
        float back[4];
        e4m3x4(lo | (hi << 16), back);
        qf[4 * w4] -= back[0]; qf[4 * w4 + 1] -= back[1];
        qf[4 * w4 + 2] -= back[2]; qf[4 * w4 + 3] -= back[3];
      }
    }
  }
  int lo_all = live ? w_lo : 0, hi_all = live ? w_hi : 0x7fffffff;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    lo_all = max(lo_all, __shfl_xor(lo_all, o));
    hi_all = min(hi_all, __shfl_xor(hi_all, o));
  }
  const float shift2 = layer_shift(L.shift, gq2, gk2, D) * 1.44269504088896341f;
  for (int t = wv; t < S.Tr; t += NW) {
    const float* k = S.qkv + (size_t)(b * S.Tr + t) * NR + NQ + (size_t)j * D;
    float ss = 0.f;
    for (int d = ln; d < D; d += 64) ss += k[d] * k[d];
    ss = wave_sum(ss);
    if (ln == 0) rk[t] = 1.0f / sqrtf(ss / (float)D + L.eps);
  }
  auto new_chunk = [&](int pos, int cc, bool value) -> v4u {
    const int t = pos - Lb;
    const int d0 = cc * EPC;
    const float* kq = S.qkv + (size_t)(b * S.Tr + t) * NR + NQ + (size_t)j * D + d0;
    float f[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) f[e] = value ? kq[NK + e] : kq[e] * rk[t] * L.k_norm[d0 + e];
    const v4u enc = encode16<kE4M3>(f);
    if (writer) *reinterpret_cast<v4u*>((value ? vc : kc) + (size_t)pos * RB + cc * 16) = enc;
    return enc;
  };

  f32x4 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // row sums of the rounded weights, on the matrix cores: an all-ones V^T
  // operand (every entry of the product is the sum of its row's weights)
  f32x4 sacc_l = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = as_bf16x8(v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  __syncthreads();  // rk is written

  // Per-lane LDS offsets within a ring slot, fixed for the item (a slot's
  // own offset is a constant of each unrolled tile below).  Score operand:
  // row 16 pt + r16 of the K tile, chunks 2 (ln >> 4) and + 1; the chunk
  // swizzle depends only on r16.  Transpose reads: slot byte
  // vr + ((dt ^ sw) << 4) = (vr | sw << 4) ^ (dt << 4), as bits 4..6 of vr
  // are zero; sw does not depend on the k-step, whose rows sit 4096 B apart.
  const int r16 = ln & 15, swr = (r16 >> 1) & 7;
  const unsigned ring_lds = (unsigned)(size_t)(__attribute__((address_space(3))) uint8_t*)ring;
  const int ka0 = (r16 * 8 + ((2 * (ln >> 4)) ^ swr)) * 16 + ph * NPT * 2048;
  const int ka1 = (r16 * 8 + ((2 * (ln >> 4) + 1) ^ swr)) * 16 + ph * NPT * 2048;
  unsigned tra;  // LDS address of dim tile 0's transpose read; tile dt: tra ^ (dt << 4)
  {
    const int q = ln & 15, m = q >> 1;
    const int vrow = 32 * ph * NKS + 4 * (ln >> 4) + (m & 3) + 16 * (m >> 2);
    const unsigned vr = Gm::RAW + vrow * 128 + 8 * (q & 1);  // within the slot
    const unsigned sw = (unsigned)((vrow >> 1) & 7);
    tra = ring_lds + (vr | (sw << 4));  // the ring is 128-B aligned: bits 4..6 are sw
  }
  // the rows' common window, uniform over the wave, in scalar registers
  const int lo_s = __builtin_amdgcn_readfirstlane(lo_all);
  const int hi_s = __builtin_amdgcn_readfirstlane(hi_all);
  const bool dead = m0 + 16 * rt >= M;

  // One tile at positions [pb, pb + 64) in ring slot SC::v.
  auto tile = [&](auto SC, int pb) {
    constexpr int SL = decltype(SC)::v;
    uint8_t* slot = ring + SL * Gm::SLOT;
    // this wave's loads of the tile have landed (the later tiles' 4 loads
    // each may still be in flight: those issued so far, up to NSLOT - 2
    // tiles ahead), then every wave's; the slot about to be refilled is free
    {
      const int later = (pe - pb - 1) / ts;  // this item's tiles after this one
      const int ahead = later < Gm::NSLOT - 2 ? later : Gm::NSLOT - 2;
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0F78);       // vmcnt(8)
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
      else __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
    }
    lds_barrier();
    {
      const int ahead = pb + ts * (Gm::NSLOT - 1);
      if (ahead < pe) issue(ahead, ring + ((SL + Gm::NSLOT - 1) % Gm::NSLOT) * Gm::SLOT);
    }
    // V rows outside the loaded range become zeros (their loads fetched the
    // head's row 0, and a masked weight times a NaN would still be NaN); the
    // step's own rows take their K and V as cache bytes
    {
      const int vlo = pb > lo_min ? pb : lo_min;
      const int vhi = Lb;
      const int n0 = pb > Lb ? pb : Lb;
      const int n1 = pb + 64 < pe ? pb + 64 : pe;
      if (pb < vlo || pb + 64 > vhi) {
        for (int q = tid; q < 64 * CPR; q += NW * 64) {
          const int row = q / CPR, cc = q - (q / CPR) * CPR;
          const int pos = pb + row;
          if (pos >= vlo && pos < vhi) continue;
          if (pos >= n0 && pos < n1) {
            *reinterpret_cast<v4u*>(slot + f8_slot(row, cc) * 16) = new_chunk(pos, cc, false);
            *reinterpret_cast<v4u*>(slot + Gm::RAW + f8_slot(row, cc) * 16) =
                new_chunk(pos, cc, true);
          } else {
            *reinterpret_cast<v4u*>(slot + Gm::RAW + f8_slot(row, cc) * 16) =
                v4u{0u, 0u, 0u, 0u};
          }
        }
        lds_barrier();
      }
    }

    if (dead) return;
    f32x4 sacc[NPT];
#pragma unroll
    for (int pq = 0; pq < NPT; ++pq) {
      const v4u a0 = *reinterpret_cast<const v4u*>(slot + pq * 2048 + ka0);
      const v4u a1 = *reinterpret_cast<const v4u*>(slot + pq * 2048 + ka1);
      const v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                        (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      sacc[pq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 3; ++k)
        sacc[pq] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qt[k], sacc[pq], 0, 0, 0,
                                                                    127, 0, 127);
    }
    // a tile inside every row's window and the chunk needs no mask (the
    // bounds are uniform: a scalar branch)
    const bool full = pb >= lo_s && pb + 63 <= hi_s && pb + 64 <= pe;
    unsigned wh[NKS][4];
#pragma unroll
    for (int pq = 0; pq < NPT; ++pq) {
      const int pt = ph * NPT + pq;
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(sacc[pq][i], qinv, -shift2));
      if (!full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = pb + 16 * pt + 4 * (ln >> 4) + i;
          e[i] = (pos >= w_lo && pos <= w_hi && pos < pe) ? e[i] : 0.f;
        }
      }
      wh[pq >> 1][2 * (pt & 1)] = cvt_pk_bf16(e[0], e[1]);
      wh[pq >> 1][2 * (pt & 1) + 1] = cvt_pk_bf16(e[2], e[3]);
    }
    auto pv = [&](auto KQ) {
      constexpr int kq = decltype(KQ)::v;
      const bf16x8 bh = as_bf16x8(v4u{wh[kq][0], wh[kq][1], wh[kq][2], wh[kq][3]});
      // V^T operand (16 dims x 32 positions, the k order of the weights:
      // slot m < 4 is position 4 g + m, slot m >= 4 position 16 + 4 g + m - 4
      // of the k-step, g = ln >> 4).  Within each 16 lanes the transpose load
      // gives lane 8 j + b byte b of the 8 bytes addressed by lane j + 2 m as
      // its byte m, so lane q addresses slot m = q >> 1's row at dims
      // 8 (q & 1) .. + 7 of the 16-dim tile, and lane i ends up with dim i
      // of the tile at the eight positions in k order.
      v2i vt[NDT];
      v_tr_reads<SL * Gm::SLOT + 4096 * kq>(tra, vt);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const v2i raw = vt[dt];
        const bf16x8 a = as_bf16x8(v4u{e4m3x2_bf16<false>((unsigned)raw.x),
                                       e4m3x2_bf16<true>((unsigned)raw.x),
                                       e4m3x2_bf16<false>((unsigned)raw.y),
                                       e4m3x2_bf16<true>((unsigned)raw.y)});
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, oacc[dt], 0, 0, 0);
      }
      sacc_l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bh, sacc_l, 0, 0, 0);
    };
    pv(F8Slot<0>());
    if constexpr (NKS > 1) pv(F8Slot<1>());
  };
  // the ring slot of a tile is a constant of each unrolled step
  for (int pb = pb0; pb < pe; pb += ts * Gm::NSLOT) {
    tile(F8Slot<0>(), pb);
    if (pb + ts < pe) tile(F8Slot<1>(), pb + ts);
    if constexpr (Gm::NSLOT > 2)
      if (pb + 2 * ts < pe) tile(F8Slot<2>(), pb + 2 * ts);
    if constexpr (Gm::NSLOT > 3)
      if (pb + 3 * ts < pe) tile(F8Slot<3>(), pb + 3 * ts);
  }
  float lsum = sacc_l[0];
  if constexpr (NPH == 2) {
    float* xs = reinterpret_cast<float*>(ring) + rt * (NDT * 4 + 1) * 64;
    lds_barrier();
    if (ph == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[(dt * 4 + i) * 64 + ln] = oacc[dt][i];
      xs[NDT * 4 * 64 + ln] = lsum;
    }
    lds_barrier();
    if (ph == 1) return;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][i] += xs[(dt * 4 + i) * 64 + ln];
    lsum += xs[NDT * 4 * 64 + ln];
  }
  if (m0 + 16 * rt >= M) return;
  float* part = S.part + ((size_t)item * ROWS + 16 * rt + (ln & 15)) * (D + 1);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[16 * dt + 4 * (ln >> 4) + i] = oacc[dt][i];
  if (ln < 16) part[D] = lsum;
}

template <int KDT, int D, int NW, int NPH>
__device__ void phase_attn_mfma(const LayerArgs& L, const StepArgs& S, const AttnPlan* P,
                                uint8_t* lds, int vb, int nvb) {
  const int n_items = P->item0[S.n_req];
  for (int item = vb; item < n_items; item += nvb) {
    if constexpr (KDT == kE4M3 && D == 128 && NW == 4)
      attn_item_f8<NPH>(L, S, P, item, lds);
    else
      attn_item_mfma<KDT, D, NW, NPH>(L, S, P, item, lds);
    __syncthreads();
  }
}

}  // namespace msk
