// Expert FFN for steps of several tokens: only the distinct selected experts
// are streamed, each once for all the tokens routed to it.
//
// The union of selected experts (ascending ids, each with its slots
// t * K + j in ascending order) is built once per call into the workspace.
// The (expert, row block) tasks are laid out expert-major and every
// workgroup takes one contiguous, equally long range of them, so a
// workgroup meets one or two experts: it stages the input vectors of that
// expert's tokens in LDS and its waves take the range's tasks in turn (wave
// w the tasks w, w + 4, ..., so the waves read neighbouring rows together),
// each streaming its rows two buffers deep, as the one-token kernels do.  An expert with more
// tokens than the staging holds is streamed once per group of tokens.
//
// down writes y[slot][c] = down_e[c] . act[slot]; the combine then forms
// out[t][c] = h[t][c] + sum_j w[t][j] * y[t*K + j][c] in slot order.
#pragma once
#include "phases_t1.h"


namespace msk {

// Input vectors staged in LDS are stored in 16-B granules in a rotated order:
// a lane reads its chunk of consecutive inputs, so in a plain layout the 16
// lanes of one LDS read pass would sit a chunk's worth of bytes apart and
// share a few bank groups.  Rotating each chunk's granules by the chunk index
// (or a part of it) gives the 16 lanes of a pass 16 distinct bank groups.
// fp32 and bf16 weights meet fp32 inputs (a granule is 4 floats); NVFP4
// weights meet fp16 inputs (a granule is 8 halves, a chunk's 32 inputs are 4
// granules).  Granule G of a vector is stored at tn_gran<DT>(G), relative to
// the vector's own start.
template <int DT>
__device__ __forceinline__ int tn_gran(int G) {
  if constexpr (DT == kNVFP4) return (G & ~3) | ((G + (G >> 4)) & 3);
  else if constexpr (DT == kBF16) return (G & ~1) | ((G ^ (G >> 4)) & 1);
  else return G;
}

// LDS floats one staged vector of n inputs takes (fp16 pairs for NVFP4).
template <int DT>
__host__ __device__ constexpr int tn_vec_floats(int n) { return DT == kNVFP4 ? n / 2 : n; }

// n inputs from global memory into LDS in that order (all threads).  NVFP4
// takes them as fp16 (nearest even, two per word, element 2i low), unscaled
// when the vector's largest magnitude lies in [2^-8, 2^15) (fp16 then holds
// every input to its own relative precision unless it is 2^-6 times the
// largest or smaller); otherwise a second pass stores them times the power of
// two that brings the largest into [2^13, 2^14).  Returns the factor that
// undoes the scaling (1 for the other types).  red: kWaves floats of LDS.
template <int DT>
__device__ __forceinline__ float tn_stage(const float* src, int n, float* dst, float* red) {
  if constexpr (DT == kNVFP4) {
    auto pass = [&](float up) {
      float m = 0.f;
      for (int c = threadIdx.x * 8; c < n; c += blockDim.x * 8) {
        const v4f a = *reinterpret_cast<const v4f*>(src + c);
        const v4f b = *reinterpret_cast<const v4f*>(src + c + 4);
        m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                           fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w)))));
        *reinterpret_cast<v4u*>(dst + tn_gran<DT>(c >> 3) * 4) =
            v4u{cvt_pk_f16(a.x * up, a.y * up), cvt_pk_f16(a.z * up, a.w * up),
                cvt_pk_f16(b.x * up, b.y * up), cvt_pk_f16(b.z * up, b.w * up)};
      }
      return m;
    };
    const float m = block_max(pass(1.f), red);
    if (m >= 0x1p-8f && m < 0x1p15f) return 1.f;
    if (!(m > 0.f) || !(m < __builtin_huge_valf())) return 1.f;  // all zero, or not finite
    int ex = 0;
    frexpf(m, &ex);  // m < 2^ex
    lds_barrier();   // every wave's first-pass stores are done before they are replaced
    pass(ldexpf(1.f, 14 - ex));
    return ldexpf(1.f, ex - 14);
  } else {
    for (int c = threadIdx.x * 4; c < n; c += blockDim.x * 4)
      *reinterpret_cast<v4f*>(dst + tn_gran<DT>(c >> 2) * 4) = *reinterpret_cast<const v4f*>(src + c);
    return 1.f;
  }
}

// The nv <= NVMAX input vectors of a group into LDS, vector v from src(v)
// (src must give a readable vector for every v < NVMAX) to dst + v *
// tn_vec_floats(n), in tn_stage's format; down[v] gets the factor that undoes
// the scaling.  Each thread issues the loads of VB vectors times C chunks
// before it stores any of them: a loop that stored each chunk as it arrived
// would wait for every load in turn, and, the load counter being in order,
// for every weight load issued before it.  The LDS stores start after a
// barrier, so the previous group's readers may still be running at entry.
// NT is the workgroup size as a constant: blockDim.x is read from the
// dispatch packet by a global load, which would wait behind the weight loads.
template <int DT, int NVMAX, int VB, int C, int NT, class Src>
__device__ __forceinline__ void tn_stage_group(int nv, int n, Src&& src, float* dst, float* red,
                                               float (&down)[NVMAX]) {
  constexpr int EPC = DT == kNVFP4 ? 8 : 4;  // inputs per thread per chunk
  constexpr int step = NT * EPC;
  const int stride = tn_vec_floats<DT>(n);
#pragma unroll
  for (int v = 0; v < NVMAX; ++v) down[v] = 1.f;
  if constexpr (C == 0) {  // vector by vector, as tn_stage goes
    lds_barrier();
#pragma unroll
    for (int v = 0; v < NVMAX; ++v)
      if (v < nv) down[v] = tn_stage<DT>(src(v), n, dst + v * stride, red);
  } else if constexpr (DT == kNVFP4) {
    if (n > C * step) {  // longer than one batch: the two-pass staging
      lds_barrier();
#pragma unroll
      for (int v = 0; v < NVMAX; ++v)
        if (v < nv) down[v] = tn_stage<DT>(src(v), n, dst + v * stride, red);
      return;
    }
#pragma unroll
    for (int v0 = 0; v0 < NVMAX; v0 += VB) {
      if (v0 >= nv) break;
      v4f x[VB][C][2];
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        const float* sp = src(v0 + b < NVMAX ? v0 + b : 0);
#pragma unroll
        for (int q = 0; q < C; ++q) {
          const int c = (int)threadIdx.x * 8 + q * step;
          const int cl = c < n ? c : 0;
          x[b][q][0] = *reinterpret_cast<const v4f*>(sp + cl);
          x[b][q][1] = *reinterpret_cast<const v4f*>(sp + cl + 4);
        }
      }
      if (v0 == 0) lds_barrier();
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        const int v = v0 + b;
        if (v >= NVMAX || v >= nv) break;
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < C; ++q)
          if ((int)threadIdx.x * 8 + q * step < n)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              m = fmaxf(m, fmaxf(fmaxf(fabsf(x[b][q][h].x), fabsf(x[b][q][h].y)),
                                 fmaxf(fabsf(x[b][q][h].z), fabsf(x[b][q][h].w))));
        m = block_max<NT / 64>(m, red);
        float up = 1.f;
        if (!(m >= 0x1p-8f && m < 0x1p15f) && m > 0.f && m < __builtin_huge_valf()) {
          int ex = 0;
          frexpf(m, &ex);  // m < 2^ex
          up = ldexpf(1.f, 14 - ex);
          down[v] = ldexpf(1.f, ex - 14);
        }
#pragma unroll
        for (int q = 0; q < C; ++q) {
          const int c = (int)threadIdx.x * 8 + q * step;
          if (c < n) {
            const v4f a = x[b][q][0], bb = x[b][q][1];
            *reinterpret_cast<v4u*>(dst + v * stride + tn_gran<DT>(c >> 3) * 4) =
                v4u{cvt_pk_f16(a.x * up, a.y * up), cvt_pk_f16(a.z * up, a.w * up),
                    cvt_pk_f16(bb.x * up, bb.y * up), cvt_pk_f16(bb.z * up, bb.w * up)};
          }
        }
      }
    }
  } else {
    // one batch: loads, a barrier (which also keeps the compiler from moving
    // any load down to its store), stores; a chunk past the end reloads and
    // rewrites chunk 0 with the same value
    auto batch = [&](int c0) {
#pragma unroll
      for (int v0 = 0; v0 < NVMAX; v0 += VB) {
        if (v0 >= nv) break;
        v4f x[VB][C];
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          const float* sp = src(v0 + b < NVMAX ? v0 + b : 0);
#pragma unroll
          for (int q = 0; q < C; ++q) {
            const int c = c0 + q * step;
            x[b][q] = *reinterpret_cast<const v4f*>(sp + (c < n ? c : 0));
          }
        }
        lds_barrier();
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          const int v = v0 + b;
          if (v >= NVMAX || v >= nv) break;
#pragma unroll
          for (int q = 0; q < C; ++q) {
            const int c = c0 + q * step;
            *reinterpret_cast<v4f*>(dst + v * stride + tn_gran<DT>((c < n ? c : 0) >> 2) * 4) =
                x[b][q];
          }
        }
      }
    };
    if (n <= C * step) {
      batch((int)threadIdx.x * 4);  // straight-line: no loop to merge wait states over
    } else {
      lds_barrier();
#pragma unroll
      for (int v = 0; v < NVMAX; ++v)
        if (v < nv) tn_stage<DT>(src(v), n, dst + v * stride, red);
    }
  }
}

// The SUB inputs of sub-block `sub` of chunk `ch` of a staged fp32 vector.
template <int DT>
__device__ __forceinline__ void tn_load(const float* v, int ch, int sub, float* a) {
  using W = WT<DT>;
  const int G = (ch * W::EPL + sub * W::SUB) >> 2;
  const v4f x = *reinterpret_cast<const v4f*>(v + tn_gran<DT>(G) * 4);
  a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
  if constexpr (W::SUB == 8) {
    const v4f y = *reinterpret_cast<const v4f*>(v + tn_gran<DT>(G + 1) * 4);
    a[4] = y.x; a[5] = y.y; a[6] = y.z; a[7] = y.w;
  }
}

// NVFP4: the 8 fp16 inputs of sub-block `sub` of chunk `ch` (one granule).
__device__ __forceinline__ v4u tn_load_f16(const float* v, int ch, int sub) {
  return *reinterpret_cast<const v4u*>(v + tn_gran<kNVFP4>(ch * 4 + sub) * 4);
}

// NV padded to a power of two, and log2 of a power of two up to 16.
constexpr int tn_nvp(int nv) { return nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : 8; }
constexpr int tn_log2(int p) { return p <= 1 ? 0 : p == 2 ? 1 : p == 4 ? 2 : p == 8 ? 3 : 4; }

// Like stream_t1, for nv <= NV input vectors in LDS (stored by tn_stage):
// the sums W_r . in_v (NVFP4: with block scales, matrix scale left out) of a
// task's R rows and nv vectors, reduced over the wave together
// (reduce_scatter): out(k, sum) gets in lane l the sum of index
// l >> (6 - log2 P), index r NVP + v, P = R NVP, NVP = tn_nvp(NV).
template <int DT, int R, int U, int NV, int NB = 2, class ActFn, class RowFn, class OutFn,
          class PreFn>
__device__ __forceinline__ void stream_tn(int ntask, int ncols, int nv, ActFn&& actfn,
                                          RowFn&& rowfn, OutFn&& out, PreFn&& pre) {
  using W = WT<DT>;
  const int ln = lane_id();
  const int nch = ncols / W::EPL;
  const int NI = (nch + 64 * U - 1) / (64 * U);
  const int total = ntask * NI;
  v4u Wb[NB][U][R];
  unsigned Sb[NB][U][R];
  float acc[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[r][v] = 0.f;

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
      // every lane loads (a clamped chunk past the row end, which compute
      // skips), so the number of loads in flight is the same on every path
      // and the waits before each compute step count exactly to that step's
      // loads.  Nothing may touch the loaded values here: a select on them
      // would wait for the refill right after issuing it.
      // addresses as a scalar row base plus one 32-bit lane offset shared by
      // the rows (no per-row 64-bit address registers to keep alive)
      const int ch = (i * U + u) * 64 + ln;
      const unsigned cc = (unsigned)(ch < nch ? ch : nch - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        w[u][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wr[r] + cc * 16u));
        // the lane's two scale bytes inside an aligned dword (a 16-bit load
        // here made the compiler wait for the refills at the next step)
        if constexpr (DT == kNVFP4)
          s[u][r] = scale_dword(sr[r], cc);
        else
          s[u][r] = 0u;
      }
    }
  };
  auto compute = [&](const v4u(&w)[U][R], const unsigned(&s)[U][R], At at) {
    const int k = at.k, i = at.i;
    const uint8_t* sr[R];  // NVFP4: the scale rows again, for their alignment
    if constexpr (DT == kNVFP4) {
      const uint8_t* wr[R];
      rowfn(k, wr, sr);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // no branch on the chunk: a lane past the row end computes on its
      // clamped chunk and adds nothing (a branch here would make the
      // compiler's waits for the loads in flight conservative)
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
      if constexpr (DT == kNVFP4) {
        // e2m1 pairs -> fp16 pairs (exact), dotted with the fp16 inputs two
        // products at a time into fp32; the block scale multiplies each
        // 8-element sum
#pragma unroll
        for (int sub = 0; sub < W::NSUB; ++sub) {
          v4u a[NV];
#pragma unroll
          for (int v = 0; v < NV; ++v)
            if (v < nv) a[v] = tn_load_f16(actfn(v), cl, sub);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const unsigned word = sub == 0 ? w[u][r].x : sub == 1 ? w[u][r].y
                                : sub == 2 ? w[u][r].z : w[u][r].w;
            const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0);
            const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1);
            const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2);
            const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              if (v < nv) {
                // the pairs are taken out of the 8-vector with a shuffle: a
                // bit cast of each 32-bit word to a pair compiled to the
                // first word for all four
                const f16x8 x = __builtin_bit_cast(f16x8, a[v]);
                float d = __builtin_amdgcn_fdot2(p0, __builtin_shufflevector(x, x, 0, 1), 0.f, false);
                d = __builtin_amdgcn_fdot2(p1, __builtin_shufflevector(x, x, 2, 3), d, false);
                d = __builtin_amdgcn_fdot2(p2, __builtin_shufflevector(x, x, 4, 5), d, false);
                d = __builtin_amdgcn_fdot2(p3, __builtin_shufflevector(x, x, 6, 7), d, false);
                acc[r][v] = fmaf((sub >> 1) ? sc[r].y : sc[r].x, d, acc[r][v]);
              }
            }
          }
        }
      } else {
        // the inputs first, then one weight row at a time: only one row's
        // decoded values are live at once (one sub-block per chunk)
        float a[NV][W::SUB];
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (v < nv) tn_load<DT>(actfn(v), cl, 0, a[v]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float fw[W::SUB];
          decode_sub<DT>(w[u][r], 0, fw);
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            if (v < nv) {
              float d = 0.f;
#pragma unroll
              for (int e = 0; e < W::SUB; ++e) d = fmaf(fw[e], a[v][e], d);
              acc[r][v] += in ? d : 0.f;
            }
          }
        }
      }
    }
    if (i == NI - 1) {
      // value (r, v) at index r * NVP + v (NV padded to a power of two);
      // out(k, sum) gets in each lane the total of index lane >> (6 - log2 P)
      constexpr int NVP = tn_nvp(NV);
      float a[R * NVP];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int v = 0; v < NVP; ++v) a[r * NVP + v] = (v < NV && v < nv) ? acc[r][v] : 0.f;
      out(k, reduce_scatter<R * NVP>(a));
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[r][v] = 0.f;
    }
  };
  // NB buffers rotate: step f computes in buffer f % NB, whose refill (step
  // f + NB) goes out right after, so NB - 1 buffers stay in flight while one
  // is computed.  The refills are issued on every iteration (past the end
  // they repeat the last step's addresses, unused), so the loop holds no
  // conditional load; peeling the last steps off instead costs registers
  // (and occupancy) here
  const int last = total - 1;
  const At at_last{last / NI, last - (last / NI) * NI};
  At c[NB];
  c[0] = At{0, 0};
#pragma unroll
  for (int b = 1; b < NB; ++b) c[b] = next(c[b - 1]);
  if (total > 0) {
    // every buffer's loads ahead of the next buffer's, as inside the loop:
    // the compiler's waits at the loop head hold for the entry path too
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      issue(Wb[b], Sb[b], b <= last ? c[b] : at_last);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  pre();
  for (int f = 0; f < total; f += NB) {
    At n[NB];
    n[0] = next(c[NB - 1]);
#pragma unroll
    for (int b = 1; b < NB; ++b) n[b] = next(n[b - 1]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b == 0 || f + b < total) compute(Wb[b], Sb[b], c[b]);
      issue(Wb[b], Sb[b], f + NB + b <= last ? n[b] : at_last);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) c[b] = n[b];
  }
}

// The union into global memory (one workgroup).
// lds: a Union followed by kUnionIdxInts ints and kMaxExperts + 1 64-bit
// words of scratch.
constexpr int kUnionIdxInts = kMaxTok * kMaxTopK + 16;
constexpr size_t kUnionLds = sizeof(Union) + kUnionIdxInts * sizeof(int) + (kMaxExperts + 1) * 8;
static_assert(sizeof(Union) % 8 == 0, "the selection after the union is read as int pairs");
__device__ inline void union_to_global(const int* idx, int T, int K, int E, Union* lds, Union* dst) {
  build_union(idx, T, K, E, lds, reinterpret_cast<int*>(lds + 1));
  const int* s = reinterpret_cast<const int*>(lds);
  int* d = reinterpret_cast<int*>(dst);
  for (int i = threadIdx.x; i < (int)(sizeof(Union) / 4); i += blockDim.x) d[i] = s[i];
}

// This workgroup's contiguous share [t0, t1) of `total` tasks.
__device__ __forceinline__ void wg_range(long long total, int& t0, int& t1) {
  t0 = (int)(total * blockIdx.x / gridDim.x);
  t1 = (int)(total * (blockIdx.x + 1) / gridDim.x);
}

// Runs body(ui, a, b, s0, nv) for every (expert ui of the union, group of at
// most NVMAX of its slots starting at slot index s0) that the workgroup's
// task range meets, with that expert's tasks [a, b) of the range; `stage`
// fills the LDS inputs for the group.  Every wave calls body for every group.
template <int NVMAX, class Body>
__device__ __forceinline__ void for_expert_groups(const Union* U, int nrt, Body&& body) {
  const int n = U->n;
  int t0, t1;
  wg_range((long long)n * nrt, t0, t1);
  int tau = t0;
  while (tau < t1) {
    const int ui = tau / nrt;
    const int seg_end = (ui + 1) * nrt < t1 ? (ui + 1) * nrt : t1;
    const int s0 = U->off[ui], ns = U->off[ui + 1] - s0;
    for (int sg = 0; sg < ns; sg += NVMAX) {
      const int nv = ns - sg < NVMAX ? ns - sg : NVMAX;
      body(ui, tau, seg_end, s0 + sg, nv);
    }
    tau = seg_end;
  }
}

// Rows per task and 16-B chunks per lane per step, as measured best on the
// GPU: NVFP4's decode needs the registers, so it streams one chunk deep.
// Buffers per stream (NB): two; three measured no faster for either type, nor
// did other row and chunk counts, nor fewer NVFP4 workgroups per CU.
template <int DT> struct TnShape;
// Staging: GU_VB / DN_VB input vectors of GU_C / DN_C chunks per thread are
// loaded per batch (C = 0: vector by vector with tn_stage).  Batched loads
// measured faster only for NVFP4's down projection (a single batch of three
// fp32 vectors at expert width 2048); elsewhere they measured the same or
// slower, and NVFP4's gate/up would lose a wave per SIMD to the registers.
template <> struct TnShape<kF32> {
  enum { GU_RW = 2, GU_U = 2, DN_R = 2, DN_U = 2, GU_VB = 1, GU_C = 0, DN_VB = 1, DN_C = 0,
         GU_NB = 2, DN_NB = 2 };
};
template <> struct TnShape<kBF16> {
  enum { GU_RW = 2, GU_U = 2, DN_R = 2, DN_U = 2, GU_VB = 1, GU_C = 0, DN_VB = 1, DN_C = 0,
         GU_NB = 2, DN_NB = 2 };
};
template <> struct TnShape<kNVFP4> {
  enum { GU_RW = 2, GU_U = 1, DN_R = 4, DN_U = 1, GU_VB = 1, GU_C = 0, DN_VB = 3, DN_C = 1,
         GU_NB = 2, DN_NB = 2 };
};

// act[s][f] = silu(gate_e[f] . u[t]) * (up_e[f] . u[t]) for slot s = t*K + j.
// Tasks: (expert, RW rows of gate and the same RW rows of up); NWV waves per
// workgroup share the staged inputs.
template <int DT, int NVMAX, int NWV = kWaves>
__device__ void gateup_tn(const LayerArgs& L, const StepArgs& S, const Union* U, float* act_lds,
                          float* red) {
  constexpr int RW = TnShape<DT>::GU_RW, R = 2 * RW, UU = TnShape<DT>::GU_U;
  const int nrt = L.F / RW;
  const size_t rb = expert_row_bytes(DT, L.H);
  const size_t sb = (size_t)L.H / 16;
  const int wv = wave_id();
  for_expert_groups<NVMAX>(U, nrt, [&](int ui, int a, int b, int sidx, int nv) {
    const int e = U->list[ui];
    const int nt = b - a;
    const int nmine = my_count(wv, NWV, nt);
    // matrix scales in scalar registers before the stream (see slot below)
    const float ggs = DT == kNVFP4 ? uniform_f(L.gg[e]) : 1.f;
    const float gus = DT == kNVFP4 ? uniform_f(L.gu[e]) : 1.f;
    // the group's slots in registers before any weight load is issued: a
    // global load inside the stream would wait behind the prefetches
    int slot[NVMAX];
#pragma unroll
    for (int v = 0; v < NVMAX; ++v)
      slot[v] = __builtin_amdgcn_readfirstlane(U->slots[sidx + (v < nv ? v : 0)]);
    float down[NVMAX];  // undoes the staging's scaling of each input
    auto pre = [&]() {
      // LDS-only barriers: the weight loads just issued stay in flight
      tn_stage_group<DT, NVMAX, TnShape<DT>::GU_VB, TnShape<DT>::GU_C, NWV * 64>(
          nv, L.H, [&](int v) { return S.u + (size_t)(slot[v] / L.K) * L.H; }, act_lds, red,
          down);
      lds_barrier();
    };
    nv_dispatch<NVMAX>(nv, [&](auto nvc) {
      constexpr int NV = decltype(nvc)::value;
      stream_tn<DT, R, UU, NV, TnShape<DT>::GU_NB>(
          nmine, L.H, nv, [&](int v) { return act_lds + v * tn_vec_floats<DT>(L.H); },
          [&](int k, auto& wr, auto& sr) {
            const int f0 = (a + wv + k * NWV - ui * nrt) * RW;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
              const size_t row = (size_t)e * L.F + f0 + r;
              wr[r] = L.wg + row * rb;
              wr[RW + r] = L.wu + row * rb;
              sr[r] = DT == kNVFP4 ? L.sg + row * sb : nullptr;
              sr[RW + r] = DT == kNVFP4 ? L.su + row * sb : nullptr;
            }
          },
          [&](int k, float sum) {
            // gate value (r, v) at index r NVP + v, its up value P / 2 later:
            // 32 lanes on
            const int f0 = (a + wv + k * NWV - ui * nrt) * RW;
            const int ln = lane_id();
            constexpr int NVP = tn_nvp(NV), LP = tn_log2(R * NVP);
            auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum),
                                                       false, false);
            const float upv = __uint_as_float(sw[1]);  // lanes < 32: lane + 32's value
            const int idx = ln >> (6 - LP), r = idx / NVP, v = idx - (idx / NVP) * NVP;
            const bool lead = ln < 32 && (ln & ((64 >> LP) - 1)) == 0;
#pragma unroll
            for (int q = 0; q < NV; ++q)  // constant slot indices (no private array)
              if (lead && v == q && q < nv)
                S.act[(size_t)slot[q] * L.F + f0 + r] =
                    silu(sum * (ggs * down[q])) * (upv * (gus * down[q]));
          },
          pre);
    });
  });
}

// y[s][c] = down_e[c] . act[s] (times the NVFP4 matrix scale) for the slots
// s routed to expert e.  Tasks: (expert, RD output rows).
template <int DT, int NVMAX, int NWV = kWaves>
__device__ void down_tn(const LayerArgs& L, const StepArgs& S, const Union* U, float* act_lds,
                        float* red, float* y) {
  constexpr int RD = TnShape<DT>::DN_R, UU = TnShape<DT>::DN_U;
  const int nrt = L.H / RD;
  const size_t rb = expert_row_bytes(DT, L.F);
  const size_t sb = (size_t)L.F / 16;
  const int wv = wave_id();
  for_expert_groups<NVMAX>(U, nrt, [&](int ui, int a, int b, int sidx, int nv) {
    const int e = U->list[ui];
    const int nt = b - a;
    const int nmine = my_count(wv, NWV, nt);
    const float gds = DT == kNVFP4 ? uniform_f(L.gd[e]) : 1.f;
    int slot[NVMAX];  // in registers before the stream (see gateup_tn)
#pragma unroll
    for (int v = 0; v < NVMAX; ++v)
      slot[v] = __builtin_amdgcn_readfirstlane(U->slots[sidx + (v < nv ? v : 0)]);
    float down[NVMAX];  // undoes the staging's scaling of each input
    auto pre = [&]() {
      tn_stage_group<DT, NVMAX, TnShape<DT>::DN_VB, TnShape<DT>::DN_C, NWV * 64>(
          nv, L.F, [&](int v) { return S.act + (size_t)slot[v] * L.F; }, act_lds, red, down);
      lds_barrier();
    };
    nv_dispatch<NVMAX>(nv, [&](auto nvc) {
      constexpr int NV = decltype(nvc)::value;
      stream_tn<DT, RD, UU, NV, TnShape<DT>::DN_NB>(
          nmine, L.F, nv, [&](int v) { return act_lds + v * tn_vec_floats<DT>(L.F); },
          [&](int k, auto& wr, auto& sr) {
            const int c0 = (a + wv + k * NWV - ui * nrt) * RD;
#pragma unroll
            for (int r = 0; r < RD; ++r) {
              const size_t row = (size_t)e * L.H + c0 + r;
              wr[r] = L.wd + row * rb;
              sr[r] = DT == kNVFP4 ? L.sd + row * sb : nullptr;
            }
          },
          [&](int k, float sum) {
            const int c0 = (a + wv + k * NWV - ui * nrt) * RD;
            const int ln = lane_id();
            constexpr int NVP = tn_nvp(NV), LP = tn_log2(RD * NVP);
            const int idx = ln >> (6 - LP), r = idx / NVP, v = idx - (idx / NVP) * NVP;
            const bool lead = (ln & ((64 >> LP) - 1)) == 0;
#pragma unroll
            for (int q = 0; q < NV; ++q)  // constant slot indices (no private array)
              if (lead && v == q && q < nv)
                y[(size_t)slot[q] * L.H + c0 + r] = sum * (gds * down[q]);
          },
          pre);
    });
  });
}

// out[t][c] = h[t][c] + sum_j w[t][j] * y[t*K + j][c], j ascending; slots
// whose expert id is out of range add nothing.
__device__ inline void down_combine(const LayerArgs& L, const StepArgs& S, const float* h,
                                    const float* y, float* out) {
  const int n4 = S.T * L.H / 4;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
    const int t = (i * 4) / L.H, c = i * 4 - t * L.H;
    v4f acc = *reinterpret_cast<const v4f*>(h + (size_t)t * L.H + c);
    // eight slots' loads in flight at once, then added in slot order
    for (int j0 = 0; j0 < L.K; j0 += 8) {
      v4f yy[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q < L.K ? j0 + q : L.K - 1;
        yy[q] = *reinterpret_cast<const v4f*>(y + ((size_t)t * L.K + j) * L.H + c);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (j0 + q >= L.K) break;
        const int s = t * L.K + j0 + q;
        const int e = S.idx[s];
        if (e < 0 || e >= L.E) continue;
        const float w = S.wts[s];
        acc.x = fmaf(w, yy[q].x, acc.x);
        acc.y = fmaf(w, yy[q].y, acc.y);
        acc.z = fmaf(w, yy[q].z, acc.z);
        acc.w = fmaf(w, yy[q].w, acc.w);
      }
    }
    *reinterpret_cast<v4f*>(out + (size_t)t * L.H + c) = acc;
  }
}

}  // namespace msk
