// Kernel parameter blocks shared by the host planner and the device code.
#pragma once
#include <stdint.h>

namespace msk {

constexpr int kMaxReq = 64;
constexpr int kMaxTok = 64;
constexpr int kMaxLayers = 64;      // layers per whole-step call
constexpr int kMaxFusedLayers = 4;  // layers of the persistent timeline kernel (kernel arguments)
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 256;
constexpr int kRowGroup = 8;       // query rows handled together by attention
constexpr int kBlockThreads = 256; // every kernel uses 4 waves of 64
constexpr int kWaves = kBlockThreads / 64;

enum Dt : int { kF32 = 0, kBF16 = 1, kE4M3 = 2, kNVFP4 = 3 };

// Kernel phases, as numbered by the timing calls of the C ABI.
enum Phase : int {
  kPhQkv = 0, kPhAttn, kPhCombine, kPhWo, kPhRouter, kPhTopk, kPhGateUp, kPhDown, kPhStep,
  kPhUnion, kPhMoeSum, kPhPrep, kPhDenseSum, kNumPhases
};

// Distinct selected experts in ascending order, and per expert the slots
// (t * K + j) routed to it in ascending order.
struct Union {
  int n;                       // distinct experts
  int list[kMaxExperts];       // expert ids
  int off[kMaxExperts + 1];    // slot ranges in `slots`
  int start[kMaxExperts];      // per expert id: first position in slots
  int slots[kMaxTok * kMaxTopK];
};

// One layer's shapes, weights, cache and attention plan.
struct LayerArgs {
  int H, Hq, Hkv, D, E, K, F, window;
  float eps, shift, qscale;  // qscale = 1/sqrt(D)
  int ddt, edt, kdt;
  const float *attn_norm, *q_norm, *k_norm, *ffn_norm;
  const uint8_t *wq, *wk, *wv, *wo, *wr, *wg, *wu, *wd;
  const uint8_t *sg, *su, *sd;
  const float *gg, *gu, *gd;
  uint8_t *kc, *vc;
  long long cap;
  int chunk;    // cache positions per attention work item (multiple of 64)
  int n_items;  // attention work items of this layer
  int nrg;      // query row groups per kv head: ceil(G * Tr / rg_rows)
  int rg_rows;  // query rows per row group (and per partial-sum block)
  int attn_nw;  // 0: vector attention (rg_rows = kRowGroup); else waves of
                // the matrix-core attention, rg_rows = 16 * attn_nw / attn_nph
  int attn_nph; // matrix-core attention: waves sharing each 16-row tile (1, 2)
};

// Cache range one request's tokens read in one layer: from the window start of
// its first draft token (rounded down to 64 positions for the matrix-core
// items, align64) to one past its last draft token's own position.  The
// vector items start at the window itself, so that a window of 64 k
// positions is k items per kv head, not k + 1.
__host__ __device__ inline void req_span(int L, int Tr, int W, bool align64, int& base, int& end) {
  const int lo = W > 0 ? (L - W + 1 > 0 ? L - W + 1 : 0) : 0;
  base = align64 ? lo & ~63 : lo;
  end = L + Tr;
}

// Default bound, in polls, of every device-side wait: past it a wait gives up
// and sets the workspace's error flag instead of hanging the GPU.
constexpr unsigned kSpinLimit = 1u << 22;

// Buffers of one step; the per-layer arrays follow the layer index.
struct StepArgs {
  int n_req, Tr, T, n_layers;
  int kv_len[kMaxReq];
  const float *x_in;    // layer 0 input [T][H]
  float *x_out;         // last layer output [T][H] (may equal x_in)
  float *layer_out;     // [n_layers][T][H] or null
  int *topk_out;        // [n_layers][T][K] or null
  int *win_out;         // [n_layers][T][2] or null
  float *attn_o_out;    // [T][Hq*D] or null (single layer calls)
  // workspace
  float *qkv;           // [T][Hq*D + 2*Hkv*D]
  float *part;          // attention partials [items][rg_rows][D + 1]
  float *attn_o;        // [T][Hq*D]
  float *h;             // [T][H]
  float *u;             // [T][H]
  float *logits;        // [T][E]
  int *idx;             // [T][K]
  float *wts;           // [T][K]
  float *act;           // [T*K][F]
  float *xa, *xb;       // [T][H] layer ping-pong
  Union *uni;           // distinct selected experts and their slots
  float *ybuf;          // [T*K][H] per-slot expert outputs (several tokens)
  unsigned short *a3;   // [3][T][max(H, Hq*D)] bf16 terms of a projection's input
  float *dpart;         // dense partial tiles
  unsigned *sync;       // kSyncBytes of barrier and counter words (zero between calls)
  long long *stamps;    // optional timeline [blocks][kStamps] of 100 MHz counter values
  unsigned spin_limit;  // polls before a device-side wait gives up
};

// K slices of a matrix-core dense projection with N rows (blocks of 64) and
// K columns (tiles of 128): about one (row block, slice) item per resident
// workgroup (two per CU), at least three k-tiles per slice.
__host__ __device__ inline int dense_slices(int N, int K) {
  const int n_rb = (N + 63) / 64;
  const int tiles = K / 128;
  const int ks = (512 + n_rb - 1) / n_rb;
  const int most = tiles / 3 > 1 ? tiles / 3 : 1;
  return ks < 1 ? 1 : (ks > most ? most : ks);
}

// The workspace starts with kSyncBytes of words that every entry point finds
// at the same place and that are zero between calls: the persistent kernel's
// tree barrier (word 0 its generation, word 1 the error flag, word 32 and
// words 64 + 32 g for g < 8 its arrival counters), at kTopkCountWord, the
// arrival counter of the several-token top-k kernel, and the attention
// counters below.
constexpr int kSyncBytes = 16384;
constexpr int kTopkCountWord = 1024;
// Words kAttnCountWord .. + kAttnCountMax: the attention items' arrival
// counters, one per (request, kv head, row group), when the last item of a
// group sums the group's partials.
constexpr int kAttnCountWord = 2048;
constexpr int kAttnCountMax = kSyncBytes / 4 - kAttnCountWord;

// Buffers of the prefill expert FFN (msk_moe_prefill; see phases_prefill.h).
// Most slots of one expert in one matrix-product item: kPfChunkFp4 for NVFP4
// experts, kPfChunk for bf16 experts (the smaller one sizes the chunk list).
constexpr int kPfChunk = 128;
constexpr int kPfChunkFp4 = 160;

struct PfChunk {
  int e, pos0, n;  // expert, first grouped position, slots (1 .. the chunk limit)
};

struct PfArgs {
  int T;                 // tokens
  const int* idx;        // [T][K] selected experts (out of range: the slot adds nothing)
  const float* u;        // [T][H] expert input
  int* off;              // [E + 1] first grouped position of each expert; off[E] = slots placed
  int* nchunk;           // chunks listed
  PfChunk* chunk;        // [T K / kPfChunk + E] chunks, by expert
  int* cur;              // [E] next grouped position of each expert (placement cursor)
  int* perm;             // [T K] slot at grouped position pos
  int* pos;              // [T K] grouped position of slot s (-1: not placed)
  int* pe;               // [T K] expert at grouped position pos
  int* ue;               // [T K] the input row of pos's token holds u * 2^-ue[pos]
  int* ae;               // [T K] activation row pos holds act * 2^-ae[pos]
  unsigned short* a;     // [T][H] inputs by token: fp16 (NVFP4 experts), or
                         // [2][T][H] two bf16 terms (bf16 experts)
  float* gu;             // [T K][2 F] gate and up products by position
  unsigned short* act;   // [T K][F] activations by position, as a
  float* y;              // [T K][H] expert outputs by slot
};

constexpr int kStamps = 32;  // timeline slots per workgroup (phase ends, per layer)

}  // namespace msk
