// ld_stages.hpp - the stages of one decode step as workgroup-level device
// functions.  Every execution mode calls these same functions: one kernel
// per stage (whole-kernel wait or tile-flag overlap) or one persistent
// kernel that runs them back to back.  A stage's workgroups loop over its
// tiles (persistent style), issue the loads of their first weight block,
// then wait for the stage's input to be signalled ready, compute, and
// finally signal their own completion once.
//
// Stage list per layer (the layer step list of a dense Llama decoder):
//   QKV  : q|k|v = Wqkv . n(x)       (RMSNorm folded in: gain on the staged
//                                      inputs, 1/rms factor on the outputs)
//   ATTN : RoPE on q and the new k, bf16 K/V append at the position,
//          split-KV grouped-query attention, last-arriver combine
//   O    : x' = x + Wo . o
//   GU   : h = silu(Wg . n(x')) * (Wu . n(x'))   (the fused first MLP stage
//          of "Deep Kernel Fusion for Transformers", Summary)
//   D    : x'' = x' + Wd . h          (the separate second MLP stage, Key
//                                      points, "Fusion scope")
// then LM : logits = Wlm . n(x), greedy argmax by the last-arriving workgroup.
#pragma once

#include "ld_common.hpp"
#include "ld_gemv.hpp"
#include "ld_mfma.hpp"
#include "ld_params.hpp"

namespace ld {

// Per-stage tile shapes of the VALU engine: NR rows x UC chunks per block,
// PF blocks in flight per wave.
constexpr int kNrQkv = 1, kUcQkv = 4, kPfQkv = 2;
constexpr int kNrO = 1, kUcO = 4, kPfO = 2;
constexpr int kPairsGu = 1, kUcGu = 4, kPfGu = 2;  // one (gate, up) row pair per task
constexpr int kNrD = 1, kUcD = 8, kPfD = 2;
// Down's input (the SwiGLU output, 8192 to 28672 columns) is staged with the
// loads of 4 column groups per thread in flight at batch 1
template <int NB>
constexpr int kStageGroupsD = NB == 1 ? 4 : 1;
constexpr int kNrLm = 2, kUcLm = 4, kPfLm = 2;
// the norm-free stages (O, Down) may take their input in column chunks of
// whole blocks, which the host sizes the staging area for.  Column chunks
// in a build (gemv_stage's KCM): none in the persistent kernel's one-row
// build (the host requires whole input rows to fit a CU's staging area, so
// one row always does), the register-lean form elsewhere (the full form
// made the persistent kernel's 2- to 8-row builds spill).
template <int NB, int MR>
constexpr int kKcMode = (NB == 1 && MR == kMfmaRingBig) ? 0 : 1;
static_assert(kUcO * kChunk * 4 <= kKChunkMinBytes && kUcD * kChunk * 4 <= kKChunkMinBytes,
              "a block's columns must fit the staging area");

__device__ __forceinline__ const uint16_t* layer_w(const Params& P, int l, int64_t off) {
  return P.W.layer0 + (int64_t)l * P.W.layer_stride + off;
}

__device__ __forceinline__ uint32_t* stage_ctr(const Params& P, int l, int slot) {
  return P.K.ctr + ((int64_t)l * kStageCtrs + slot) * kCtrWords;
}

__device__ __forceinline__ uint32_t* split_ctr(const Params& P, int l, int b, int kvh) {
  return P.K.split_ctr + (((int64_t)l * P.D.max_batch + b) * P.D.nkv + kvh) * 16;
}

// The long-context combine phase's counters of layer l: 0 = attention items
// done, 1 = workgroups past the wait for them.
__device__ __forceinline__ uint32_t* aph_ctr(const Params& P, int l, int which) {
  return P.K.aph + ((int64_t)l * 2 + which) * kCtrWords;
}

__device__ __forceinline__ SyncArgs sync_of(const Params& P) {
  return SyncArgs{P.K.err, P.K.watchdog};
}

__device__ __forceinline__ int clamp_pos(const Params& P, int b) {
  const int p = P.S.pos[b];
  return ((unsigned)p < (unsigned)P.D.max_seq) ? p : 0;
}

// Batch rows whose inputs of length K fit the LDS staging area at once.
__device__ __forceinline__ int batch_tile(const Params& P, int K, int NB) {
  const int fit = (int)(P.S.x_cap / ((size_t)K * 4));
  return max(1, min(NB, fit));
}

// LDS staging bytes of the batch tiles of whole rows the O and SwiGLU stages
// read (hidden-size and attention-output rows): the persistent kernel keeps
// SwiGLU weight blocks copied ahead of time above this, so the O stage, even
// when it takes its input in column chunks, stays below it.
template <int NB>
__device__ __forceinline__ size_t row_stage_bytes(const Params& P) {
  const Dims& D = P.D;
  return max((size_t)batch_tile(P, D.H, NB) * D.H, (size_t)batch_tile(P, D.qd, NB) * D.qd) * 4;
}

__device__ __forceinline__ void signal_if(const Params& P, uint32_t* ctr, int who) {
  if (!P.S.wait) wg_signal(ctr, who);
}

// ---- row-count counters (tile-granular readiness, see ld_params.hpp)

__device__ __forceinline__ uint32_t* qg_ctr(const Params& P, int l, int g) {
  return P.K.qg_ctr + ((int64_t)l * P.D.nkv + g) * kCtrWords;
}
__device__ __forceinline__ uint32_t* hc_ctr(const Params& P, int l, int c) {
  return P.K.hc_ctr + ((int64_t)l * P.D.nhc + c) * kCtrWords;
}
// kv group of a QKV output row (q rows of its query heads, then k, then v)
__device__ __forceinline__ int qkv_group(const Dims& D, int row) {
  if (row < D.qd) return row / (D.group * D.d);
  row -= D.qd;
  if (row >= D.kvd) row -= D.kvd;
  return row / D.d;
}
// rows of the QKV output in one kv group, and of the SwiGLU output in chunk c
__device__ __forceinline__ uint32_t qkv_group_rows(const Dims& D) { return (uint32_t)((D.group + 2) * D.d); }
__device__ __forceinline__ uint32_t h_chunk_rows(const Dims& D, int c) {
  return (uint32_t)min(kHChunk, D.I - c * kHChunk);
}
__device__ __forceinline__ bool tile_counting(const Params& P) { return !P.S.wait && P.S.tile_sync; }
// At stage entry: the workgroup's row counts start at zero (the stage's own
// barriers order this before its first epilogue).
__device__ __forceinline__ void counts_clear(const Params& P, Scratch& sc, int n) {
  if (tile_counting(P) && tid() < n) sc.cnt[tid()] = 0;
}
// One output row written (counted once per row, whatever the batch).
__device__ __forceinline__ void count_row(Scratch& sc, int i) { atomicAdd(&sc.cnt[i], 1); }
// After the workgroup's outputs are stored: every wave waits for its stores,
// then counter i gains the rows the workgroup wrote for it (leaf `who`).
__device__ __forceinline__ void wg_signal_counts(const Params& P, Scratch& sc, uint32_t* (*ctr)(const Params&, int, int),
                                                 int l, int n, int who) {
  wave_drain();
  __syncthreads();
  if (tid() < n && sc.cnt[tid()] > 0)
    __hip_atomic_fetch_add(ctr(P, l, tid()) + (who & (kLeaves - 1)) * kLeafStride, (uint32_t)sc.cnt[tid()],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Optional timeline: thread 0 of each workgroup stores the constant-rate
// clock (s_memrealtime) at stage entry (ev 0), after the readiness wait
// (ev 1), after the compute (ev 2) and at stage exit (ev 3), at
// trace[((layer * 8 + stage) * 4 + ev) * kTraceWgs + wg].
constexpr int kTraceWgs = 1024;
__device__ __forceinline__ void trace_ev(const Params& P, int l, int stage, int ev, int wg) {
  if (P.K.trace != nullptr && tid() == 0 && wg < kTraceWgs)
    P.K.trace[(((int64_t)l * 8 + stage) * 4 + ev) * kTraceWgs + wg] = __builtin_amdgcn_s_memrealtime();
}

// ----------------------------------------------------------------- QKV

template <int NB, int MR = kMfmaRingSmall>
__device__ __forceinline__ void stage_qkv(const Params& P, int l, int wg, int nwg, char* smem) {
  constexpr int NR = kNrQkv, UC = kUcQkv;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int rows_total = D.qkv_rows, K = D.H, B = P.S.B;
  const uint16_t* Wm = layer_w(P, l, P.W.o_wqkv);
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  if (l == 0 && wg == 0 && tid() < B) {
    const int t = P.S.tokens[tid()], p = P.S.pos[tid()];
    if ((unsigned)t >= (unsigned)D.V) raise_error(P.K.err, kErrToken);
    if ((unsigned)p >= (unsigned)D.max_seq) raise_error(P.K.err, kErrPos);
    // a sequence's tokens take consecutive positions
    const int j = tid() % P.S.M;
    if (j > 0 && p != P.S.pos[tid() - j] + j) raise_error(P.K.err, kErrPos);
  }
  trace_ev(P, l, kSQkv, 0, wg);
  Scratch& scq = *reinterpret_cast<Scratch*>(smem);
  counts_clear(P, scq, D.nkv);
  const bool counting = tile_counting(P);
  auto wait = [&](int = 0, int = 0) {
    if (!P.S.wait && l > 0) wg_wait(sync_of(P), stage_ctr(P, l - 1, kCD), P.S.t_d, kSQkv);
    trace_ev(P, l, kSQkv, 1, wg);
  };
  const XSrc src{l == 0 ? nullptr : P.K.xa, K, P.W.embed, P.S.tokens, D.V};
  float* out = P.K.qkv;
  static_assert(NR * NB <= kWave, "one task's results take one lane each");
  HeldStores<(NB > 1)> held;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch& sc) {
    const int base = held.reserve(NR * NB);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NR + r;
        if (b < nb && row < rows_total && lane == base + r * NB + b)
          held.hold(out + (int64_t)(b0 + b) * rows_total + row, acc[r][b] * sc.rs[b]);
      }
    if (counting && b0 == 0 && lane == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (t * NR + r < rows_total) count_row(sc, qkv_group(D, t * NR + r));
    }
  };
  const uint32_t wbytes = (uint32_t)((int64_t)rows_total * K * 2);
  if constexpr (NB >= kMfmaMinBatch) {
    Scratch& sc = *reinterpret_cast<Scratch*>(smem);
    auto epe = [&](int tile, int r, int b, int bl, int, const float* v) -> float {
      const int row = tile * 16 + r;
      if (row < rows_total) {
        st_coh(out + (int64_t)b * rows_total + row, v[0] * sc.rs[bl]);
        if (counting && b == 0) count_row(sc, qkv_group(D, row));
      }
      return 0.f;
    };
    const MatRows mr{Wm, {Wm, Wm}, rows_total, K};
    const int ntile = (rows_total + 15) / 16;
    if (l == 0) {  // the embedding rows, staged with the gain applied
      mfma_stage<kMfmaNbt<NB, MR>, 1, MR>(mr, ntile, K, Wm, wbytes, src,
                                          layer_w(P, l, P.W.o_attn_norm), true, D.eps, B,
                                          P.S.x_cap, wait, epe, [](int, int) {}, wg, nwg, smem);
    } else {  // the previous layer's Down stage wrote its output as fragments
      XSrc fs{nullptr, K, nullptr, nullptr, 0};
      fs.frag = P.K.xa_f;
      fs.kp = D.Hp;
      fs.ss = P.K.ss_a;
      fs.ss_n = fs.ss_ld = D.Ht;
      mfma_stage_frag<kMfmaNbt<NB, MR>, 1, MR>(mr, ntile, K, Wm, wbytes, fs, true, D.eps, B,
                                               P.S.x_cap, wait, epe, [](int, int) {}, wg, nwg,
                                               smem);
    }
  } else {
    gemv_stage<NR, UC, NB, kPfQkv>(rowfn, (rows_total + NR - 1) / NR, K, Wm, wbytes, src,
                                   layer_w(P, l, P.W.o_attn_norm), true, D.eps, B,
                                   batch_tile(P, K, NB), wait, epi, wg, nwg, smem);
    held.flush();
  }
  trace_ev(P, l, kSQkv, 2, wg);
  if (counting)
    wg_signal_counts(P, scq, qg_ctr, l, D.nkv, wg);
  else
    signal_if(P, stage_ctr(P, l, kCQkv), wg);
  trace_ev(P, l, kSQkv, 3, wg);
}

// ------------------------------------------------------------ attention
//
// Split-KV grouped-query decode attention.  A work item is (sequence b, kv
// head, split s): positions [n0, n1) of 0..p, the splits of a sequence
// balanced to at most T positions each.  T is chosen per step from the batch
// size alone (the host never reads positions), so a batch-1 step spreads over
// many workgroups.  One workgroup per item:
//  - the split's cached K and V rows are copied into LDS with direct-to-LDS
//    loads; they do not depend on this step's QKV outputs, so the first
//    item's copies are issued before the readiness wait;
//  - the group's q heads are rotated to p into LDS; the split holding p also
//    rotates the new key, rounds k and v to bf16, appends them to the cache
//    and places them in the tiles;
//  - scores (q . K_t) / sqrt(d): one lane per (position, 8 channels), the
//    8-channel partial dot products summed across the position's lanes;
//  - the split's softmax statistics per head, then the unnormalised output
//    sum_t e_t V_t over fixed position slices;
//  - a single split writes o / l directly; otherwise each split stores
//    (m, l, o) and the last-arriving split combines all splits in fixed order.

// Position slices of the output sum: one (slice, head, 8 channels) item per
// thread of a 512-thread workgroup, at most 16 slices.  It depends on the
// shape only, so every mode adds the same numbers in the same order.
__host__ __device__ constexpr int attn_parts(int group, int d) {
  return 512 / (group * (d / 8)) < 1 ? 1 : 512 / (group * (d / 8)) > 16 ? 16 : 512 / (group * (d / 8));
}
__host__ __device__ constexpr size_t attn_tiles_bytes(int group, int d, int T, int max_splits) {
  // K and V tiles [T][d] bf16
  return (void)group, (void)max_splits, (size_t)2 * T * d * 2;
}
__host__ __device__ constexpr size_t attn_smem_bytes(int group, int d, int T, int max_splits) {
  return (size_t)group * d * 4                                     /* rotated q */
         + (attn_tiles_bytes(group, d, T, max_splits) + 15) / 16 * 16
         + (size_t)group * T * 4                                   /* scores / weights */
         + (size_t)attn_parts(group, d) * group * d * 4            /* output slices */
         + (size_t)group * 2 * 4;                                  /* (max, sum) per head */
}

// Attention output of row b, column c (head-major) for the O stage: fp32 for
// the VALU engine, a split-bf16 pair in B-fragment order when the step runs
// on the MFMA engine (16 rows and more), which loads it as it is.
__device__ __forceinline__ void st_ao(const Params& P, int b, int c, float v) {
  if (P.S.B >= kMfmaMinBatch)
    st_coh_u(P.K.ao_f + frag_word(b, c, P.D.qdp), split_pair(v));
  else
    st_coh(P.K.ao + (int64_t)b * P.D.qd + c, v);
}

constexpr int kCombBatch = 16;  // splits combined from registers in one round of loads
template <int N>
struct CInt {
  static constexpr int value = N;
};

// Row b of the step (token j = b % M of sequence slot = b / M, at position
// p = p0 + j, where p0 is the sequence's first position of this step).
struct AttnItem {
  int b, kvh, s, ns, p, slot, p0;
};

// Item `it` of the step (sequence-major, then kv head, then split).
// MULTI: the step may hold several tokens per sequence (P.S.M > 1); the
// persistent kernel is built without it (decode steps only), which keeps its
// scalar registers from spilling.
template <bool MULTI>
__device__ __forceinline__ bool attn_item_at(const Params& P, const Scratch& sc, int T, int it,
                                             AttnItem& a) {
  int base = 0;
  const int M = MULTI ? P.S.M : 1;
  for (int b = 0; b < P.S.B; ++b) {
    const int slot = b / M, p0 = sc.pos[slot * M];
    const int p = min(p0 + (b - slot * M), P.D.max_seq - 1);
    const int ns = (p + T) / T, cnt = P.D.nkv * ns;
    if (it < base + cnt) {
      a.b = b;
      a.slot = slot;
      a.p0 = p0;
      a.p = p;
      a.ns = ns;
      a.kvh = (it - base) / ns;
      a.s = it - base - a.kvh * ns;
      return true;
    }
    base += cnt;
  }
  return false;
}

struct AttnLds {
  float* qs;     // [group][d] rotated q
  uint16_t* Ks;  // [T][d]
  uint16_t* Vs;  // [T][d]
  float* Sc;     // [group][T]
  float* op;     // [parts][group][d]
  float* ml;     // [group][2]
};

__device__ __forceinline__ AttnLds attn_lds(const Dims& D, char* smem) {
  AttnLds s;
  char* base = smem + kScratchBytes;
  const int T = D.split_len;
  s.qs = reinterpret_cast<float*>(base);
  s.Ks = reinterpret_cast<uint16_t*>(base + (size_t)D.group * D.d * 4);
  s.Vs = s.Ks + (size_t)T * D.d;
  char* after = reinterpret_cast<char*>(s.Ks) +
                (attn_tiles_bytes(D.group, D.d, T, D.max_splits) + 15) / 16 * 16;
  s.Sc = reinterpret_cast<float*>(after);
  s.op = s.Sc + (size_t)D.group * T;
  s.ml = s.op + (size_t)attn_parts(D.group, D.d) * D.group * D.d;
  return s;
}

__device__ __forceinline__ int64_t attn_cache_off(const Params& P, int l, int b, int kvh) {
  const Dims& D = P.D;
  return ((((int64_t)l * D.max_batch + b) * D.nkv + kvh) * D.max_seq) * (int64_t)D.d;
}

// Copy the item's cached K and V rows into the LDS tiles (1 KB per wave
// instruction, direct to LDS).  With skip_wave0 the polling wave issues none,
// so its spin loads never wait behind these copies.
__device__ __forceinline__ void attn_copy_tiles(const Params& P, int l, const AttnItem& a, char* smem,
                                bool skip_wave0) {
  const Dims& D = P.D;
  const AttnLds s = attn_lds(D, smem);
  const int len = a.p + 1;
  const int n0 = (a.s * len) / a.ns, n1 = ((a.s + 1) * len) / a.ns;
  const int ncached = max(0, min(n1, a.p0) - n0);  // rows before this step's tokens
  const int bytes = ncached * D.d * 2;
  const int nw = nwaves(), w0 = (skip_wave0 && nw > 1) ? 1 : 0, w = wave_id(), lane = lane_id();
  if (w < w0 || bytes <= 0) return;
  const int64_t off = attn_cache_off(P, l, a.slot, a.kvh) + (int64_t)n0 * D.d;
  const char* ksrc = reinterpret_cast<const char*>(P.K.kc + off);
  const char* vsrc = reinterpret_cast<const char*>(P.K.vc + off);
  const int chunks = (bytes + 1023) >> 10;
  for (int c = w - w0; c < 2 * chunks; c += nw - w0) {
    const bool isv = c >= chunks;
    const int cb = (isv ? c - chunks : c) << 10;
    const int o = cb + lane * 16;
    char* dst = reinterpret_cast<char*>(isv ? s.Vs : s.Ks) + cb;
    if (o < bytes)
      __builtin_amdgcn_global_load_lds((isv ? vsrc : ksrc) + o,
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  }
}

// G, DH: the GQA group and head_dim when known at compile time (0: read from
// the dimensions); the arithmetic is the same either way, the known-shape
// forms only fold the index math (slice bounds, lane groups) into constants.
template <bool MULTI, int G = 0, int DH = 0>
__device__ __forceinline__ void attn_item(const Params& P, int l, const AttnItem& a, char* smem) {
  // head_dim is a power of two (checked on the host): index math uses shifts
  const Dims& D = P.D;
  const int d = DH > 0 ? DH : D.d, half = d / 2, group = G > 0 ? G : D.group, w8 = d / 8;
  const int T = D.split_len;
  const int ld = 31 - __builtin_clz(d), lw8 = ld - 3;
  const int tid = ld::tid(), nth = blockDim.x, lane = lane_id(), wave = wave_id();
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  const AttnLds s = attn_lds(D, smem);
  const int b = a.b, kvh = a.kvh, p = a.p, nsplit = a.ns;
  const int len = p + 1;
  const int n0 = (a.s * len) / nsplit, n1 = ((a.s + 1) * len) / nsplit;
  const int n = n1 - n0;
  // positions [q_lo, n1) of the split belong to this step's tokens of the
  // sequence: their k and v come from the QKV outputs of rows
  // slot * M + (q - p0), not from the cache, and the sequence's last token
  // appends them to the cache (each position is appended once)
  const int M = MULTI ? P.S.M : 1;
  const int q_lo = max(n0, a.p0), nnew = max(0, n1 - q_lo);
  const bool appends = (b - a.slot * M) == M - 1;
  const float* qkv = P.K.qkv + (int64_t)b * D.qkv_rows;
  const float* rope = P.K.rope + (int64_t)p * half * 2;
  const int64_t cache_off = attn_cache_off(P, l, a.slot, kvh);
  uint16_t* kc = P.K.kc + cache_off;
  uint16_t* vc = P.K.vc + cache_off;

  // ---- q heads of this group (one (head, pair) per thread: group * half <=
  // 512) and the split's new k and v rows
  trace_ev(P, l, 6, 0, blockIdx.x);
  const bool qthread = tid < group * half;
  const int qg = tid >> (ld - 1), qi = tid & (half - 1);
  // new row e (position q = q_lo + e), pair i: its k, v and the cos/sin of q
  const int rstep = nth / half, i = tid & (half - 1);
  struct NewRow {
    float k0, k1, v0, v1, c, sn;
  };
  auto load_row = [&](int e) {
    const int q = q_lo + e;
    const float* kh = P.K.qkv + (int64_t)(a.slot * M + (q - a.p0)) * D.qkv_rows + D.qd +
                      (int64_t)kvh * d;
    const float* vh = kh + D.kvd;
    const float* rq = P.K.rope + (int64_t)q * half * 2;
    return NewRow{ld_coh(kh + i), ld_coh(kh + i + half), ld_coh(vh + i), ld_coh(vh + i + half),
                  rq[2 * i], rq[2 * i + 1]};
  };
  // rotate the key at q, round k and v to bf16, place them in the tiles (and
  // append them to the cache)
  auto store_row = [&](int e, const NewRow& w) {
    const int q = q_lo + e;
    const uint16_t ka = f2bf(w.k0 * w.c - w.k1 * w.sn), kb = f2bf(w.k0 * w.sn + w.k1 * w.c);
    const uint16_t va = f2bf(w.v0), vb = f2bf(w.v1);
    if (appends) {
      kc[(int64_t)q * d + i] = ka;
      kc[(int64_t)q * d + i + half] = kb;
      vc[(int64_t)q * d + i] = va;
      vc[(int64_t)q * d + i + half] = vb;
    }
    s.Ks[(q - n0) * d + i] = ka;
    s.Ks[(q - n0) * d + i + half] = kb;
    s.Vs[(q - n0) * d + i] = va;
    s.Vs[(q - n0) * d + i + half] = vb;
  };
  // the q loads and the (first pass of) new rows share one round trip
  float q0 = 0.f, q1 = 0.f, cq = 0.f, sq = 0.f;
  if (qthread) {
    const float* qh = qkv + (int64_t)(kvh * group + qg) * d;
    q0 = ld_coh(qh + qi);
    q1 = ld_coh(qh + qi + half);
    cq = rope[2 * qi];
    sq = rope[2 * qi + 1];
  }
  auto rotate_q = [&] {  // rotate q (rotate-half pairs) into LDS
    if (qthread) {
      s.qs[qg * d + qi] = q0 * cq - q1 * sq;
      s.qs[qg * d + qi + half] = q0 * sq + q1 * cq;
    }
  };
  if (!MULTI || M == 1) {
    // a decode step: at most one new row, position p, in the last split;
    // thread tid < half holds pair tid, whose cos/sin it loaded as a q thread
    const bool newrow = (n1 == len) && tid < half;
    NewRow w0{};
    if (newrow) {
      const float* kh = qkv + D.qd + (int64_t)kvh * d;
      const float* vh = kh + D.kvd;
      w0 = NewRow{ld_coh(kh + tid), ld_coh(kh + tid + half), ld_coh(vh + tid),
                  ld_coh(vh + tid + half), cq, sq};
    }
    rotate_q();
    if (newrow) store_row(p - q_lo, w0);
  } else if constexpr (MULTI) {
    const int e0 = tid / half;
    NewRow w0{};
    if (e0 < nnew) w0 = load_row(e0);
    rotate_q();
    if (e0 < nnew) store_row(e0, w0);
    for (int e = e0 + rstep; e < nnew; e += rstep) store_row(e, load_row(e));
  }
  wave_drain();  // direct-to-LDS copies have landed
  __syncthreads();
  trace_ev(P, l, 7, 0, blockIdx.x);

  // ---- scores: lane (t, c8) takes channels [8 c8, 8 c8 + 8) of position t
  // for every head; the w8 lanes of a position are aligned within a wave
  for (int idx = tid; idx < n * w8; idx += nth) {
    const int t = idx >> lw8, c8 = idx & (w8 - 1);
    const u32x4 kw = *reinterpret_cast<const u32x4*>(s.Ks + t * d + c8 * 8);
    const float kf[8] = {bf16lo(kw.x), bf16hi(kw.x), bf16lo(kw.y), bf16hi(kw.y),
                         bf16lo(kw.z), bf16hi(kw.z), bf16lo(kw.w), bf16hi(kw.w)};
#pragma unroll 4
    for (int g = 0; g < group; ++g) {
      const float4 qa = *reinterpret_cast<const float4*>(s.qs + g * d + c8 * 8);
      const float4 qb = *reinterpret_cast<const float4*>(s.qs + g * d + c8 * 8 + 4);
      float acc = qa.x * kf[0];
      acc = fmaf(qa.y, kf[1], acc);
      acc = fmaf(qa.z, kf[2], acc);
      acc = fmaf(qa.w, kf[3], acc);
      acc = fmaf(qb.x, kf[4], acc);
      acc = fmaf(qb.y, kf[5], acc);
      acc = fmaf(qb.z, kf[6], acc);
      acc = fmaf(qb.w, kf[7], acc);
      acc = lane_group_sum(acc, w8);
      if (c8 == w8 - 1) s.Sc[g * T + t] = acc * D.attn_scale;
    }
  }
  __syncthreads();
  // ---- split-local softmax statistics per head
  for (int g = wave; g < group; g += nwaves()) {
    float m = -INFINITY;
    for (int u = lane; u < n; u += kWave) m = fmaxf(m, s.Sc[g * T + u]);
    m = wave_max(m);
    float sum = 0.f;
    for (int u = lane; u < n; u += kWave) {
      const float e = expf(s.Sc[g * T + u] - m);
      s.Sc[g * T + u] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      s.ml[2 * g] = m;
      s.ml[2 * g + 1] = sum;
    }
  }
  __syncthreads();
  trace_ev(P, l, 7, 1, blockIdx.x);
  // ---- unnormalised output sum_t e_t V_t: item (position slice, head, 8
  // channels); per position one 16-byte V read and one broadcast weight, two
  // independent accumulator sets; the slices are then added in fixed order
  const int parts = attn_parts(group, d);
  const int gd = group * d;
  for (int it = tid; it < parts * group * w8; it += nth) {
    const int c8 = it & (w8 - 1);
    const int slg = it >> lw8;  // slice * group + head
    const int sl = slg / group, g = slg - sl * group;
    const int u0 = (sl * n) / parts, u1 = ((sl + 1) * n) / parts;
    const float* e = s.Sc + g * T;
    const uint16_t* vcol = s.Vs + c8 * 8;
    float x[8], y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = y[k] = 0.f;
    int u = u0;
    for (; u + 2 <= u1; u += 2) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(vcol + u * d);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(vcol + (u + 1) * d);
      const float ea = e[u], eb = e[u + 1];
      x[0] = fmaf(ea, bf16lo(va.x), x[0]); x[1] = fmaf(ea, bf16hi(va.x), x[1]);
      x[2] = fmaf(ea, bf16lo(va.y), x[2]); x[3] = fmaf(ea, bf16hi(va.y), x[3]);
      x[4] = fmaf(ea, bf16lo(va.z), x[4]); x[5] = fmaf(ea, bf16hi(va.z), x[5]);
      x[6] = fmaf(ea, bf16lo(va.w), x[6]); x[7] = fmaf(ea, bf16hi(va.w), x[7]);
      y[0] = fmaf(eb, bf16lo(vb.x), y[0]); y[1] = fmaf(eb, bf16hi(vb.x), y[1]);
      y[2] = fmaf(eb, bf16lo(vb.y), y[2]); y[3] = fmaf(eb, bf16hi(vb.y), y[3]);
      y[4] = fmaf(eb, bf16lo(vb.z), y[4]); y[5] = fmaf(eb, bf16hi(vb.z), y[5]);
      y[6] = fmaf(eb, bf16lo(vb.w), y[6]); y[7] = fmaf(eb, bf16hi(vb.w), y[7]);
    }
    if (u < u1) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(vcol + u * d);
      const float ea = e[u];
      x[0] = fmaf(ea, bf16lo(va.x), x[0]); x[1] = fmaf(ea, bf16hi(va.x), x[1]);
      x[2] = fmaf(ea, bf16lo(va.y), x[2]); x[3] = fmaf(ea, bf16hi(va.y), x[3]);
      x[4] = fmaf(ea, bf16lo(va.z), x[4]); x[5] = fmaf(ea, bf16hi(va.z), x[5]);
      x[6] = fmaf(ea, bf16lo(va.w), x[6]); x[7] = fmaf(ea, bf16hi(va.w), x[7]);
    }
    float4* o4 = reinterpret_cast<float4*>(s.op + sl * gd + g * d + c8 * 8);
    o4[0] = make_float4(x[0] + y[0], x[1] + y[1], x[2] + y[2], x[3] + y[3]);
    o4[1] = make_float4(x[4] + y[4], x[5] + y[5], x[6] + y[6], x[7] + y[7]);
  }
  __syncthreads();
  const int oc = kvh * gd;  // this group's first output column
  for (int r = tid; r < gd; r += nth) {
    const int g = r >> ld, i = r & (d - 1);
    float o = 0.f;
#pragma unroll 4
    for (int sl = 0; sl < parts; ++sl) o += s.op[sl * gd + r];
    if (nsplit == 1) {
      st_ao(P, b, oc + r, o / s.ml[2 * g + 1]);
    } else {
      float* pp = P.K.part + (((int64_t)b * D.nq + kvh * group + g) * D.max_splits + a.s) * (d + 2);
      st_coh(pp + 2 + i, o);
      if (i == 0) {
        st_coh(pp, s.ml[2 * g]);
        st_coh(pp + 1, s.ml[2 * g + 1]);
      }
    }
  }
  trace_ev(P, l, 7, 2, blockIdx.x);
  // a step with a long context combines its splits in a phase of its own
  // (stage_attn): the item only counts itself as done
  const bool phase = __builtin_amdgcn_readfirstlane(sc.attn_phase) != 0;
  if (nsplit > 1 && phase) {
    wg_signal(aph_ctr(P, l, 0), blockIdx.x);
    return;
  }
  if (nsplit > 1) {
    // last-arriving split combines all splits in fixed order
    wave_drain();
    __syncthreads();
    if (tid == 0) {
      uint32_t* ctr = split_ctr(P, l, b, kvh);
      const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = (old == (uint32_t)(nsplit - 1));
      if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sc.flag[0] = last;
    }
    __syncthreads();
    trace_ev(P, l, 7, 3, blockIdx.x);
    if (!sc.flag[0]) return;
    // M = max_s m_s, f_s = e^(m_s - M), L = sum_s l_s f_s and, per output
    // channel, o = (sum_s o_s f_s) / L: per channel, the splits in ascending
    // order, kCombBatch splits' (m, l, o) loaded per round; from a second
    // round on (more than kCombBatch splits: a long context) the running L
    // and O are rescaled by e^(M_old - M_new) when the maximum grows.  With
    // more output channels than threads (CPT = 2) a thread takes two
    // adjacent channels of one head, which share the round's m and l loads;
    // each channel's arithmetic is the same either way.
    const float* pbase = P.K.part + ((int64_t)b * D.nq + kvh * group) * D.max_splits * (d + 2);
    auto combine = [&](auto cpt) {
      constexpr int CPT = decltype(cpt)::value;
      for (int r = tid * CPT; r < gd; r += nth * CPT) {
        const int g = r >> ld, i = r & (d - 1);
        const float* q = pbase + (int64_t)g * D.max_splits * (d + 2);
        float M = -INFINITY, L = 0.f, O[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) O[c] = 0.f;
        for (int s0 = 0; s0 < nsplit; s0 += kCombBatch) {
          float mv[kCombBatch], lv[kCombBatch], ov[kCombBatch][CPT];
#pragma unroll
          for (int u = 0; u < kCombBatch; ++u) {
            if (s0 + u < nsplit) {
              const float* rec = q + (s0 + u) * (d + 2);
              mv[u] = ld_coh(rec);
              lv[u] = ld_coh(rec + 1);
#pragma unroll
              for (int c = 0; c < CPT; ++c) ov[u][c] = ld_coh(rec + 2 + i + c);
            }
          }
          float Mn = M;
#pragma unroll
          for (int u = 0; u < kCombBatch; ++u)
            if (s0 + u < nsplit) Mn = fmaxf(Mn, mv[u]);
          if (s0 > 0) {  // (first round: L = O = 0, nothing to rescale)
            const float e = expf(M - Mn);
            L *= e;
#pragma unroll
            for (int c = 0; c < CPT; ++c) O[c] *= e;
          }
          M = Mn;
#pragma unroll
          for (int u = 0; u < kCombBatch; ++u) {
            if (s0 + u < nsplit) {
              const float f = expf(mv[u] - M);
              L = fmaf(lv[u], f, L);
#pragma unroll
              for (int c = 0; c < CPT; ++c) O[c] = fmaf(ov[u][c], f, O[c]);
            }
          }
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) st_ao(P, b, oc + r + c, O[c] / L);
      }
    };
    // (two channels per thread only where the shape is known at compile
    // time: the general form stays one channel per thread, which keeps the
    // persistent kernel's register use where it was)
    if constexpr (G > 0 && DH > 0)
      combine(CInt<(G * DH > kBlockThreads) ? 2 : 1>{});
    else
      combine(CInt<1>{});
  }
  signal_if(P, stage_ctr(P, l, kCAttn), b * D.nkv + kvh);
  if (phase) wg_signal(aph_ctr(P, l, 0), blockIdx.x);  // (an unsplit row of a phase step)
}

// The split combine of one (row b, kv head) in the combine phase: the same
// arithmetic as the last-arriving split's (per channel, the splits in
// ascending order, kCombBatch per round of loads, rescaled from a second
// round on), CPT adjacent channels of one head per thread.
template <int CPT>
__device__ __forceinline__ void attn_combine_unit(const Params& P, int b, int kvh, int nsplit) {
  const Dims& D = P.D;
  const int d = D.d, group = D.group, gd = group * d, ld = 31 - __builtin_clz(d);
  const int tid = ld::tid(), nth = blockDim.x;
  const float* pbase = P.K.part + ((int64_t)b * D.nq + kvh * group) * D.max_splits * (d + 2);
  const int oc = kvh * gd;
  for (int r = tid * CPT; r < gd; r += nth * CPT) {
    const int g = r >> ld, i = r & (d - 1);
    const float* q = pbase + (int64_t)g * D.max_splits * (d + 2);
    float M = -INFINITY, L = 0.f, O[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) O[c] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kCombBatch) {
      float mv[kCombBatch], lv[kCombBatch], ov[kCombBatch][CPT];
#pragma unroll
      for (int u = 0; u < kCombBatch; ++u) {
        if (s0 + u < nsplit) {
          const float* rec = q + (s0 + u) * (d + 2);
          mv[u] = ld_coh(rec);
          lv[u] = ld_coh(rec + 1);
#pragma unroll
          for (int c = 0; c < CPT; ++c) ov[u][c] = ld_coh(rec + 2 + i + c);
        }
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < kCombBatch; ++u)
        if (s0 + u < nsplit) Mn = fmaxf(Mn, mv[u]);
      if (s0 > 0) {
        const float e = expf(M - Mn);
        L *= e;
#pragma unroll
        for (int c = 0; c < CPT; ++c) O[c] *= e;
      }
      M = Mn;
#pragma unroll
      for (int u = 0; u < kCombBatch; ++u) {
        if (s0 + u < nsplit) {
          const float f = expf(mv[u] - M);
          L = fmaf(lv[u], f, L);
#pragma unroll
          for (int c = 0; c < CPT; ++c) O[c] = fmaf(ov[u][c], f, O[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) st_ao(P, b, oc + r + c, O[c] / L);
  }
}

template <int G, int DH>
struct AttnShape {
  static constexpr int g = G, dh = DH;
};

// `idle_hook()` runs in a workgroup that has no attention item, without
// waiting for the stage's input (the persistent kernel issues the SwiGLU
// stage's first weight loads there).
template <bool MULTI, class Hook>
__device__ __forceinline__ void stage_attn(const Params& P, int l, int wg, int nwg, char* smem,
                           const Hook& idle_hook) {
  const Dims& D = P.D;
  trace_ev(P, l, kSAttn, 0, wg);
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  // split length: the step's (from its batch size), or longer when the
  // step's contexts would otherwise make far more items than workgroups (a
  // long context), up to the LDS tiles' capacity.  It depends on the
  // positions and the grid only, so every workgroup (and every mode) finds
  // the same one.  Positions and split length are found once per kernel.
  if (!sc.pos_ok) {
    if (tid() < P.S.B) sc.pos[tid()] = clamp_pos(P, tid());
    __syncthreads();
    if (tid() == 0) {
      int64_t total = 0;
      for (int b = 0; b < P.S.B; ++b) total += sc.pos[b] + 1;
      const int64_t need = (total * D.nkv + nwg - 1) / nwg;
      int T = P.S.T;
      if (need > T) T = (int)min((int64_t)P.S.Tmax, (need + 31) / 32 * 32);
      sc.attn_T = T;
      // the items (row b at position p_b has (p_b + T) / T splits), and the
      // combine phase when some row has more splits than one round of the
      // combine takes (a long context)
      const int M = MULTI ? P.S.M : 1;
      int items = 0, maxns = 0;
      for (int b = 0; b < P.S.B; ++b) {
        const int slot = b / M;
        const int p = min(sc.pos[slot * M] + (b - slot * M), D.max_seq - 1);
        const int ns = (p + T) / T;
        items += D.nkv * ns;
        maxns = max(maxns, ns);
      }
      sc.attn_items = items;
      sc.attn_phase = maxns > kCombBatch;
      sc.pos_ok = 1;
    }
    __syncthreads();
  }
  const int T = __builtin_amdgcn_readfirstlane(sc.attn_T);
  AttnItem a;
  const bool any = attn_item_at<MULTI>(P, sc, T, wg, a);
  // the first item's cached rows are copied while this stage's input is
  // still being produced.  A workgroup without an item reads none of this
  // stage's input, so it does not wait for it: its hook starts at once (the
  // persistent kernel's SwiGLU weight loads then drain while the items
  // compute, instead of during their combine), and the next stage's wait on
  // this stage's counter orders it after the QKV stage as before.
  // the item's input: with tile-granular readiness the q, k and v rows of
  // its own kv group (each item waits for its group), otherwise the whole
  // QKV stage (one wait covers every item)
  auto wait_input = [&](int kvh) {
    if (P.S.wait) return;
    if (P.S.tile_sync)
      wg_wait(sync_of(P), qg_ctr(P, l, kvh), P.S.n_sig * qkv_group_rows(D) + P.S.inject, kSAttn);
    else
      wg_wait(sync_of(P), stage_ctr(P, l, kCQkv), P.S.t_qkv + P.S.inject, kSAttn);
  };
  if (any) {
    attn_copy_tiles(P, l, a, smem, !P.S.wait);
    wait_input(a.kvh);
  } else {
    idle_hook();
  }
  trace_ev(P, l, kSAttn, 1, wg);
  // the item loop of one shape (the dispatch stays outside the loop, so each
  // loop's hoisted index math is computed on its own path only)
  auto items = [&](auto shape) {
    for (int it = wg;;) {
      attn_item<MULTI, decltype(shape)::g, decltype(shape)::dh>(P, l, a, smem);
      __syncthreads();  // LDS is reused by the next item
      it += nwg;
      if (!attn_item_at<MULTI>(P, sc, T, it, a)) break;
      attn_copy_tiles(P, l, a, smem, false);
      if (P.S.tile_sync) wait_input(a.kvh);
    }
  };
  // the shapes of the Llama-1B, 8B and 70B configurations run with their
  // index math folded; any other shape takes the general form
  if (any) {
    if (D.group == 4 && D.d == 64)
      items(AttnShape<4, 64>{});
    else if (D.group == 4 && D.d == 128)
      items(AttnShape<4, 128>{});
    else if (D.group == 8 && D.d == 128)
      items(AttnShape<8, 128>{});
    else
      items(AttnShape<0, 0>{});
  }
  // combine phase (long context): once every item has stored its partial
  // results, the (row, kv head) combines are dealt to the whole grid instead
  // of running one after another in whichever workgroups arrived last
  if (__builtin_amdgcn_readfirstlane(sc.attn_phase) != 0) {
    const int n_items = __builtin_amdgcn_readfirstlane(sc.attn_items);
    wg_wait(sync_of(P), aph_ctr(P, l, 0), (uint32_t)n_items, kSAttn);
    // the last workgroup past the wait clears the item counter for the next
    // layer (every other one has passed it)
    if (tid() == 0) sc.flag[2] = last_arriver(aph_ctr(P, l, 1), wg, nwg);
    __syncthreads();
    if (sc.flag[2] && tid() < kLeaves)
      __hip_atomic_store(aph_ctr(P, l, 0) + tid() * kLeafStride, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    const int M = MULTI ? P.S.M : 1;
    for (int u = wg; u < P.S.B * D.nkv; u += nwg) {
      const int b = u / D.nkv, kvh = u - b * D.nkv, slot = b / M;
      const int p = min(sc.pos[slot * M] + (b - slot * M), D.max_seq - 1);
      const int ns = (p + T) / T;
      if (ns > 1) {
        if (D.group * D.d > (int)blockDim.x)
          attn_combine_unit<2>(P, b, kvh, ns);
        else
          attn_combine_unit<1>(P, b, kvh, ns);
        signal_if(P, stage_ctr(P, l, kCAttn), u);
      }
    }
  }
  (void)D;
  trace_ev(P, l, kSAttn, 3, wg);
}

// ----------------------------------------------------------- O-proj

template <int NB, int MR = kMfmaRingSmall>
__device__ __forceinline__ void stage_o(const Params& P, int l, int wg, int nwg, char* smem) {
  constexpr int NR = kNrO, UC = kUcO;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int rows_total = D.H, K = D.qd, B = P.S.B;
  const uint16_t* Wm = layer_w(P, l, P.W.o_wo);
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  trace_ev(P, l, kSO, 0, wg);
  const XSrc src{P.K.ao, K, nullptr, nullptr, 0};
  // residual input: the layer input (the embedding row for layer 0)
  const float* xa = P.K.xa;
  const uint16_t* emb = P.W.embed;
  const int* tok = P.S.tokens;
  float* xb = P.K.xb;
  auto residual = [&](int bb, int row) -> float {
    if (l == 0) {
      int tk = tok[bb];
      tk = ((unsigned)tk < (unsigned)D.V) ? tk : 0;
      return bf16f(emb[(int64_t)tk * D.H + row]);
    }
    return ld_coh(xa + (int64_t)bb * D.H + row);
  };
  // VALU engine: the residuals of this wave's first task are loaded before
  // the readiness wait (the layer input is complete once this layer's QKV
  // stage has run), so the epilogue does not wait for them
  const int t0 = wg * nwaves() + wave_id();
  float pre[NR][NB];
  auto wait = [&](int = 0, int = 0) {
    if constexpr (NB < kMfmaMinBatch) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int row = t0 * NR + r;
          pre[r][b] = (b < B && row < rows_total && lane == ((r * NB + b) & (kWave - 1)))
                          ? residual(b, row)
                          : 0.f;
        }
    }
    if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, l, kCAttn), P.S.t_attn, kSO);
    trace_ev(P, l, kSO, 1, wg);
  };
  HeldStores<(NB > 1)> held;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch&) {
    const int base = held.reserve(NR * NB);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NR + r;
        if (b < nb && row < rows_total && lane == base + r * NB + b) {
          const int bb = b0 + b;
          const float res = (t == t0 && b0 == 0) ? pre[r][b] : residual(bb, row);
          held.hold(xb + (int64_t)bb * D.H + row, res + acc[r][b]);
        }
      }
  };
  const uint32_t wbytes = (uint32_t)((int64_t)rows_total * K * 2);
  if constexpr (NB >= kMfmaMinBatch) {
    // x' = x + Wo . o, stored as fp32 (the Down stage's residual) and as
    // fragments with the SwiGLU stage's norm gain, with its sums of squares
    const uint16_t* gm = layer_w(P, l, P.W.o_mlp_norm);
    auto epe = [&](int tile, int r, int b, int, int, const float* v) -> float {
      const int row = tile * 16 + r;
      if (row >= rows_total) return 0.f;
      float res;
      if (l == 0) {
        int tk = tok[b];
        tk = ((unsigned)tk < (unsigned)D.V) ? tk : 0;
        res = bf16f(emb[(int64_t)tk * D.H + row]);
      } else {
        res = ld_coh(xa + (int64_t)b * D.H + row);
      }
      const float x = res + v[0];
      st_coh(xb + (int64_t)b * D.H + row, x);
      st_coh_u(P.K.xb_f + frag_word(b, row, D.Hp), split_pair(x * bf16f(gm[row])));
      return x;
    };
    XSrc fs{nullptr, K, nullptr, nullptr, 0};
    fs.frag = P.K.ao_f;
    fs.kp = D.qdp;
    const int ntile = (rows_total + 15) / 16;
    const SplitK sk{P.K.mpart, P.K.mctr, kSplitK<NB, MR> ? mfma_splits(ntile, K, nwg) : 1};
    mfma_stage_frag<kMfmaNbt<NB, MR>, 1, MR>(MatRows{Wm, {Wm, Wm}, rows_total, K}, ntile, K, Wm,
                                             wbytes, fs, false, D.eps, B, P.S.x_cap, wait, epe,
                                             [](int, int) {}, wg, nwg, smem, sk, false, P.K.ss_b,
                                             D.Ht);
  } else {
    gemv_stage<NR, UC, NB, kPfO, 1, kKcMode<NB, MR>>(rowfn, (rows_total + NR - 1) / NR, K, Wm, wbytes, src, nullptr,
                                 false, D.eps, B, batch_tile(P, K, NB), wait, epi, wg, nwg, smem,
                                 (uint32_t)min((size_t)P.S.x_cap, row_stage_bytes<NB>(P)));
    held.flush();
  }
  trace_ev(P, l, kSO, 2, wg);
  signal_if(P, stage_ctr(P, l, kCO), wg);
  trace_ev(P, l, kSO, 3, wg);
}

// -------------------------------------------------------- fused SwiGLU

// A task holds kPairsGu (gate, up) row pairs.  The two tilings of the fused
// stage ("Deep Kernel Fusion for Transformers", Key points, "Fusion scope"):
//  - column-major (weight reuse, the default): each weight tile, once in
//    registers, is multiplied with every staged batch row, so the weights
//    stream once per step;
//  - row-major (activation reuse): one batch tile (a single row on the VALU
//    engine, 16 rows on the MFMA engine) stays staged while the whole weight
//    stream passes it, so the weights stream once per batch tile (the repeat
//    passes read what the first left in the memory-side cache when it fits).
// Both add the same numbers in the same order (bitwise-equal results); they
// coincide at batch 1 and, on the MFMA engine, at 16 rows.
// SwiGLU task t: gate rows and up rows t * kPairsGu .. + kPairsGu (gate and
// up lie in one layer block, so one buffer covers both).
struct GuRows {
  const uint16_t* Wg;
  const uint16_t* Wu;
  int I, K;
  __device__ __forceinline__ void operator()(int t, const uint16_t* (&rows)[2 * kPairsGu]) const {
#pragma unroll
    for (int r = 0; r < kPairsGu; ++r) {
      const int row = t * kPairsGu + r;
      rows[r] = row < I ? Wg + (int64_t)row * K : nullptr;
      rows[kPairsGu + r] = row < I ? Wu + (int64_t)row * K : nullptr;
    }
  }
};
using GuBlock = WBlock<2 * kPairsGu, kUcGu>;
using GuStream = WStream<2 * kPairsGu, kUcGu, GuRows>;

__device__ __forceinline__ GuRows gu_rows(const Params& P, int l) {
  return GuRows{layer_w(P, l, P.W.o_wg), layer_w(P, l, P.W.o_wu), P.D.I, P.D.H};
}
__device__ __forceinline__ int gu_tiles(const Params& P) { return (P.D.I + kPairsGu - 1) / kPairsGu; }

// Idle-time SwiGLU blocks of the persistent kernel: besides the register
// ring, up to kGuLdsBlocks more blocks per wave are copied into the top of
// the LDS staging area, as far as the staged input rows of the O and SwiGLU
// stages leave room (those rows sit at the bottom of the same area).
constexpr int kGuLdsBlocks = 2;
constexpr int kGuBlockBytes = kBlockLdsBytes<2 * kPairsGu, kUcGu>;

template <int NB>
__device__ __forceinline__ int gu_lds_blocks(const Params& P) {
  const size_t need = row_stage_bytes<NB>(P);
  const size_t room = P.S.x_cap > need ? P.S.x_cap - need : 0;
  return min(kGuLdsBlocks, (int)(room / ((size_t)kGuBlockBytes * nwaves())));
}
__device__ __forceinline__ char* gu_lds_base(const Params& P, char* smem, int nl) {
  const size_t per_wave = (size_t)nl * kGuBlockBytes;
  return smem + kScratchBytes + P.S.x_cap - nwaves() * per_wave + wave_id() * per_wave;
}

// Issue this wave's first SwiGLU weight blocks of layer l into the ring and
// copy the next ones into LDS (the persistent kernel calls it while attention
// runs).  Returns the number of blocks per wave placed in LDS.
template <int NB>
__device__ __forceinline__ int gu_prefetch(const Params& P, int l, int wg, int nwg,
                                           GuBlock (&ring)[kPfGu], char* smem) {
  const GuRows rows = gu_rows(P, l);
  const GuStream ws(rows, gu_tiles(P), P.D.H, layer_w(P, l, 0), (uint32_t)(P.W.layer_stride * 2),
                    wg, nwg);
  gemv_prefetch(ws, ring, true);
  const int nl = gu_lds_blocks<NB>(P);
  char* dst = gu_lds_base(P, smem, nl);
  for (int q = 0; q < nl; ++q) ws.copy_to_lds(kPfGu + q, dst + q * kGuBlockBytes, lane_id());
  return nl;
}

template <int NB, int MR = kMfmaRingSmall>
__device__ __forceinline__ void stage_gu(const Params& P, int l, int wg, int nwg, char* smem,
                         GuBlock (&ring)[kPfGu], bool prefetched, int lds_blocks = 0) {
  constexpr int NP = kPairsGu, NR = 2 * kPairsGu;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int I = D.I, K = D.H, B = P.S.B;
  const GuRows rows = gu_rows(P, l);
  const GuStream ws(rows, gu_tiles(P), K, layer_w(P, l, 0), (uint32_t)(P.W.layer_stride * 2), wg,
                    nwg);
  trace_ev(P, l, kSGu, 0, wg);
  Scratch& scg = *reinterpret_cast<Scratch*>(smem);
  counts_clear(P, scg, D.nhc);
  const bool counting = tile_counting(P);
  auto wait = [&](int = 0, int = 0) {
    if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, l, kCO), P.S.t_o, kSGu);
    trace_ev(P, l, kSGu, 1, wg);
  };
  const XSrc src{P.K.xb, K, nullptr, nullptr, 0};
  float* h = P.K.hbuf;
  HeldStores<(NB > 1)> held;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch& sc) {
    const int base = held.reserve(NP * NB);
#pragma unroll
    for (int r = 0; r < NP; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NP + r;
        if (b < nb && row < I && lane == base + r * NB + b) {
          const float a = acc[r][b] * sc.rs[b], u = acc[NP + r][b] * sc.rs[b];
          held.hold(h + (int64_t)(b0 + b) * I + row, a / (1.0f + expf(-a)) * u);
        }
      }
    if (counting && b0 == 0 && lane == 0) {
#pragma unroll
      for (int r = 0; r < NP; ++r)
        if (t * NP + r < I) count_row(sc, (t * NP + r) / kHChunk);
    }
  };
  const int bw = (P.S.gu_variant == kGuRow) ? 1 : batch_tile(P, K, NB);
  if constexpr (NB >= kMfmaMinBatch) {
    (void)ring;
    (void)prefetched;
    (void)bw;
    Scratch& sc = *reinterpret_cast<Scratch*>(smem);
    auto epe = [&](int tile, int r, int b, int bl, int, const float* v) -> float {
      const int row = tile * 16 + r;
      if (row >= I) return 0.f;
      const float a = v[0] * sc.rs[bl], u = v[1] * sc.rs[bl];
      // for the Down stage (MFMA engine too): fragments of split-bf16 pairs
      st_coh_u(P.K.h_f + frag_word(b, row, D.Ip), split_pair(a / (1.0f + expf(-a)) * u));
      if (counting && b == 0) count_row(sc, row / kHChunk);
      return 0.f;
    };
    (void)h;
    XSrc fs{nullptr, K, nullptr, nullptr, 0};  // the O stage's output as fragments
    fs.frag = P.K.xb_f;
    fs.kp = D.Hp;
    fs.ss = P.K.ss_b;
    fs.ss_n = fs.ss_ld = D.Ht;
    mfma_stage_frag<kMfmaNbt<NB, MR>, 2, MR>(
        MatRows{layer_w(P, l, 0), {rows.Wg, rows.Wu}, I, K}, (I + 15) / 16, K, layer_w(P, l, 0),
        (uint32_t)(P.W.layer_stride * 2), fs, true, D.eps, B, P.S.x_cap, wait, epe,
        [](int, int) {}, wg, nwg, smem, SplitK{nullptr, nullptr, 1}, P.S.gu_variant == kGuRow);
  } else {
    gemv_run<NR, kUcGu, NB, kPfGu>(ws, ring, prefetched, src, layer_w(P, l, P.W.o_mlp_norm), true,
                                   D.eps, B, bw, wait, epi, smem,
                                   lds_blocks > 0 ? gu_lds_base(P, smem, lds_blocks) : nullptr,
                                   lds_blocks);
    held.flush();
  }
  trace_ev(P, l, kSGu, 2, wg);
  if (counting)
    wg_signal_counts(P, scg, hc_ctr, l, D.nhc, wg);
  else
    signal_if(P, stage_ctr(P, l, kCGu), wg);
  trace_ev(P, l, kSGu, 3, wg);
}

// ------------------------------------------------- unfused-MLP ablation
//
// The fused SwiGLU stage measured against two unfused forms of the same
// first MLP stage (the fused form, Deep Kernel Fusion for Transformers, "Key
// points" / "Fusion scope", never writes the projections out):
//  - two kernels: one GEMV over the gate and up rows writing both
//    projections (kMlpBoth), then silu(g) * u;
//  - four kernels: the gate GEMV (kMlpGate), the up GEMV (kMlpUp), silu(g)
//    in place, then the product.
// Every form adds the same numbers in the same order as the fused stage (the
// same staged input and norm factor, the same chunk order and reductions per
// row, the same activation formula), so all three give bitwise-equal
// results.  Whole-kernel-wait launches only: they wait on nothing and signal
// nothing.  (The kMlp* codes are in ld_params.hpp.)

template <int NB, int MR = kMfmaRingSmall>
__device__ __forceinline__ void stage_mlp_proj(const Params& P, int l, int which, int wg, int nwg,
                                               char* smem) {
  const Dims& D = P.D;
  const int lane = lane_id();
  const int I = D.I, K = D.H, B = P.S.B;
  const XSrc src{P.K.xb, K, nullptr, nullptr, 0};
  const uint16_t* base = layer_w(P, l, 0);
  const uint32_t bytes = (uint32_t)(P.W.layer_stride * 2);
  const uint16_t* gain = layer_w(P, l, P.W.o_mlp_norm);
  const int bw = batch_tile(P, K, NB);
  auto nowait = [] {};
  if constexpr (NB >= kMfmaMinBatch) {
    // MFMA engine: the fused stage's call (the O stage's fragments and sums
    // of squares, the same tiling and K order), with an epilogue that stores
    // the scaled projections instead of the activation
    (void)lane, (void)src, (void)gain, (void)bw, (void)nowait;
    Scratch& sc = *reinterpret_cast<Scratch*>(smem);
    XSrc fs{nullptr, K, nullptr, nullptr, 0};
    fs.frag = P.K.xb_f;
    fs.kp = D.Hp;
    fs.ss = P.K.ss_b;
    fs.ss_n = fs.ss_ld = D.Ht;
    const bool row_major = P.S.gu_variant == kGuRow;
    auto none = [](int = 0, int = 0) {};
    if (which == kMlpBoth) {
      const GuRows rows = gu_rows(P, l);
      auto epe = [&](int tile, int r, int b, int bl, int, const float* v) -> float {
        const int row = tile * 16 + r;
        if (row < I) {
          st_coh(P.K.gbuf + (int64_t)b * I + row, v[0] * sc.rs[bl]);
          st_coh(P.K.ubuf + (int64_t)b * I + row, v[1] * sc.rs[bl]);
        }
        return 0.f;
      };
      mfma_stage_frag<kMfmaNbt<NB, MR>, 2, MR>(
          MatRows{base, {rows.Wg, rows.Wu}, I, K}, (I + 15) / 16, K, base, bytes, fs, true, D.eps,
          B, P.S.x_cap, none, epe, [](int, int) {}, wg, nwg, smem, SplitK{nullptr, nullptr, 1},
          row_major);
    } else {
      const uint16_t* Wm = which == kMlpGate ? layer_w(P, l, P.W.o_wg) : layer_w(P, l, P.W.o_wu);
      float* out = which == kMlpGate ? P.K.gbuf : P.K.ubuf;
      auto epe = [&](int tile, int r, int b, int bl, int, const float* v) -> float {
        const int row = tile * 16 + r;
        if (row < I) st_coh(out + (int64_t)b * I + row, v[0] * sc.rs[bl]);
        return 0.f;
      };
      mfma_stage_frag<kMfmaNbt<NB, MR>, 1, MR>(
          MatRows{base, {Wm, Wm}, I, K}, (I + 15) / 16, K, base, bytes, fs, true, D.eps, B,
          P.S.x_cap, none, epe, [](int, int) {}, wg, nwg, smem, SplitK{nullptr, nullptr, 1},
          row_major);
    }
    return;
  }
  if (which == kMlpBoth) {
    constexpr int NP = kPairsGu, NR = 2 * kPairsGu;
    const GuRows rows = gu_rows(P, l);
    const GuStream ws(rows, gu_tiles(P), K, base, bytes, wg, nwg);
    HeldStores<(NB > 1)> held_g, held_u;  // the stores wait for the end of the stream, as in the fused stage
    auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch& sc) {
      const int base = held_g.reserve(NP * NB);
      held_u.reserve(NP * NB);
#pragma unroll
      for (int r = 0; r < NP; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int row = t * NP + r;
          if (b < nb && row < I && lane == base + r * NB + b) {
            held_g.hold(P.K.gbuf + (int64_t)(b0 + b) * I + row, acc[r][b] * sc.rs[b]);
            held_u.hold(P.K.ubuf + (int64_t)(b0 + b) * I + row, acc[NP + r][b] * sc.rs[b]);
          }
        }
    };
    GuBlock ring[kPfGu];
    gemv_run<NR, kUcGu, NB, kPfGu>(ws, ring, false, src, gain, true, D.eps, B, bw, nowait, epi, smem);
    held_g.flush();
    held_u.flush();
  } else {
    const uint16_t* Wm = which == kMlpGate ? layer_w(P, l, P.W.o_wg) : layer_w(P, l, P.W.o_wu);
    float* out = which == kMlpGate ? P.K.gbuf : P.K.ubuf;
    auto rowfn = [&](int t, const uint16_t* (&rows)[1]) {
      rows[0] = t < I ? Wm + (int64_t)t * K : nullptr;
    };
    HeldStores<(NB > 1)> held;
    auto epi = [&](int t, int b0, int nb, float (&acc)[1][NB], Scratch& sc) {
      const int base = held.reserve(NB);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (b < nb && t < I && lane == base + b)
          held.hold(out + (int64_t)(b0 + b) * I + t, acc[0][b] * sc.rs[b]);
    };
    gemv_stage<1, kUcGu, NB, kPfGu>(rowfn, I, K, base, bytes, src, gain, true, D.eps, B, bw, nowait,
                                    epi, wg, nwg, smem);
    held.flush();
  }
}

// The elementwise kernels of the unfused forms over [B][I]: silu(g) in place
// (kMlpSilu), h = g * u (kMlpMul), or h = silu(g) * u (kMlpSiluMul).  From 16
// rows h goes where the Down stage's MFMA engine reads it, as the fused
// stage writes it: split-bf16 pairs in B-fragment order.
__device__ __forceinline__ void mlp_elementwise(const Params& P, int op, int64_t i) {
  float* g = P.K.gbuf;
  const float a = ld_coh(g + i);
  if (op == kMlpSilu) {
    st_coh(g + i, a / (1.0f + expf(-a)));
  } else {
    const float u = ld_coh(P.K.ubuf + i);
    const float s = op == kMlpSiluMul ? a / (1.0f + expf(-a)) : a;
    if (P.S.B >= kMfmaMinBatch) {
      const int b = (int)(i / P.D.I), row = (int)(i - (int64_t)b * P.D.I);
      st_coh_u(P.K.h_f + frag_word(b, row, P.D.Ip), split_pair(s * u));
    } else {
      st_coh(P.K.hbuf + i, s * u);
    }
  }
}

// ---------------------------------------------------------- Down-proj

template <int NB, int MR = kMfmaRingSmall>
__device__ __forceinline__ void stage_d(const Params& P, int l, int wg, int nwg, char* smem) {
  constexpr int NR = kNrD, UC = kUcD;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int rows_total = D.H, K = D.I, B = P.S.B;
  const uint16_t* Wm = layer_w(P, l, P.W.o_wd);
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  trace_ev(P, l, kSD, 0, wg);
  const XSrc src{P.K.hbuf, K, nullptr, nullptr, 0};
  const float* xb = P.K.xb;
  float* xa = P.K.xa;
  // VALU engine: the residuals of this wave's first task (the O stage's
  // output, complete before the SwiGLU stage this one waits for) are loaded
  // before the readiness wait
  const int t0 = wg * nwaves() + wave_id();
  float pre[NR][NB];
  auto wait = [&](int k0 = 0, int k1 = 0x7FFFFFFF) {
    if constexpr (NB < kMfmaMinBatch) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int row = t0 * NR + r;
          pre[r][b] = (b < B && row < rows_total && lane == ((r * NB + b) & (kWave - 1)))
                          ? ld_coh(xb + (int64_t)b * D.H + row)
                          : 0.f;
        }
    }
    if (!P.S.wait) {
      if (P.S.tile_sync) {
        // only the SwiGLU output chunks of the workgroup's K range [k0, k1)
        // (all of them for the VALU engine), polled together
        const int c0 = k0 / kHChunk, c1 = min(D.nhc, (min(k1, D.I) + kHChunk - 1) / kHChunk);
        const uint32_t n = P.S.n_sig;
        wg_wait_all(sync_of(P), hc_ctr(P, l, c0), c1 - c0,
                    [&](int i) { return n * h_chunk_rows(D, c0 + i); }, kSD);
      } else {
        wg_wait(sync_of(P), stage_ctr(P, l, kCGu), P.S.t_gu, kSD);
      }
    }
    trace_ev(P, l, kSD, 1, wg);
  };
  HeldStores<(NB > 1)> held;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch&) {
    const int base = held.reserve(NR * NB);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NR + r;
        if (b < nb && row < rows_total && lane == base + r * NB + b) {
          const int64_t o = (int64_t)(b0 + b) * D.H + row;
          const float res = (t == t0 && b0 == 0) ? pre[r][b] : ld_coh(xb + o);
          held.hold(xa + o, res + acc[r][b]);
        }
      }
  };
  const uint32_t wbytes = (uint32_t)((int64_t)rows_total * K * 2);
  if constexpr (NB >= kMfmaMinBatch) {
    // x'' = x' + Wd . h, stored as fp32 (the next layer's residual) and as
    // fragments with the norm gain of its consumer (the next layer's QKV
    // stage, or the LM head after the last layer), with its sums of squares
    const uint16_t* gn = l + 1 < D.L ? layer_w(P, l + 1, P.W.o_attn_norm) : P.W.final_norm;
    auto epe = [&](int tile, int r, int b, int, int, const float* v) -> float {
      const int row = tile * 16 + r;
      if (row >= rows_total) return 0.f;
      const int64_t o = (int64_t)b * D.H + row;
      const float x = ld_coh(xb + o) + v[0];
      st_coh(xa + o, x);
      st_coh_u(P.K.xa_f + frag_word(b, row, D.Hp), split_pair(x * bf16f(gn[row])));
      return x;
    };
    XSrc fs{nullptr, K, nullptr, nullptr, 0};  // the SwiGLU output as fragments
    fs.frag = P.K.h_f;
    fs.kp = D.Ip;
    const int ntile = (rows_total + 15) / 16;
    const SplitK sk{P.K.mpart, P.K.mctr + kMctrPasses * ntile,
                    kSplitK<NB, MR> ? mfma_splits(ntile, K, nwg) : 1};
    mfma_stage_frag<kMfmaNbt<NB, MR>, 1, MR>(MatRows{Wm, {Wm, Wm}, rows_total, K}, ntile, K, Wm,
                                             wbytes, fs, false, D.eps, B, P.S.x_cap, wait, epe,
                                             [](int, int) {}, wg, nwg, smem, sk, false, P.K.ss_a,
                                             D.Ht);
  } else {
    gemv_stage<NR, UC, NB, kPfD, kStageGroupsD<NB>, kKcMode<NB, MR>>(rowfn, (rows_total + NR - 1) / NR, K, Wm,
                                                     wbytes, src, nullptr, false, D.eps, B,
                                                     batch_tile(P, K, NB), wait, epi, wg, nwg,
                                                     smem, P.S.x_cap);
    held.flush();
  }
  trace_ev(P, l, kSD, 2, wg);
  signal_if(P, stage_ctr(P, l, kCD), wg);
  trace_ev(P, l, kSD, 3, wg);
}

// ------------------------------------------------- LM head + argmax

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Per-wave running argmax of the LM head, placed after the staged inputs.
struct Best {
  float v[kMaxWaves][64];
  int i[kMaxWaves][64];
};
constexpr int kBestBytes = (int)sizeof(Best);

template <int NB, int MR = kMfmaRingSmall>
__device__ __forceinline__ void stage_lm(const Params& P, int wg, int nwg, char* smem) {
  constexpr int NR = kNrLm, UC = kUcLm;
  const Dims& D = P.D;
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  Best& bs = *reinterpret_cast<Best*>(smem + kScratchBytes + P.S.x_cap);
  const int lane = lane_id(), wave = wave_id();
  const int rows_total = D.V, K = D.H, B = P.S.B;
  const uint16_t* Wm = P.W.lm;
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  trace_ev(P, D.L, kSLm, 0, wg);
  auto wait = [&](int = 0, int = 0) {
    if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, D.L - 1, kCD), P.S.t_d, kSLm);
    trace_ev(P, D.L, kSLm, 1, wg);
  };
  for (int b = lane; b < 64; b += kWave) {
    bs.v[wave][b] = -INFINITY;
    bs.i[wave][b] = 0x7FFFFFFF;
  }
  const XSrc src{P.K.xa, K, nullptr, nullptr, 0};
  float* logits = P.S.logits;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch& s) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        float bv = bs.v[wave][b0 + b];
        int bi = bs.i[wave][b0 + b];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int row = t * NR + r;
          if (row < rows_total) {
            const float v = acc[r][b] * s.rs[b];
            if (lane == ((r * NB + b) & (kWave - 1))) logits[(int64_t)(b0 + b) * D.V + row] = v;
            if (better(v, row, bv, bi)) {
              bv = v;
              bi = row;
            }
          }
        }
        if (lane == 0) {
          bs.v[wave][b0 + b] = bv;
          bs.i[wave][b0 + b] = bi;
        }
      }
    }
  };
  const uint32_t wbytes = (uint32_t)((int64_t)rows_total * K * 2);
  if constexpr (NB >= kMfmaMinBatch) {
    // logits, and each lane's running best per batch tile (the lane holds one
    // batch row of each tile); merged into the wave's slots per batch pass
    constexpr int NBT = kMfmaNbt<NB, MR>;
    float bv[NBT];
    int bi[NBT];
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt) {
      bv[bt] = -INFINITY;
      bi[bt] = 0x7FFFFFFF;
    }
    auto epe = [&](int tile, int r, int b, int bl, int bt, const float* v) -> float {
      const int row = tile * 16 + r;
      if (row >= rows_total) return 0.f;
      const float val = v[0] * sc.rs[bl];
      logits[(int64_t)b * D.V + row] = val;
      if (better(val, row, bv[bt], bi[bt])) {
        bv[bt] = val;
        bi[bt] = row;
      }
      return 0.f;
    };
    auto pass_end = [&](int b0, int nb) {
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt) {
        float v = bv[bt];
        int i = bi[bt];
        // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same batch row
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
          const float ov = __shfl_xor(v, off, kWave);
          const int oi = __shfl_xor(i, off, kWave);
          if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
          }
        }
        const int bl = bt * 16 + lane;
        if (lane < 16 && bl < nb) {
          bs.v[wave][b0 + bl] = v;
          bs.i[wave][b0 + bl] = i;
        }
        bv[bt] = -INFINITY;
        bi[bt] = 0x7FFFFFFF;
      }
    };
    XSrc fs{nullptr, K, nullptr, nullptr, 0};  // the last Down stage's output as fragments
    fs.frag = P.K.xa_f;
    fs.kp = D.Hp;
    fs.ss = P.K.ss_a;
    fs.ss_n = fs.ss_ld = D.Ht;
    mfma_stage_frag<NBT, 1, MR>(MatRows{Wm, {Wm, Wm}, rows_total, K}, (rows_total + 15) / 16, K,
                                Wm, wbytes, fs, true, D.eps, B, P.S.x_cap, wait, epe, pass_end, wg,
                                nwg, smem);
  } else {
    gemv_stage<NR, UC, NB, kPfLm>(rowfn, (rows_total + NR - 1) / NR, K, Wm, wbytes, src,
                                  P.W.final_norm, true, D.eps, B, batch_tile(P, K, NB), wait, epi,
                                  wg, nwg, smem);
  }
  trace_ev(P, D.L, kSLm, 2, wg);
  __syncthreads();
  // this workgroup's best per sequence -> partials
  for (int b = tid(); b < B; b += blockDim.x) {
    float bv = bs.v[0][b];
    int bi = bs.i[0][b];
    for (int w = 1; w < nwaves(); ++w)
      if (better(bs.v[w][b], bs.i[w][b], bv, bi)) {
        bv = bs.v[w][b];
        bi = bs.i[w][b];
      }
    st_coh(P.K.lm_val + (int64_t)wg * D.max_batch + b, bv);
    st_coh_i(P.K.lm_idx + (int64_t)wg * D.max_batch + b, bi);
  }
  wave_drain();
  __syncthreads();
  if (tid() == 0) sc.flag[1] = last_arriver(P.K.lm_ctr, wg, nwg);
  __syncthreads();
  trace_ev(P, D.L, kSLm, 3, wg);
  if (!sc.flag[1] || P.S.next == nullptr) return;
  // last arriver: reduce the partials of every workgroup, per sequence.  Wave
  // w takes rows w, w + nw, ... four at a time, its lanes reading the
  // partials of workgroups lane, lane + 64, ... (every load of a round issued
  // before any is used; a clamped index past the end reads a valid partial
  // that is not compared), then a wave-wide argmax.  The comparison (larger
  // value, then lower index; NaN never wins) makes the result independent of
  // the order.
  constexpr int RB = 4, WU = 4;  // rows and workgroup partials per lane per round
  const int nw = nwaves();
  for (int r0 = wave; r0 < B; r0 += RB * nw) {
    float bv[RB];
    int bi[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      bv[k] = -INFINITY;
      bi[k] = 0x7FFFFFFF;
    }
    for (int w0 = lane; w0 < nwg; w0 += WU * kWave) {
      float v[RB][WU];
      int ix[RB][WU];
#pragma unroll
      for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int u = 0; u < WU; ++u) {
          const int b = min(r0 + k * nw, B - 1), w = min(w0 + u * kWave, nwg - 1);
          v[k][u] = ld_coh(P.K.lm_val + (int64_t)w * D.max_batch + b);
          ix[k][u] = ld_coh_i(P.K.lm_idx + (int64_t)w * D.max_batch + b);
        }
#pragma unroll
      for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int u = 0; u < WU; ++u)
          if (w0 + u * kWave < nwg && better(v[k][u], ix[k][u], bv[k], bi[k])) {
            bv[k] = v[k][u];
            bi[k] = ix[k][u];
          }
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv[k], off, kWave);
        const int oi = __shfl_xor(bi[k], off, kWave);
        if (better(ov, oi, bv[k], bi[k])) {
          bv[k] = ov;
          bi[k] = oi;
        }
      }
      const int b = r0 + k * nw;
      if (lane == 0 && b < B) P.S.next[b] = (bi[k] == 0x7FFFFFFF) ? 0 : bi[k];
    }
  }
}

}  // namespace ld
