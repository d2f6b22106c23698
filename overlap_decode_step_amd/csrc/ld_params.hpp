// ld_params.hpp - argument blocks shared by the host runtime and the kernels.
// Plain structs passed by value as kernel arguments.
#pragma once

#include <stdint.h>

namespace ld {

// Stage-completion counters: per layer one counter per stage (each counter
// is a set of leaves, see ld_common.hpp).
enum : int { kCQkv = 0, kCAttn = 1, kCO = 2, kCGu = 3, kCD = 4, kStageCtrs = 5 };

// One counter: kLeaves leaf words 128 bytes apart, plus a root slot.
constexpr int kLeaves = 16;
constexpr int kLeafStride = 32;  // uint32 slots between leaves (128 bytes)
constexpr int kCtrWords = (kLeaves + 1) * kLeafStride;

// Tile-granular readiness.  Besides its stage counter, a stage can signal
// row-count counters: the QKV stage one per (layer, kv group), counting the
// q, k and v rows of the group it has written, and the SwiGLU stage one per
// (layer, chunk of kHChunk rows of its output), so that an attention item
// waits only for its own group's projections and the Down stage takes its
// input chunk by chunk (a split-K range waits only for its own chunks).
// A counter's target after n signalling steps is n times the rows it covers.
constexpr int kHChunk = 1024;
constexpr int kMaxTileCtrs = 64;  // kv groups, and chunks, per layer at most

// The norm-free stages of the VALU engine (O, Down) can stage their input in
// column chunks of whole weight blocks: the staging area must hold at least
// one such chunk of one row (8 KB-wide blocks of 8 x 512 bf16 columns, fp32
// inputs); the stages with a deferred norm stage whole rows.
constexpr int kKChunkMinBytes = 8 * 512 * 4;

// Stage ids (watchdog error codes and schedule bookkeeping).  kSMlpProj is
// the projection kernel of the unfused-MLP ablation (kernel lookup only).
enum : int { kSQkv = 1, kSAttn = 2, kSO = 3, kSGu = 4, kSD = 5, kSLm = 6, kSMlpProj = 7 };

// Device error word codes (low byte; a timeout carries the stage id << 8).
constexpr int kErrToken = 1;
constexpr int kErrPos = 2;
constexpr int kErrTimeout = 3;

// Batches from here on take the MFMA engine; smaller ones the VALU engine.
constexpr int kMfmaMinBatch = 16;
// Split-K stages of the MFMA engine (64-row kernels): at most kMaxKSplit K
// ranges, and one last-arriver counter per (batch pass of 16 rows, tile) and
// stage.
constexpr int kMaxKSplit = 4;
constexpr int kMctrPasses = 4;  // batch passes at max_batch 64

// SwiGLU tiling variants (chosen offline per batch size).
enum : int { kGuCol = 0, kGuRow = 1 };

// Unfused-MLP ablation: projection kernels (gate rows, up rows, or both into
// separate outputs) and elementwise ops (silu in place, product, silu-product).
enum : int { kMlpGate = 0, kMlpUp = 1, kMlpBoth = 2 };
enum : int { kMlpSilu = 0, kMlpMul = 1, kMlpSiluMul = 2 };

// K rounded up to whole 32-wide MFMA K steps.
constexpr int round32(int k) { return (k + 31) / 32 * 32; }

// Word offset of element (b, k) of an activation matrix stored in the MFMA
// engine's B-fragment order (see ld_mfma.hpp): 2 KB per (16-row batch tile,
// 32-wide K step), two 1 KB halves, lane l = 16 * ((k / 8) % 4) + b % 16
// holding columns 8 (k / 8) .. + 3 of its row in the first half and + 4 .. + 7
// in the second, 16 bytes each, so one 16-byte load per lane reads a
// contiguous 1 KB.  kp: K rounded up to 32.
constexpr int64_t frag_word(int b, int k, int kp) {
  return ((((int64_t)(b >> 4) * (kp >> 5) + (k >> 5)) * 2 + ((k >> 2) & 1)) * 64 +
          ((((k >> 3) & 3) << 4) | (b & 15))) * 4 +
         (k & 3);
}

struct Dims {
  int L, H, nq, nkv, d, I, V, group;
  int qd, kvd, qkv_rows;
  int max_batch, max_seq;
  int split_len, max_splits;  // longest attention split (LDS tiles), splits per sequence at most
  int tied;
  int Hp, qdp, Ip;  // hidden, n_q * head_dim and intermediate rounded up to 32
  int Ht;           // 16-row output tiles of a hidden-sized projection
  int nhc;          // chunks of kHChunk rows of the SwiGLU output
  float eps;
  float attn_scale;  // 1 / sqrt(head_dim)
};

// Weight arena: every layer block has the same layout.
// Largest weight buffer one buffer resource covers (32-bit byte offsets,
// with room above for the out-of-range offset of masked loads).
constexpr size_t kMaxWeightBuffer = 0xFFFF0000u;

struct Weights {
  const uint16_t* embed;       // [V, H]
  const uint16_t* lm;          // [V, H] (== embed when tied)
  const uint16_t* final_norm;  // [H]
  const uint16_t* layer0;      // first layer block
  int64_t layer_stride;        // elements between layer blocks
  int64_t o_attn_norm, o_wqkv, o_wo, o_mlp_norm, o_wg, o_wu, o_wd;  // offsets in a block
};

struct Work {
  uint16_t* kc;   // K cache [L][maxB][nkv][max_seq][d]
  uint16_t* vc;   // V cache, same layout
  float* xa;      // residual stream after each layer [maxB][H]
  float* xb;      // residual stream after attention [maxB][H]
  float* qkv;     // raw q|k|v projections [maxB][qkv_rows]
  float* ao;      // attention output [maxB][qd]
  float* part;    // attention split partials [maxB][nq][max_splits][d + 2]
  float* hbuf;    // SwiGLU output [maxB][I]
  float* gbuf;    // unfused-MLP ablation: gate projections [maxB][I]
  float* ubuf;    // unfused-MLP ablation: up projections [maxB][I]
  float* lm_val;  // argmax partials [max_wg][maxB]
  int* lm_idx;
  const float* rope;  // [max_seq][d/2][2] (cos, sin)
  uint32_t* ctr;        // stage counters [L][kStageCtrs][counter words]
  uint32_t* lm_ctr;     // LM-head last-arriver counter
  uint32_t* split_ctr;  // attention last-arriver counters [L][maxB][nkv][16]
  uint32_t* mctr;       // split-K last-arriver counters: O, then Down, [kMctrPasses][tiles]
  uint32_t* aph;        // long-context combine phase: per layer, items done, then workgroups past [L][2][counter words]
  uint32_t* qg_ctr;     // QKV rows written per (layer, kv group) [L][nkv][counter words]
  uint32_t* hc_ctr;     // SwiGLU rows written per (layer, chunk) [L][nhc][counter words]
  float* mpart;         // split-K partial tiles [kMaxKSplit][maxB][H]
  // MFMA engine (16 rows and more): activations handed from one of its stages
  // to the next in B-fragment order (frag_word; batch rows padded to 16) as
  // split-bf16 pairs with the consumer's norm gain applied, and the sums of
  // squares of the two residual streams per (row, 16-row output tile)
  uint32_t* xa_f;  // layer output, for the next QKV stage or the LM head [Bp][Hp]
  uint32_t* xb_f;  // O-stage output, for the SwiGLU stage [Bp][Hp]
  uint32_t* ao_f;  // attention output, for the O stage [Bp][qdp]
  uint32_t* h_f;   // SwiGLU output, for the Down stage [Bp][Ip]
  float* ss_a;     // sums of squares of xa [maxB][Ht]
  float* ss_b;     // sums of squares of xb [maxB][Ht]
  int* err;
  uint64_t* trace;  // optional stage timestamps (see trace_ev), nullptr = off
  uint64_t watchdog;
  int max_wg;
};

struct Step {
  const int* tokens;
  const int* pos;
  float* logits;
  int* next;
  int B;
  int wait;        // 1: whole-kernel-wait mode, stream order only (no counter waits)
  int gu_variant;  // kGuCol / kGuRow
  // cumulative counter targets once this step's signals are in
  uint32_t t_qkv, t_attn, t_o, t_gu, t_d, t_lm;
  uint32_t inject;  // debug: added to one wait target to force a watchdog timeout
  uint32_t n_sig;   // signalling steps enqueued so far, this one included
  int tile_sync;    // 1: attention and Down wait on the row-count counters
  uint32_t x_cap;   // bytes of LDS for staged input vectors
  int T;            // attention split length of this step (<= Dims::split_len)
  int Tmax;         // longest split a long context may take (<= Dims::split_len)
  int M;            // tokens per sequence: rows b*M .. b*M + M - 1 are sequence b's
                    // consecutive positions (KV cache slot b); 1 for a decode step
};

struct Params {
  Dims D;
  Weights W;
  Work K;
  Step S;
};

}  // namespace ld
