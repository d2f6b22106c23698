/*
 * ld_oracle.h - CPU oracle for the small-batch decode step of a dense
 * Llama-style decoder.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke
 * check and the benchmark's CPU-baseline leg use it; the GPU library never
 * includes, links or calls it.
 *
 * What it computes.  One decode step per sequence: embedding row, then per
 * layer RMSNorm -> Q/K/V projections -> rotary position embedding -> append
 * K/V to the cache -> grouped-query attention over positions 0..p -> output
 * projection + residual -> RMSNorm -> SwiGLU (Up and Gate projections, SiLU
 * on the gate, elementwise product) -> Down projection + residual; then the
 * final RMSNorm, the LM head and a greedy argmax.
 *
 * Sources.  The workload is single-sequence (batch-1) decode of Llama-3.2-1B,
 * which is memory-bound (Hazy Research, "Look Ma, No Bubbles! Designing a
 * Low-Latency Megakernel for Llama-1B", introduction).  The MLP is two stages:
 * a first stage of Up and Gate GEMMs, the SiLU activation and the elementwise
 * product, and a separate Down projection ("Deep Kernel Fusion for
 * Transformers", Summary; Key points, "Fusion scope"); SiLU gates the Gate
 * branch as in Shazeer's GLU variants, which that page lists among its
 * references.  The pages print no formula for RMSNorm, RoPE or attention; the
 * oracle takes the standard Llama definitions (pre-norm residual blocks,
 * rotate-half RoPE pairs (i, i + d/2), 1/sqrt(d) scaled softmax attention,
 * contiguous GQA groups), one reading per silent point.
 *
 * Arithmetic.  Weights and the KV cache are bf16; everything else is `real`,
 * which is float in the reference build (liblo32) and double in the
 * self-check build (liblo64).  Every dot product sums in ascending index
 * order.  No blocking, fusion or reordering.
 *
 * Parity pins: every function below is pinned by closed forms, invariants or
 * brute force in the CPU test suite (see the test module for the oracle).
 */
#ifndef LD_ORACLE_H
#define LD_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifndef LO_REAL
#define LO_REAL float
#endif
typedef LO_REAL lo_real;

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, tied;
  float rms_eps, rope_theta;
} lo_config;

/* Weight kinds for lo_weight(). */
enum {
  LO_W_EMBED = 0,     /* [vocab, hidden] */
  LO_W_ATTN_NORM = 1, /* [hidden] per layer */
  LO_W_Q = 2,         /* [n_q*d, hidden] */
  LO_W_K = 3,         /* [n_kv*d, hidden] */
  LO_W_V = 4,         /* [n_kv*d, hidden] */
  LO_W_O = 5,         /* [hidden, n_q*d] */
  LO_W_MLP_NORM = 6,  /* [hidden] */
  LO_W_GATE = 7,      /* [intermediate, hidden] */
  LO_W_UP = 8,        /* [intermediate, hidden] */
  LO_W_DOWN = 9,      /* [hidden, intermediate] */
  LO_W_FINAL_NORM = 10, /* [hidden] */
  LO_W_LM_HEAD = 11   /* [vocab, hidden]; the embedding when tied */
};

typedef struct lo_model lo_model;
typedef struct lo_kv lo_kv;

/* bf16 helpers (round to nearest, ties to even). */
uint16_t lo_bf16_round(float f);
float lo_bf16_widen(uint16_t b);

/* Model: weights zero, norm gains 1.0.  NULL on bad config or no memory. */
lo_model* lo_model_create(const lo_config* cfg);
void lo_model_free(lo_model* m);
/* Fill every matrix from the seeded generator, ~N(0, w_std); gains stay 1.0. */
int lo_model_synth(lo_model* m, uint64_t seed, float w_std);
/* Mutable bf16 storage of one weight (row-major); rows/cols out. */
uint16_t* lo_weight(lo_model* m, int kind, int layer, int64_t* rows, int64_t* cols);

/* KV cache [layer][seq][kv_head][pos][d], bf16, zero-filled. */
lo_kv* lo_kv_create(const lo_config* cfg, int32_t max_batch, int32_t max_seq);
void lo_kv_free(lo_kv* kv);
/* Positions 0..prefill_len[b]-1 of every (layer, seq, kv head) from the
 * seeded generator, ~N(0, kv_std). */
int lo_kv_synth(lo_kv* kv, uint64_t seed, float kv_std, const int32_t* prefill_len);
/* As lo_kv_synth, but cache slot s holds logical sequence seq0 + s (so a
 * small cache can stand for chosen sequences of a large batch). */
int lo_kv_synth_from(lo_kv* kv, uint64_t seed, float kv_std, const int32_t* prefill_len,
                     int32_t seq0);
uint16_t* lo_kv_k(lo_kv* kv, int layer, int seq, int kv_head); /* [max_seq][d] */
uint16_t* lo_kv_v(lo_kv* kv, int layer, int seq, int kv_head);

/* --- single operations (each pinned on its own) --- */
lo_real lo_silu(lo_real a);
/* out = (x * r) * g with r = 1 / sqrt(mean(x^2) + eps); g may be NULL (= 1). */
void lo_rmsnorm(const lo_real* x, const uint16_t* g, int32_t n, float eps, lo_real* out);
/* y[i] = sum_j W[i][j] * x[j], W bf16 [rows, cols] row-major. */
void lo_matvec(const uint16_t* W, int64_t rows, int64_t cols, const lo_real* x, lo_real* y);
/* Rotate one head h[0..d) to position p (pairs (i, i + d/2)). */
void lo_rope(lo_real* h, int32_t d, int32_t p, float theta);
/* In-place softmax of s[0..n). */
void lo_softmax(lo_real* s, int32_t n);
/* One head of decode attention over positions 0..len-1 of K/V ([len][d] bf16). */
void lo_attention_head(const lo_real* q, const uint16_t* K, const uint16_t* V, int32_t len,
                       int32_t d, lo_real* out);
/* SwiGLU first stage: h[i] = silu(Wg[i].xn) * (Wu[i].xn). */
void lo_swiglu(const uint16_t* Wg, const uint16_t* Wu, int64_t inter, int64_t hidden,
               const lo_real* xn, lo_real* h);
/* Index of the largest value; the lowest index wins ties. */
int32_t lo_argmax(const lo_real* v, int64_t n);

/* Intermediates of one (seq, layer) of a step, for tests; NULL fields skipped.
 * Sizes: xn/x_attn/xn2/x_out [hidden]; q/o [n_q*d]; k/v [n_kv*d] (after
 * RoPE for q/k); hh [intermediate]. */
typedef struct {
  int32_t seq, layer;
  lo_real *xn, *q, *k, *v, *o, *x_attn, *xn2, *hh, *x_out;
} lo_trace;

/* One decode step for B sequences.  tokens[b] in [0, vocab), pos[b] in
 * [0, max_seq): the slot the new K/V is written to; attention covers 0..pos[b].
 * logits [B, vocab] (float, as the GPU path), next [B] (may be NULL),
 * trace may be NULL.  Returns 0, or -1 on bad arguments. */
int lo_decode_step(const lo_model* m, lo_kv* kv, const int32_t* tokens, int32_t B,
                   const int32_t* pos, float* logits, int32_t* next, lo_trace* trace);

/* One sequence only: cache slot `seq` decodes `token` at position `pos`.
 * logits [vocab]; next may be NULL. */
int lo_decode_one(const lo_model* m, lo_kv* kv, int32_t seq, int32_t token, int32_t pos,
                  float* logits, int32_t* next);

/* Bytes of lo_real in this build (4 or 8), so callers can tell the builds apart. */
int32_t lo_real_bytes(void);

#ifdef __cplusplus
}
#endif
#endif
