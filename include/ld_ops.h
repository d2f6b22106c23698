/*
 * ld_ops.h - inspection, tuning and test hooks of libld.so (see ld.h for the
 * decode-step ABI and its conventions).  All functions here are synchronous
 * unless stated otherwise and return ld_status codes.
 */
#ifndef LD_OPS_H
#define LD_OPS_H

#include "ld.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Logical weights.  Matrices are bf16 row-major [out, in]; norm gains are
 * [1, hidden].  LD_W_LM_HEAD aliases LD_W_EMBED when the model is tied. */
enum {
  LD_W_EMBED = 0,      /* [vocab, hidden] */
  LD_W_ATTN_NORM = 1,  /* per layer [1, hidden] */
  LD_W_Q = 2,          /* [n_q*d, hidden] */
  LD_W_K = 3,          /* [n_kv*d, hidden] */
  LD_W_V = 4,          /* [n_kv*d, hidden] */
  LD_W_O = 5,          /* [hidden, n_q*d] */
  LD_W_MLP_NORM = 6,   /* [1, hidden] */
  LD_W_GATE = 7,       /* [intermediate, hidden] */
  LD_W_UP = 8,         /* [intermediate, hidden] */
  LD_W_DOWN = 9,       /* [hidden, intermediate] */
  LD_W_FINAL_NORM = 10,/* [1, hidden] */
  LD_W_LM_HEAD = 11    /* [vocab, hidden] */
};

/* SwiGLU tilings ("Deep Kernel Fusion for Transformers", Key points, "Fusion
 * scope": row-major favours activation reuse, column-major weight reuse). */
enum { LD_SWIGLU_COL = 0, LD_SWIGLU_ROW = 1 };

/* Shape of one logical weight (rows, cols out). */
ld_status ld_weight_shape(ld_model* m, int32_t kind, int32_t layer, int64_t* rows, int64_t* cols);

/* Copy one logical weight to host memory (host_dst: rows*cols bf16). */
ld_status ld_read_weight(ld_model* m, int32_t kind, int32_t layer, uint16_t* host_dst);

/* Overwrite one logical weight from host memory (the host-copy path for
 * real or hand-built weights).  Rejects LD_W_LM_HEAD on a tied model. */
ld_status ld_write_weight(ld_model* m, int32_t kind, int32_t layer, const uint16_t* host_src);

/* Copy K and/or V cache rows [pos0, pos0+npos) of (layer, seq, kv_head) to
 * host memory (npos*head_dim bf16 each; either pointer may be NULL). */
ld_status ld_read_kv(ld_model* m, int32_t layer, int32_t seq, int32_t kv_head, int32_t pos0,
                     int32_t npos, uint16_t* k_dst, uint16_t* v_dst);

/* Force the SwiGLU tiling of one batch size in every mode / query the one the
 * current mode uses. */
ld_status ld_set_swiglu_variant(ld_model* m, int32_t batch, int32_t variant);
int32_t ld_get_swiglu_variant(const ld_model* m, int32_t batch);

/* Unfused-MLP ablation (Deep Kernel Fusion for Transformers, "Key points",
 * "Fusion scope": the fused first MLP stage never writes the projections
 * out).  LD_MLP_FUSED (the default) runs the fused SwiGLU stage;
 * LD_MLP_TWO_KERNELS one GEMV writing the gate and up projections, then a
 * silu-product kernel; LD_MLP_FOUR_KERNELS the gate GEMV, the up GEMV, silu
 * in place and the product.  All three give bitwise-equal results, on both
 * engines (below 16 rows the VALU engine, from 16 the MFMA engine, whose
 * projections are the fused stage's tiles with a different epilogue and
 * whose product kernel writes the Down stage's split-bf16 fragments).  The
 * unfused forms apply to the whole-kernel-wait mode only (the other modes
 * always run the fused stage).  Returns LD_EINVAL for an unknown variant. */
enum { LD_MLP_FUSED = 0, LD_MLP_TWO_KERNELS = 1, LD_MLP_FOUR_KERNELS = 2 };
ld_status ld_set_mlp_variant(ld_model* m, int32_t variant);

/* Readiness granularity of the tile-flag and persistent modes (MegaOps
 * summary, "In plain words": a consumer starts once the particular pieces of
 * shared data it needs are ready).  LD_SYNC_TILE: each attention item waits
 * only for the q, k and v rows of its own kv group, and the Down stage only
 * for the SwiGLU output chunks (1024 rows each) of the K range it reads (all
 * of them on the VALU engine, its own range in a split-K stage of the MFMA
 * engine), through row-count counters.  LD_SYNC_STAGE: those consumers wait
 * for their whole producer stage.  LD_SYNC_AUTO (the default): LD_SYNC_TILE
 * in the tile-flag mode below 64 rows, LD_SYNC_STAGE otherwise (the faster
 * of the two as measured on MI355X).  Results are bitwise the same either
 * way.  Shapes with more than 64 kv groups or SwiGLU chunks per layer always
 * use LD_SYNC_STAGE.  Returns LD_EINVAL for another value. */
enum { LD_SYNC_STAGE = 0, LD_SYNC_TILE = 1, LD_SYNC_AUTO = 2 };
ld_status ld_set_sync(ld_model* m, int32_t granularity);

/* Spin limit of every device-side readiness wait (default 2 s). */
ld_status ld_set_watchdog(ld_model* m, double seconds);

/* Failure injection from the host: the next ld_decode_step's attention stage
 * waits for one more producer signal than will ever arrive, so its wait runs
 * into the watchdog (tile-flag and persistent modes).  Every kernel still
 * exits; ld_device_error() then reports LD_ETIMEOUT and resets the counters. */
ld_status ld_debug_inject_stall(ld_model* m);

/* Debug mechanisms (race and protocol checks; off by default).
 *
 * ld_set_debug(m, LD_DEBUG_POISON): before every following decode step (same
 * stream, asynchronous like the step) every activation, partial-result and
 * hand-off buffer of the work arena, the caller's logits rows and next
 * tokens, and the KV-cache rows the step appends (each row's position, every
 * layer and kv head) are filled with quiet NaNs.  A stage that reads a word
 * before its producer wrote it then turns the logits into NaN; a correct
 * step returns exactly the logits it returns without the poison.  Fragment
 * buffers of the MFMA engine whose K (hidden, n_q d or intermediate) is not a
 * multiple of 32 are left out (their padding columns must stay zero).
 * flags 0 turns it off; LD_EINVAL for an unknown flag.
 *
 * ld_audit(m): synchronises, then checks every readiness counter against
 * what the steps enqueued so far imply: each layer's stage counters equal the
 * host's running totals (their leaves added modulo 2^32), the row-count
 * counters the tile-granular steps times the rows of their kv group or
 * SwiGLU chunk, and every last-arriver counter (LM head, attention splits,
 * split K) and the device error word zero.  Returns LD_OK, LD_EAUDIT with up
 * to four mismatches in ld_last_error(), or LD_ESTATE before ld_alloc_kv.
 * After LD_ETIMEOUT (which resets the counters) the audit starts over.
 *
 * Environment (read when a model is created): LD_MODE = wait | flags | mega
 * | graph sets the starting mode, LD_WATCHDOG_US the watchdog in
 * microseconds; another value makes ld_init_weights return LD_EINVAL. */
enum { LD_DEBUG_POISON = 1 };
ld_status ld_set_debug(ld_model* m, int32_t flags);
ld_status ld_audit(ld_model* m);

/* Stage timeline (profiling).  When dev_buf is not NULL every decode kernel
 * stores, for each workgroup w < 1024, the GPU's constant 100 MHz clock
 * (s_memrealtime) at stage entry (ev 0), after the readiness wait (ev 1),
 * after the compute (ev 2) and at stage exit (ev 3), as uint64 at
 * dev_buf[((layer * 8 + stage) * 4 + ev) * 1024 + w]; stage ids 1..5 are
 * QKV, attention, O, SwiGLU, Down and the LM head is stage 6 of layer
 * n_layers.  Slots 6 and 7 of a layer hold the attention items' own events,
 * for each workgroup's last item: (6, 0) item start, (7, 0) its K/V tiles and
 * new rows in LDS, (7, 1) scores and softmax done, (7, 2) outputs stored,
 * (7, 3) split counter returned (several splits only).  NULL turns it off.
 * bytes >= ld_trace_bytes(cfg). */
size_t ld_trace_bytes(const ld_config* cfg);
ld_status ld_set_trace(ld_model* m, void* dev_buf, size_t bytes);

/* Work buffers of the last decode step, for inspection (synchronous).
 * Copies rows [0, rows) of one fp32 buffer to host memory:
 *   LD_ACT_X    - the residual stream after the last layer   [rows, hidden]
 *   LD_ACT_QKV  - the last layer's q|k|v projections, before the rotary
 *                 embedding (q rows, then k, then v)        [rows, (n_q + 2 n_kv) d]
 *   LD_ACT_ATTN - the last layer's attention output         [rows, n_q d]
 *   LD_ACT_H    - the last layer's SwiGLU output             [rows, intermediate]
 * From 16 rows the attention and SwiGLU outputs hold each value as the MFMA
 * engine's split-bf16 pair (bf16(v) in the low half, bf16(v - bf16(v)) in the
 * high half of the 32-bit word), the form in which the next stage reads them.
 * Returns LD_EINVAL for an unknown buffer or rows outside [1, max_batch],
 * LD_ESTATE before ld_alloc_kv. */
enum { LD_ACT_X = 0, LD_ACT_QKV = 1, LD_ACT_ATTN = 2, LD_ACT_H = 3 };
ld_status ld_read_activation(ld_model* m, int32_t which, int32_t rows, float* host_dst);

/* Launch geometry: out[0] CUs, out[1] grid of the whole-kernel-wait kernels,
 * out[2] grid of the tile-flag kernels, out[3] persistent grid at batch 1,
 * out[4] attention split length, out[5] current mode.  n >= 6. */
ld_status ld_launch_info(const ld_model* m, int32_t* out, int32_t n);

#ifdef __cplusplus
}
#endif
#endif
