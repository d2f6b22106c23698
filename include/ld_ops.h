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

/* Force / query the SwiGLU tiling used for one batch size. */
ld_status ld_set_swiglu_variant(ld_model* m, int32_t batch, int32_t variant);
int32_t ld_get_swiglu_variant(const ld_model* m, int32_t batch);

/* Unfused-MLP ablation (Deep Kernel Fusion for Transformers, "Key points",
 * "Fusion scope": the fused first MLP stage never writes the projections
 * out).  LD_MLP_FUSED (the default) runs the fused SwiGLU stage;
 * LD_MLP_TWO_KERNELS one GEMV writing the gate and up projections, then a
 * silu-product kernel; LD_MLP_FOUR_KERNELS the gate GEMV, the up GEMV, silu
 * in place and the product.  All three give bitwise-equal results.  The
 * unfused forms apply to the whole-kernel-wait mode only (the other modes
 * always run the fused stage) and to batches below 16 (the VALU engine): a
 * step outside that returns LD_EINVAL.  Returns LD_EINVAL for an unknown
 * variant. */
enum { LD_MLP_FUSED = 0, LD_MLP_TWO_KERNELS = 1, LD_MLP_FOUR_KERNELS = 2 };
ld_status ld_set_mlp_variant(ld_model* m, int32_t variant);

/* Spin limit of every device-side readiness wait (default 2 s). */
ld_status ld_set_watchdog(ld_model* m, double seconds);

/* Failure injection from the host: the next ld_decode_step's attention stage
 * waits for one more producer signal than will ever arrive, so its wait runs
 * into the watchdog (tile-flag and persistent modes).  Every kernel still
 * exits; ld_device_error() then reports LD_ETIMEOUT and resets the counters. */
ld_status ld_debug_inject_stall(ld_model* m);

/* Stage timeline (profiling).  When dev_buf is not NULL every decode kernel
 * stores, for each workgroup w < 1024, the GPU's constant 100 MHz clock
 * (s_memrealtime) at stage entry (ev 0), after the readiness wait (ev 1),
 * after the compute (ev 2) and at stage exit (ev 3), as uint64 at
 * dev_buf[((layer * 8 + stage) * 4 + ev) * 1024 + w]; stage ids 1..5 are
 * QKV, attention, O, SwiGLU, Down and the LM head is stage 6 of layer
 * n_layers.  NULL turns it off.  bytes >= ld_trace_bytes(cfg). */
size_t ld_trace_bytes(const ld_config* cfg);
ld_status ld_set_trace(ld_model* m, void* dev_buf, size_t bytes);

/* Launch geometry: out[0] CUs, out[1] grid of the whole-kernel-wait kernels,
 * out[2] grid of the tile-flag kernels, out[3] persistent grid at batch 1,
 * out[4] attention split length, out[5] current mode.  n >= 6. */
ld_status ld_launch_info(const ld_model* m, int32_t* out, int32_t n);

#ifdef __cplusplus
}
#endif
#endif
