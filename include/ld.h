/*
 * ld.h - C ABI of libld.so: the small-batch decode step of a dense
 * Llama-style decoder on one MI355X (gfx950), with stages that hand work to
 * each other through per-tile readiness counters instead of whole-kernel
 * waits.
 *
 * What the step computes (per sequence): embedding row; per layer RMSNorm,
 * the Q/K/V projection with rotary position embedding and K/V append,
 * grouped-query attention over the cache, the output projection with
 * residual, RMSNorm, the fused SwiGLU first stage and the Down projection
 * with residual; then the final RMSNorm, the LM head (fp32 logits) and a
 * greedy argmax.  The workload is batch-1 Llama-3.2-1B decode, which is
 * memory-bound (Hazy Research, "Look Ma, No Bubbles! Designing a
 * Low-Latency Megakernel for Llama-1B", introduction); the MLP is split into
 * a fused Up/Gate/SiLU/product stage and a separate Down projection ("Deep
 * Kernel Fusion for Transformers", Key points, "Fusion scope").
 *
 * Execution modes (all share the same stage code; below batch 16 they give
 * bitwise-equal results, except the tile-flag mode where a long context
 * lengthens the attention splits past half a CU's tile area.  From 16 on
 * they agree to rounding: the MFMA engine's split of each tile's K steps
 * over waves depends on the mode's grid, and the tile-flag mode splits
 * attention into shorter KV ranges, since two of its stage kernels share a
 * CU's LDS):
 *   LD_MODE_WAIT  - one kernel per stage on one stream; each kernel starts
 *                   when the previous one has finished (the conventional
 *                   whole-kernel wait of the MegaOps summary, "In plain
 *                   words").
 *   LD_MODE_FLAGS - the same kernels on two alternating streams; a consumer's
 *                   workgroups start as soon as the tiles they read are
 *                   signalled ready (MegaOps summary, "Keep kernels
 *                   separate"; multi-streaming and prefetch, "What the
 *                   control can show").
 *   LD_MODE_MEGA  - one persistent kernel per step whose workgroups walk
 *                   the stages in order, synchronising on the same counters
 *                   (the megakernel of the Hazy post).  Its grid is one
 *                   workgroup per CU and all of them must run at once: the
 *                   GPU must not be shared with other work during the step
 *                   (otherwise the step ends in LD_ETIMEOUT, not a hang).
 *                   The tile-flag mode assumes the same of its two
 *                   co-resident stage kernels.
 *   LD_MODE_GRAPH - the whole-kernel-wait step captured into a HIP graph
 *                   and replayed (the graph-of-kernels alternative to a
 *                   megakernel argued in "Megakernel Debate Sparks CUDA
 *                   Infrastructure Community Feud").  A step is captured on
 *                   the library's own stream the first time it is called
 *                   with a given (batch, tokens, positions, logits,
 *                   next_tokens) and SwiGLU tiling, and later steps with the
 *                   same arguments replay it on the caller's stream, so the
 *                   contents of those buffers may change between steps but
 *                   not their addresses.  Up to 8 argument sets are kept
 *                   (least recently captured dropped first); they are
 *                   released by ld_free.  A capture failure returns LD_EHIP.
 *
 * Conventions.
 *  - Every pointer documented "dev" is device memory on the current HIP
 *    device; "host" is host memory.  `stream` is a hipStream_t (NULL = the
 *    legacy default stream), passed as void* so this header needs no HIP
 *    include.
 *  - Buffers handed in belong to the caller and must outlive the model; the
 *    library frees only memory it allocated itself.
 *  - Host-visible argument errors return LD_EINVAL before anything is
 *    enqueued; ld_last_error() describes the latest error of a model.
 *  - ld_decode_step does no host synchronisation: it is asynchronous on
 *    `stream`.  Device-side input errors (token outside [0, vocab), position
 *    outside [0, max_seq)) and watchdog timeouts set a device error word and
 *    the step completes with unspecified outputs; read the word with
 *    ld_device_error().
 *  - A model is not thread-safe; use one model per host thread.
 */
#ifndef LD_H
#define LD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ld_model ld_model;

typedef enum {
  LD_OK = 0,
  LD_EINVAL = -1,   /* bad argument (host-side check) */
  LD_ENOMEM = -2,   /* allocation failed or caller buffer too small */
  LD_EHIP = -3,     /* a HIP runtime call failed */
  LD_ETIMEOUT = -4, /* a device-side wait exceeded the watchdog */
  LD_ESTATE = -5,   /* call out of order (e.g. decode before ld_alloc_kv) */
  LD_EDEVICE = -6,  /* device input error (bad token or position) */
  LD_EAUDIT = -7    /* ld_audit found a counter off its expected value */
} ld_status;

typedef enum { LD_MODE_WAIT = 0, LD_MODE_FLAGS = 1, LD_MODE_MEGA = 2, LD_MODE_GRAPH = 3 } ld_mode;

/* Model shape.  Weights are bf16 row-major [out, in]; norm gains bf16. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, tied;
  float rms_eps, rope_theta;
} ld_config;

/* Bytes of the weight arena for `cfg` (0 if the shape is unsupported).
 * Requirements: hidden, intermediate and n_q_heads*head_dim multiples of 8;
 * head_dim even and <= 256; n_q_heads a multiple of n_kv_heads. */
size_t ld_weights_bytes(const ld_config* cfg);

/* Create a model and fill its weights on the device from the seeded
 * generator: matrices ~N(0, w_std) (Irwin-Hall(4) approximation, keyed by
 * (seed, tensor, logical index)), norm gains 1.0.  dev_buf: dev arena of at
 * least ld_weights_bytes(cfg) bytes, or NULL to let the library allocate it.
 * Work is enqueued on `stream`; *out is valid on return. */
ld_status ld_init_weights(ld_model** out, const ld_config* cfg, void* dev_buf, size_t bytes,
                          uint64_t seed, float w_std, void* stream);

/* Bytes of the KV-cache + workspace arena for max_batch sequences of up to
 * max_seq positions each. */
size_t ld_kv_bytes(const ld_config* cfg, int32_t max_batch, int32_t max_seq);

/* Carve the bf16 KV cache [layer][seq][kv_head][pos][head_dim], the fp32
 * workspaces and the readiness counters; zero the counters and the device
 * error word.  dev_buf: dev arena of >= ld_kv_bytes() bytes or NULL.
 * Synchronous. */
ld_status ld_alloc_kv(ld_model* m, void* dev_buf, size_t bytes, int32_t max_batch,
                      int32_t max_seq);

/* Fill positions [0, prefill_len[b]) of every (layer, seq b, kv head) with
 * seeded ~N(0, kv_std) bf16 values (treated as already-rotated keys).
 * prefill_len: host [max_batch]. */
ld_status ld_fill_kv(ld_model* m, uint64_t seed, float kv_std, const int32_t* prefill_len,
                     void* stream);

/* ld_fill_kv without any device allocation, for callers that cannot
 * allocate (code under stream capture, serving loops, harnesses that forbid
 * hipMalloc): the same fill, bit for bit, but the device copy of the
 * lengths lives in a static device array of the library (64 int32 per GPU,
 * held until the process ends) instead of a buffer from hipMalloc.  The
 * lengths are passed to the device as kernel arguments, so prefill_len (host
 * [max_batch]) may be reused when the call returns.  Asynchronous on
 * `stream`; no allocation, free or synchronisation.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams)
 * race.  Returns LD_EINVAL if max_batch exceeds 64 or a length lies outside
 * [0, max_seq], LD_ESTATE before ld_alloc_kv, LD_EHIP on a launch failure. */
ld_status ld_fill_kv_static(ld_model* m, uint64_t seed, float kv_std, const int32_t* prefill_len,
                            void* stream);

/* Select the execution mode for later steps (see the list above).  Returns
 * LD_EINVAL for an unknown mode, and for LD_MODE_FLAGS when two of its stage
 * kernels cannot share a CU for this shape (a hidden-size input row, or two
 * weight blocks' columns of the O and Down stages' column chunks, must fit
 * half a CU's LDS; no Llama-1B, 8B or 70B configuration is refused). */
ld_status ld_set_mode(ld_model* m, ld_mode mode);

/* One decode step for `batch` sequences (1 <= batch <= max_batch).
 *   tokens      dev int32 [batch]: input token of each sequence
 *   positions   dev int32 [batch]: slot the new K/V is written to (= tokens
 *               already in the cache); attention covers 0..positions[b]
 *   logits      dev fp32 [batch, vocab] (out)
 *   next_tokens dev int32 [batch] greedy argmax, lowest index on ties (out,
 *               may be NULL)
 * The KV cache of slot positions[b] is overwritten. */
ld_status ld_decode_step(ld_model* m, const int32_t* tokens, int32_t batch,
                         const int32_t* positions, float* logits, int32_t* next_tokens,
                         void* stream);

/* Several consecutive tokens per sequence in one step (a prefill chunk, or
 * the verification of drafted tokens): the prompt-processing setting of the
 * MegaOps summary's prefill comparisons ("A multi-GPU check"), here on one
 * GPU, with every GEMV a GEMM over batch * tokens_per_seq rows.  Row
 * r = b * tokens_per_seq + j is token
 * j of sequence b (KV cache slot b):
 *   tokens      dev int32 [batch * tokens_per_seq] (in)
 *   positions   dev int32 [batch * tokens_per_seq]: positions[r] =
 *               positions[b * tokens_per_seq] + j, each < max_seq (a device
 *               error otherwise, like a bad position)
 *   logits      dev fp32 [batch * tokens_per_seq, vocab] (out)
 *   next_tokens dev int32 [batch * tokens_per_seq] or NULL (out)
 * Token j attends to positions 0 .. positions[r] of its sequence, that is
 * the cache plus this step's tokens 0 .. j; all of the step's K and V rows
 * are appended.  The result equals tokens_per_seq single-token steps in
 * order (teacher forced).  batch * tokens_per_seq must be in
 * [1, max_batch] and tokens_per_seq >= 1 (LD_EINVAL otherwise); 16 rows and
 * more run on the MFMA engine.  tokens_per_seq = 1 is ld_decode_step.  The
 * persistent kernel is built for decode steps only: tokens_per_seq > 1 in
 * LD_MODE_MEGA returns LD_EINVAL. */
ld_status ld_decode_step_tokens(ld_model* m, const int32_t* tokens, int32_t tokens_per_seq,
                                int32_t batch, const int32_t* positions, float* logits,
                                int32_t* next_tokens, void* stream);

/* Offline choice of the SwiGLU tiling ("Deep Kernel Fusion for Transformers",
 * Summary: a profiler benchmarks the tiling variants on the target before
 * inference and keeps the fastest; Key points, "Code and limitations": no
 * dispatch cost at run time).  For each batch size in batches[0..n) (each
 * <= max_batch) times whole decode steps in the model's current mode with the
 * column-major and the row-major tiling, alternating, 5 rounds of 3 steps
 * after 2 warm-up steps each, every sequence at position min(max_seq - 1,
 * 1024); the row-major tiling is recorded for that (mode, batch) only if its
 * median beats the column-major median by more than 1%.  Writes the mode's
 * table (choices and both medians) as JSON to table_path unless NULL.
 * Synchronous; needs ld_alloc_kv; allocates its own small step buffers.
 * Overwrites the workspace and the KV cache row at that position of
 * sequences 0..batch-1 (refill the cache afterwards if it matters).  A
 * device error during the steps is returned as by ld_device_error. */
ld_status ld_tune(ld_model* m, const int32_t* batches, int32_t n, const char* table_path);

/* Load a table written by ld_tune (same shape required) into the mode it was
 * tuned in (the current mode if the table names none). */
ld_status ld_load_tuning(ld_model* m, const char* table_path);

/* Synchronise the device, return LD_OK / LD_ETIMEOUT / LD_EDEVICE from the
 * device error word, and clear it. */
ld_status ld_device_error(ld_model* m);

/* Message of the latest error on `m` (or of the latest failed
 * ld_init_weights when m is NULL). Never NULL. */
const char* ld_last_error(const ld_model* m);

/* Free the model and any memory the library allocated. */
void ld_free(ld_model* m);

#ifdef __cplusplus
}
#endif
#endif
