/*
 * ld_synth.h - seeded synthetic inputs for the decode-step workloads.
 *
 * This module is the only code shared by the CPU oracle and the GPU library.
 * It generates inputs (weights, KV-cache prefill, first tokens, per-sequence
 * KV lengths) and holds none of the decode step's arithmetic.
 *
 * Every value is a pure function of (seed, tensor id, logical index), so any
 * physical layout can be filled in any order, on the host or on the device,
 * and gives the same bytes.
 *
 * Mixer: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  For a stream key
 * k, element n of the stream is mix64(k + (n + 1) * GAMMA), which is exactly
 * the n-th output of a SplitMix64 generator seeded with k.
 *
 * "Approximately N(0, sigma)" values: the four 16-bit fields of one 64-bit
 * hash are summed (Irwin-Hall with n = 4 over the discrete uniform on
 * [0, 65535]); z = sum - 131070 is an exact integer with mean 0 and variance
 * (65536^2 - 1) / 3.  The value is bf16(float(z) * kappa) with
 * kappa = (float)(sigma / sqrt((65536^2 - 1) / 3)): one IEEE fp32 multiply
 * then round-to-nearest-even to bf16, so host and device agree bit for bit.
 *
 * Uniform integers in [lo, hi]: lo + ((hash >> 32) * (hi - lo + 1)) >> 32
 * (Lemire's multiply-shift range reduction).
 */
#ifndef LD_SYNTH_H
#define LD_SYNTH_H

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define LS_FN __host__ __device__ static inline
#else
#define LS_FN static inline
#endif

/* Seeds used by the workloads: weights 1, KV prefill 2, first tokens 3, KV lengths 4. */
#define LS_SEED_WEIGHTS 1ull
#define LS_SEED_KV 2ull
#define LS_SEED_TOKENS 3ull
#define LS_SEED_KVLEN 4ull

/* Tensor ids (one independent stream each). */
#define LS_T_EMBED 1ull
#define LS_T_FINAL_NORM 2ull
#define LS_T_LM_HEAD 3ull
/* per-layer tensors: LS_T_LAYER(l, kind) */
#define LS_K_ATTN_NORM 0
#define LS_K_WQ 1
#define LS_K_WK 2
#define LS_K_WV 3
#define LS_K_WO 4
#define LS_K_MLP_NORM 5
#define LS_K_WG 6
#define LS_K_WU 7
#define LS_K_WD 8
#define LS_T_LAYER(l, kind) (0x1000ull + (uint64_t)(l) * 16ull + (uint64_t)(kind))
#define LS_T_KCACHE(l) (0x100000ull + 2ull * (uint64_t)(l))
#define LS_T_VCACHE(l) (0x100000ull + 2ull * (uint64_t)(l) + 1ull)
#define LS_T_TOKENS 0x200000ull
#define LS_T_KVLEN 0x200001ull

/* Logical index of KV element (seq b, kv head h, position pos, channel i). */
LS_FN uint64_t ls_kv_index(uint64_t b, uint64_t n_kv, uint64_t h, uint64_t pos,
                           uint64_t d, uint64_t i) {
  return ((b * n_kv + h) << 32) + pos * d + i;
}

LS_FN uint64_t ls_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

#define LS_GAMMA 0x9E3779B97F4A7C15ull

/* Stream key for (seed, tensor). */
LS_FN uint64_t ls_key(uint64_t seed, uint64_t tensor) {
  return ls_mix64(seed ^ ls_mix64(tensor * LS_GAMMA + 0x632BE59BD9B4E019ull));
}

/* 64-bit hash of element `index` of the stream with key `key`. */
LS_FN uint64_t ls_hash(uint64_t key, uint64_t index) {
  return ls_mix64(key + (index + 1ull) * LS_GAMMA);
}

/* fp32 -> bf16 bits, round to nearest, ties to even (inputs here are finite). */
LS_FN uint16_t ls_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Irwin-Hall(4) integer z in [-131070, 131070]. */
LS_FN int32_t ls_irwin_hall4(uint64_t h) {
  int32_t s = (int32_t)(h & 0xFFFFu) + (int32_t)((h >> 16) & 0xFFFFu) +
              (int32_t)((h >> 32) & 0xFFFFu) + (int32_t)((h >> 48) & 0xFFFFu);
  return s - 131070;
}

/* Approximately N(0, sigma) bf16 element; kappa from ls_kappa(sigma). */
LS_FN uint16_t ls_normal_bf16(uint64_t key, uint64_t index, float kappa) {
  float v = (float)ls_irwin_hall4(ls_hash(key, index)) * kappa;
  return ls_bf16_bits(v);
}

/* Uniform integer in [lo, hi] for element `index` of the stream `key`. */
LS_FN int32_t ls_uniform_int(uint64_t key, uint64_t index, int32_t lo, int32_t hi) {
  uint64_t h = ls_hash(key, index);
  uint64_t span = (uint64_t)(int64_t)(hi - lo) + 1ull;
  return lo + (int32_t)(((h >> 32) * span) >> 32);
}

#include <math.h>
/* Scale that maps the Irwin-Hall(4) integer to standard deviation sigma.
 * Computed on the host only; the device receives the fp32 result. */
#if defined(__HIPCC__)
__host__
#endif
static inline float ls_kappa(float sigma) {
  return (float)((double)sigma / sqrt((65536.0 * 65536.0 - 1.0) / 3.0));
}

/* bf16 bits of 1.0 (norm gains are 1.0 in every workload). */
#define LS_BF16_ONE ((uint16_t)0x3F80u)

#endif /* LD_SYNTH_H */
