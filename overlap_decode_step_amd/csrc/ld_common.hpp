// ld_common.hpp - shared device definitions for the decode-step kernels
// (gfx950, wave64): bf16 helpers, wave reductions, readiness counters and
// the argument blocks every stage reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ld_params.hpp"

namespace ld {

constexpr int kWave = 64;
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWave * kWaves;  // 256 threads per workgroup
constexpr int kChunk = kWave * 8;         // bf16 elements covered by one 16-byte load per lane

// ----------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0x7FFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Eight bf16 (one 16-byte word) dotted with eight floats, accumulated in order.
__device__ __forceinline__ float dot8(const uint4& w, const float* x, float acc) {
  acc = fmaf(bf16lo(w.x), x[0], acc);
  acc = fmaf(bf16hi(w.x), x[1], acc);
  acc = fmaf(bf16lo(w.y), x[2], acc);
  acc = fmaf(bf16hi(w.y), x[3], acc);
  acc = fmaf(bf16lo(w.z), x[4], acc);
  acc = fmaf(bf16hi(w.z), x[5], acc);
  acc = fmaf(bf16lo(w.w), x[6], acc);
  acc = fmaf(bf16hi(w.w), x[7], acc);
  return acc;
}

// ------------------------------------------------------------ reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Sum over the workgroup; every thread gets the result.  `red` holds kWaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[w];
  return s;
}

// ------------------------------------------------- readiness counters
//
// A producer workgroup writes its tiles, passes a workgroup barrier (which
// waits for every wave's stores), and one thread adds 1 to the counter with
// release semantics at agent scope.  A consumer's first thread spins on an
// acquire load until the counter reaches the cumulative target of this step
// (counters only grow; targets are compared modulo 2^32), then releases the
// workgroup through a barrier.  This is the tile-level hand-off between
// dependent kernels of the MegaOps summary ("In plain words": a later kernel
// starts once the pieces of shared data it needs are ready).  The spin is
// bounded by a watchdog: on timeout (or once another workgroup has timed
// out) it records an error and returns, so every kernel always exits.

struct SyncArgs {
  uint32_t* ctr;        // counter arena
  int* err;             // device error word
  uint64_t watchdog;    // spin limit in s_memrealtime ticks (100 MHz)
};

__device__ __forceinline__ bool reached(uint32_t v, uint32_t target) {
  return (int32_t)(v - target) >= 0;
}

__device__ __forceinline__ void raise_error(int* err, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-wide wait for *ctr >= target.  Must be called by every thread.
__device__ __forceinline__ void wg_wait(const SyncArgs& s, const uint32_t* ctr, uint32_t target,
                                        int stage) {
  if (threadIdx.x == 0) {
    uint32_t v = __hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    if (!reached(v, target)) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if (reached(v, target)) break;
        // another workgroup already timed out: stop waiting so the grid drains
        if ((__hip_atomic_load(s.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xFF) ==
            kErrTimeout)
          break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > s.watchdog) {
          raise_error(s.err, kErrTimeout | (stage << 8));
          break;
        }
      }
    }
  }
  __syncthreads();
}

// Workgroup-wide signal: every thread calls it after writing its outputs.
__device__ __forceinline__ void wg_signal(uint32_t* ctr) {
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace ld
