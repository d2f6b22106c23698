// ld_common.hpp - shared device definitions for the decode-step kernels
// (gfx950, wave64): bf16 helpers, wave reductions, coherent loads/stores and
// the readiness counters every stage uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ld_params.hpp"

namespace ld {

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;              // waves per workgroup at most (1024 threads)
constexpr int kChunk = kWave * 8;          // bf16 elements covered by one 16-byte load per lane

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Threads per workgroup of every decode kernel.
constexpr int kBlockThreads = 512;

// The thread index through an empty volatile asm: values derived from it
// cannot be hoisted out of the persistent kernel's layer loop, where they
// would stay live (in registers) across every stage.  Its range is restated
// so that tests against it still fold.
__device__ __forceinline__ int tid() {
  int v = (int)threadIdx.x;
  asm volatile("" : "+v"(v));
  __builtin_assume(v >= 0 && v < kBlockThreads);
  return v;
}
__device__ __forceinline__ int nwaves() { return blockDim.x >> 6; }
// the wave index is uniform: keep it (and what is derived from it) scalar
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return tid() & (kWave - 1); }

// ----------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0x7FFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------ reductions
//
// Wave-wide reductions with DPP lane moves (VALU, a few cycles each) instead
// of LDS permutes: pairs and quads inside each 4-lane group, rotations inside
// each 16-lane row, then row broadcasts 15 -> next row and 31 -> upper half;
// lane 63 ends with the total, which is read back as a uniform value.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1, 0xF>(0.f, v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E, 0xF>(0.f, v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x124, 0xF>(0.f, v);  // row_ror:4
  v += dpp_f<0x128, 0xF>(0.f, v);  // row_ror:8
  v += dpp_f<0x142, 0xA>(0.f, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(0.f, v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  const float lo = -INFINITY;
  v = fmaxf(v, dpp_f<0xB1, 0xF>(lo, v));
  v = fmaxf(v, dpp_f<0x4E, 0xF>(lo, v));
  v = fmaxf(v, dpp_f<0x124, 0xF>(lo, v));
  v = fmaxf(v, dpp_f<0x128, 0xF>(lo, v));
  v = fmaxf(v, dpp_f<0x142, 0xA>(lo, v));
  v = fmaxf(v, dpp_f<0x143, 0xC>(lo, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u<0xB1, 0xF>(0u, v);
  v += dpp_u<0x4E, 0xF>(0u, v);
  v += dpp_u<0x124, 0xF>(0u, v);
  v += dpp_u<0x128, 0xF>(0u, v);
  v += dpp_u<0x142, 0xA>(0u, v);
  v += dpp_u<0x143, 0xC>(0u, v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over aligned groups of w lanes (w = 1..32, a power of two).  DPP row
// rotations move data to higher lanes, so the total is valid in the last
// lane of each group.
__device__ __forceinline__ float lane_group_sum(float v, int w) {
  if (w > 1) v += dpp_f<0xB1, 0xF>(0.f, v);     // + lane ^ 1
  if (w > 2) v += dpp_f<0x4E, 0xF>(0.f, v);     // + lane ^ 2
  if (w > 4) v += dpp_f<0x124, 0xF>(0.f, v);    // row_ror:4 (lane 7 of 8 gets lanes 0..3)
  if (w > 8) v += dpp_f<0x128, 0xF>(0.f, v);    // row_ror:8 (lane 15 of 16 gets lanes 0..7)
  if (w > 16) v += __shfl_up(v, 16, kWave);     // lane 31 of 32 gets lanes 0..15
  return v;
}

// ------------------------------------------- coherent (agent-scope) access
//
// Activations, partial results and counters pass between workgroups that may
// sit on different XCDs, each with its own L2.  They are written with
// agent-scope stores (write-through past the non-coherent L2) and read with
// agent-scope loads (which miss any stale L2 copy), so no L2 write-back or
// invalidate is needed at each hand-off; weights are read-only and use
// ordinary non-temporal loads.

__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ int ld_coh_i(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// eight consecutive floats (32-byte aligned) through four 64-bit coherent loads
__device__ __forceinline__ void ld_coh8(const float* p, float* o) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t v = __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    o[2 * i] = __uint_as_float((uint32_t)v);
    o[2 * i + 1] = __uint_as_float((uint32_t)(v >> 32));
  }
}

// ------------------------------------------------- readiness counters
//
// A stage signals completion through 16 "leaf" counters, each on its own
// 128-byte line; workgroup w adds 1 to leaf w % 16 once its outputs are
// stored, and a consumer sums the leaves (one wave-wide load) and compares
// with the cumulative number of signals expected by the end of this step
// (counters only grow; comparisons are modulo 2^32).  This is the tile-level
// hand-off between dependent stages of the MegaOps summary ("In plain
// words": a later kernel starts once the pieces of shared data it needs are
// ready).  Ordering: every wave waits for its own stores to complete
// (s_waitcnt 0), the workgroup barrier makes that true for all waves, then
// one relaxed atomic add publishes it; the consumer issues its data loads
// only after it has seen the count.  The spin is bounded by a watchdog: on
// timeout, or once another workgroup has timed out, it records an error and
// returns, so every kernel always exits.

struct SyncArgs {
  int* err;           // device error word
  uint64_t watchdog;  // spin limit in s_memrealtime ticks (100 MHz)
};

__device__ __forceinline__ bool reached(uint32_t v, uint32_t target) {
  return (int32_t)(v - target) >= 0;
}

__device__ __forceinline__ void raise_error(int* err, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// All of this wave's memory operations have completed.
__device__ __forceinline__ void wave_drain() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup-wide wait until the leaves of `ctr` sum to >= target.  Every
// thread calls it.  Wave 0 polls with kPollDepth loads in flight and a short
// sleep between polls.  (Deeper polling, or polling without the sleep, was
// measured slower: the extra coherent loads on the counter lines delay the
// stages' own memory traffic more than they shorten the hand-off.)
constexpr int kPollDepth = 1;

// One poll: one load per lane, unconditional (a load under a lane mask, or a
// second load whose value is needed at once, would make the compiler wait for
// every poll in flight).  Lanes 0..15 read the leaves, lane 16 the device
// error word, the others a leaf again (ignored).
__device__ __forceinline__ uint32_t poll_once(const uint32_t* ctr, const int* err, int lane) {
  const uint32_t* a = lane == kLeaves ? reinterpret_cast<const uint32_t*>(err)
                                      : ctr + (lane & (kLeaves - 1)) * kLeafStride;
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wg_wait(const SyncArgs& s, const uint32_t* ctr, uint32_t target,
                                        int stage) {
  // wave_id() is scalar, so the poll loop is uniform control flow with one
  // exit per round; that lets the compiler wait for the oldest poll only
  if (wave_id() == 0) {
    const int lane = lane_id();
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint32_t v[kPollDepth];
#pragma unroll
    for (int j = 0; j < kPollDepth; ++j) v[j] = poll_once(ctr, s.err, lane);
    bool done = false;
    while (!done) {
#pragma unroll
      for (int j = 0; j < kPollDepth; ++j) {
        const uint32_t sum = wave_sum_u32(lane < kLeaves ? v[j] : 0u);
        const int e = __builtin_amdgcn_readlane((int)v[j], kLeaves);
        // reached, or another workgroup already timed out (let the grid drain)
        done = done || reached(sum, target) || (e & 0xFF) == kErrTimeout;
        v[j] = poll_once(ctr, s.err, lane);
        __builtin_amdgcn_s_sleep(1);
      }
      if (!done && __builtin_amdgcn_s_memrealtime() - t0 > s.watchdog) {
        if (lane == 0) raise_error(s.err, kErrTimeout | (stage << 8));
        done = true;
      }
    }
  }
  __syncthreads();
}

// Workgroup-wide wait until each of the n counters ctr0 + i * kCtrWords
// (i < n) has reached target(i).  Wave 0 polls four counters per wave-wide
// load (lane 16 c + leaf reads leaf `leaf` of counter c), adds each counter's
// 16 leaves within its lane row, and repeats until every counter has reached
// its target (or another workgroup timed out); same watchdog as wg_wait.
template <class TargetFn>
__device__ __forceinline__ void wg_wait_all(const SyncArgs& s, const uint32_t* ctr0, int n,
                                            const TargetFn& target, int stage) {
  if (n > 0 && wave_id() == 0) {
    const int lane = lane_id(), sub = lane >> 4, leaf = lane & (kLeaves - 1);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool done = false;
    while (!done) {
      bool all = true;
      for (int g = 0; g < n; g += 4) {
        const int i = g + sub;
        uint32_t v = __hip_atomic_load(ctr0 + (int64_t)min(i, n - 1) * kCtrWords + leaf * kLeafStride,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v += dpp_u<0xB1, 0xF>(0u, v);   // quad_perm [1,0,3,2]
        v += dpp_u<0x4E, 0xF>(0u, v);   // quad_perm [2,3,0,1]
        v += dpp_u<0x124, 0xF>(0u, v);  // row_ror:4
        v += dpp_u<0x128, 0xF>(0u, v);  // row_ror:8: every lane of the row holds its sum
        const bool ok = i >= n || reached(v, target(i));
        all = all && __ballot(ok) == ~0ull;
      }
      const int e = ld_coh_i(s.err);
      done = all || (e & 0xFF) == kErrTimeout;
      if (!done) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > s.watchdog) {
          if (lane == 0) raise_error(s.err, kErrTimeout | (stage << 8));
          done = true;
        }
      }
    }
  }
  __syncthreads();
}

// Workgroup-wide signal after this workgroup's outputs are stored.
__device__ __forceinline__ void wg_signal(uint32_t* ctr, int who) {
  wave_drain();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(ctr + (who & (kLeaves - 1)) * kLeafStride, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Last-arriver detection within one step: each of the n participants calls
// it once (one thread, after its results are stored and drained).  Returns
// true for exactly one caller, the last, and leaves the counter at zero for
// the next step.  Two levels: leaf who % 16, then a root slot.
__device__ __forceinline__ bool last_arriver(uint32_t* ctr, int who, int n) {
  const int leaf = who & (kLeaves - 1);
  const uint32_t per = (uint32_t)((n - leaf + kLeaves - 1) / kLeaves);
  const int nleaf = n < kLeaves ? n : kLeaves;
  uint32_t* lp = ctr + leaf * kLeafStride;
  const uint32_t old = __hip_atomic_fetch_add(lp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1u != per) return false;
  __hip_atomic_store(lp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t* root = ctr + kLeaves * kLeafStride;
  const uint32_t r = __hip_atomic_fetch_add(root, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (r + 1u != (uint32_t)nleaf) return false;
  __hip_atomic_store(root, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

}  // namespace ld
