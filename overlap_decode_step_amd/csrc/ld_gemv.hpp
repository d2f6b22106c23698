// ld_gemv.hpp - weight-streaming GEMV engine for small batches (VALU path).
//
// Each wave owns NR weight rows at a time and streams them in blocks of UC
// 512-element chunks: every lane issues one 16-byte non-temporal load per
// (row, chunk), so a block keeps NR*UC KB in flight per wave.  The bf16
// weights are widened in registers and multiplied with fp32 activations
// (fp32 FMA); each lane's partial sums are reduced across the wave with
// butterfly shuffles.  There is no cross-wave reduction: waves are
// independent, which keeps the engine latency-tolerant and free of barriers.
//
// Decode at batch 1 is bound by streaming the weights from HBM (Hazy
// Research, "Look Ma, No Bubbles!", introduction), so the engine's job is to
// keep enough 16-byte loads in flight on every CU; arithmetic per weight byte
// is B/2 FMAs.
#pragma once

#include "ld_common.hpp"

namespace ld {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot8v(const u32x4& w, const float* x, float acc) {
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

// Input-vector accessor: eight consecutive fp32 inputs of batch row b at
// column k (k % 8 == 0).  Either an fp32 activation matrix or, for the first
// layer, the widened bf16 embedding rows of the input tokens.  An optional
// bf16 gain multiplies the inputs (RMSNorm gain; the 1/rms factor itself is
// deferred to the epilogue).
struct XIn {
  const float* x;         // [B][ldx] fp32, or nullptr for embedding rows
  int ldx;
  const uint16_t* emb;    // [V][ldx] bf16 when x == nullptr
  const int* tokens;      // [B]
  int V;
  const uint16_t* gain;   // [K] bf16 or nullptr

  __device__ __forceinline__ void raw8(int b, int k, float* o) const {
    if (x) {
      const float4* p = reinterpret_cast<const float4*>(x + (int64_t)b * ldx + k);
      const float4 a = p[0], c = p[1];
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
      o[4] = c.x; o[5] = c.y; o[6] = c.z; o[7] = c.w;
    } else {
      int t = tokens[b];
      t = ((unsigned)t < (unsigned)V) ? t : 0;
      const u32x4 w = *reinterpret_cast<const u32x4*>(emb + (int64_t)t * ldx + k);
      o[0] = bf16lo(w.x); o[1] = bf16hi(w.x); o[2] = bf16lo(w.y); o[3] = bf16hi(w.y);
      o[4] = bf16lo(w.z); o[5] = bf16hi(w.z); o[6] = bf16lo(w.w); o[7] = bf16hi(w.w);
    }
  }

  __device__ __forceinline__ void load8(int b, int k, float* o) const {
    raw8(b, k, o);
    if (gain) {
      const u32x4 g = *reinterpret_cast<const u32x4*>(gain + k);
      o[0] *= bf16lo(g.x); o[1] *= bf16hi(g.x); o[2] *= bf16lo(g.y); o[3] *= bf16hi(g.y);
      o[4] *= bf16lo(g.z); o[5] *= bf16hi(g.z); o[6] *= bf16lo(g.w); o[7] *= bf16hi(g.w);
    }
  }
};

// Deferred RMSNorm factors r_b = 1/sqrt(sum_k x_bk^2 / K + eps) for b < B,
// computed by the whole workgroup into rs[0..B).  red: kWaves floats of LDS.
__device__ __forceinline__ void norm_scales(const XIn& xin, int B, int K, float eps, float* rs,
                                            float* red) {
  for (int b = 0; b < B; ++b) {
    float ss = 0.f;
    for (int k = threadIdx.x * 8; k < K; k += kThreads * 8) {
      float v[8];
      xin.raw8(b, k, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    }
    ss = block_sum(ss, red);
    if (threadIdx.x == 0) rs[b] = 1.0f / sqrtf(ss / (float)K + eps);
  }
  __syncthreads();
}

// A block of weights held in registers: NR rows x UC chunks, one 16-byte
// word per lane each.
template <int NR, int UC>
struct WBlock {
  u32x4 w[NR][UC];

  // rows[r] points at row r of the task (nullptr = masked row).
  __device__ __forceinline__ void load(const uint16_t* const (&rows)[NR], int K, int c0, int lane) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int k = (c0 + u) * kChunk + lane * 8;
        if (rows[r] != nullptr && k < K)
          w[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows[r] + k));
        else
          w[r][u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // acc[r][b] += W[r, chunk] . x[b0 + b, chunk] for b < nb (nb <= NB).
  template <int NB>
  __device__ __forceinline__ void fma(const XIn& xin, int b0, int nb, int K, int c0, int lane,
                                      float (&acc)[NR][NB]) const {
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int k = (c0 + u) * kChunk + lane * 8;
      if (k < K) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < nb) {
            float xv[8];
            xin.load8(b0 + b, k, xv);
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r][b] = dot8v(w[r][u], xv, acc[r][b]);
          }
        }
      }
    }
  }
};

// Drive one wave over its tasks.  A task is (batch tile bt, row tile t) with
// task index = bt * ntile + t; RowFn(t, rows) fills the NR row pointers of
// tile t; Epi(t, b0, nb, acc) consumes the wave-reduced sums (every lane
// holds every sum).  `blk` may already hold block 0 of the first task
// (prefetched before a readiness wait).
template <int NR, int UC, int NB, class RowFn, class Epi>
__device__ __forceinline__ void gemv_waves(const RowFn& rowfn, int ntile, int nbt, int K,
                                           const XIn& xin, int B, Epi& epi, WBlock<NR, UC>& blk,
                                           bool prefetched, int first, int stride, int lane) {
  const int nch = (K + kChunk - 1) / kChunk;
  const int ntask = ntile * nbt;
  const uint16_t* rows[NR];
  int t = first;
  if (t < ntask) {
    rowfn(t % ntile, rows);
    if (!prefetched) blk.load(rows, K, 0, lane);
  }
  for (; t < ntask; t += stride) {
    const int tile = t % ntile, bt = t / ntile;
    const int b0 = bt * NB, nb = min(NB, B - b0);
    float acc[NR][NB];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
    for (int c0 = 0;;) {
      blk.template fma<NB>(xin, b0, nb, K, c0, lane, acc);
      c0 += UC;
      if (c0 >= nch) break;
      blk.load(rows, K, c0, lane);
    }
    // start streaming the next task's first block before reducing this one
    const int tn = t + stride;
    if (tn < ntask) {
      rowfn(tn % ntile, rows);
      blk.load(rows, K, 0, lane);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
    epi(tile, b0, nb, acc);
  }
}

}  // namespace ld
