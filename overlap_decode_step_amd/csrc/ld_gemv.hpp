// ld_gemv.hpp - weight-streaming GEMV engine for small batches (VALU path).
//
// Decode at batch 1 is bound by streaming the weights from HBM (Hazy
// Research, "Look Ma, No Bubbles!", introduction).  The engine keeps many
// 16-byte non-temporal loads in flight on every CU:
//  - each wave owns NR weight rows at a time (a task) and streams them in
//    blocks of UC 512-element chunks, one 16-byte load per lane per (row,
//    chunk); the first block of a stage is issued before the stage waits for
//    its input (prefetch across the readiness wait);
//  - the input vectors (fp32, RMSNorm gain applied) are staged once per stage
//    into LDS with coherent loads, together with the sum of squares of the
//    deferred RMSNorm; the FMA loop then reads them with ds_read_b128;
//  - bf16 weights are widened in registers and multiplied in fp32; each
//    lane's partial sums are reduced across the wave with shuffles, so waves
//    never wait for each other inside a stage.
#pragma once

#include "ld_common.hpp"

namespace ld {

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

// Where a stage's input vectors come from: an fp32 activation matrix written
// by another workgroup (read coherently), or, for the first layer, the bf16
// embedding rows of the input tokens (read-only weights).
struct XSrc {
  const float* x;       // [B][ldx] fp32, or nullptr for embedding rows
  int ldx;
  const uint16_t* emb;  // [V][ldx] bf16 when x == nullptr
  const int* tokens;    // [B]
  int V;

  __device__ __forceinline__ void raw8(int b, int k, float* o) const {
    if (x) {
      ld_coh8(x + (int64_t)b * ldx + k, o);
    } else {
      int t = tokens[b];
      t = ((unsigned)t < (unsigned)V) ? t : 0;
      const u32x4 w = *reinterpret_cast<const u32x4*>(emb + (int64_t)t * ldx + k);
      o[0] = bf16lo(w.x); o[1] = bf16hi(w.x); o[2] = bf16lo(w.y); o[3] = bf16hi(w.y);
      o[4] = bf16lo(w.z); o[5] = bf16hi(w.z); o[6] = bf16lo(w.w); o[7] = bf16hi(w.w);
    }
  }
};

// Shared-memory scratch at the start of a workgroup's dynamic LDS.
struct Scratch {
  float red[kMaxWaves][8];
  float rs[64];  // deferred-norm factors of the staged batch rows
  float bestv[kMaxWaves][64];
  int besti[kMaxWaves][64];
  int flag[4];
};
constexpr int kScratchBytes = (int)((sizeof(Scratch) + 255) / 256 * 256);

// Stage batch rows [b0, b0+nb) of the input into LDS: xs[b*K + k] =
// x[b0+b][k] * gain[k] (gain may be null).  With `norm`, also
// rs[b] = 1/sqrt(sum_k x^2 / K + eps) over the raw inputs.  nb <= NB.
template <int NB>
__device__ __forceinline__ void stage_x(const XSrc& src, int b0, int nb, int K,
                                        const uint16_t* gain, bool norm, float eps, float* xs,
                                        Scratch& sc) {
  float ss[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) ss[b] = 0.f;
  const int n8 = K >> 3;
  for (int j = threadIdx.x; j < n8; j += blockDim.x) {
    float g[8];
    if (gain) {
      const u32x4 gw = *reinterpret_cast<const u32x4*>(gain + j * 8);
      g[0] = bf16lo(gw.x); g[1] = bf16hi(gw.x); g[2] = bf16lo(gw.y); g[3] = bf16hi(gw.y);
      g[4] = bf16lo(gw.z); g[5] = bf16hi(gw.z); g[6] = bf16lo(gw.w); g[7] = bf16hi(gw.w);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        float v[8];
        src.raw8(b0 + b, j * 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss[b] = fmaf(v[i], v[i], ss[b]);
        if (gain) {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] *= g[i];
        }
        float4* d = reinterpret_cast<float4*>(xs + (int64_t)b * K + j * 8);
        d[0] = make_float4(v[0], v[1], v[2], v[3]);
        d[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
  if (norm) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float s = wave_sum(ss[b]);
      if (lane_id() == 0) sc.red[wave_id()][b] = s;
    }
    __syncthreads();
    if (threadIdx.x < nb) {
      float s = 0.f;
      for (int w = 0; w < nwaves(); ++w) s += sc.red[w][threadIdx.x];
      sc.rs[threadIdx.x] = 1.0f / sqrtf(s / (float)K + eps);
    }
  }
  __syncthreads();
}

// A block of weights held in registers: NR rows x UC chunks, one 16-byte
// word per lane each.
template <int NR, int UC>
struct WBlock {
  u32x4 w[NR][UC];

  // rows[r]: row r of the task (nullptr = masked row).
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

  // acc[r][b] += W[r, block] . xs[b, block] for b < nb, inputs in LDS [nb][K].
  template <int NB>
  __device__ __forceinline__ void fma(const float* xs, int nb, int K, int c0, int lane,
                                      float (&acc)[NR][NB]) const {
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int k = (c0 + u) * kChunk + lane * 8;
      if (k < K) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < nb) {
            const float4* p = reinterpret_cast<const float4*>(xs + (int64_t)b * K + k);
            const float4 a = p[0], c = p[1];
            const float xv[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r][b] = dot8v(w[r][u], xv, acc[r][b]);
          }
        }
      }
    }
  }
};

// One GEMV stage for one workgroup: rows are split into tiles of NR rows
// (RowFn(tile, rows) fills the row pointers), tiles are dealt to the waves of
// the whole grid, the batch is processed in tiles of at most `bw` rows that
// fit the LDS staging area.  Epi(tile, b0, nb, acc) consumes wave-reduced
// sums (every lane holds every sum).  Wait(): the readiness wait, called once
// after the first block has been issued.
template <int NR, int UC, int NB, class RowFn, class WaitFn, class Epi>
__device__ __forceinline__ void gemv_stage(const RowFn& rowfn, int ntile, int K, const XSrc& src,
                                           const uint16_t* gain, bool norm, float eps, int B,
                                           int bw, const WaitFn& wait, Epi& epi, int wg, int nwg,
                                           char* smem) {
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  float* xs = reinterpret_cast<float*>(smem + kScratchBytes);
  const int lane = lane_id();
  const int first = wg * nwaves() + wave_id(), stride = nwg * nwaves();
  const int nch = (K + kChunk - 1) / kChunk;
  const int nbt = (B + bw - 1) / bw;
  const uint16_t* rows[NR];
  WBlock<NR, UC> blk;
  bool have = false;  // blk holds block 0 of task `first`
  if (first < ntile) {
    rowfn(first, rows);
    blk.load(rows, K, 0, lane);
    have = true;
  }
  wait();
  for (int bt = 0; bt < nbt; ++bt) {
    const int b0 = bt * bw, nb = min(bw, B - b0);
    stage_x<NB>(src, b0, nb, K, gain, norm, eps, xs, sc);
    for (int t = first; t < ntile; t += stride) {
      if (!have) {
        rowfn(t, rows);
        blk.load(rows, K, 0, lane);
      }
      have = false;
      float acc[NR][NB];
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
      for (int c0 = 0;;) {
        blk.template fma<NB>(xs, nb, K, c0, lane, acc);
        c0 += UC;
        if (c0 >= nch) break;
        blk.load(rows, K, c0, lane);
      }
      // issue the next task's first block before reducing this one
      const int tn = t + stride;
      if (tn < ntile || (bt + 1 < nbt && first < ntile)) {
        rowfn(tn < ntile ? tn : first, rows);
        blk.load(rows, K, 0, lane);
        have = true;
      }
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
      epi(t, b0, nb, acc, sc);
    }
    if (bt + 1 < nbt) __syncthreads();  // every wave is done with xs before restaging
  }
}

}  // namespace ld
