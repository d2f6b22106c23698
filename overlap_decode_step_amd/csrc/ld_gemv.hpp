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
  float rs[64];   // deferred-norm factors of the staged batch rows
  int pos[64];    // positions of the step (valid once pos_ok is set)
  int pos_ok;
  int flag[4];
};

// Every decode kernel starts with this (the scratch area persists across
// the stages of the persistent kernel).
__device__ __forceinline__ void scratch_init(char* smem) {
  if (threadIdx.x == 0) reinterpret_cast<Scratch*>(smem)->pos_ok = 0;
  __syncthreads();
}
constexpr int kScratchBytes = (int)((sizeof(Scratch) + 255) / 256 * 256);

// Reductions across a workgroup use a fixed partition of kRedThreads
// threads, so every execution mode (1024- or 512-thread workgroups) adds the
// same numbers in the same order and produces bitwise-equal results.
constexpr int kRedThreads = 512;

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
  if (threadIdx.x < kRedThreads) {
    for (int j = threadIdx.x; j < n8; j += kRedThreads) {
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
  }
  if (norm) {
    if (threadIdx.x < kRedThreads) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float s = wave_sum(ss[b]);
        if (lane_id() == 0) sc.red[wave_id()][b] = s;
      }
    }
    __syncthreads();
    if (threadIdx.x < nb) {
      float s = 0.f;
      for (int w = 0; w < kRedThreads / kWave; ++w) s += sc.red[w][threadIdx.x];
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

  // rows[r]: row r of the task (nullptr = masked row); columns >= kend masked.
  __device__ __forceinline__ void load(const uint16_t* const (&rows)[NR], int kend, int c0,
                                       int lane) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int k = (c0 + u) * kChunk + lane * 8;
        if (rows[r] != nullptr && k < kend)
          w[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows[r] + k));
        else
          w[r][u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // acc[r][b] += W[r, block] . xs[b, block] for b < nb; inputs in LDS with
  // row stride ldx; columns >= kend skipped.
  template <int NB>
  __device__ __forceinline__ void fma(const float* xs, int ldx, int nb, int kend, int c0, int lane,
                                      float (&acc)[NR][NB]) const {
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int k = (c0 + u) * kChunk + lane * 8;
      if (k < kend) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < nb) {
            const float4* p = reinterpret_cast<const float4*>(xs + (int64_t)b * ldx + k);
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

// One GEMV stage for one workgroup.  Rows are split into tiles of NR rows
// (RowFn(tile, rows) fills the row pointers) and the K dimension into KS
// slices; a task is (tile, slice) and tasks are dealt to the waves of the
// whole grid in rounds.  The KS slices of a tile land on KS neighbouring
// waves of one workgroup and are added through LDS in fixed order.  The batch
// is processed in tiles of at most `bw` rows that fit the LDS staging area.
// Epi(tile, b0, nb, acc, scratch) consumes the reduced sums (every lane of the
// calling wave holds every sum).  Wait(): the readiness wait, called once
// after the first block has been issued.
template <int NR, int UC, int NB, int KS, class RowFn, class WaitFn, class Epi>
__device__ __forceinline__ void gemv_stage(const RowFn& rowfn, int ntile, int K, const XSrc& src,
                                           const uint16_t* gain, bool norm, float eps, int B,
                                           int bw, const WaitFn& wait, Epi& epi, int wg, int nwg,
                                           char* smem) {
  static_assert(NR * NB <= 8 || KS == 1, "K-split partials must fit the scratch row");
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  float* xs = reinterpret_cast<float*>(smem + kScratchBytes);
  const int lane = lane_id(), wave = wave_id();
  const int first = wg * nwaves() + wave, stride = nwg * nwaves();
  const int nch = (K + kChunk - 1) / kChunk;
  const int nchp = (nch + KS - 1) / KS;  // chunks per K slice
  const int ntask = ntile * KS;
  const int rounds = (ntask + stride - 1) / stride;
  const int nbt = (B + bw - 1) / bw;
  auto slice = [&](int t, int& c0, int& kend) {
    const int kp = t % KS;
    c0 = kp * nchp;
    kend = min(K, (kp + 1) * nchp * kChunk);
  };
  const uint16_t* rows[NR];
  WBlock<NR, UC> blk;
  bool have = false;  // blk holds block 0 of task `first`
  // Prefetch across the wait, except in wave 0: it polls the readiness
  // counter, and loads return in order, so weight loads in flight would delay
  // every poll it makes.
  if (first < ntask && wave != 0) {
    int c0, kend;
    slice(first, c0, kend);
    rowfn(first / KS, rows);
    blk.load(rows, kend, c0, lane);
    have = true;
  }
  wait();
  for (int bt = 0; bt < nbt; ++bt) {
    const int b0 = bt * bw, nb = min(bw, B - b0);
    stage_x<NB>(src, b0, nb, K, gain, norm, eps, xs, sc);
    for (int r = 0; r < rounds; ++r) {
      const int t = first + r * stride;
      float acc[NR][NB];
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[i][b] = 0.f;
      if (t < ntask) {
        int c0, kend;
        slice(t, c0, kend);
        if (!have) {
          rowfn(t / KS, rows);
          blk.load(rows, kend, c0, lane);
        }
        have = false;
        const int cend = min(nch, c0 + nchp);
        for (int c = c0;;) {
          blk.template fma<NB>(xs, K, nb, kend, c, lane, acc);
          c += UC;
          if (c >= cend) break;
          blk.load(rows, kend, c, lane);
        }
        // issue the next task's first block before reducing this one
        const int tn = t + stride;
        const int tnext = tn < ntask ? tn : ((bt + 1 < nbt) ? first : -1);
        if (tnext >= 0) {
          int c1, k1;
          slice(tnext, c1, k1);
          rowfn(tnext / KS, rows);
          blk.load(rows, k1, c1, lane);
          have = true;
        }
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[i][b] = wave_sum(acc[i][b]);
      }
      if constexpr (KS == 1) {
        if (t < ntask) epi(t, b0, nb, acc, sc);
      } else {
        // slices of one tile sit on waves wave - wave % KS .. + KS - 1
        if (lane == 0) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) sc.red[wave][i * NB + b] = acc[i][b];
        }
        __syncthreads();
        if (t < ntask && wave % KS == 0) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              float v = 0.f;
              for (int q = 0; q < KS; ++q) v += sc.red[wave + q][i * NB + b];
              acc[i][b] = v;
            }
          epi(t / KS, b0, nb, acc, sc);
        }
        __syncthreads();
      }
    }
    if (bt + 1 < nbt) __syncthreads();  // every wave is done with xs before restaging
  }
}

}  // namespace ld
