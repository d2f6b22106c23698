// ld_mfma.hpp - bf16 MFMA engine of the decode step for batches of 16 and
// more (gfx950 matrix cores).
//
// From batch 16 up, the step is a skinny dense contraction Y[B,N] = X[B,K] .
// W[N,K]^T, and fp32 VALU FMAs fed from LDS run out of issue slots and LDS
// bandwidth before HBM does.  Here each 16-row tile of W is the A operand of
// v_mfma_f32_16x16x32_bf16 (weights are bf16, exact), and the activations are
// the B operand, split into two bf16 halves x = hi + lo with lo = bf16(x - hi)
// so that the product keeps about 16 mantissa bits of x: two MFMAs per tile,
// fp32 accumulation.
//
// Layout of one MFMA (checked on the device): lane l holds A[l%16][8*(l/16)+j]
// and B[8*(l/16)+j][l%16] for j < 8, and D[4*(l/16)+i][l%16] for i < 4.
//
// Work split: the N rows are cut into 16-row tiles dealt round-robin to the
// workgroups; a workgroup's 8 waves form WR x WK (WR = tiles side by side,
// WK = waves sharing a tile by interleaved 32-wide K steps), chosen from the
// number of tiles per workgroup.  The inputs are staged in LDS in K chunks,
// batch rows padded to 16, rows padded by 16 bytes against bank conflicts; a
// batch larger than the staging area allows is done in batch passes.  After
// the K loop, WK > 1 partial tiles are added through LDS in fixed order and
// the waves with wk == 0 call the per-element epilogue.
#pragma once

#include "ld_common.hpp"
#include "ld_gemv.hpp"

namespace ld {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaMinBatch = 16;  // batches from here on take this engine
constexpr int kMfmaTileMats = 2;   // 16-row tiles x matrices a wave accumulates at once
constexpr int kMfmaRing = 4;       // K steps of weight fragments in flight per wave
constexpr int kMfmaPad = 8;        // bf16 elements of padding per staged row
constexpr int kMfmaMinChunk = 512; // smallest K chunk (a wave's 64 lanes stage one row)

// Batch tiles of 16 a wave accumulates at once for a kernel built for NB
// batch rows: at most 2 (32 rows) within 128 VGPRs; larger batches take
// several batch passes.
template <int NB>
constexpr int kMfmaNbt = NB / 16 < 2 ? NB / 16 : 2;

// LDS bytes per staged batch row: hi and lo bf16 halves of a chunk of `kc`
// columns (plus padding), and the row's per-wave sums of squares (at most 16
// waves).
__host__ __device__ constexpr size_t mfma_row_bytes(int kc) {
  return (size_t)(kc + kMfmaPad) * 4 + 16 * 4;
}
// Staged rows of one batch pass (a multiple of 16) for a staging area of
// `cap` bytes, and the K chunk (a multiple of kMfmaMinChunk, no longer than K
// needs).
__host__ __device__ constexpr int mfma_pass_rows(int B, uint32_t cap) {
  return (int)(cap / mfma_row_bytes(kMfmaMinChunk)) / 16 * 16 < ((B + 15) / 16) * 16
             ? (int)(cap / mfma_row_bytes(kMfmaMinChunk)) / 16 * 16
             : ((B + 15) / 16) * 16;
}
__host__ __device__ constexpr int mfma_chunk(int rows, int K, uint32_t cap) {
  return (int)((cap / rows - 16 * 4) / 4 - kMfmaPad) / kMfmaMinChunk * kMfmaMinChunk <
                 (K + kMfmaMinChunk - 1) / kMfmaMinChunk * kMfmaMinChunk
             ? (int)((cap / rows - 16 * 4) / 4 - kMfmaPad) / kMfmaMinChunk * kMfmaMinChunk
             : (K + kMfmaMinChunk - 1) / kMfmaMinChunk * kMfmaMinChunk;
}

__device__ __forceinline__ uint16_t bf16_rn(float f) { return f2bf(f); }

// Rows of NT weight matrices in one buffer: tile t, matrix j, row r (0..15).
struct MatRows {
  const uint16_t* base;
  const uint16_t* m[2];
  int nrows, K;
  __device__ __forceinline__ uint32_t operator()(int t, int j, int r) const {
    const int row = t * 16 + r;
    return row < nrows ? (uint32_t)(((m[j] - base) + (int64_t)row * K) * 2) : kOob;
  }
};

// Epe(tile, r, b, bl, bt, v[NT]) gets the raw dot products of row 16*tile +
// r (r < 16) and batch row b, which is row bl = 16*bt + (lane % 16) of the
// current batch pass; sc.rs[bl] holds b's deferred-norm factor when `norm`.
// It is called only for b < B, by the lanes that hold the values; rows past
// the matrix end are the callee's to skip.  PassEnd(b0, nb) runs (in every
// thread) after each batch pass.
template <int NBT, int NT, class WaitFn, class Epe, class PassEnd>
__device__ __forceinline__ void mfma_stage(const MatRows& mr, int ntile, int K, const uint16_t* wbase,
                           uint32_t wbytes, const XSrc& src, const uint16_t* gain, bool norm,
                           float eps, int B, uint32_t x_cap, const WaitFn& wait, Epe& epe,
                           const PassEnd& pass_end, int wg, int nwg, char* smem) {
  constexpr int MT = kMfmaTileMats / NT;  // tiles per wave per tile pass
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  char* xbase = smem + kScratchBytes;
  const int lane = lane_id(), wave = wave_id(), nw = nwaves(), t = tid(), nth = blockDim.x;
  // ---- decomposition (uniform across the grid)
  const int tpw = (ntile + nwg - 1) / nwg;
  int WR = 1;
  while (WR < tpw && WR < nw) WR *= 2;
  const int WK = nw / WR, wr = wave % WR, wk = wave / WR;
  const int cnt = wg < ntile ? (ntile - 1 - wg) / nwg + 1 : 0;     // this workgroup's tiles
  const int mt = cnt > wr ? (cnt - 1 - wr) / WR + 1 : 0;            // this wave's tiles
  const int ntpass = ((tpw + WR - 1) / WR + MT - 1) / MT;  // tile passes
  const int prow = min(mfma_pass_rows(B, x_cap), NBT * 16);        // batch rows per pass
  const int nbpass = (B + prow - 1) / prow;
  const int KC = mfma_chunk(prow, K, x_cap), ldx = KC + kMfmaPad;
  const int nchunk = (K + KC - 1) / KC;
  uint16_t* xh = reinterpret_cast<uint16_t*>(xbase);
  uint16_t* xl = xh + (size_t)prow * ldx;
  float* red = reinterpret_cast<float*>(xbase);  // WK partial tiles (after the K loop)

  wait();
  for (int bp = 0; bp < nbpass; ++bp) {
    const int b0 = bp * prow, nb = min(prow, B - b0);
    // deferred-norm sums of squares of this pass's rows, accumulated over the
    // chunks in fixed order: per chunk, wave w's share of row b goes to
    // ssw[b * nw + w] (one value per wave) and is added in wave order
    float* ssw = reinterpret_cast<float*>(xbase + (size_t)prow * ldx * 4);  // [prow][16]
    float ssacc = 0.f;  // thread t < nb keeps row b0 + t's running sum
    for (int tp = 0; tp < ntpass; ++tp) {
      const int m0 = tp * MT;
      f32x4 acc[MT][NT][NBT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int bt = 0; bt < NBT; ++bt) acc[m][j][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
      uint32_t roff[MT][NT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          roff[m][j] = (m0 + m < mt) ? mr(wg + (wr + (m0 + m) * WR) * nwg, j, lane & 15) : kOob;
      const __amdgpu_buffer_rsrc_t rs = weight_rsrc(wbase, wbytes);
      for (int c = 0; c < nchunk; ++c) {
        const int kc0 = c * KC;
        // ---- stage rows [b0, b0 + prow) x columns [kc0, kc0 + KC): x * gain as
        // bf16 hi and lo; one 8-column group per thread per round (KC / 8 >=
        // 64 threads per row, so a wave's lanes share a row in each round)
        __syncthreads();  // the previous chunk's tiles and partial sums are consumed
        const int gpr = KC / 8;  // groups per row
        for (int g = t; g < prow * gpr; g += nth) {
          const int b = g / gpr, k = kc0 + (g - b * gpr) * 8;
          float v[8];
          float s2 = 0.f;
          if (b < nb && k < K) {
            src.raw8(b0 + b, k, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) s2 = fmaf(v[i], v[i], s2);
            if (gain) {
              const u32x4 gw = *reinterpret_cast<const u32x4*>(gain + k);
              v[0] *= bf16lo(gw.x); v[1] *= bf16hi(gw.x); v[2] *= bf16lo(gw.y); v[3] *= bf16hi(gw.y);
              v[4] *= bf16lo(gw.z); v[5] *= bf16hi(gw.z); v[6] *= bf16lo(gw.w); v[7] *= bf16hi(gw.w);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
          }
          uint16_t h[8], lo[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            h[i] = bf16_rn(v[i]);
            lo[i] = bf16_rn(v[i] - bf16f(h[i]));
          }
          const int o = b * ldx + (k - kc0);
          *reinterpret_cast<u32x4*>(xh + o) =
              u32x4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                    h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
          *reinterpret_cast<u32x4*>(xl + o) =
              u32x4{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16),
                    lo[4] | ((uint32_t)lo[5] << 16), lo[6] | ((uint32_t)lo[7] << 16)};
          if (norm && tp == 0) {
            // a round covers whole rows per wave: the wave's lanes share row b
            const float ws = wave_sum(s2);
            if (lane == 0) ssw[b * 16 + (g - b * gpr) / kWave] = ws;
          }
        }
        __syncthreads();
        if (norm && tp == 0 && t < nb) {
          // this chunk's per-wave shares of row b0 + t, in fixed order
          const int waves_per_row = gpr / kWave;
          float s = 0.f;
          for (int w = 0; w < waves_per_row; ++w) s += ssw[t * 16 + w];
          ssacc += s;
        }
        // ---- this wave's K steps of the chunk: s = wk, wk + WK, ...
        const int ns = min(KC, K - kc0 + 31) / 32;  // steps in this chunk
        const int nq = ns > wk ? (ns - 1 - wk) / WK + 1 : 0;
        u32x4 ring[kMfmaRing][MT][NT];
        auto issue = [&](u32x4 (&f)[MT][NT], int q) {
          const int k = kc0 + (wk + q * WK) * 32 + (lane >> 4) * 8;
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              const uint32_t off = (q < nq && roff[m][j] != kOob && k < K) ? roff[m][j] + 2u * k : kOob;
              f[m][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNt);
            }
        };
#pragma unroll
        for (int j = 0; j < kMfmaRing; ++j) issue(ring[j], j);
        for (int q0 = 0; q0 < nq; q0 += kMfmaRing) {
#pragma unroll
          for (int jj = 0; jj < kMfmaRing; ++jj) {
            const int q = q0 + jj;
            if (q < nq) {
              const int kl = (wk + q * WK) * 32 + (lane >> 4) * 8;  // column in the chunk
#pragma unroll
              for (int bt = 0; bt < NBT; ++bt) {
                if (bt * 16 < prow) {
                  // this batch tile's hi and lo fragments, used by every tile
                  const int o = (bt * 16 + (lane & 15)) * ldx + kl;
                  const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xh + o));
                  const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + o));
#pragma unroll
                  for (int m = 0; m < MT; ++m) {
                    if (m0 + m < mt) {
#pragma unroll
                      for (int j = 0; j < NT; ++j) {
                        const bf16x8 a = __builtin_bit_cast(bf16x8, ring[jj][m][j]);
                        acc[m][j][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[m][j][bt], 0, 0, 0);
                        acc[m][j][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[m][j][bt], 0, 0, 0);
                      }
                    }
                  }
                }
              }
            }
            issue(ring[jj], q + kMfmaRing);
          }
        }
      }
      // ---- norms of this batch pass (first tile pass only)
      if (norm && tp == 0) {
        __syncthreads();
        if (t < nb) sc.rs[t] = 1.0f / sqrtf(ssacc / (float)K + eps);
      }
      // ---- add the WK partial tiles in fixed order, then the epilogue
      __syncthreads();  // LDS staging area is free
      const int tiles_here = min(MT, max(0, mt - m0));
      if (WK > 1) {
        // wave (wr, wk) stores its partial tiles; the tile count per wave is
        // at most 1 when WK > 1 (WR >= tiles per workgroup)
        const int per = NT * NBT * 4 * kWave;  // floats per wave
        float* mine = red + (size_t)wave * per;
        if (tiles_here > 0) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
              for (int i = 0; i < 4; ++i) mine[((j * NBT + bt) * 4 + i) * kWave + lane] = acc[0][j][bt][i];
        }
        __syncthreads();
        if (wk == 0 && tiles_here > 0) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float s = acc[0][j][bt][i];
                for (int q = 1; q < WK; ++q)
                  s += red[(size_t)(wr + q * WR) * per + ((j * NBT + bt) * 4 + i) * kWave + lane];
                acc[0][j][bt][i] = s;
              }
        }
      }
      if (wk == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < tiles_here) {
            const int tile = wg + (wr + (m0 + m) * WR) * nwg;
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
              const int b = bt * 16 + (lane & 15);
              if (bt * 16 < prow && b < nb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  float v[NT];
#pragma unroll
                  for (int j = 0; j < NT; ++j) v[j] = acc[m][j][bt][i];
                  epe(tile, (lane >> 4) * 4 + i, b0 + b, b, bt, v);
                }
              }
            }
          }
        }
      }
    }
    pass_end(b0, nb);
  }
}

}  // namespace ld
