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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// x as the packed pair (bf16(x) | bf16(x - bf16(x)) << 16), both halves
// rounded to nearest even by the hardware conversion: the form in which the
// engine stages its inputs.  Producers feeding an MFMA stage directly write
// this form, so the stage copies it without a conversion pass.
__device__ __forceinline__ uint32_t split_pair(float x) {
  const float hi = (float)(__bf16)x;
  const bf16x2 hl = {(__bf16)x, (__bf16)(x - hi)};
  return __builtin_bit_cast(uint32_t, hl);
}

constexpr int kMfmaTileMats = 2;   // 16-row tiles x matrices a wave accumulates at once
// K steps of weight fragments in flight per wave: the persistent kernel has
// 256 VGPRs per wave, the stage kernels 128
constexpr int kMfmaRingBig = 8, kMfmaRingSmall = 4;
// ... but 6 when a wave accumulates 4 batch tiles (64 rows) from LDS
// fragments: with 8 the 64-row builds spilled (the persistent kernel 50
// VGPRs, the O stage kernel 19); with 6 they spill 5 and 0, and batch 64 went
// 3.94 -> 3.79 ms (MEGA) and 4.49 -> 4.35 ms (WAIT) at the Llama-1B shape
constexpr int kMfmaRing64 = 6;
constexpr int kMfmaPad = 4;        // 4-byte elements of padding per staged row (16 bytes)
// Tiles per workgroup at least: a stage with fewer tiles than this many per
// workgroup runs on ntile / kMfmaMinTiles workgroups, the others skip it.
// Every participating workgroup stages the whole input, so this trades
// staging traffic (B x K x 4 bytes per workgroup) against streaming lanes.
constexpr int kMfmaMinTiles = 1;
constexpr int kMfmaMinChunk = 512; // smallest K chunk (a wave's 64 lanes stage one row)
constexpr int kSc1 = 16;           // cache policy: agent-coherent (sc1)

// Batch tiles of 16 a wave accumulates at once for a kernel built for NB
// batch rows and a weight ring of MR steps: at most 2 (32 rows) within the
// stage kernels' 128 VGPRs, 4 (64 rows) in the persistent kernel's 256;
// larger batches take several batch passes, each streaming the weights again.
template <int NB, int MR>
constexpr int kMfmaNbt = MR == kMfmaRingBig ? (NB / 16 < 4 ? NB / 16 : 4) : (NB / 16 < 2 ? NB / 16 : 2);

// LDS bytes per staged batch row: hi and lo bf16 halves of a chunk of `kc`
// columns (plus padding), and the row's per-wave sums of squares (at most 16
// waves).
__host__ __device__ constexpr size_t mfma_row_bytes(int kc) {
  return (size_t)(kc + kMfmaPad) * 4 + 16 * 4;
}
// Staged rows of one batch pass (a multiple of 16) for a staging area of
// `cap` bytes, and the K chunk.
__host__ __device__ constexpr int mfma_pass_rows(int B, uint32_t cap) {
  return (int)(cap / mfma_row_bytes(kMfmaMinChunk)) / 16 * 16 < ((B + 15) / 16) * 16
             ? (int)(cap / mfma_row_bytes(kMfmaMinChunk)) / 16 * 16
             : ((B + 15) / 16) * 16;
}
__host__ __device__ constexpr int mfma_chunk(int rows, int K, uint32_t cap) {
  // a power of two from kMfmaMinChunk up: the largest that fits, and no
  // longer than K needs (the staging maps 512 threads onto its 8-column groups)
  int kc = kMfmaMinChunk;
  while (kc < K && (size_t)rows * mfma_row_bytes(2 * kc) <= cap && 2 * kc <= 4096) kc *= 2;
  return kc;
}


// Split K (64-row kernels).  Every workgroup of a stage stages the
// batch rows it multiplies, B x K x 4 bytes, so at 64 rows a narrow matrix
// (the O and Down projections) moves many times its own weight bytes as
// staging traffic.  Such a stage splits K into S ranges: workgroup wg takes
// range wg % S and deals the tiles among the nwg / S workgroups of its range,
// so it stages only K / S columns.  Each range's partial tile goes to a
// scratch buffer, part[((s * B + b) * nrows + row], and a per-(batch pass,
// tile) counter elects the last arriving range, which adds the S partials in
// range order and calls the epilogue with the sum.  (At 16 rows the extra
// round trips cost more than the staging saved.)
struct SplitK {
  float* part;
  uint32_t* ctr;
  int S;
};
// Split K runs in the 64-row builds with 256 VGPRs (the persistent kernel,
// and the whole-kernel-wait kernels at 64 rows); measured there: batch 64
// 5.03 -> 4.53 ms (WAIT), 4.52 -> 4.14 ms (MEGA).  In the tile-flag mode's
// 128-VGPR builds it spilled registers and was 2% slower.
template <int NB, int MR>
constexpr bool kSplitK = NB >= 16 && MR == kMfmaRingBig;

// The largest power of two up to kMaxKSplit that divides the grid, leaves
// every range at least kMfmaMinChunk columns and at most 8 tiles per
// workgroup.
__host__ __device__ constexpr int mfma_splits(int ntile, int K, int nwg) {
  int S = 1;
  while (2 * S <= kMaxKSplit && nwg % (2 * S) == 0 && K / (2 * S) >= kMfmaMinChunk &&
         ntile * 2 * S <= 8 * nwg)
    S *= 2;
  return S;
}

// Activations handed from one MFMA stage to the next are stored in the order
// the B operand is loaded in, as split-bf16 pairs (split_pair) with the
// consumer's RMSNorm gain already applied: for K step s (32 columns) of batch
// tile bt (16 rows) the 64 lanes' fragments lie in one 2 KB block, lane l
// holding the 8 consecutive columns 8 (l / 16) .. + 7 of batch row l % 16 (32
// contiguous bytes).  A wave then loads a B fragment with two 16-byte loads
// per lane straight from memory, like its weight fragments, with no staging
// copy, conversion pass or workgroup barrier.  kp: the matrix's K rounded up
// to a multiple of 32 (the padding columns stay zero).  Word offset of
// element (b, k):
// frag_word(b, k, kp) (ld_params.hpp).

// Weight-and-activation ring depth (K steps in flight per wave) of a stage
// that loads its B fragments from memory: each step holds kMfmaTileMats
// weight fragments (4 VGPRs each) and NBT pairs of 16-byte activation loads
// (8 VGPRs per batch tile), within kDirectRingVgprs of the 256-VGPR builds
// and kDirectRingVgprsSmall of the 128-VGPR ones (more spilled registers).
// With one batch tile (16 rows) the 256-VGPR builds take 128, a ring of 8
// steps: 1-2% faster than 6 at batch 16 (Llama-1B 1.670 -> 1.649 ms MEGA, 8B
// and 70B likewise), the persistent kernel then spilling one VGPR.
constexpr int kDirectRingVgprs = 96, kDirectRingVgprs16 = 128, kDirectRingVgprsSmall = 56;
template <int NBT, int RING>
constexpr int kDirectRingRaw =
    (RING == kMfmaRingBig ? (NBT == 1 ? kDirectRingVgprs16 : kDirectRingVgprs) : kDirectRingVgprsSmall) /
    (4 * kMfmaTileMats + 8 * NBT);
template <int NBT, int RING>
constexpr int kDirectRing =
    kDirectRingRaw<NBT, RING> < 2 ? 2 : (kDirectRingRaw<NBT, RING> > RING ? RING : kDirectRingRaw<NBT, RING>);

// Deferred-norm sums from a fragment source: ss[b * ss_ld + q], q < ss_n,
// are the producer's sums of squares per (batch row, 16-row output tile).
// Row b of a pass is read by the kSsGroup threads t = 8 b .. 8 b + 7, thread
// p adding tiles p, p + 8, ... in ascending order, U of its loads issued
// before any is used (a clamped index past the end reads a valid word that
// is not added); the group then adds its 8 partials in a fixed tree
// (lane_group_sum), the sum landing in its last lane.  The group size is
// fixed, so every pass size, tiling and mode adds the same numbers in the
// same order.
constexpr int kSsGroup = 8;
__device__ __forceinline__ float ss_partial(const XSrc& src, int b0, int nb, int t) {
  constexpr int U = 16, G = kSsGroup;
  const int b = t / G, p = t - b * G;
  float s2 = 0.f;
  if (b < nb) {
    const float* row = src.ss + (int64_t)(b0 + b) * src.ss_ld;
    for (int q0 = p; q0 < src.ss_n; q0 += U * G) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld_coh(row + min(q0 + u * G, src.ss_n - 1));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (q0 + u * G < src.ss_n) s2 += v[u];
    }
  }
  return s2;
}

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
// the matrix end are the callee's to skip; it returns the value it stored
// (0 for a skipped row).  PassEnd(b0, nb) runs (in every thread) after each
// batch pass.
//
// SRC: where the B fragments come from.
//  kSrcConvert: src.x (fp32) or the embedding rows, staged in LDS in K chunks
//    and converted there to split-bf16 pairs, gain applied, norm sums taken.
//  kSrcFragLds: src.frag (B-fragment order, pairs, gain applied), its blocks
//    copied as they are into LDS once per chunk and shared by the waves;
//  kSrcDirect: src.frag loaded one K step at a time into registers through
//    the weight ring, no LDS (each wave reads only its own K steps, so used
//    when a workgroup holds one column of tiles).
// With a fragment source the deferred-norm factors come from src.ss, the
// sums of squares the producer stored per (batch row, 16-row output tile).
// With ss_out the stage stores those sums for its own outputs: ss_out[b *
// ss_ld + tile] = sum over the tile's rows of the squares of what Epe
// returned.  All three give the MFMAs the same fragments in the same order.
enum : int { kSrcConvert = 0, kSrcFragLds = 1, kSrcDirect = 2 };
template <int NBT, int NT, int RING, int SRC = kSrcConvert, class WaitFn, class Epe, class PassEnd>
__device__ __forceinline__ void mfma_stage(const MatRows& mr, int ntile, int K, const uint16_t* wbase,
                                           uint32_t wbytes, const XSrc& src, const uint16_t* gain,
                                           bool norm, float eps, int B, uint32_t x_cap,
                                           const WaitFn& wait, Epe& epe, const PassEnd& pass_end,
                                           int wg, int nwg, char* smem,
                                           const SplitK& sk = SplitK{nullptr, nullptr, 1},
                                           bool row_major = false, float* ss_out = nullptr,
                                           int ss_ld = 0) {
  constexpr int MT = kMfmaTileMats / NT;  // tiles per wave per tile pass
  constexpr bool DIRECT = SRC == kSrcDirect, FRAG = SRC != kSrcConvert;
  constexpr int RR = DIRECT ? kDirectRing<NBT, RING>                // K steps in flight per wave
                            : (NBT >= 4 && RING > kMfmaRing64 ? kMfmaRing64 : RING);
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  char* xbase = smem + kScratchBytes;
  const int lane = lane_id(), wave = wave_id(), nw = nwaves(), t = tid(), nth = blockDim.x;
  // ---- K range of this workgroup (split K: norm-free single-matrix stages)
  const int S = sk.S, ks = wg % S;
  const int Kfull = K;
  const int Ks = S > 1 ? ((K + S - 1) / S + 31) / 32 * 32 : K;
  const int ks0 = ks * Ks;
  K = max(0, min(Kfull, ks0 + Ks) - ks0);  // columns of this range
  wg /= S;
  nwg /= S;
  // ---- decomposition (uniform across the workgroups of a range)
  nwg = min(nwg, max(1, ntile / kMfmaMinTiles));
  if (wg >= nwg || K <= 0) return;
  const int tpw = (ntile + nwg - 1) / nwg;
  int WR = 1;
  while (WR < tpw && WR < nw) WR *= 2;
  const int WK = nw / WR, wr = wave % WR, wk = wave / WR;
  const int cnt = wg < ntile ? (ntile - 1 - wg) / nwg + 1 : 0;     // this workgroup's tiles
  const int mt = cnt > wr ? (cnt - 1 - wr) / WR + 1 : 0;            // this wave's tiles
  const int ntpass = ((tpw + WR - 1) / WR + MT - 1) / MT;            // tile passes
  // batch rows per pass: as many as the staging area and the accumulators
  // allow (column-major: every batch row meets each weight fragment while it
  // is in registers), or 16 (row-major: one batch tile stays staged while the
  // whole weight stream passes, once per tile).  The K chunk is the
  // column-major one in both, so both add the same numbers in the same order.
  const int prow_col = DIRECT ? NBT * 16 : min(mfma_pass_rows(B, x_cap), NBT * 16);
  const int prow = row_major ? 16 : prow_col;
  const int nbpass = (B + prow - 1) / prow;
  // (reading fragments from memory, the whole K range is one chunk)
  const int KC = DIRECT ? round32(K) : mfma_chunk(prow_col, K, x_cap);
  const int ldx = KC + kMfmaPad;  // staged row stride (4-byte words)
  const int nchunk = (K + KC - 1) / KC;
  const int cs = KC / 32;                 // 32-wide K steps per chunk
  const int spc = (cs + WK - 1) / WK;     // this wave's step slots per chunk (wave wk takes
                                          // steps wk, wk + WK, ...)
  const int nslot = nchunk * spc;
  // staged rows [prow][ldx] of 4-byte words: the fp32 inputs as copied, then
  // each word rewritten in place as the pair (bf16 hi | bf16 lo << 16)
  uint32_t* xw = reinterpret_cast<uint32_t*>(xbase);
  float* ssw = reinterpret_cast<float*>(xbase + (size_t)prow * ldx * 4);  // [prow] row sums
  float* red = reinterpret_cast<float*>(xbase);  // WK partial tiles (after the K loop)
  const __amdgpu_buffer_rsrc_t rs = weight_rsrc(wbase, wbytes);

  uint32_t roff[MT][NT];
  auto set_tiles = [&](int m0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        roff[m][j] = (m0 + m < mt) ? mr(wg + (wr + (m0 + m) * WR) * nwg, j, lane & 15) : kOob;
  };
  // weight fragments of slot i (chunk i / spc, step wk + WK * (i % spc));
  // past the end, or past K, the loads are masked
  auto issue = [&](u32x4 (&f)[MT][NT], int i) {
    const int c = i / spc, st = wk + (i - c * spc) * WK;
    const int k = c * KC + st * 32 + (lane >> 4) * 8;
    const bool ok = i < nslot && st < cs;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const uint32_t off = (ok && roff[m][j] != kOob && k < K) ? roff[m][j] + 2u * (ks0 + k) : kOob;
        f[m][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNt);
      }
  };
  // direct mode: the B fragments of slot i for batch tiles bt < NBT of the
  // pass starting at row b0 (agent-coherent loads: other workgroups stored
  // them during this step); masked past the stream or the pass
  const __amdgpu_buffer_rsrc_t frs =
      weight_rsrc(reinterpret_cast<const uint16_t*>(src.frag), DIRECT ? (uint32_t)((size_t)((B + 15) / 16) * src.kp * 64) : 0u);
  auto issue_b = [&](u32x4 (&fb)[NBT][2], int i, int b0, int nb) {
    if constexpr (DIRECT) {
      const int st = wk + i * WK;
      const bool ok = i < nslot && st < cs;
      const int sg = (ks0 >> 5) + st;  // K step in the whole matrix
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt) {
        const bool okb = ok && bt * 16 < min(prow, nb);
        const uint32_t off = okb ? (uint32_t)((((int64_t)((b0 >> 4) + bt) * (src.kp >> 5) + sg) * 128 + lane) * 16) : 0u;
        const __amdgpu_buffer_rsrc_t r = okb ? frs : weight_rsrc(reinterpret_cast<const uint16_t*>(src.frag), 0u);
        fb[bt][0] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1);
        fb[bt][1] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 1024u, 0, kSc1);
      }
    } else {
      (void)fb, (void)i, (void)b0, (void)nb;
    }
  };
  float ssacc = 0.f;  // thread t < nb: row b0 + t's running sum of squares
  // ---- stage rows [b0, b0 + prow) x columns [kc0, kc0 + KC) of chunk c
  auto stage_chunk = [&](int b0, int nb, int c, bool sums) {
    const int kc0 = c * KC;
    __syncthreads();  // the previous chunk's pairs and partial sums are consumed
    if constexpr (SRC == kSrcFragLds) {
      // the chunk's fragment blocks (2 KB per batch tile and K step, two
      // contiguous 1 KB halves) copied as they are: LDS holds [tile][step of
      // the chunk][half][lane] 16-byte words, one 1 KB half per wave
      // instruction (agent-coherent: other workgroups wrote them this step)
      (void)sums;
      const int ntl = (min(prow, nb) + 15) / 16, spk = KC >> 5;
      const int ns = min(spk, (K - kc0 + 31) >> 5);  // steps of this chunk
      const int s0 = (ks0 + kc0) >> 5;                // its first step in the matrix
      const char* fb = reinterpret_cast<const char*>(src.frag);
      for (int i = wave; i < ntl * ns * 2; i += nw) {
        const int bt = i / (ns * 2), r = i - bt * (ns * 2), s = r >> 1, h = r & 1;
        const char* g = fb + ((((int64_t)((b0 >> 4) + bt) * (src.kp >> 5) + s0 + s) * 2 + h) << 10) + lane * 16;
        char* dst = reinterpret_cast<char*>(xw) + (((size_t)(bt * spk + s) * 2 + h) << 10);
        __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)dst, 16, 0, kSc1);
      }
      wave_drain();
      __syncthreads();
      return;
    }
    const int gpr = KC / 8;  // 8-column groups per row (a multiple of 64)
    const int ngroup = prow * gpr;
    if (src.x != nullptr) {
      // fp32 activations: direct-to-LDS copies of 1 KB per wave instruction,
      // all issued before any wait (agent-coherent: other workgroups wrote
      // them during this step)
      const int kn = min(KC, K - kc0), pieces = (kn + 255) / 256;
      for (int i = wave; i < nb * pieces; i += nw) {
        const int b = i / pieces, pc = i - b * pieces;
        const int k = pc * 256 + lane * 4;
        char* dst = reinterpret_cast<char*>(xw + (size_t)b * ldx + pc * 256);
        if (k < kn)
          __builtin_amdgcn_global_load_lds(src.x + (int64_t)(b0 + b) * src.ldx + ks0 + kc0 + k,
                                           (__attribute__((address_space(3))) void*)dst, 16, 0,
                                           kSc1);
      }
      wave_drain();
      __syncthreads();
      if (src.pairs) {
        // already split-bf16 pairs: only the columns of the last 32-wide K
        // step past K (if K is not a multiple of 32) must read as zeros
        const int kpad = min(KC, ((kn + 31) / 32) * 32);
        for (int i = t; i < nb * (kpad - kn); i += nth) {
          const int b = i / (kpad - kn), k = kn + (i - b * (kpad - kn));
          xw[(size_t)b * ldx + k] = 0u;
        }
        if (kpad > kn) __syncthreads();
        return;
      }
    }
    // thread t takes 8-column group j = t % gpr of the rows h, h + tpc, ...
    // (h = t / gpr, tpc = threads per column group), so it loads its gain
    // once: inputs (from the copy, or the bf16 embedding rows of the first
    // layer) -> norm partial sums, gain, and each element rewritten as the
    // pair (bf16 hi, bf16 lo) by the hardware conversion (round to nearest
    // even); rows past the batch and columns past K become zeros
    const int tpc = nth / gpr, j = t % gpr, h = t / gpr;
    const int kk = j * 8, k = kc0 + kk;
    float g8[8];
    if (gain && k < K) {
      const u32x4 gw = *reinterpret_cast<const u32x4*>(gain + ks0 + k);
      g8[0] = bf16lo(gw.x); g8[1] = bf16hi(gw.x); g8[2] = bf16lo(gw.y); g8[3] = bf16hi(gw.y);
      g8[4] = bf16lo(gw.z); g8[5] = bf16hi(gw.z); g8[6] = bf16lo(gw.w); g8[7] = bf16hi(gw.w);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) g8[i] = 1.f;
    }
    for (int b = h; b < prow; b += tpc) {
      uint32_t* w = xw + (size_t)b * ldx + kk;
      float v[8];
      if (b < nb && k < K) {
        if (src.x != nullptr) {
          const u32x4 p0 = *reinterpret_cast<const u32x4*>(w);
          const u32x4 p1 = *reinterpret_cast<const u32x4*>(w + 4);
          v[0] = __uint_as_float(p0.x); v[1] = __uint_as_float(p0.y);
          v[2] = __uint_as_float(p0.z); v[3] = __uint_as_float(p0.w);
          v[4] = __uint_as_float(p1.x); v[5] = __uint_as_float(p1.y);
          v[6] = __uint_as_float(p1.z); v[7] = __uint_as_float(p1.w);
        } else {
          src.raw8(b0 + b, ks0 + k, v);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
      }
      if (sums) {
        float s2 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s2 = fmaf(v[i], v[i], s2);
        // the wave's 64 lanes hold 64 column groups of row b
        s2 = wave_sum(s2);
        if (lane == 0) ssw[b * 16 + (j >> 6)] = s2;
      }
      uint32_t pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = split_pair(v[i] * g8[i]);
      *reinterpret_cast<u32x4*>(w) = u32x4{pr[0], pr[1], pr[2], pr[3]};
      *reinterpret_cast<u32x4*>(w + 4) = u32x4{pr[4], pr[5], pr[6], pr[7]};
    }
    __syncthreads();
    if (sums && t < nb) {
      // the row's per-wave shares, in fixed order
      float sr = 0.f;
      for (int q = 0; q < gpr / kWave; ++q) sr += ssw[t * 16 + q];
      ssacc += sr;
    }
  };


  u32x4 ring[RR][MT][NT];
  u32x4 bring[DIRECT ? RR : 1][NBT][2];
  set_tiles(0);
  if (wave != 0) {  // weight loads across the wait, except in the polling wave
#pragma unroll
    for (int j = 0; j < RR; ++j) issue(ring[j], j);
  }
  wait(ks0, ks0 + K);  // (the K range this workgroup reads)
  for (int bp = 0; bp < nbpass; ++bp) {
    const int b0 = bp * prow, nb = min(prow, B - b0);
    ssacc = 0.f;
    for (int tp = 0; tp < ntpass; ++tp) {
      const int m0 = tp * MT;
      const bool sums = norm && tp == 0;
      if (bp > 0 || tp > 0) set_tiles(m0);
      if (bp > 0 || tp > 0 || wave == 0) {
#pragma unroll
        for (int j = 0; j < RR; ++j) issue(ring[j], j);
      }
      if constexpr (DIRECT) {
#pragma unroll
        for (int j = 0; j < RR; ++j) issue_b(bring[j], j, b0, nb);
      }
      f32x4 acc[MT][NT][NBT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int bt = 0; bt < NBT; ++bt) acc[m][j][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!DIRECT) stage_chunk(b0, nb, 0, sums);
      // fragment source: this thread's share of the norm sums, read before
      // the K loop (its loads overlap the first K steps' loads)
      float ssp = 0.f;
      if constexpr (FRAG) {
        if (sums) ssp = ss_partial(src, b0, nb, t);
      }
      // ---- one ring over the whole K stream; a chunk boundary restages the
      // inputs while the next chunk's weight loads are already in flight
      for (int i0 = 0; i0 < nslot; i0 += RR) {
#pragma unroll
        for (int jj = 0; jj < RR; ++jj) {
          const int i = i0 + jj;
          const int c = i / spc, st = wk + (i - c * spc) * WK;
          if constexpr (!DIRECT) {
            if (i < nslot && i == c * spc && c > 0) stage_chunk(b0, nb, c, sums);
          }
          if (i < nslot && st < cs && c * KC + st * 32 < K) {
            const int kl = st * 32 + (lane >> 4) * 8;  // column in the chunk
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
              if (bt * 16 < prow) {
                // this batch tile's hi and lo fragments, used by every tile
                u32x4 p0, p1;
                if constexpr (DIRECT) {
                  p0 = bring[jj][bt][0];
                  p1 = bring[jj][bt][1];
                } else if constexpr (SRC == kSrcFragLds) {
                  const char* q = reinterpret_cast<const char*>(xw) +
                                  ((((size_t)bt * (KC >> 5) + st) * 2) << 10) + lane * 16;
                  p0 = *reinterpret_cast<const u32x4*>(q);
                  p1 = *reinterpret_cast<const u32x4*>(q + 1024);
                } else {
                  const uint32_t* w = xw + (size_t)(bt * 16 + (lane & 15)) * ldx + kl;
                  p0 = *reinterpret_cast<const u32x4*>(w);
                  p1 = *reinterpret_cast<const u32x4*>(w + 4);
                }
                // (hi | lo << 16) pairs -> 8 hi halves, 8 lo halves
                const u32x4 hh{(p0.x & 0xFFFFu) | (p0.y << 16), (p0.z & 0xFFFFu) | (p0.w << 16),
                               (p1.x & 0xFFFFu) | (p1.y << 16), (p1.z & 0xFFFFu) | (p1.w << 16)};
                const u32x4 ll{(p0.x >> 16) | (p0.y & 0xFFFF0000u),
                               (p0.z >> 16) | (p0.w & 0xFFFF0000u),
                               (p1.x >> 16) | (p1.y & 0xFFFF0000u),
                               (p1.z >> 16) | (p1.w & 0xFFFF0000u)};
                const bf16x8 bh = __builtin_bit_cast(bf16x8, hh);
                const bf16x8 bl = __builtin_bit_cast(bf16x8, ll);
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
          issue(ring[jj], i + RR);
          if constexpr (DIRECT) issue_b(bring[jj], i + RR, b0, nb);
        }
      }
      // ---- norms of this batch pass (first tile pass only)
      if constexpr (FRAG) {
        // from the producer's sums of squares (ss_partial, read before the
        // K loop): each row's group of kSsGroup threads adds its partials
        if (sums) {
          const float s2 = lane_group_sum(ssp, kSsGroup);
          __syncthreads();
          const int b = t / kSsGroup;
          if (b < nb && t - b * kSsGroup == kSsGroup - 1)
            sc.rs[b] = 1.0f / sqrtf(s2 / (float)Kfull + eps);
        }
      } else if (sums) {
        __syncthreads();
        if (t < nb) sc.rs[t] = 1.0f / sqrtf(ssacc / (float)Kfull + eps);
      }
      // ---- add the WK partial tiles in fixed order, then the epilogue
      __syncthreads();  // LDS staging area is free
      const int tiles_here = min(MT, max(0, mt - m0));
      if (WK > 1) {
        // wave (wr, wk) stores its partial tile; a wave has at most one tile
        // when WK > 1 (WR >= tiles per workgroup)
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
                float sum = acc[0][j][bt][i];
                for (int q = 1; q < WK; ++q)
                  sum += red[(size_t)(wr + q * WR) * per + ((j * NBT + bt) * 4 + i) * kWave + lane];
                acc[0][j][bt][i] = sum;
              }
        }
      }
      if (wk == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < tiles_here) {
            const int tile = wg + (wr + (m0 + m) * WR) * nwg;
            bool split = false;
            if constexpr (NT == 1) split = S > 1;
            if (split) {
              // this range's partial tile, then the last arriving range adds
              // all S partials in range order
#pragma unroll
              for (int bt = 0; bt < NBT; ++bt) {
                const int b = bt * 16 + (lane & 15);
                if (bt * 16 < prow && b < nb) {
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    const int row = tile * 16 + (lane >> 4) * 4 + i;
                    if (row < mr.nrows)
                      st_coh(sk.part + ((int64_t)ks * B + b0 + b) * mr.nrows + row, acc[m][0][bt][i]);
                  }
                }
              }
              wave_drain();
              uint32_t last = 0;
              if (lane == 0) {
                uint32_t* c = sk.ctr + (int64_t)bp * ntile + tile;
                const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                last = old == (uint32_t)(S - 1);
                if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
              if (!__shfl(last, 0)) continue;
            }
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
              const int b = bt * 16 + (lane & 15);
              float s2 = 0.f;  // squares of the stored values of this lane's 4 rows
              if (bt * 16 < prow && b < nb) {
                if (split) {
                  // every range's partials of the lane's 4 rows in one round
                  // of loads, then added in range order
                  float pv[4][kMaxKSplit];
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    const int row = tile * 16 + (lane >> 4) * 4 + i;
#pragma unroll
                    for (int q = 0; q < kMaxKSplit; ++q)
                      pv[i][q] = (q < S && row < mr.nrows)
                                     ? ld_coh(sk.part + ((int64_t)q * B + b0 + b) * mr.nrows + row)
                                     : 0.f;
                  }
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    float v[NT] = {pv[i][0]};
#pragma unroll
                    for (int q = 1; q < kMaxKSplit; ++q)
                      if (q < S) v[0] += pv[i][q];
                    const float r = epe(tile, (lane >> 4) * 4 + i, b0 + b, b, bt, v);
                    s2 = fmaf(r, r, s2);
                  }
                } else {
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    float v[NT];
#pragma unroll
                    for (int j = 0; j < NT; ++j) v[j] = acc[m][j][bt][i];
                    const float r = epe(tile, (lane >> 4) * 4 + i, b0 + b, b, bt, v);
                    s2 = fmaf(r, r, s2);
                  }
                }
              }
              if (ss_out != nullptr) {
                // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the tile's 16 rows of
                // one batch row: their sum, in a fixed order
                s2 += __shfl_xor(s2, 16, kWave);
                s2 += __shfl_xor(s2, 32, kWave);
                if (lane < 16 && bt * 16 < prow && b < nb)
                  st_coh(ss_out + (int64_t)(b0 + b) * ss_ld + tile, s2);
              }
            }
          }
        }
      }
    }
    pass_end(b0, nb);
  }
}

// A fragment-source stage: direct loads when every workgroup holds a single
// column of 16-row tiles (its waves then split K, so no wave loads another's
// fragments), otherwise one LDS copy of the fragments shared by the waves.
// (The decomposition is mfma_stage's: tiles per workgroup of a K range.)
template <int NBT, int NT, int RING, class WaitFn, class Epe, class PassEnd>
__device__ __forceinline__ void mfma_stage_frag(const MatRows& mr, int ntile, int K,
                                                const uint16_t* wbase, uint32_t wbytes,
                                                const XSrc& src, bool norm, float eps, int B,
                                                uint32_t x_cap, const WaitFn& wait, Epe& epe,
                                                const PassEnd& pass_end, int wg, int nwg,
                                                char* smem,
                                                const SplitK& sk = SplitK{nullptr, nullptr, 1},
                                                bool row_major = false, float* ss_out = nullptr,
                                                int ss_ld = 0) {
  const int nwr = min(nwg / sk.S, max(1, ntile / kMfmaMinTiles));
  // (64-row passes would hold 32 VGPRs of fragments per K step: they share one copy)
  if constexpr (NBT <= 2) {
    if ((ntile + nwr - 1) / nwr <= 1) {
      mfma_stage<NBT, NT, RING, kSrcDirect>(mr, ntile, K, wbase, wbytes, src, nullptr, norm, eps, B,
                                          x_cap, wait, epe, pass_end, wg, nwg, smem, sk, row_major,
                                          ss_out, ss_ld);
      return;
    }
  }
  mfma_stage<NBT, NT, RING, kSrcFragLds>(mr, ntile, K, wbase, wbytes, src, nullptr, norm, eps, B,
                                           x_cap, wait, epe, pass_end, wg, nwg, smem, sk,
                                           row_major, ss_out, ss_ld);
}

}  // namespace ld
