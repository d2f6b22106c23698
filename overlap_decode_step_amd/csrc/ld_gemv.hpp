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
  // MFMA engine only: x holds each value as its split-bf16 pair (the
  // producer wrote split_pair(v)), staged as copied, with no conversion pass;
  // only for inputs without an RMSNorm gain or norm
  bool pairs = false;
  // MFMA engine only: the same inputs as split-bf16 pairs in B-fragment
  // order (frag_word, K rounded up to kp), the consumer's gain applied, read
  // straight into registers; with a deferred norm, ss[b * ss_ld + t] for t <
  // ss_n are the producer's sums of squares per output tile of row b
  const uint32_t* frag = nullptr;
  int kp = 0;
  const float* ss = nullptr;
  int ss_n = 0, ss_ld = 0;

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
  int attn_T;     // the attention stage's split length (set with pos)
  int attn_items; // its items, and whether the step combines its splits in a
  int attn_phase; // phase of its own (set with pos)
  int flag[4];
  int cnt[kMaxTileCtrs];  // rows this workgroup wrote per row-count counter
};

// A stage's write-through results held in registers until the wave's
// weight stream is done.  A wave's memory operations complete in order, so a
// write-through store issued between weight loads holds back every later
// load until memory acknowledges it.  With DEFER each lane keeps at most one
// pending (address, value): reserve(n) hands out the next n lane slots for
// one task's results and first writes the pending ones when the wave's 64
// slots are used up, and flush() writes them.  Without DEFER, hold() stores
// at once and every task uses lane slots from 0.  Deferring was measured
// faster from batch 2 (batch 4: 2.5-3%) and slower at batch 1 (1-2%), where
// a wave holds one result per task.
template <bool DEFER>
struct HeldStores {
  float* ptr = nullptr;
  float val = 0.f;
  int used = 0;  // slots handed out (the same in every lane)

  __device__ __forceinline__ void flush() {
    if constexpr (DEFER) {
      if (ptr != nullptr) st_coh(ptr, val);
      ptr = nullptr;
      used = 0;
    }
  }
  __device__ __forceinline__ int reserve(int n) {
    if constexpr (!DEFER) return (void)n, 0;
    if (used + n > kWave) flush();
    const int base = used;
    used += n;
    return base;
  }
  __device__ __forceinline__ void hold(float* p, float v) {
    if constexpr (DEFER) {
      ptr = p;
      val = v;
    } else {
      st_coh(p, v);
    }
  }
};

// Every decode kernel starts with this (the scratch area persists across
// the stages of the persistent kernel).
__device__ __forceinline__ void scratch_init(char* smem) {
  if (tid() == 0) reinterpret_cast<Scratch*>(smem)->pos_ok = 0;
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
// A thread's column groups are j = tid, tid + kRedThreads, ...  With U > 1
// (single-row inputs) it issues the loads of U groups before it uses any, so
// a wide input costs one round trip per U groups rather than one per group;
// the groups are added in the same order.  (A gain, if any, is read when a
// group is used: the callers that group have none.)
template <int NB, int U = 1>
__device__ __forceinline__ void stage_x(const XSrc& src, int b0, int nb, int K,
                                        const uint16_t* gain, bool norm, float eps, float* xs,
                                        Scratch& sc) {
  float ss[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) ss[b] = 0.f;
  const int n8 = K >> 3;
  if constexpr (U > 1) {
    static_assert(NB == 1, "grouped staging holds one row's groups");
    if (tid() < kRedThreads) {
      for (int j0 = tid(); j0 < n8; j0 += U * kRedThreads) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (j0 + u * kRedThreads < n8) src.raw8(b0, (j0 + u * kRedThreads) * 8, v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * kRedThreads;
          if (j >= n8) break;
#pragma unroll
          for (int i = 0; i < 8; ++i) ss[0] = fmaf(v[u][i], v[u][i], ss[0]);
          if (gain) {
            const u32x4 gw = *reinterpret_cast<const u32x4*>(gain + j * 8);
            v[u][0] *= bf16lo(gw.x); v[u][1] *= bf16hi(gw.x); v[u][2] *= bf16lo(gw.y);
            v[u][3] *= bf16hi(gw.y); v[u][4] *= bf16lo(gw.z); v[u][5] *= bf16hi(gw.z);
            v[u][6] *= bf16lo(gw.w); v[u][7] *= bf16hi(gw.w);
          }
          float4* d = reinterpret_cast<float4*>(xs + j * 8);
          d[0] = make_float4(v[u][0], v[u][1], v[u][2], v[u][3]);
          d[1] = make_float4(v[u][4], v[u][5], v[u][6], v[u][7]);
        }
      }
    }
  } else if (tid() < kRedThreads) {
    for (int j = tid(); j < n8; j += kRedThreads) {
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
    if (tid() < kRedThreads) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float s = wave_sum(ss[b]);
        if (lane_id() == 0) sc.red[wave_id()][b] = s;
      }
    }
    __syncthreads();
    if (tid() < nb) {
      float s = 0.f;
      for (int w = 0; w < kRedThreads / kWave; ++w) s += sc.red[w][tid()];
      sc.rs[tid()] = 1.0f / sqrtf(s / (float)K + eps);
    }
  }
  __syncthreads();
}

// Weights are read through buffer loads: the row's byte offset goes in the
// scalar offset operand (it is the same for the whole wave), the lane's
// column offset in a vector register shared by all rows of a block.  A masked
// row uses a zero-length buffer, whose loads return zeros without touching
// memory, so every wave issues the same loads on every path; that keeps the
// compiler's memory-counter waits exact for a ring of blocks in flight.  A
// lane whose columns lie past the row end rereads the row's last 16 bytes
// (the FMA skips those lanes).  Cache policy: non-temporal (weights are
// streamed once per step).
constexpr uint32_t kOob = 0xFFFFFFFFu;  // row offset of a masked row
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, raw (untyped) access
constexpr int kNt = 2;                  // cache policy: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// A block of weights held in registers: NR rows x UC chunks, one 16-byte
// word per lane each.
template <int NR, int UC>
struct WBlock {
  u32x4 w[NR][UC];

  // roff[r]: byte offset of row r in the buffer [base, base + bytes), or kOob
  // (masked row); rows have K columns.
  __device__ __forceinline__ void load(const uint16_t* base, uint32_t bytes,
                                       const uint32_t (&roff)[NR], int K, int c0, int lane) {
    uint32_t voff[UC];
#pragma unroll
    for (int u = 0; u < UC; ++u)
      voff[u] = (uint32_t)min(((c0 + u) * kChunk + lane * 8) * 2, K * 2 - 16);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const bool ok = roff[r] != kOob;
      const __amdgpu_buffer_rsrc_t rs = weight_rsrc(base, ok ? bytes : 0u);
      const uint32_t so = ok ? roff[r] : 0u;
#pragma unroll
      for (int u = 0; u < UC; ++u) w[r][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[u], so, kNt);
    }
  }

  // A block copied to LDS by WStream::copy_to_lds (chunk (r, u) at
  // (r * UC + u) KB, 16 bytes per lane).
  __device__ __forceinline__ void load_lds(const char* src, int lane) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int u = 0; u < UC; ++u)
        w[r][u] = *reinterpret_cast<const u32x4*>(src + (r * UC + u) * 1024 + lane * 16);
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

// One wave's weight stream in a GEMV stage.  Rows are split into tiles of NR
// rows (RowFn(tile, rows) fills the row pointers, nullptr for a masked row;
// all rows lie in the buffer [wbase, wbase + wbytes)), one tile per task.
// Round q deals tiles [q * stride, (q + 1) * stride) to the grid's waves in
// order, so at any time the whole grid streams one contiguous window of the
// matrix (measured faster than giving each XCD its own contiguous range;
// dealing fewer tiles to the workgroups busy with attention was measured
// slower too).  The wave's tasks are streamed as one sequence of blocks of UC
// chunks.
template <int NR, int UC, class RowFn>
struct WStream {
  const RowFn& rowfn;
  const uint16_t* wbase;
  uint32_t wbytes;
  int K, nch, bpt, first, stride, nblk;

  __device__ __forceinline__ WStream(const RowFn& f, int ntile, int K_, const uint16_t* base,
                                     uint32_t bytes, int wg, int nwg)
      : rowfn(f), wbase(base), wbytes(bytes), K(K_) {
    nch = (K + kChunk - 1) / kChunk;
    bpt = (nch + UC - 1) / UC;  // blocks per task
    first = wg * nwaves() + wave_id();
    stride = nwg * nwaves();
    const int ntask = first < ntile ? (ntile - 1 - first) / stride + 1 : 0;
    nblk = ntask * bpt;
  }
  __device__ __forceinline__ int task(int q) const { return first + q * stride; }

  // Block i of the stream into blk; past the end every row is masked.
  __device__ __forceinline__ void issue(WBlock<NR, UC>& blk, int i, int lane) const {
    const int q = i / bpt;
    uint32_t roff[NR];
    const uint16_t* rows[NR];
    rowfn(task(q), rows);
#pragma unroll
    for (int r = 0; r < NR; ++r)
      roff[r] = __builtin_amdgcn_readfirstlane(
          (i < nblk && rows[r] != nullptr)
              ? (uint32_t)(reinterpret_cast<const char*>(rows[r]) - reinterpret_cast<const char*>(wbase))
              : kOob);
    blk.load(wbase, wbytes, roff, K, (i - q * bpt) * UC, lane);
  }

  // Block i copied straight into LDS at dst (NR * UC KB, laid out for
  // WBlock::load_lds), with direct-to-LDS loads; nothing for masked rows,
  // columns past K or blocks past the end.
  __device__ __forceinline__ void copy_to_lds(int i, char* dst, int lane) const {
    if (i >= nblk) return;
    const int q = i / bpt, c0 = (i - q * bpt) * UC;
    const uint16_t* rows[NR];
    rowfn(task(q), rows);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int k = (c0 + u) * kChunk + lane * 8;
        if (rows[r] != nullptr && k < K)
          __builtin_amdgcn_global_load_lds(rows[r] + k,
                                           (__attribute__((address_space(3))) void*)(
                                               dst + (r * UC + u) * 1024),
                                           16, 0, kNt);
      }
    }
  }
};

// LDS bytes of one block of NR rows x UC chunks.
template <int NR, int UC>
constexpr int kBlockLdsBytes = NR * UC * 1024;

// Issue the first PF blocks of a stream into a ring.  Called right before the
// stage's readiness wait it skips wave 0, which polls the counters (loads
// return in order, so weight loads in flight would delay every poll); called
// long before (`all_waves`: the persistent kernel issues the SwiGLU stage's
// first blocks while attention runs) every wave takes part.
template <int NR, int UC, int PF, class RowFn>
__device__ __forceinline__ void gemv_prefetch(const WStream<NR, UC, RowFn>& ws,
                                              WBlock<NR, UC> (&ring)[PF], bool all_waves = false) {
  if (all_waves || wave_id() != 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) ws.issue(ring[j], j, lane_id());
  }
}

// One GEMV stage for one workgroup: each wave streams its blocks keeping PF
// in flight (the ring); unless `prefetched` (by gemv_prefetch with all_waves),
// the first PF are issued here, before the stage waits for its input in waves
// other than 0 and after it in wave 0.  With `lds`, this wave's blocks PF ..
// PF + nl - 1 were already copied to LDS there (WStream::copy_to_lds, long
// before): blocks are consumed in stream order, the first PF from the ring,
// then those from LDS, then the rest streamed through the ring.  The batch is
// processed in tiles of at most `bw` rows that fit the LDS staging area; each
// batch tile streams the weights again (LDS blocks are used by a single batch
// tile only).  Epi(tile, b0, nb, acc, scratch) consumes the reduced sums
// (every lane of the calling wave holds every sum).
template <int NR, int UC, int NB, int PF, int SU = 1, class RowFn, class WaitFn, class Epi>
__device__ __forceinline__ void gemv_run(const WStream<NR, UC, RowFn>& ws,
                                         WBlock<NR, UC> (&ring)[PF], bool prefetched,
                                         const XSrc& src, const uint16_t* gain, bool norm, float eps,
                                         int B, int bw, const WaitFn& wait, Epi& epi, char* smem,
                                         const char* lds = nullptr, int nl_req = 0) {
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  float* xs = reinterpret_cast<float*>(smem + kScratchBytes);
  const int lane = lane_id(), wave = wave_id();
  const int K = ws.K, nch = ws.nch, bpt = ws.bpt, nblk = ws.nblk;
  const int nbt = (B + bw - 1) / bw;
  // blocks taken from LDS, and the register stream: block regblk(r)
  const int nl = (lds != nullptr && nbt == 1) ? max(0, min(nl_req, nblk - PF)) : 0;
  const int nreg = nblk - nl;
  auto regblk = [&](int r) { return r < nreg ? (r < PF ? r : r + nl) : nblk; };
  if (!prefetched) gemv_prefetch(ws, ring);
  wait();
  for (int bt = 0; bt < nbt; ++bt) {
    const int b0 = bt * bw, nb = min(bw, B - b0);
    // (its input loads also wait for any earlier loads of this wave: the
    // copies to LDS have landed once this returns)
    stage_x<NB, SU>(src, b0, nb, K, gain, norm, eps, xs, sc);
    if (bt > 0 || (wave == 0 && !prefetched)) {
#pragma unroll
      for (int j = 0; j < PF; ++j) ws.issue(ring[j], j, lane);
    }
    float acc[NR][NB];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
    auto consume = [&](const WBlock<NR, UC>& blk, int i) {
      const int q = i / bpt, c = (i - q * bpt) * UC;
      blk.template fma<NB>(xs, K, nb, K, c, lane, acc);
      if (c + UC >= nch) {  // last block of task q
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
        epi(ws.task(q), b0, nb, acc, sc);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
      }
    };
    auto lds_blocks = [&]() {
      for (int q = 0; q < nl; ++q) {
        WBlock<NR, UC> blk;
        blk.load_lds(lds + q * kBlockLdsBytes<NR, UC>, lane);
        consume(blk, PF + q);
      }
    };
    for (int r0 = 0; r0 < nreg; r0 += PF) {
      if (r0 == PF) lds_blocks();
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int r = r0 + j;
        if (r < nreg) consume(ring[j], regblk(r));
        ws.issue(ring[j], regblk(r + PF), lane);
      }
    }
    if (nreg <= PF) lds_blocks();
    if (bt + 1 < nbt) __syncthreads();  // every wave is done with xs before restaging
  }
}

// Stage columns [k0, k0 + kn) of batch rows [b0, b0 + nb) into xs with row
// stride ldx (inputs without gain or norm).  A thread takes the 8-column
// groups j = tid, tid + blockDim, ... and keeps V groups' loads in flight
// (V groups of one row, V / 2 of two rows, ..., or one group of V rows)
// before it stores any.
template <int NB, int V>
__device__ __forceinline__ void stage_x_cols(const XSrc& src, int b0, int nb, int k0, int kn,
                                             int ldx, float* xs) {
  constexpr int RB = NB < V ? NB : V, U = V / RB;  // rows and groups per round
  const int n8 = kn >> 3, nth = blockDim.x;
  for (int j0 = tid(); j0 < n8; j0 += U * nth) {
    for (int r0 = 0; r0 < nb; r0 += RB) {
      float v[U][RB][8];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < RB; ++b)
          if (r0 + b < nb && j0 + u * nth < n8) src.raw8(b0 + r0 + b, k0 + (j0 + u * nth) * 8, v[u][b]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < RB; ++b)
          if (r0 + b < nb && j0 + u * nth < n8) {
            float4* d = reinterpret_cast<float4*>(xs + (int64_t)(r0 + b) * ldx + (j0 + u * nth) * 8);
            d[0] = make_float4(v[u][b][0], v[u][b][1], v[u][b][2], v[u][b][3]);
            d[1] = make_float4(v[u][b][4], v[u][b][5], v[u][b][6], v[u][b][7]);
          }
    }
  }
  __syncthreads();
}

// K-chunked GEMV: for inputs whose whole rows would not fit the LDS staging
// area for the batch (gemv_run would then stream the weights once per batch
// tile), the batch is staged in column chunks of KC (a multiple of a block's
// UC * kChunk columns) and each wave takes its tasks in groups of G, whose
// per-lane sums stay in registers from chunk to chunk.  Per chunk, the
// group's tasks are streamed one after another, each over its blocks in the
// chunk.  A task's lanes add the same blocks in the same order as in
// gemv_run (its blocks in increasing column order, then one wave sum), so
// the results are bitwise the same, but the weights stream once per batch
// tile of bw rows, where bw * KC fits the staging area rather than bw * K.
// The stream is a fixed sequence per (group, chunk) segment of G tasks x
// nbp blocks (the chunk's blocks padded to a multiple of PF with masked
// ones; missing tasks masked too), the same in every wave, so the chunk
// restaging barriers line up; the ring of PF blocks runs across segments.
template <int NR, int UC, int NB, int PF, int G, int V, class RowFn, class WaitFn, class Epi>
__device__ __forceinline__ void gemv_run_kc(const WStream<NR, UC, RowFn>& ws, int ntile,
                                            WBlock<NR, UC> (&ring)[PF], const XSrc& src, int B,
                                            int bw, int KC, const WaitFn& wait, Epi& epi,
                                            char* smem) {
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  float* xs = reinterpret_cast<float*>(smem + kScratchBytes);
  const int lane = lane_id(), wave = wave_id();
  const int K = ws.K, bpt = ws.bpt;
  const int bpc = KC / (UC * kChunk);               // blocks per chunk per task
  const int nkc = (K + KC - 1) / KC;                // chunks
  const int nbp = (bpc + PF - 1) / PF * PF;         // padded blocks per segment row
  const int first0 = ws.first - wave;               // the workgroup's wave 0
  const int ntask0 = first0 < ntile ? (ntile - 1 - first0) / ws.stride + 1 : 0;
  const int ntask = ws.nblk / bpt;                  // this wave's tasks
  const int ngr = (ntask0 + G - 1) / G;             // groups (the same in every wave)
  const int seg = G * nbp, nseq = ngr * nkc * seg;
  // element e of the sequence -> block of the task-major stream (masked
  // past the end of a task, a chunk or the wave's tasks)
  auto block_of = [&](int e) -> int {
    if (e >= nseq) return ws.nblk;
    const int gk = e / seg, r = e - gk * seg;
    const int g = gk / nkc, kc = gk - g * nkc;
    const int t = r / nbp, cb = r - t * nbp;
    const int q = g * G + t, bk = kc * bpc + cb;
    return (q < ntask && cb < bpc && bk < bpt) ? q * bpt + bk : ws.nblk;
  };
  const int nbt = (B + bw - 1) / bw;
  for (int bt = 0; bt < nbt; ++bt) {
    const int b0 = bt * bw, nb = min(bw, B - b0);
    if (bt == 0) {
      // the first blocks before the readiness wait, except in the polling wave
      if (wave != 0) {
#pragma unroll
        for (int j = 0; j < PF; ++j) ws.issue(ring[j], block_of(j), lane);
      }
      wait();
    }
    if (bt > 0 || wave == 0) {
#pragma unroll
      for (int j = 0; j < PF; ++j) ws.issue(ring[j], block_of(j), lane);
    }
    for (int g = 0; g < ngr; ++g) {
      float acc[G][NR][NB];
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[t][r][b] = 0.f;
      for (int kc = 0; kc < nkc; ++kc) {
        const int k0 = kc * KC;
        if (bt > 0 || g > 0 || kc > 0) __syncthreads();  // every wave is done with xs
        stage_x_cols<NB, V>(src, b0, nb, k0, min(KC, K - k0), KC, xs);
        const float* xk = xs - k0;  // column k of row b at xk[b * KC + k]
        const int ebase = (g * nkc + kc) * seg;
#pragma unroll
        for (int t = 0; t < G; ++t) {
          for (int c0 = 0; c0 < nbp; c0 += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j) {
              const int e = ebase + t * nbp + c0 + j;
              const int blk = block_of(e);
              if (blk < ws.nblk) ring[j].template fma<NB>(xk, KC, nb, K, (blk % bpt) * UC, lane, acc[t]);
              ws.issue(ring[j], block_of(e + PF), lane);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < G; ++t) {
        const int q = g * G + t;
        if (q < ntask) {
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[t][r][b] = wave_sum(acc[t][r][b]);
          epi(ws.task(q), b0, nb, acc[t], sc);
        }
      }
    }
  }
}

// A whole GEMV stage with its own ring.  KCM > 0 and xcap (the LDS staging
// area's bytes) given: an input without gain or norm may be taken in column
// chunks (gemv_run_kc) when that needs fewer passes over the weights than
// whole rows in batch tiles (ties keep whole rows).  A chunk of PF blocks
// per task keeps the ring full; a chunk of one block (half the ring's slots
// then masked padding) is used only where it saves a further pass.  KCM = 1
// (the register-lean form every build with the path uses): at most 2 tasks
// and 2 staged groups in registers; KCM = 2: up to 4 of each.
template <int NR, int UC, int NB, int PF, int SU = 1, int KCM = 0, class RowFn, class WaitFn,
          class Epi>
__device__ __forceinline__ void gemv_stage(const RowFn& rowfn, int ntile, int K,
                                           const uint16_t* wbase, uint32_t wbytes, const XSrc& src,
                                           const uint16_t* gain, bool norm, float eps, int B,
                                           int bw, const WaitFn& wait, Epi& epi, int wg, int nwg,
                                           char* smem, uint32_t xcap = 0) {
  const WStream<NR, UC, RowFn> ws(rowfn, ntile, K, wbase, wbytes, wg, nwg);
  WBlock<NR, UC> ring[PF];
  if constexpr (KCM > 0) {
    const int rows = min(B, NB);
    if (xcap > 0 && gain == nullptr && !norm && (int64_t)K * 4 * rows > (int64_t)xcap) {
      constexpr int CB = UC * kChunk;  // columns of one block
      auto passes = [&](int w) { return w > 0 ? (rows + w - 1) / w : 0x7FFF; };
      const int fitw = (int)(xcap / ((uint32_t)K * 4));
      const int w2 = min(rows, (int)(xcap / ((uint32_t)PF * CB * 4)));  // chunks of PF blocks
      const int w1 = min(rows, (int)(xcap / ((uint32_t)CB * 4)));       // chunks of one block
      int bwk = 0, KC = 0;
      if (passes(w2) < passes(fitw)) {
        bwk = w2;
        KC = min((K + PF * CB - 1) / (PF * CB), (int)(xcap / ((uint32_t)w2 * PF * CB * 4))) * PF * CB;
      }
      if (passes(w1) < min(passes(fitw), passes(w2))) {
        bwk = w1;
        KC = min((K + CB - 1) / CB, (int)(xcap / ((uint32_t)w1 * CB * 4))) * CB;
      }
      if (bwk > 0) {
        constexpr int GM = KCM == 1 ? 2 : 4, V = KCM == 1 ? 2 : 4;
        const int first0 = wg * nwaves();
        const int ntask0 = first0 < ntile ? (ntile - 1 - first0) / (nwg * nwaves()) + 1 : 0;
        if (ntask0 <= 1)
          gemv_run_kc<NR, UC, NB, PF, 1, V>(ws, ntile, ring, src, B, bwk, KC, wait, epi, smem);
        else if (ntask0 <= 2 || GM == 2 || NB > 4)
          gemv_run_kc<NR, UC, NB, PF, 2, V>(ws, ntile, ring, src, B, bwk, KC, wait, epi, smem);
        else
          gemv_run_kc<NR, UC, NB, PF, GM, V>(ws, ntile, ring, src, B, bwk, KC, wait, epi, smem);
        return;
      }
    }
  }
  gemv_run<NR, UC, NB, PF, SU>(ws, ring, false, src, gain, norm, eps, B, bw, wait, epi, smem);
}

}  // namespace ld
