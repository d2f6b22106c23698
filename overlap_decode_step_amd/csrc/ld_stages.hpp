// ld_stages.hpp - the stages of one decode step as workgroup-level device
// functions.  Every execution mode calls these same functions: one kernel
// per stage (whole-kernel wait or tile-flag overlap) or one persistent
// kernel that runs them back to back.  A stage's workgroups loop over its
// tiles (persistent style), issue the loads of their first weight block,
// then wait for the stage's input to be signalled ready, compute, and
// finally signal their own completion once.
//
// Stage list per layer (the layer step list of a dense Llama decoder):
//   QKV  : q|k|v = Wqkv . n(x)       (RMSNorm folded in: gain on the staged
//                                      inputs, 1/rms factor on the outputs)
//   ATTN : RoPE on q and the new k, bf16 K/V append at the position,
//          split-KV grouped-query attention, last-arriver combine
//   O    : x' = x + Wo . o
//   GU   : h = silu(Wg . n(x')) * (Wu . n(x'))   (the fused first MLP stage
//          of "Deep Kernel Fusion for Transformers", Summary)
//   D    : x'' = x' + Wd . h          (the separate second MLP stage, Key
//                                      points, "Fusion scope")
// then LM : logits = Wlm . n(x), greedy argmax by the last-arriving workgroup.
#pragma once

#include "ld_common.hpp"
#include "ld_gemv.hpp"
#include "ld_params.hpp"

namespace ld {

// Per-stage tile shapes of the VALU engine: NR rows x UC chunks per block.
constexpr int kNrQkv = 1, kUcQkv = 4;
constexpr int kNrO = 1, kUcO = 4;
constexpr int kPairsGu = 1, kUcGu = 4;  // one (gate, up) row pair per task
constexpr int kNrD = 1, kUcD = 8;
constexpr int kNrLm = 2, kUcLm = 4;

__host__ __device__ constexpr size_t attn_smem_bytes(int group, int d, int T) {
  return (size_t)group * d * 4             /* rotated q */
         + 2 * (size_t)T * (d / 2 + 1) * 4 /* K, V tiles, rows padded by one dword */
         + (size_t)group * T * 4           /* scores */
         + (size_t)group * 2 * 4;          /* (max, sum) per head */
}

__device__ __forceinline__ const uint16_t* layer_w(const Params& P, int l, int64_t off) {
  return P.W.layer0 + (int64_t)l * P.W.layer_stride + off;
}

__device__ __forceinline__ uint32_t* stage_ctr(const Params& P, int l, int slot) {
  return P.K.ctr + ((int64_t)l * kStageCtrs + slot) * kCtrWords;
}

__device__ __forceinline__ uint32_t* split_ctr(const Params& P, int l, int b, int kvh) {
  return P.K.split_ctr + (((int64_t)l * P.D.max_batch + b) * P.D.nkv + kvh) * 16;
}

__device__ __forceinline__ SyncArgs sync_of(const Params& P) {
  return SyncArgs{P.K.err, P.K.watchdog};
}

__device__ __forceinline__ int clamp_pos(const Params& P, int b) {
  const int p = P.S.pos[b];
  return ((unsigned)p < (unsigned)P.D.max_seq) ? p : 0;
}

// Batch rows whose inputs of length K fit the LDS staging area at once.
__device__ __forceinline__ int batch_tile(const Params& P, int K, int NB) {
  const int fit = (int)(P.S.x_cap / ((size_t)K * 4));
  return max(1, min(NB, fit));
}

__device__ __forceinline__ void signal_if(const Params& P, uint32_t* ctr, int who) {
  if (!P.S.wait) wg_signal(ctr, who);
}

// ----------------------------------------------------------------- QKV

template <int NB>
__device__ void stage_qkv(const Params& P, int l, int wg, int nwg, char* smem) {
  constexpr int NR = kNrQkv, UC = kUcQkv;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int rows_total = D.qkv_rows, K = D.H, B = P.S.B;
  const uint16_t* Wm = layer_w(P, l, P.W.o_wqkv);
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  if (l == 0 && wg == 0 && threadIdx.x < B) {
    const int t = P.S.tokens[threadIdx.x], p = P.S.pos[threadIdx.x];
    if ((unsigned)t >= (unsigned)D.V) raise_error(P.K.err, kErrToken);
    if ((unsigned)p >= (unsigned)D.max_seq) raise_error(P.K.err, kErrPos);
  }
  auto wait = [&]() {
    if (!P.S.wait && l > 0) wg_wait(sync_of(P), stage_ctr(P, l - 1, kCD), P.S.t_d, kSQkv);
  };
  const XSrc src{l == 0 ? nullptr : P.K.xa, K, P.W.embed, P.S.tokens, D.V};
  float* out = P.K.qkv;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch& sc) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NR + r;
        if (b < nb && row < rows_total && lane == ((r * NB + b) & (kWave - 1)))
          st_coh(out + (int64_t)(b0 + b) * rows_total + row, acc[r][b] * sc.rs[b]);
      }
  };
  gemv_stage<NR, UC, NB>(rowfn, (rows_total + NR - 1) / NR, K, src,
                         layer_w(P, l, P.W.o_attn_norm), true, D.eps, B, batch_tile(P, K, NB),
                         wait, epi, wg, nwg, smem);
  signal_if(P, stage_ctr(P, l, kCQkv), wg);
}

// ------------------------------------------------------------ attention

// One (sequence b, kv head, split s) item: positions [s*T, min(s*T+T, p+1)).
__device__ void attn_item(const Params& P, int l, int b, int kvh, int s, int nsplit, int p,
                          char* smem) {
  const Dims& D = P.D;
  const int T = D.split_len, d = D.d, half = d / 2, group = D.group, rowd = half + 1;
  const int tid = threadIdx.x, nth = blockDim.x, lane = lane_id(), wave = wave_id();
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  float* qs = reinterpret_cast<float*>(smem + kScratchBytes);  // [group][d]
  uint32_t* Ks = reinterpret_cast<uint32_t*>(qs + group * d);  // [T][rowd]
  uint32_t* Vs = Ks + T * rowd;                                // [T][rowd]
  float* Sc = reinterpret_cast<float*>(Vs + T * rowd);         // [group][T]
  float* ml = Sc + group * T;                                  // [group][2]

  const int n0 = s * T, n1 = min(n0 + T, p + 1), n = n1 - n0;
  const bool has_new = (n1 == p + 1);
  const float* qkv = P.K.qkv + (int64_t)b * D.qkv_rows;
  const float* rope = P.K.rope + (int64_t)p * half * 2;
  const int64_t cache_off =
      ((((int64_t)l * D.max_batch + b) * D.nkv + kvh) * D.max_seq) * (int64_t)d;
  uint16_t* kc = P.K.kc + cache_off;
  uint16_t* vc = P.K.vc + cache_off;

  // q heads of this group, rotated to position p (rotate-half pairs)
  for (int idx = tid; idx < group * half; idx += nth) {
    const int g = idx / half, i = idx - g * half;
    const float* qh = qkv + (int64_t)(kvh * group + g) * d;
    const float q0 = ld_coh(qh + i), q1 = ld_coh(qh + i + half);
    const float c = rope[2 * i], sn = rope[2 * i + 1];
    qs[g * d + i] = q0 * c - q1 * sn;
    qs[g * d + i + half] = q0 * sn + q1 * c;
  }
  // cached K/V rows of this split (the new row, if any, is filled below)
  const int ncached = has_new ? n - 1 : n;
  const int w8 = d / 8;  // 16-byte words per row
  for (int idx = tid; idx < ncached * w8; idx += nth) {
    const int t = idx / w8, j = idx - t * w8;
    const u32x4 kk = *reinterpret_cast<const u32x4*>(kc + (int64_t)(n0 + t) * d + j * 8);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(vc + (int64_t)(n0 + t) * d + j * 8);
    uint32_t* kd = Ks + t * rowd + j * 4;
    uint32_t* vd = Vs + t * rowd + j * 4;
    kd[0] = kk.x; kd[1] = kk.y; kd[2] = kk.z; kd[3] = kk.w;
    vd[0] = vv.x; vd[1] = vv.y; vd[2] = vv.z; vd[3] = vv.w;
  }
  if (has_new) {
    // rotate the new key, round k and v to bf16, append them to the cache at p
    const float* kh = qkv + D.qd + (int64_t)kvh * d;
    const float* vh = qkv + D.qd + D.kvd + (int64_t)kvh * d;
    uint16_t* kl = reinterpret_cast<uint16_t*>(Ks + (n - 1) * rowd);
    uint16_t* vl = reinterpret_cast<uint16_t*>(Vs + (n - 1) * rowd);
    for (int i = tid; i < half; i += nth) {
      const float k0 = ld_coh(kh + i), k1 = ld_coh(kh + i + half);
      const float c = rope[2 * i], sn = rope[2 * i + 1];
      const uint16_t a = f2bf(k0 * c - k1 * sn), bb = f2bf(k0 * sn + k1 * c);
      const uint16_t v0 = f2bf(ld_coh(vh + i)), v1 = f2bf(ld_coh(vh + i + half));
      kc[(int64_t)p * d + i] = a;
      kc[(int64_t)p * d + i + half] = bb;
      vc[(int64_t)p * d + i] = v0;
      vc[(int64_t)p * d + i + half] = v1;
      kl[i] = a;
      kl[i + half] = bb;
      vl[i] = v0;
      vl[i + half] = v1;
    }
  }
  __syncthreads();

  // scores s_t = (q . K_t) * scale, channels summed in ascending order
  for (int idx = tid; idx < group * n; idx += nth) {
    const int g = idx / n, t = idx - g * n;
    const float* q = qs + g * d;
    const uint32_t* kr = Ks + t * rowd;
    float acc = 0.f;
    for (int j = 0; j < half; ++j) {
      const uint32_t w = kr[j];
      acc = fmaf(q[2 * j], bf16lo(w), acc);
      acc = fmaf(q[2 * j + 1], bf16hi(w), acc);
    }
    Sc[g * T + t] = acc * D.attn_scale;
  }
  __syncthreads();
  // split-local softmax statistics
  for (int g = wave; g < group; g += nwaves()) {
    float m = -INFINITY;
    for (int t = lane; t < n; t += kWave) m = fmaxf(m, Sc[g * T + t]);
    m = wave_max(m);
    float sum = 0.f;
    for (int t = lane; t < n; t += kWave) {
      const float e = expf(Sc[g * T + t] - m);
      Sc[g * T + t] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      ml[2 * g] = m;
      ml[2 * g + 1] = sum;
    }
  }
  __syncthreads();
  // unnormalised output of this split
  float* out = P.K.ao + (int64_t)b * D.qd;
  for (int idx = tid; idx < group * d; idx += nth) {
    const int g = idx / d, i = idx - g * d;
    const float* e = Sc + g * T;
    const int hi = i & 1;
    const uint32_t* vcol = Vs + (i >> 1);
    float acc = 0.f;
    for (int t = 0; t < n; ++t) {
      const uint32_t w = vcol[t * rowd];
      acc = fmaf(e[t], hi ? bf16hi(w) : bf16lo(w), acc);
    }
    const int hq = kvh * group + g;
    if (nsplit == 1) {
      st_coh(out + hq * d + i, acc / ml[2 * g + 1]);
    } else {
      float* pp = P.K.part + (((int64_t)b * D.nq + hq) * D.max_splits + s) * (d + 2);
      st_coh(pp + 2 + i, acc);
      if (i == 0) {
        st_coh(pp, ml[2 * g]);
        st_coh(pp + 1, ml[2 * g + 1]);
      }
    }
  }
  if (nsplit > 1) {
    // last-arriving split combines all splits in fixed order
    wave_drain();
    __syncthreads();
    if (tid == 0) {
      uint32_t* ctr = split_ctr(P, l, b, kvh);
      const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = (old == (uint32_t)(nsplit - 1));
      if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sc.flag[0] = last;
    }
    __syncthreads();
    if (!sc.flag[0]) return;
    for (int idx = tid; idx < group * d; idx += nth) {
      const int g = idx / d, i = idx - g * d;
      const int hq = kvh * group + g;
      const float* pp = P.K.part + ((int64_t)b * D.nq + hq) * D.max_splits * (d + 2);
      float M = -INFINITY;
      for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, ld_coh(pp + sp * (d + 2)));
      float Ls = 0.f, O = 0.f;
      for (int sp = 0; sp < nsplit; ++sp) {
        const float* q = pp + sp * (d + 2);
        const float f = expf(ld_coh(q) - M);
        Ls = fmaf(ld_coh(q + 1), f, Ls);
        O = fmaf(ld_coh(q + 2 + i), f, O);
      }
      st_coh(out + hq * d + i, O / Ls);
    }
  }
  signal_if(P, stage_ctr(P, l, kCAttn), b * D.nkv + kvh);
}

__device__ void stage_attn(const Params& P, int l, int wg, int nwg, char* smem) {
  const Dims& D = P.D;
  if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, l, kCQkv), P.S.t_qkv + P.S.inject, kSAttn);
  const int T = D.split_len, B = P.S.B;
  int total = 0;
  for (int b = 0; b < B; ++b) total += D.nkv * ((clamp_pos(P, b) + T) / T);
  for (int it = wg; it < total; it += nwg) {
    int b = 0, base = 0, ns = 0, p = 0;
    for (;; ++b) {
      p = clamp_pos(P, b);
      ns = (p + T) / T;
      if (it < base + D.nkv * ns) break;
      base += D.nkv * ns;
    }
    const int kvh = (it - base) / ns, s = (it - base) - kvh * ns;
    attn_item(P, l, b, kvh, s, ns, p, smem);
    __syncthreads();  // shared memory is reused by the next item
  }
}

// ----------------------------------------------------------- O-proj

template <int NB>
__device__ void stage_o(const Params& P, int l, int wg, int nwg, char* smem) {
  constexpr int NR = kNrO, UC = kUcO;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int rows_total = D.H, K = D.qd, B = P.S.B;
  const uint16_t* Wm = layer_w(P, l, P.W.o_wo);
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  auto wait = [&]() {
    if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, l, kCAttn), P.S.t_attn, kSO);
  };
  const XSrc src{P.K.ao, K, nullptr, nullptr, 0};
  // residual input: the layer input (the embedding row for layer 0)
  const float* xa = P.K.xa;
  const uint16_t* emb = P.W.embed;
  const int* tok = P.S.tokens;
  float* xb = P.K.xb;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch&) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NR + r;
        if (b < nb && row < rows_total && lane == ((r * NB + b) & (kWave - 1))) {
          const int bb = b0 + b;
          float res;
          if (l == 0) {
            int tk = tok[bb];
            tk = ((unsigned)tk < (unsigned)D.V) ? tk : 0;
            res = bf16f(emb[(int64_t)tk * D.H + row]);
          } else {
            res = ld_coh(xa + (int64_t)bb * D.H + row);
          }
          st_coh(xb + (int64_t)bb * D.H + row, res + acc[r][b]);
        }
      }
  };
  gemv_stage<NR, UC, NB>(rowfn, (rows_total + NR - 1) / NR, K, src, nullptr, false, D.eps, B,
                         batch_tile(P, K, NB), wait, epi, wg, nwg, smem);
  signal_if(P, stage_ctr(P, l, kCO), wg);
}

// -------------------------------------------------------- fused SwiGLU

// A task holds kPairsGu (gate, up) row pairs.  Column-major tiling (weight
// reuse, the default): the whole batch tile is multiplied with each weight
// tile while it is in registers.  Row-major tiling (activation reuse): the
// batch is cut into tiles of at most two rows, each kept in LDS while every
// weight tile streams past it.  At batch <= 2 both tilings issue the same
// loads.
template <int NB>
__device__ void stage_gu(const Params& P, int l, int wg, int nwg, char* smem) {
  constexpr int NP = kPairsGu, NR = 2 * kPairsGu, UC = kUcGu;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int I = D.I, K = D.H, B = P.S.B;
  const uint16_t* Wg = layer_w(P, l, P.W.o_wg);
  const uint16_t* Wu = layer_w(P, l, P.W.o_wu);
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int row = t * NP + r;
      rows[r] = row < I ? Wg + (int64_t)row * K : nullptr;
      rows[NP + r] = row < I ? Wu + (int64_t)row * K : nullptr;
    }
  };
  auto wait = [&]() {
    if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, l, kCO), P.S.t_o, kSGu);
  };
  const XSrc src{P.K.xb, K, nullptr, nullptr, 0};
  float* h = P.K.hbuf;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch& sc) {
#pragma unroll
    for (int r = 0; r < NP; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NP + r;
        if (b < nb && row < I && lane == ((r * NB + b) & (kWave - 1))) {
          const float a = acc[r][b] * sc.rs[b], u = acc[NP + r][b] * sc.rs[b];
          st_coh(h + (int64_t)(b0 + b) * I + row, a / (1.0f + expf(-a)) * u);
        }
      }
  };
  const int bw = (P.S.gu_variant == kGuRow) ? min(2, batch_tile(P, K, NB)) : batch_tile(P, K, NB);
  gemv_stage<NR, UC, NB>(rowfn, (I + NP - 1) / NP, K, src, layer_w(P, l, P.W.o_mlp_norm), true,
                         D.eps, B, bw, wait, epi, wg, nwg, smem);
  signal_if(P, stage_ctr(P, l, kCGu), wg);
}

// ---------------------------------------------------------- Down-proj

template <int NB>
__device__ void stage_d(const Params& P, int l, int wg, int nwg, char* smem) {
  constexpr int NR = kNrD, UC = kUcD;
  const Dims& D = P.D;
  const int lane = lane_id();
  const int rows_total = D.H, K = D.I, B = P.S.B;
  const uint16_t* Wm = layer_w(P, l, P.W.o_wd);
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  auto wait = [&]() {
    if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, l, kCGu), P.S.t_gu, kSD);
  };
  const XSrc src{P.K.hbuf, K, nullptr, nullptr, 0};
  const float* xb = P.K.xb;
  float* xa = P.K.xa;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch&) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = t * NR + r;
        if (b < nb && row < rows_total && lane == ((r * NB + b) & (kWave - 1))) {
          const int64_t o = (int64_t)(b0 + b) * D.H + row;
          st_coh(xa + o, ld_coh(xb + o) + acc[r][b]);
        }
      }
  };
  gemv_stage<NR, UC, NB>(rowfn, (rows_total + NR - 1) / NR, K, src, nullptr, false, D.eps, B,
                         batch_tile(P, K, NB), wait, epi, wg, nwg, smem);
  signal_if(P, stage_ctr(P, l, kCD), wg);
}

// ------------------------------------------------- LM head + argmax

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int NB>
__device__ void stage_lm(const Params& P, int wg, int nwg, char* smem) {
  constexpr int NR = kNrLm, UC = kUcLm;
  const Dims& D = P.D;
  Scratch& sc = *reinterpret_cast<Scratch*>(smem);
  const int lane = lane_id(), wave = wave_id();
  const int rows_total = D.V, K = D.H, B = P.S.B;
  const uint16_t* Wm = P.W.lm;
  auto rowfn = [&](int t, const uint16_t* (&rows)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = t * NR + r;
      rows[r] = row < rows_total ? Wm + (int64_t)row * K : nullptr;
    }
  };
  auto wait = [&]() {
    if (!P.S.wait) wg_wait(sync_of(P), stage_ctr(P, D.L - 1, kCD), P.S.t_d, kSLm);
  };
  for (int b = lane; b < 64; b += kWave) {
    sc.bestv[wave][b] = -INFINITY;
    sc.besti[wave][b] = 0x7FFFFFFF;
  }
  const XSrc src{P.K.xa, K, nullptr, nullptr, 0};
  float* logits = P.S.logits;
  auto epi = [&](int t, int b0, int nb, float (&acc)[NR][NB], Scratch& s) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        float bv = s.bestv[wave][b0 + b];
        int bi = s.besti[wave][b0 + b];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int row = t * NR + r;
          if (row < rows_total) {
            const float v = acc[r][b] * s.rs[b];
            if (lane == ((r * NB + b) & (kWave - 1))) logits[(int64_t)(b0 + b) * D.V + row] = v;
            if (better(v, row, bv, bi)) {
              bv = v;
              bi = row;
            }
          }
        }
        if (lane == 0) {
          s.bestv[wave][b0 + b] = bv;
          s.besti[wave][b0 + b] = bi;
        }
      }
    }
  };
  gemv_stage<NR, UC, NB>(rowfn, (rows_total + NR - 1) / NR, K, src, P.W.final_norm, true, D.eps,
                         B, batch_tile(P, K, NB), wait, epi, wg, nwg, smem);
  __syncthreads();
  // this workgroup's best per sequence -> partials
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    float bv = sc.bestv[0][b];
    int bi = sc.besti[0][b];
    for (int w = 1; w < nwaves(); ++w)
      if (better(sc.bestv[w][b], sc.besti[w][b], bv, bi)) {
        bv = sc.bestv[w][b];
        bi = sc.besti[w][b];
      }
    st_coh(P.K.lm_val + (int64_t)wg * D.max_batch + b, bv);
    st_coh_i(P.K.lm_idx + (int64_t)wg * D.max_batch + b, bi);
  }
  wave_drain();
  __syncthreads();
  if (threadIdx.x == 0) sc.flag[1] = last_arriver(P.K.lm_ctr, wg, nwg);
  __syncthreads();
  if (!sc.flag[1] || P.S.next == nullptr) return;
  // last arriver: reduce the partials of every workgroup, per sequence
  for (int b = 0; b < B; ++b) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int w = threadIdx.x; w < nwg; w += blockDim.x) {
      const float v = ld_coh(P.K.lm_val + (int64_t)w * D.max_batch + b);
      const int i = ld_coh_i(P.K.lm_idx + (int64_t)w * D.max_batch + b);
      if (better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sc.bestv[wave][0] = bv;
      sc.besti[wave][0] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < nwaves(); ++w)
        if (better(sc.bestv[w][0], sc.besti[w][0], bv, bi)) {
          bv = sc.bestv[w][0];
          bi = sc.besti[w][0];
        }
      P.S.next[b] = (bi == 0x7FFFFFFF) ? 0 : bi;
    }
    __syncthreads();
  }
}

}  // namespace ld
