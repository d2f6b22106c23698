// ld_api.cpp - host runtime behind the C ABI of include/ld.h: arena
// layout, argument validation, cumulative readiness-counter targets, the
// three launch schedules (whole-kernel wait, tile flags on two streams, one
// persistent kernel) and the offline SwiGLU tiling choice.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/ld.h"
#include "../../include/ld_ops.h"
#include "../../synth/ld_synth.h"
#include "ld_launch.h"
#include "ld_params.hpp"

using namespace ld;

constexpr int kModes = 4;  // LD_MODE_WAIT .. LD_MODE_GRAPH
// Automatic readiness granularity: row-count counters in the tile-flag mode
// below this many rows (measured, Llama-1B shape: batch 1 0.891 -> 0.872 ms,
// 4: 1.353 -> 1.326, 16: 1.900 -> 1.888; batch 64 5.578 -> 5.626 and the
// persistent kernel 0.7-1.1% slower at every batch).
constexpr int kTileSyncMaxRows = 64;

struct ld_model {
  ld_config cfg{};
  Dims D{};
  Weights W{};
  Work K{};
  void* warena = nullptr;
  bool own_w = false;
  size_t wbytes = 0;
  void* karena = nullptr;
  bool own_k = false;
  size_t kbytes = 0;
  bool kv_ready = false;
  int last_rows = 0;  // rows of the last enqueued step
  ld_mode mode = LD_MODE_MEGA;
  int device = 0;
  int n_cu = 0;
  hipStream_t s1 = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // graph mode: captured whole-kernel-wait steps, keyed by their arguments
  struct StepGraph {
    int B, M, variant;
    const void *tokens, *pos;
    void *logits, *next;
    hipGraph_t graph;
    hipGraphExec_t exec;
  };
  std::vector<StepGraph> graphs;
  hipStream_t s_cap = nullptr;  // capture stream (the caller's may be the legacy default)
  // cumulative counter totals (what every layer's counter will read once all
  // enqueued steps have finished)
  uint32_t tot_qkv = 0, tot_attn = 0, tot_o = 0, tot_gu = 0, tot_d = 0;
  // readiness granularity of the tile-flag and persistent modes, and the
  // signalling steps enqueued with row-count counters so far
  int sync = LD_SYNC_AUTO;
  uint32_t n_tile = 0;
  // SwiGLU tiling per (mode, batch size), and whether ld_tune or a loaded
  // table chose it; tile_ms[mode][b] = {column-major, row-major} median ms
  // per step measured by ld_tune
  int gu_variant[kModes][65];
  bool gu_tuned[kModes][65];
  float tile_ms[kModes][65][2];
  int mlp_variant = LD_MLP_FUSED;  // unfused-MLP ablation (whole-kernel-wait mode)
  // launch geometry per mode: grid, threads per workgroup, LDS bytes, LDS for staged inputs
  int grid_wait = 0, grid_flags = 0, grid_mega[65] = {0};  // grid_mega indexed by nb
  int thr_wait = 512, thr_flags = 512, thr_mega = 512;
  size_t smem_wait = 0, smem_flags = 0, smem_mega = 0;
  uint32_t xcap_wait = 0, xcap_flags = 0, xcap_mega = 0;
  bool flags_ok = true;
  // attention split capacity of the whole-kernel-wait, graph and persistent
  // modes (a full CU's LDS), used from 16 rows; the tile-flag mode and every
  // step below 16 rows use D.split_len (half a CU's LDS)
  int split_len_full = 0;
  // device address of the allocation-free KV fill's length array on this
  // model's device (set up at init), and its capacity
  int32_t* scratch_lens = nullptr;
  int scratch_cap = 0;
  uint64_t watchdog_ticks = 0;
  double wall_khz = 100000.0;
  uint32_t inject_next = 0;
  uint32_t* tune_ctr = nullptr;  // counter slots for standalone tuning launches
  size_t ctr_bytes = 0;          // bytes of all counters (stage, LM, split)
  // debug mechanisms (ld_set_debug): flags, and the work-arena byte ranges
  // a poisoned step fills with NaN (set by ld_alloc_kv)
  int debug = 0;
  std::vector<std::pair<size_t, size_t>> poison;
  std::string err;
};

static std::string g_err;

static ld_status fail(ld_model* m, ld_status st, const std::string& msg) {
  if (m)
    m->err = msg;
  else
    g_err = msg;
  return st;
}

#define HIPCHK(m, call)                                                                   \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail((m), LD_EHIP, std::string(#call) + ": " + hipGetErrorString(e_));       \
  } while (0)

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool cfg_ok(const ld_config* c, std::string* why) {
  if (!c) {
    *why = "null config";
    return false;
  }
  if (c->n_layers < 1 || c->hidden < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 2 || c->intermediate < 8 || c->vocab < 1) {
    *why = "non-positive dimension";
    return false;
  }
  if (c->hidden % 8 || c->intermediate % 8 || (c->n_q_heads * c->head_dim) % 8) {
    *why = "hidden, intermediate and n_q_heads*head_dim must be multiples of 8";
    return false;
  }
  if (c->head_dim < 8 || c->head_dim > 256 || (c->head_dim & (c->head_dim - 1))) {
    *why = "head_dim must be a power of two in [8, 256]";
    return false;
  }
  if (c->n_q_heads % c->n_kv_heads || c->n_q_heads / c->n_kv_heads > 8) {
    *why = "n_q_heads must be a multiple of n_kv_heads, with at most 8 query heads per group";
    return false;
  }
  {
    // every weight matrix, and each layer's block, is read through one buffer
    // resource with 32-bit offsets
    const size_t H = c->hidden, I = c->intermediate;
    const size_t qd = (size_t)c->n_q_heads * c->head_dim, kvd = (size_t)c->n_kv_heads * c->head_dim;
    const size_t layer = 2 * (2 * H + (qd + 2 * kvd) * H + H * qd + 3 * I * H) + 7 * 256;
    if (layer > kMaxWeightBuffer || (size_t)c->vocab * H * 2 > kMaxWeightBuffer) {
      *why = "a layer's weights and the LM head must each be below 4 GB";
      return false;
    }
  }
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) {
    *why = "bad rms_eps or rope_theta";
    return false;
  }
  return true;
}

// Weight arena layout (element offsets), every tensor 256-byte aligned.
struct WLayout {
  size_t embed, final_norm, lm, layer0, layer_stride;
  size_t attn_norm, wqkv, wo, mlp_norm, wg, wu, wd;  // within a layer block
  size_t total_bytes;
};

static WLayout wlayout(const ld_config* c) {
  WLayout L{};
  const size_t H = c->hidden, V = c->vocab, I = c->intermediate;
  const size_t qd = (size_t)c->n_q_heads * c->head_dim, kvd = (size_t)c->n_kv_heads * c->head_dim;
  size_t off = 0;  // bytes
  auto take = [&](size_t elems) {
    const size_t at = off;
    off = align256(off + elems * 2);
    return at / 2;
  };
  L.embed = take(V * H);
  L.final_norm = take(H);
  L.lm = c->tied ? L.embed : take(V * H);
  // layer block
  size_t lb = 0;
  auto ltake = [&](size_t elems) {
    const size_t at = lb;
    lb = align256(lb + elems * 2);
    return at / 2;
  };
  L.attn_norm = ltake(H);
  L.wqkv = ltake((qd + 2 * kvd) * H);
  L.wo = ltake(H * qd);
  L.mlp_norm = ltake(H);
  L.wg = ltake(I * H);
  L.wu = ltake(I * H);
  L.wd = ltake(H * I);
  L.layer0 = off / 2;
  L.layer_stride = lb / 2;
  L.total_bytes = off + lb * (size_t)c->n_layers;
  return L;
}

extern "C" size_t ld_weights_bytes(const ld_config* cfg) {
  std::string why;
  if (!cfg_ok(cfg, &why)) return 0;
  return wlayout(cfg).total_bytes;
}

// KV + workspace arena layout (byte offsets).
struct KLayout {
  size_t kc, vc, xa, xb, qkv, ao, part, hbuf, gbuf, ubuf, lm_val, lm_idx, rope, ctr, lm_ctr,
      split_ctr, mctr, aph, qg_ctr, hc_ctr, mpart, xa_f, xb_f, ao_f, h_f, ss_a, ss_b, err, tune_ctr, total;
  int split_len, max_splits, max_wg;
};

// LDS bytes available per CU.
static const size_t kLdsPerCu = 160 * 1024;

// Attention positions per work item: the largest multiple of 32 up to 512
// (one position per thread of the 512-thread tile-flag workgroups) whose
// tiles fit half a CU's LDS, so two tile-flag kernels still share a CU.
// Attention split lengths.  The longest split (Tmax) sizes the LDS tiles: a
// multiple of 32 up to 512 whose K and V tiles fit next to the other
// attention buffers in half a CU's LDS (two tile-flag kernels share a CU).
// A step uses T = step_split_len(Tmax, batch): short splits at small batch
// spread one sequence's attention over many workgroups, long ones at large
// batch keep the number of items (and of partial results) down.
constexpr int kMinSplit = 64;

static int step_split_len(int Tmax, int batch) {
  int T = kMinSplit;
  while (T < 32 * batch && T < Tmax) T *= 2;
  return std::min(T, Tmax);
}

static int max_splits_for(int Tmax, int max_seq) {
  const int Tmin = std::min(kMinSplit, Tmax);
  return (max_seq + Tmin - 1) / Tmin;
}

static int split_len_for(const ld_config* c, int max_seq) {
  const int group = c->n_q_heads / c->n_kv_heads;
  int T = 512;
  while (T > 32) {
    if (scratch_bytes() + attn_smem(group, c->head_dim, T, max_splits_for(T, max_seq)) <=
        kLdsPerCu / 2)
      break;
    T -= 32;
  }
  return T;
}

static KLayout klayout(const ld_config* c, int maxB, int max_seq) {
  KLayout K{};
  const size_t H = c->hidden, I = c->intermediate, d = c->head_dim;
  const size_t qd = (size_t)c->n_q_heads * d, kvd = (size_t)c->n_kv_heads * d;
  K.split_len = split_len_for(c, max_seq);
  K.max_splits = max_splits_for(K.split_len, max_seq);
  K.max_wg = 8192;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  const size_t cache = (size_t)c->n_layers * maxB * c->n_kv_heads * (size_t)max_seq * d * 2;
  K.kc = take(cache);
  K.vc = take(cache);
  K.xa = take((size_t)maxB * H * 4);
  K.xb = take((size_t)maxB * H * 4);
  K.qkv = take((size_t)maxB * (qd + 2 * kvd) * 4);
  K.ao = take((size_t)maxB * qd * 4);
  K.part = take((size_t)maxB * c->n_q_heads * K.max_splits * (d + 2) * 4);
  K.hbuf = take((size_t)maxB * I * 4);
  K.mpart = take((size_t)kMaxKSplit * maxB * H * 4);
  {
    const size_t Bp = ((size_t)maxB + 15) / 16 * 16, Ht = (H + 15) / 16;
    const size_t Hp = round32((int)H), qdp = round32((int)qd), Ip = round32((int)I);
    K.xa_f = take(Bp * Hp * 4);
    K.xb_f = take(Bp * Hp * 4);
    K.ao_f = take(Bp * qdp * 4);
    K.h_f = take(Bp * Ip * 4);
    K.ss_a = take((size_t)maxB * Ht * 4);
    K.ss_b = take((size_t)maxB * Ht * 4);
  }
  K.gbuf = take((size_t)maxB * I * 4);
  K.ubuf = take((size_t)maxB * I * 4);
  K.lm_val = take((size_t)K.max_wg * maxB * 4);
  K.lm_idx = take((size_t)K.max_wg * maxB * 4);
  K.rope = take((size_t)max_seq * (d / 2) * 2 * 4);
  // counters: contiguous so they can be cleared together
  K.ctr = take((size_t)c->n_layers * kStageCtrs * kCtrWords * 4);
  K.lm_ctr = take((size_t)kCtrWords * 4);
  K.split_ctr = take((size_t)c->n_layers * maxB * c->n_kv_heads * 16 * 4);
  K.mctr = take((size_t)2 * kMctrPasses * ((H + 15) / 16) * 4);
  K.aph = take((size_t)c->n_layers * 2 * kCtrWords * 4);
  K.qg_ctr = take((size_t)c->n_layers * c->n_kv_heads * kCtrWords * 4);
  K.hc_ctr = take((size_t)c->n_layers * ((I + kHChunk - 1) / kHChunk) * kCtrWords * 4);
  K.err = take(256);
  // private counters of standalone tuning launches (one layer's worth)
  K.tune_ctr = take(((size_t)kStageCtrs * kCtrWords + kCtrWords + (size_t)maxB * c->n_kv_heads * 16) * 4);
  K.total = off;
  return K;
}

extern "C" size_t ld_kv_bytes(const ld_config* cfg, int32_t max_batch, int32_t max_seq) {
  std::string why;
  if (!cfg_ok(cfg, &why) || max_batch < 1 || max_batch > 64 || max_seq < 1) return 0;
  return klayout(cfg, max_batch, max_seq).total;
}

static ld_status setup_launch(ld_model* m) {
  HIPCHK(m, hipGetDevice(&m->device));
  HIPCHK(m, hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, m->device));
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, m->device) == hipSuccess &&
      khz > 0)
    m->wall_khz = (double)khz;
  m->watchdog_ticks = (uint64_t)(m->wall_khz * 1000.0 * 2.0);  // 2 s
  // harness overrides from the environment: the starting mode, the watchdog
  if (const char* e = std::getenv("LD_MODE")) {
    const std::string v(e);
    if (v == "wait") m->mode = LD_MODE_WAIT;
    else if (v == "flags") m->mode = LD_MODE_FLAGS;
    else if (v == "mega") m->mode = LD_MODE_MEGA;
    else if (v == "graph") m->mode = LD_MODE_GRAPH;
    else return fail(m, LD_EINVAL, "LD_MODE must be wait, flags, mega or graph");
  }
  if (const char* e = std::getenv("LD_WATCHDOG_US")) {
    char* end = nullptr;
    const double us = std::strtod(e, &end);
    if (end == e || *end != '\0' || !(us > 0.0) || us > 3.6e9)
      return fail(m, LD_EINVAL, "LD_WATCHDOG_US must be a number of microseconds in (0, 3.6e9]");
    m->watchdog_ticks = (uint64_t)(m->wall_khz * 1e-3 * us);
  }
  HIPCHK(m, scratch_lens_ptr(&m->scratch_lens, &m->scratch_cap));
  HIPCHK(m, hipStreamCreateWithFlags(&m->s1, hipStreamNonBlocking));
  HIPCHK(m, hipStreamCreateWithFlags(&m->s_cap, hipStreamNonBlocking));
  HIPCHK(m, hipEventCreateWithFlags(&m->ev_fork, hipEventDisableTiming));
  HIPCHK(m, hipEventCreateWithFlags(&m->ev_join, hipEventDisableTiming));
  for (int md = 0; md < kModes; ++md)
    for (int b = 0; b <= 64; ++b) {
      m->gu_variant[md][b] = kGuCol;
      m->gu_tuned[md][b] = false;
      m->tile_ms[md][b][0] = m->tile_ms[md][b][1] = 0.f;
    }
  return LD_OK;
}

extern "C" ld_status ld_init_weights(ld_model** out, const ld_config* cfg, void* dev_buf,
                                     size_t bytes, uint64_t seed, float w_std, void* stream) {
  std::string why;
  if (!out) return fail(nullptr, LD_EINVAL, "null output pointer");
  *out = nullptr;
  if (!cfg_ok(cfg, &why)) return fail(nullptr, LD_EINVAL, "bad config: " + why);
  if (!(w_std >= 0.f)) return fail(nullptr, LD_EINVAL, "bad w_std");
  const WLayout L = wlayout(cfg);
  if (dev_buf && bytes < L.total_bytes) return fail(nullptr, LD_ENOMEM, "weight buffer too small");
  if (dev_buf && ((uintptr_t)dev_buf & 255)) return fail(nullptr, LD_EINVAL, "weight buffer not 256-byte aligned");
  ld_model* m = new ld_model();
  m->cfg = *cfg;
  ld_status st = setup_launch(m);
  if (st != LD_OK) {
    g_err = m->err;
    ld_free(m);
    return st;
  }
  if (dev_buf) {
    m->warena = dev_buf;
  } else {
    if (hipMalloc(&m->warena, L.total_bytes) != hipSuccess) {
      g_err = "hipMalloc of the weight arena failed";
      ld_free(m);
      return LD_ENOMEM;
    }
    m->own_w = true;
  }
  m->wbytes = L.total_bytes;
  uint16_t* base = static_cast<uint16_t*>(m->warena);
  m->W.embed = base + L.embed;
  m->W.final_norm = base + L.final_norm;
  m->W.lm = base + L.lm;
  m->W.layer0 = base + L.layer0;
  m->W.layer_stride = (int64_t)L.layer_stride;
  m->W.o_attn_norm = (int64_t)L.attn_norm;
  m->W.o_wqkv = (int64_t)L.wqkv;
  m->W.o_wo = (int64_t)L.wo;
  m->W.o_mlp_norm = (int64_t)L.mlp_norm;
  m->W.o_wg = (int64_t)L.wg;
  m->W.o_wu = (int64_t)L.wu;
  m->W.o_wd = (int64_t)L.wd;

  Dims& D = m->D;
  D.L = cfg->n_layers;
  D.H = cfg->hidden;
  D.nq = cfg->n_q_heads;
  D.nkv = cfg->n_kv_heads;
  D.d = cfg->head_dim;
  D.I = cfg->intermediate;
  D.V = cfg->vocab;
  D.group = D.nq / D.nkv;
  D.qd = D.nq * D.d;
  D.kvd = D.nkv * D.d;
  D.qkv_rows = D.qd + 2 * D.kvd;
  D.tied = cfg->tied;
  D.Hp = round32(D.H);
  D.qdp = round32(D.qd);
  D.Ip = round32(D.I);
  D.Ht = (D.H + 15) / 16;
  D.nhc = (D.I + kHChunk - 1) / kHChunk;
  D.eps = cfg->rms_eps;
  D.attn_scale = 1.0f / sqrtf((float)D.d);

  // synthetic weights from the seeded generator (logical row-major index)
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float kappa = ls_kappa(w_std);
  const int64_t H = D.H, V = D.V, I = D.I, qd = D.qd, kvd = D.kvd;
  auto gen = [&](const uint16_t* dst, int64_t n, uint64_t tensor) {
    return launch_gen_normal(const_cast<uint16_t*>(dst), n, ls_key(seed, tensor), 0, kappa, s);
  };
  auto ones = [&](const uint16_t* dst, int64_t n) {
    return launch_fill16(const_cast<uint16_t*>(dst), n, LS_BF16_ONE, s);
  };
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t x) {
    if (e == hipSuccess) e = x;
  };
  chk(gen(m->W.embed, V * H, LS_T_EMBED));
  chk(ones(m->W.final_norm, H));
  if (!cfg->tied) chk(gen(m->W.lm, V * H, LS_T_LM_HEAD));
  for (int l = 0; l < D.L; ++l) {
    const uint16_t* lb = m->W.layer0 + (int64_t)l * m->W.layer_stride;
    chk(ones(lb + L.attn_norm, H));
    chk(gen(lb + L.wqkv, qd * H, LS_T_LAYER(l, LS_K_WQ)));
    chk(gen(lb + L.wqkv + qd * H, kvd * H, LS_T_LAYER(l, LS_K_WK)));
    chk(gen(lb + L.wqkv + (qd + kvd) * H, kvd * H, LS_T_LAYER(l, LS_K_WV)));
    chk(gen(lb + L.wo, H * qd, LS_T_LAYER(l, LS_K_WO)));
    chk(ones(lb + L.mlp_norm, H));
    chk(gen(lb + L.wg, I * H, LS_T_LAYER(l, LS_K_WG)));
    chk(gen(lb + L.wu, I * H, LS_T_LAYER(l, LS_K_WU)));
    chk(gen(lb + L.wd, H * I, LS_T_LAYER(l, LS_K_WD)));
  }
  if (e != hipSuccess) {
    g_err = std::string("weight generation launch failed: ") + hipGetErrorString(e);
    ld_free(m);
    return LD_EHIP;
  }
  *out = m;
  return LD_OK;
}

static ld_status compute_grids(ld_model* m) {
  const Dims& D = m->D;
  const int maxnb = nb_for_batch(D.max_batch);
  const size_t scratch = scratch_bytes(), best = best_bytes();
  // whole-kernel wait and persistent modes: one 512-thread workgroup per CU,
  // whose staging area holds one whole input row of every stage
  const size_t kmax = (size_t)std::max(std::max(D.H, D.I), D.qd) * 4;  // longest staged input row
  const uint32_t xcap_full = (uint32_t)((kLdsPerCu - scratch - best) / 256 * 256);
  if (kmax > xcap_full) return fail(m, LD_EINVAL, "input rows longer than the LDS staging area");
  m->xcap_wait = m->xcap_mega = xcap_full;
  const size_t attn_full = attn_smem(D.group, D.d, m->split_len_full, D.max_splits);
  m->smem_wait = m->smem_mega = scratch + std::max<size_t>(xcap_full + best, attn_full);
  if (m->smem_mega > kLdsPerCu) return fail(m, LD_EINVAL, "stage tiles do not fit in LDS");
  // tile-flag mode: two consecutive stage kernels share each CU, so each
  // 512-thread workgroup gets at most half the LDS
  const size_t half = kLdsPerCu / 2;
  m->xcap_flags = (uint32_t)(half - scratch - best);
  const size_t attn_half = attn_smem(D.group, D.d, D.split_len, D.max_splits);
  m->smem_flags = scratch + std::max<size_t>(m->xcap_flags + best, attn_half);
  // (the stages with a deferred norm stage whole hidden-size rows there; O
  // and Down may take theirs in column chunks of two blocks)
  const size_t kmax_flags = std::max((size_t)D.H * 4, (size_t)2 * kKChunkMinBytes);
  m->flags_ok = (kmax_flags <= m->xcap_flags) && (m->smem_flags <= half);
  for (int nb = 1; nb <= maxnb; nb *= 2) {
    for (int st = 0; st <= kSLm; ++st) {
      const size_t sm = (st == 0) ? m->smem_mega : std::max(m->smem_wait, m->smem_flags);
      HIPCHK(m, set_max_dynamic_smem(st, nb, sm));
      if (st > 0 && nb == 64) HIPCHK(m, set_max_dynamic_smem(st, nb, m->smem_wait, true));
    }
    HIPCHK(m, set_max_dynamic_smem(kSMlpProj, nb, m->smem_wait));
    if (nb == 64) HIPCHK(m, set_max_dynamic_smem(kSMlpProj, nb, m->smem_wait, true));
    int occ = 0;
    HIPCHK(m, occupancy(0, nb, m->thr_mega, m->smem_mega, &occ));
    if (occ < 1) return fail(m, LD_EINVAL, "persistent kernel does not fit on a CU");
    m->grid_mega[nb] = std::min(occ * m->n_cu, m->K.max_wg);
    for (int st = kSQkv; st <= kSLm; ++st) {
      int o1 = 0, o2 = 0;
      HIPCHK(m, occupancy(st, nb, m->thr_wait, m->smem_wait, &o1, nb == 64));
      HIPCHK(m, occupancy(st, nb, m->thr_flags, m->smem_flags, &o2));
      if (o1 < 1) return fail(m, LD_EINVAL, "stage kernel does not fit on a CU");
      if (o2 < 2) m->flags_ok = false;  // two tile-flag kernels must fit side by side
    }
  }
  m->grid_wait = m->n_cu;
  m->grid_flags = m->n_cu;
  return LD_OK;
}

extern "C" ld_status ld_alloc_kv(ld_model* m, void* dev_buf, size_t bytes, int32_t max_batch,
                                 int32_t max_seq) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (m->kv_ready) return fail(m, LD_ESTATE, "KV arena already allocated");
  if (max_batch < 1 || max_batch > 64) return fail(m, LD_EINVAL, "max_batch must be in [1, 64]");
  if (max_seq < 1) return fail(m, LD_EINVAL, "max_seq must be >= 1");
  const KLayout KL = klayout(&m->cfg, max_batch, max_seq);
  if (dev_buf && bytes < KL.total) return fail(m, LD_ENOMEM, "KV buffer too small");
  if (dev_buf && ((uintptr_t)dev_buf & 255)) return fail(m, LD_EINVAL, "KV buffer not 256-byte aligned");
  HIPCHK(m, hipDeviceSynchronize());
  if (dev_buf) {
    m->karena = dev_buf;
  } else {
    if (hipMalloc(&m->karena, KL.total) != hipSuccess)
      return fail(m, LD_ENOMEM, "hipMalloc of the KV arena failed");
    m->own_k = true;
  }
  m->kbytes = KL.total;
  char* base = static_cast<char*>(m->karena);
  Work& K = m->K;
  K.kc = reinterpret_cast<uint16_t*>(base + KL.kc);
  K.vc = reinterpret_cast<uint16_t*>(base + KL.vc);
  K.xa = reinterpret_cast<float*>(base + KL.xa);
  K.xb = reinterpret_cast<float*>(base + KL.xb);
  K.qkv = reinterpret_cast<float*>(base + KL.qkv);
  K.ao = reinterpret_cast<float*>(base + KL.ao);
  K.part = reinterpret_cast<float*>(base + KL.part);
  K.hbuf = reinterpret_cast<float*>(base + KL.hbuf);
  K.gbuf = reinterpret_cast<float*>(base + KL.gbuf);
  K.ubuf = reinterpret_cast<float*>(base + KL.ubuf);
  K.lm_val = reinterpret_cast<float*>(base + KL.lm_val);
  K.lm_idx = reinterpret_cast<int*>(base + KL.lm_idx);
  K.rope = reinterpret_cast<const float*>(base + KL.rope);
  K.ctr = reinterpret_cast<uint32_t*>(base + KL.ctr);
  K.lm_ctr = reinterpret_cast<uint32_t*>(base + KL.lm_ctr);
  K.split_ctr = reinterpret_cast<uint32_t*>(base + KL.split_ctr);
  K.mctr = reinterpret_cast<uint32_t*>(base + KL.mctr);
  K.aph = reinterpret_cast<uint32_t*>(base + KL.aph);
  K.qg_ctr = reinterpret_cast<uint32_t*>(base + KL.qg_ctr);
  K.hc_ctr = reinterpret_cast<uint32_t*>(base + KL.hc_ctr);
  K.mpart = reinterpret_cast<float*>(base + KL.mpart);
  K.xa_f = reinterpret_cast<uint32_t*>(base + KL.xa_f);
  K.xb_f = reinterpret_cast<uint32_t*>(base + KL.xb_f);
  K.ao_f = reinterpret_cast<uint32_t*>(base + KL.ao_f);
  K.h_f = reinterpret_cast<uint32_t*>(base + KL.h_f);
  K.ss_a = reinterpret_cast<float*>(base + KL.ss_a);
  K.ss_b = reinterpret_cast<float*>(base + KL.ss_b);
  K.err = reinterpret_cast<int*>(base + KL.err);
  m->ctr_bytes = KL.err - KL.ctr;
  K.max_wg = KL.max_wg;
  m->tune_ctr = reinterpret_cast<uint32_t*>(base + KL.tune_ctr);
  m->D.max_batch = max_batch;
  m->D.max_seq = max_seq;
  m->D.split_len = KL.split_len;
  m->split_len_full = KL.split_len;
  while (m->split_len_full + 32 <= 512 &&
         scratch_bytes() + attn_smem(m->D.group, m->D.d, m->split_len_full + 32, KL.max_splits) <= kLdsPerCu)
    m->split_len_full += 32;
  m->D.max_splits = KL.max_splits;

  // poisoned steps: the activations, partial results and fragment buffers
  // (xa .. the RoPE table, contiguous), except a fragment buffer whose K is
  // not a multiple of 32: its padding columns must stay zero (the MFMA engine
  // multiplies them by masked, zero, weights)
  {
    m->poison.clear();
    const bool keep[4] = {m->D.H % 32 == 0, m->D.H % 32 == 0, m->D.qd % 32 == 0, m->D.I % 32 == 0};
    const size_t fb[5] = {KL.xa_f, KL.xb_f, KL.ao_f, KL.h_f, KL.ss_a};
    m->poison.push_back({KL.xa, KL.xa_f - KL.xa});
    for (int i = 0; i < 4; ++i)
      if (keep[i]) m->poison.push_back({fb[i], fb[i + 1] - fb[i]});
    m->poison.push_back({KL.ss_a, KL.rope - KL.ss_a});
  }
  // zero everything except the caches, then counters and error word
  HIPCHK(m, hipMemset(base + KL.xa, 0, KL.total - KL.xa));
  // RoPE table: angle p * theta^(-2i/d) in double, cos and sin rounded to fp32
  const int half = m->D.d / 2;
  std::vector<float> rope((size_t)max_seq * half * 2);
  for (int p = 0; p < max_seq; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)m->cfg.rope_theta, -2.0 * i / (double)m->D.d);
      const double a = (double)p * inv;
      rope[((size_t)p * half + i) * 2] = (float)std::cos(a);
      rope[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
    }
  HIPCHK(m, hipMemcpy(base + KL.rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));
  m->tot_qkv = m->tot_attn = m->tot_o = m->tot_gu = m->tot_d = 0;
  m->n_tile = 0;
  ld_status st = compute_grids(m);
  if (st != LD_OK) return st;
  m->K.watchdog = m->watchdog_ticks;
  m->kv_ready = true;
  return LD_OK;
}

extern "C" ld_status ld_fill_kv(ld_model* m, uint64_t seed, float kv_std,
                                const int32_t* prefill_len, void* stream) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  if (!prefill_len) return fail(m, LD_EINVAL, "null prefill_len");
  const int B = m->D.max_batch;
  for (int b = 0; b < B; ++b)
    if (prefill_len[b] < 0 || prefill_len[b] > m->D.max_seq)
      return fail(m, LD_EINVAL, "prefill length outside [0, max_seq]");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* len_dev = nullptr;
  HIPCHK(m, hipMalloc(&len_dev, B * sizeof(int)));
  hipError_t e = hipMemcpy(len_dev, prefill_len, B * sizeof(int), hipMemcpyHostToDevice);
  const float kappa = ls_kappa(kv_std);
  const int64_t per_layer = (int64_t)B * m->D.nkv * m->D.max_seq * m->D.d;
  for (int l = 0; l < m->D.L && e == hipSuccess; ++l)
    e = launch_gen_kv(m->K.kc + l * per_layer, m->K.vc + l * per_layer, len_dev, B, m->D.nkv,
                      m->D.max_seq, m->D.d, ls_key(seed, LS_T_KCACHE(l)),
                      ls_key(seed, LS_T_VCACHE(l)), kappa, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(len_dev);
  if (e != hipSuccess) return fail(m, LD_EHIP, std::string("KV fill failed: ") + hipGetErrorString(e));
  return LD_OK;
}

extern "C" ld_status ld_fill_kv_static(ld_model* m, uint64_t seed, float kv_std,
                                       const int32_t* prefill_len, void* stream) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  if (!prefill_len) return fail(m, LD_EINVAL, "null prefill_len");
  const int B = m->D.max_batch;
  if (B > m->scratch_cap)
    return fail(m, LD_EINVAL, "max_batch exceeds the static length array (" +
                                  std::to_string(m->scratch_cap) + " entries)");
  for (int b = 0; b < B; ++b)
    if (prefill_len[b] < 0 || prefill_len[b] > m->D.max_seq)
      return fail(m, LD_EINVAL, "prefill length outside [0, max_seq]");
  if (m->scratch_lens == nullptr) return fail(m, LD_EHIP, "static length array unavailable");
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIPCHK(m, launch_put_lens(m->scratch_lens, prefill_len, B, s));
  const float kappa = ls_kappa(kv_std);
  const int64_t per_layer = (int64_t)B * m->D.nkv * m->D.max_seq * m->D.d;
  for (int l = 0; l < m->D.L; ++l)
    HIPCHK(m, launch_gen_kv(m->K.kc + l * per_layer, m->K.vc + l * per_layer, m->scratch_lens, B,
                            m->D.nkv, m->D.max_seq, m->D.d, ls_key(seed, LS_T_KCACHE(l)),
                            ls_key(seed, LS_T_VCACHE(l)), kappa, s));
  return LD_OK;
}

extern "C" ld_status ld_set_mode(ld_model* m, ld_mode mode) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (mode != LD_MODE_WAIT && mode != LD_MODE_FLAGS && mode != LD_MODE_MEGA &&
      mode != LD_MODE_GRAPH)
    return fail(m, LD_EINVAL, "unknown mode");
  if (mode == LD_MODE_FLAGS && m->kv_ready && !m->flags_ok)
    return fail(m, LD_EINVAL, "tile-flag mode cannot keep two stage kernels of this shape on a CU");
  m->mode = mode;
  return LD_OK;
}

static Params make_params(ld_model* m) {
  Params P{};
  P.D = m->D;
  P.W = m->W;
  P.K = m->K;
  P.S.M = 1;
  return P;
}

// Captured steps bake in the weight and work arena addresses (fixed once the
// KV arena exists) and the SwiGLU tiling (part of the key); they are released
// with the model.
static void drop_graphs(ld_model* m) {
  for (auto& g : m->graphs) {
    (void)hipGraphExecDestroy(g.exec);
    (void)hipGraphDestroy(g.graph);
  }
  m->graphs.clear();
}
constexpr size_t kMaxGraphs = 8;  // captured argument sets kept per model

// The whole-kernel-wait step: one kernel per stage, in order, on one stream.
static hipError_t enqueue_wait_kernels(ld_model* m, const Params& P, hipStream_t s) {
  const int L = m->D.L;
  for (int l = 0; l < L; ++l) {
    for (int stage : {kSQkv, kSAttn, kSO, kSGu, kSD}) {
      const hipError_t e = launch_stage(stage, P, l, m->grid_wait, m->thr_wait, m->smem_wait, s);
      if (e != hipSuccess) return e;
    }
  }
  return launch_stage(kSLm, P, 0, m->grid_wait, m->thr_wait, m->smem_wait, s);
}

// Enqueue one step in the current mode.
// B rows: M consecutive tokens of each of B / M sequences.
static ld_status enqueue_step(ld_model* m, const int32_t* tokens, int32_t B, int32_t M,
                              const int32_t* pos, float* logits, int32_t* next, hipStream_t s0) {
  Params P = make_params(m);
  P.S.tokens = tokens;
  P.S.pos = pos;
  P.S.logits = logits;
  P.S.next = next;
  P.S.B = B;
  P.S.M = M;
  m->last_rows = B;
  if (m->debug & LD_DEBUG_POISON) {
    PoisonRanges r{};
    char* base = static_cast<char*>(m->karena);
    for (const auto& pr : m->poison) {
      r.p[r.count] = reinterpret_cast<uint32_t*>(base + pr.first);
      r.n[r.count++] = (int64_t)(pr.second / 4);
    }
    r.p[r.count] = reinterpret_cast<uint32_t*>(logits);
    r.n[r.count++] = (int64_t)B * m->D.V;
    if (next) {
      r.p[r.count] = reinterpret_cast<uint32_t*>(next);
      r.n[r.count++] = B;
    }
    HIPCHK(m, launch_poison(r, m->K.kc, m->K.vc, pos, B, M, m->D.L, m->D.max_batch, m->D.nkv,
                            m->D.max_seq, m->D.d, s0));
  }
  // split length: from 16 rows the modes with a full CU's LDS take longer
  // splits (fewer items and partial results); below 16 rows every mode uses
  // the same splits, so they add the same numbers in the same order.  The
  // long-context rule (on the device: far more items than workgroups) may
  // lengthen them up to the mode's whole tile area at any batch size.
  if (m->mode != LD_MODE_FLAGS) P.D.split_len = m->split_len_full;
  P.S.T = step_split_len(B >= kMfmaMinBatch ? P.D.split_len : m->D.split_len, B);
  P.S.Tmax = P.D.split_len;
  P.S.gu_variant = m->gu_variant[m->mode][B];
  P.S.inject = m->inject_next;
  m->inject_next = 0;
  const int L = m->D.L;
  const uint32_t attn_inc = (uint32_t)(B * m->D.nkv);
  // tile-granular readiness needs at most kMaxTileCtrs groups and chunks
  // (automatic: row-count counters in the tile-flag mode below 64 rows, where
  // they were measured faster, whole-stage counters otherwise)
  const bool want = m->sync == LD_SYNC_TILE ||
                    (m->sync == LD_SYNC_AUTO && m->mode == LD_MODE_FLAGS && B < kTileSyncMaxRows);
  const bool tile = want && m->D.nkv <= kMaxTileCtrs && m->D.nhc <= kMaxTileCtrs;
  auto add_targets = [&](int g) {
    // a step signals either the QKV and SwiGLU stage counters or their
    // row-count counters, and only the counters it signals advance
    if (tile) {
      m->n_tile += 1;
    } else {
      m->tot_qkv += g;
      m->tot_gu += g;
    }
    P.S.tile_sync = tile ? 1 : 0;
    P.S.n_sig = m->n_tile;
    m->tot_attn += attn_inc;
    m->tot_o += g;
    m->tot_d += g;
    P.S.t_qkv = m->tot_qkv;
    P.S.t_attn = m->tot_attn;
    P.S.t_o = m->tot_o;
    P.S.t_gu = m->tot_gu;
    P.S.t_d = m->tot_d;
  };
  if (m->mode == LD_MODE_MEGA) {
    const int g = m->grid_mega[nb_for_batch(B)];
    add_targets(g);
    P.S.wait = 0;
    P.S.x_cap = m->xcap_mega;
    HIPCHK(m, launch_mega(P, g, m->thr_mega, m->smem_mega, s0));
    return LD_OK;
  }
  if (m->mode == LD_MODE_GRAPH && P.S.inject == 0) {
    // the whole-kernel-wait step captured once per argument set (on the
    // library's own stream) and replayed on the caller's stream
    P.S.wait = 1;
    P.S.x_cap = m->xcap_wait;
    ld_model::StepGraph* hit = nullptr;
    for (auto& g : m->graphs)
      if (g.B == B && g.M == M && g.variant == P.S.gu_variant && g.tokens == tokens &&
          g.pos == pos && g.logits == logits && g.next == next)
        hit = &g;
    if (!hit) {
      if (m->graphs.size() >= kMaxGraphs) {
        (void)hipGraphExecDestroy(m->graphs.front().exec);
        (void)hipGraphDestroy(m->graphs.front().graph);
        m->graphs.erase(m->graphs.begin());
      }
      ld_model::StepGraph g{B, M, P.S.gu_variant, tokens, pos, logits, next, nullptr, nullptr};
      HIPCHK(m, hipStreamBeginCapture(m->s_cap, hipStreamCaptureModeThreadLocal));
      const hipError_t e = enqueue_wait_kernels(m, P, m->s_cap);
      const hipError_t e2 = hipStreamEndCapture(m->s_cap, &g.graph);
      HIPCHK(m, e);
      HIPCHK(m, e2);
      const hipError_t e3 = hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0);
      if (e3 != hipSuccess) {
        (void)hipGraphDestroy(g.graph);
        HIPCHK(m, e3);
      }
      m->graphs.push_back(g);
      hit = &m->graphs.back();
    }
    HIPCHK(m, hipGraphLaunch(hit->exec, s0));
    return LD_OK;
  }
  // whole-kernel wait (also graph mode with a watchdog test target pending)
  const bool flags = (m->mode == LD_MODE_FLAGS);
  if (flags && !m->flags_ok)
    return fail(m, LD_EINVAL, "tile-flag mode cannot keep two stage kernels of this shape on a CU");
  const int g = flags ? m->grid_flags : m->grid_wait;
  const int thr = flags ? m->thr_flags : m->thr_wait;
  const size_t smem = flags ? m->smem_flags : m->smem_wait;
  if (flags) add_targets(g);  // whole-kernel-wait kernels do not signal
  P.S.wait = flags ? 0 : 1;
  P.S.x_cap = flags ? m->xcap_flags : m->xcap_wait;
  hipStream_t ss[2] = {s0, m->s1};
  if (flags) {
    HIPCHK(m, hipEventRecord(m->ev_fork, s0));
    HIPCHK(m, hipStreamWaitEvent(m->s1, m->ev_fork, 0));
  }
  int k = 0;
  auto launch = [&](int stage, int l) -> hipError_t {
    hipStream_t s = flags ? ss[k & 1] : s0;
    ++k;
    return launch_stage(stage, P, l, g, thr, smem, s);
  };
  // the first MLP stage: fused, or an unfused form of the ablation
  const int mlp = flags ? LD_MLP_FUSED : m->mlp_variant;
  auto launch_mlp = [&](int l) -> hipError_t {
    if (mlp == LD_MLP_FUSED) return launch(kSGu, l);
    hipError_t e;
    if (mlp == LD_MLP_TWO_KERNELS) {
      if ((e = launch_mlp_proj(kMlpBoth, P, l, g, thr, smem, s0)) != hipSuccess) return e;
      return launch_mlp_elem(kMlpSiluMul, P, s0);
    }
    if ((e = launch_mlp_proj(kMlpGate, P, l, g, thr, smem, s0)) != hipSuccess) return e;
    if ((e = launch_mlp_proj(kMlpUp, P, l, g, thr, smem, s0)) != hipSuccess) return e;
    if ((e = launch_mlp_elem(kMlpSilu, P, s0)) != hipSuccess) return e;
    return launch_mlp_elem(kMlpMul, P, s0);
  };
  for (int l = 0; l < L; ++l) {
    HIPCHK(m, launch(kSQkv, l));
    HIPCHK(m, launch(kSAttn, l));
    HIPCHK(m, launch(kSO, l));
    HIPCHK(m, launch_mlp(l));
    HIPCHK(m, launch(kSD, l));
  }
  HIPCHK(m, launch(kSLm, 0));
  if (flags) {
    HIPCHK(m, hipEventRecord(m->ev_join, m->s1));
    HIPCHK(m, hipStreamWaitEvent(s0, m->ev_join, 0));
  }
  return LD_OK;
}

extern "C" ld_status ld_decode_step(ld_model* m, const int32_t* tokens, int32_t batch,
                                    const int32_t* positions, float* logits, int32_t* next_tokens,
                                    void* stream) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  if (batch < 1 || batch > m->D.max_batch) return fail(m, LD_EINVAL, "batch outside [1, max_batch]");
  if (!tokens || !positions || !logits) return fail(m, LD_EINVAL, "null tokens, positions or logits");
  if (((uintptr_t)tokens & 3) || ((uintptr_t)positions & 3) || ((uintptr_t)logits & 3) ||
      ((uintptr_t)next_tokens & 3))
    return fail(m, LD_EINVAL, "unaligned pointer");
  return enqueue_step(m, tokens, batch, 1, positions, logits, next_tokens,
                      static_cast<hipStream_t>(stream));
}

extern "C" ld_status ld_decode_step_tokens(ld_model* m, const int32_t* tokens,
                                           int32_t tokens_per_seq, int32_t batch,
                                           const int32_t* positions, float* logits,
                                           int32_t* next_tokens, void* stream) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  if (tokens_per_seq < 1) return fail(m, LD_EINVAL, "tokens_per_seq must be >= 1");
  if (tokens_per_seq > 1 && m->mode == LD_MODE_MEGA)
    return fail(m, LD_EINVAL, "several tokens per sequence need the wait, tile-flag or graph mode");
  if (batch < 1 || (int64_t)batch * tokens_per_seq > m->D.max_batch)
    return fail(m, LD_EINVAL, "batch * tokens_per_seq outside [1, max_batch]");
  if (!tokens || !positions || !logits) return fail(m, LD_EINVAL, "null tokens, positions or logits");
  if (((uintptr_t)tokens & 3) || ((uintptr_t)positions & 3) || ((uintptr_t)logits & 3) ||
      ((uintptr_t)next_tokens & 3))
    return fail(m, LD_EINVAL, "unaligned pointer");
  return enqueue_step(m, tokens, batch * tokens_per_seq, tokens_per_seq, positions, logits,
                      next_tokens, static_cast<hipStream_t>(stream));
}

extern "C" ld_status ld_device_error(ld_model* m) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return LD_OK;
  HIPCHK(m, hipDeviceSynchronize());
  int w = 0;
  HIPCHK(m, hipMemcpy(&w, m->K.err, sizeof(int), hipMemcpyDeviceToHost));
  if (w == 0) return LD_OK;
  const int zero = 0;
  HIPCHK(m, hipMemcpy(m->K.err, &zero, sizeof(int), hipMemcpyHostToDevice));
  const int code = w & 0xFF, stage = w >> 8;
  if (code == kErrTimeout) {
    // the counters no longer match the host's totals: reset both
    HIPCHK(m, hipMemset(m->K.ctr, 0, m->ctr_bytes));
    HIPCHK(m, hipDeviceSynchronize());
    m->tot_qkv = m->tot_attn = m->tot_o = m->tot_gu = m->tot_d = 0;
    m->n_tile = 0;
    char buf[96];
    snprintf(buf, sizeof buf, "device wait timed out in stage %d", stage);
    return fail(m, LD_ETIMEOUT, buf);
  }
  return fail(m, LD_EDEVICE, code == kErrToken ? "token outside [0, vocab)" : "position outside [0, max_seq)");
}

extern "C" const char* ld_last_error(const ld_model* m) {
  return m ? m->err.c_str() : g_err.c_str();
}

extern "C" void ld_free(ld_model* m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  if (m->own_w && m->warena) (void)hipFree(m->warena);
  if (m->own_k && m->karena) (void)hipFree(m->karena);
  drop_graphs(m);
  if (m->s1) (void)hipStreamDestroy(m->s1);
  if (m->s_cap) (void)hipStreamDestroy(m->s_cap);
  if (m->ev_fork) (void)hipEventDestroy(m->ev_fork);
  if (m->ev_join) (void)hipEventDestroy(m->ev_join);
  delete m;
}

extern "C" ld_status ld_set_mlp_variant(ld_model* m, int32_t variant) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (variant != LD_MLP_FUSED && variant != LD_MLP_TWO_KERNELS && variant != LD_MLP_FOUR_KERNELS)
    return fail(m, LD_EINVAL, "unknown MLP variant");
  m->mlp_variant = variant;
  return LD_OK;
}

// ------------------------------------------------------------- tuning

static const char* mode_name(int mode) {
  return mode == LD_MODE_WAIT ? "wait" : mode == LD_MODE_FLAGS ? "flags" : mode == LD_MODE_MEGA ? "mega" : "graph";
}

static ld_status write_table(ld_model* m, const char* path) {
  FILE* f = fopen(path, "w");
  if (!f) return fail(m, LD_EINVAL, std::string("cannot write ") + path);
  const ld_config& c = m->cfg;
  const int md = m->mode;
  fprintf(f, "{\"shape\": [%d, %d, %d, %d, %d, %d, %d], \"mode\": \"%s\", \"swiglu\": {", c.n_layers,
          c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.intermediate, c.vocab, mode_name(md));
  bool first = true;
  for (int b = 1; b <= 64; ++b)
    if (m->gu_tuned[md][b]) {
      fprintf(f, "%s\"%d\": \"%s\"", first ? "" : ", ", b, m->gu_variant[md][b] == kGuRow ? "row" : "col");
      first = false;
    }
  fprintf(f, "}, \"ms_per_step_col_row\": [");
  first = true;
  for (int b = 1; b <= 64; ++b)
    if (m->gu_tuned[md][b] && m->tile_ms[md][b][0] > 0.f) {
      fprintf(f, "%s[%d, %.5f, %.5f]", first ? "" : ", ", b, m->tile_ms[md][b][0], m->tile_ms[md][b][1]);
      first = false;
    }
  fprintf(f, "]}\n");
  fclose(f);
  return LD_OK;
}

// The tuning pass: for each batch size, whole decode steps in the model's
// current mode, the two tilings alternating in rounds (kTuneRounds rounds of
// kTuneSteps steps each, after warm-up), median ms per step of each; the
// row-major tiling is kept only if its median beats the column-major one by
// more than kTuneMargin (run-to-run noise on one GPU is below that).
constexpr int kTuneRounds = 5, kTuneSteps = 3;
constexpr float kTuneMargin = 0.01f;

extern "C" ld_status ld_tune(ld_model* m, const int32_t* batches, int32_t n, const char* table_path) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  if (!batches || n < 1) return fail(m, LD_EINVAL, "no batch sizes");
  for (int i = 0; i < n; ++i)
    if (batches[i] < 1 || batches[i] > m->D.max_batch)
      return fail(m, LD_EINVAL, "tuning batch outside [1, max_batch]");
  const int md = m->mode;
  const int maxB = m->D.max_batch;
  const int p = std::min(m->D.max_seq - 1, 1024);
  HIPCHK(m, hipDeviceSynchronize());
  // the steps' inputs and outputs (tokens 0.., every sequence at position p)
  int32_t* dtok = nullptr;
  float* dlog = nullptr;
  HIPCHK(m, hipMalloc(&dtok, (size_t)2 * maxB * sizeof(int32_t)));
  hipError_t he = hipMalloc(&dlog, (size_t)maxB * m->D.V * sizeof(float));
  std::vector<int32_t> host(2 * maxB);
  for (int b = 0; b < maxB; ++b) {
    host[b] = b % m->D.V;
    host[maxB + b] = p;
  }
  if (he == hipSuccess) he = hipMemcpy(dtok, host.data(), host.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (he == hipSuccess) he = hipEventCreate(&e0);
  if (he == hipSuccess) he = hipEventCreate(&e1);
  ld_status st = he == hipSuccess ? LD_OK : fail(m, LD_EHIP, std::string("tuning setup: ") + hipGetErrorString(he));
  for (int i = 0; i < n && st == LD_OK; ++i) {
    const int B = batches[i];
    std::vector<float> t[2];
    auto run = [&](int variant, int steps) -> ld_status {
      m->gu_variant[md][B] = variant;
      for (int s = 0; s < steps; ++s) {
        const ld_status r = enqueue_step(m, dtok, B, 1, dtok + maxB, dlog, nullptr, nullptr);
        if (r != LD_OK) return r;
      }
      return LD_OK;
    };
    for (int v = 0; v < 2 && st == LD_OK; ++v) st = run(v == 0 ? kGuCol : kGuRow, 2);
    for (int r = 0; r < kTuneRounds && st == LD_OK; ++r)
      for (int v = 0; v < 2 && st == LD_OK; ++v) {
        he = hipEventRecord(e0, nullptr);
        if (he == hipSuccess) st = run(v == 0 ? kGuCol : kGuRow, kTuneSteps);
        if (st == LD_OK && he == hipSuccess) he = hipEventRecord(e1, nullptr);
        if (he == hipSuccess && st == LD_OK) he = hipEventSynchronize(e1);
        float ms = 0.f;
        if (he == hipSuccess && st == LD_OK) he = hipEventElapsedTime(&ms, e0, e1);
        if (he != hipSuccess && st == LD_OK) st = fail(m, LD_EHIP, std::string("tuning: ") + hipGetErrorString(he));
        t[v].push_back(ms / kTuneSteps);
      }
    if (st != LD_OK) break;
    for (auto& x : t) std::sort(x.begin(), x.end());
    const float col = t[0][kTuneRounds / 2], row = t[1][kTuneRounds / 2];
    m->gu_variant[md][B] = (row < col * (1.0f - kTuneMargin)) ? kGuRow : kGuCol;
    m->gu_tuned[md][B] = true;
    m->tile_ms[md][B][0] = col;
    m->tile_ms[md][B][1] = row;
  }
  (void)hipDeviceSynchronize();
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(dtok);
  (void)hipFree(dlog);
  if (st != LD_OK) return st;
  int w = 0;
  HIPCHK(m, hipMemcpy(&w, m->K.err, sizeof(int), hipMemcpyDeviceToHost));
  if (w != 0) return ld_device_error(m);
  if (table_path) return write_table(m, table_path);
  return LD_OK;
}

extern "C" ld_status ld_load_tuning(ld_model* m, const char* table_path) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!table_path) return fail(m, LD_EINVAL, "null path");
  FILE* f = fopen(table_path, "r");
  if (!f) return fail(m, LD_EINVAL, std::string("cannot read ") + table_path);
  std::string txt;
  char buf[4096];
  size_t k;
  while ((k = fread(buf, 1, sizeof buf, f)) > 0) txt.append(buf, k);
  fclose(f);
  const ld_config& c = m->cfg;
  char shape[160];
  snprintf(shape, sizeof shape, "\"shape\": [%d, %d, %d, %d, %d, %d, %d]", c.n_layers, c.hidden,
           c.n_q_heads, c.n_kv_heads, c.head_dim, c.intermediate, c.vocab);
  if (txt.find(shape) == std::string::npos) return fail(m, LD_EINVAL, "tuning table is for another shape");
  const size_t sw = txt.find("\"swiglu\"");
  if (sw == std::string::npos) return fail(m, LD_EINVAL, "tuning table has no swiglu entry");
  size_t p = txt.find('{', sw);
  const size_t end = txt.find('}', p);
  if (p == std::string::npos || end == std::string::npos) return fail(m, LD_EINVAL, "malformed tuning table");
  int md = m->mode;
  const size_t mk = txt.find("\"mode\"");
  if (mk != std::string::npos) {
    const size_t q = txt.find('"', txt.find(':', mk) + 1);
    if (q == std::string::npos) return fail(m, LD_EINVAL, "malformed tuning table");
    if (txt.compare(q + 1, 5, "wait\"") == 0) md = LD_MODE_WAIT;
    else if (txt.compare(q + 1, 6, "flags\"") == 0) md = LD_MODE_FLAGS;
    else if (txt.compare(q + 1, 5, "mega\"") == 0) md = LD_MODE_MEGA;
    else if (txt.compare(q + 1, 6, "graph\"") == 0) md = LD_MODE_GRAPH;
    else return fail(m, LD_EINVAL, "unknown mode in tuning table");
  }
  int parsed[65];
  bool have[65] = {false};
  while (true) {
    const size_t q = txt.find('"', p + 1);
    if (q == std::string::npos || q > end) break;
    const int b = atoi(txt.c_str() + q + 1);
    const size_t v = txt.find('"', txt.find(':', q) + 1);
    if (b < 1 || b > 64 || v == std::string::npos || v > end) return fail(m, LD_EINVAL, "malformed tuning table");
    if (txt.compare(v + 1, 3, "row") == 0) parsed[b] = kGuRow;
    else if (txt.compare(v + 1, 3, "col") == 0) parsed[b] = kGuCol;
    else return fail(m, LD_EINVAL, "unknown tiling in tuning table");
    have[b] = true;
    p = txt.find('"', v + 1);
    if (p == std::string::npos || p > end) break;
  }
  for (int b = 1; b <= 64; ++b)
    if (have[b]) {
      m->gu_variant[md][b] = parsed[b];
      m->gu_tuned[md][b] = true;
    }
  return LD_OK;
}

// --------------------------------------------------- inspection / tests

static ld_status weight_ptr(ld_model* m, int kind, int layer, uint16_t** p, int64_t* rows,
                            int64_t* cols) {
  const Dims& D = m->D;
  const bool per_layer = !(kind == LD_W_EMBED || kind == LD_W_FINAL_NORM || kind == LD_W_LM_HEAD);
  if (per_layer && (layer < 0 || layer >= D.L)) return fail(m, LD_EINVAL, "layer out of range");
  uint16_t* lb = const_cast<uint16_t*>(m->W.layer0) + (per_layer ? (int64_t)layer * m->W.layer_stride : 0);
  const int64_t H = D.H, I = D.I, qd = D.qd, kvd = D.kvd;
  switch (kind) {
    case LD_W_EMBED: *p = const_cast<uint16_t*>(m->W.embed); *rows = D.V; *cols = H; break;
    case LD_W_FINAL_NORM: *p = const_cast<uint16_t*>(m->W.final_norm); *rows = 1; *cols = H; break;
    case LD_W_LM_HEAD: *p = const_cast<uint16_t*>(m->W.lm); *rows = D.V; *cols = H; break;
    case LD_W_ATTN_NORM: *p = lb + m->W.o_attn_norm; *rows = 1; *cols = H; break;
    case LD_W_Q: *p = lb + m->W.o_wqkv; *rows = qd; *cols = H; break;
    case LD_W_K: *p = lb + m->W.o_wqkv + qd * H; *rows = kvd; *cols = H; break;
    case LD_W_V: *p = lb + m->W.o_wqkv + (qd + kvd) * H; *rows = kvd; *cols = H; break;
    case LD_W_O: *p = lb + m->W.o_wo; *rows = H; *cols = qd; break;
    case LD_W_MLP_NORM: *p = lb + m->W.o_mlp_norm; *rows = 1; *cols = H; break;
    case LD_W_GATE: *p = lb + m->W.o_wg; *rows = I; *cols = H; break;
    case LD_W_UP: *p = lb + m->W.o_wu; *rows = I; *cols = H; break;
    case LD_W_DOWN: *p = lb + m->W.o_wd; *rows = H; *cols = I; break;
    default: return fail(m, LD_EINVAL, "unknown weight kind");
  }
  return LD_OK;
}

extern "C" ld_status ld_weight_shape(ld_model* m, int32_t kind, int32_t layer, int64_t* rows,
                                     int64_t* cols) {
  if (!m || !rows || !cols) return fail(m, LD_EINVAL, "null argument");
  uint16_t* p;
  return weight_ptr(m, kind, layer, &p, rows, cols);
}

extern "C" ld_status ld_read_weight(ld_model* m, int32_t kind, int32_t layer, uint16_t* host_dst) {
  if (!m || !host_dst) return fail(m, LD_EINVAL, "null argument");
  uint16_t* p;
  int64_t r, c;
  ld_status st = weight_ptr(m, kind, layer, &p, &r, &c);
  if (st != LD_OK) return st;
  HIPCHK(m, hipDeviceSynchronize());
  HIPCHK(m, hipMemcpy(host_dst, p, (size_t)(r * c) * 2, hipMemcpyDeviceToHost));
  return LD_OK;
}

extern "C" ld_status ld_write_weight(ld_model* m, int32_t kind, int32_t layer,
                                     const uint16_t* host_src) {
  if (!m || !host_src) return fail(m, LD_EINVAL, "null argument");
  uint16_t* p;
  int64_t r, c;
  ld_status st = weight_ptr(m, kind, layer, &p, &r, &c);
  if (st != LD_OK) return st;
  if (kind == LD_W_LM_HEAD && m->cfg.tied) return fail(m, LD_EINVAL, "tied model: write the embedding");
  HIPCHK(m, hipDeviceSynchronize());
  HIPCHK(m, hipMemcpy(p, host_src, (size_t)(r * c) * 2, hipMemcpyHostToDevice));
  return LD_OK;
}

extern "C" ld_status ld_read_kv(ld_model* m, int32_t layer, int32_t seq, int32_t kv_head,
                                int32_t pos0, int32_t npos, uint16_t* k_dst, uint16_t* v_dst) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  const Dims& D = m->D;
  if (layer < 0 || layer >= D.L || seq < 0 || seq >= D.max_batch || kv_head < 0 ||
      kv_head >= D.nkv || pos0 < 0 || npos < 0 || pos0 + npos > D.max_seq)
    return fail(m, LD_EINVAL, "KV slice out of range");
  const int64_t off = ((((int64_t)layer * D.max_batch + seq) * D.nkv + kv_head) * D.max_seq + pos0) * D.d;
  HIPCHK(m, hipDeviceSynchronize());
  if (k_dst) HIPCHK(m, hipMemcpy(k_dst, m->K.kc + off, (size_t)npos * D.d * 2, hipMemcpyDeviceToHost));
  if (v_dst) HIPCHK(m, hipMemcpy(v_dst, m->K.vc + off, (size_t)npos * D.d * 2, hipMemcpyDeviceToHost));
  return LD_OK;
}

extern "C" ld_status ld_read_activation(ld_model* m, int32_t which, int32_t rows,
                                        float* host_dst) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  if (!host_dst || rows < 1 || rows > m->D.max_batch) return fail(m, LD_EINVAL, "bad rows or buffer");
  const Dims& D = m->D;
  const float* src = nullptr;
  size_t width = 0;
  switch (which) {
    case LD_ACT_X: src = m->K.xa; width = D.H; break;
    case LD_ACT_QKV: src = m->K.qkv; width = D.qkv_rows; break;
    case LD_ACT_ATTN: src = m->K.ao; width = D.qd; break;
    case LD_ACT_H: src = m->K.hbuf; width = D.I; break;
    default: return fail(m, LD_EINVAL, "unknown work buffer");
  }
  HIPCHK(m, hipDeviceSynchronize());
  if ((which == LD_ACT_ATTN || which == LD_ACT_H) && m->last_rows >= kMfmaMinBatch) {
    // the MFMA engine's steps keep these in B-fragment order: gather rows
    const uint32_t* f = which == LD_ACT_ATTN ? m->K.ao_f : m->K.h_f;
    const int kp = which == LD_ACT_ATTN ? D.qdp : D.Ip;
    std::vector<uint32_t> tmp((size_t)((D.max_batch + 15) / 16 * 16) * kp);
    HIPCHK(m, hipMemcpy(tmp.data(), f, tmp.size() * 4, hipMemcpyDeviceToHost));
    uint32_t* out = reinterpret_cast<uint32_t*>(host_dst);
    for (int b = 0; b < rows; ++b)
      for (size_t c = 0; c < width; ++c) out[(size_t)b * width + c] = tmp[frag_word(b, (int)c, kp)];
    return LD_OK;
  }
  HIPCHK(m, hipMemcpy(host_dst, src, (size_t)rows * width * 4, hipMemcpyDeviceToHost));
  return LD_OK;
}

extern "C" ld_status ld_set_swiglu_variant(ld_model* m, int32_t batch, int32_t variant) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (batch < 1 || batch > 64 || (variant != LD_SWIGLU_COL && variant != LD_SWIGLU_ROW))
    return fail(m, LD_EINVAL, "bad batch or variant");
  for (int md = 0; md < kModes; ++md) m->gu_variant[md][batch] = variant == LD_SWIGLU_ROW ? kGuRow : kGuCol;
  return LD_OK;
}

extern "C" int32_t ld_get_swiglu_variant(const ld_model* m, int32_t batch) {
  if (!m || batch < 1 || batch > 64) return -1;
  return m->gu_variant[m->mode][batch] == kGuRow ? LD_SWIGLU_ROW : LD_SWIGLU_COL;
}

extern "C" ld_status ld_set_sync(ld_model* m, int32_t granularity) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (granularity != LD_SYNC_STAGE && granularity != LD_SYNC_TILE && granularity != LD_SYNC_AUTO)
    return fail(m, LD_EINVAL, "unknown readiness granularity");
  m->sync = granularity;
  return LD_OK;
}

extern "C" ld_status ld_set_watchdog(ld_model* m, double seconds) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!(seconds > 0.0) || seconds > 3600.0) return fail(m, LD_EINVAL, "watchdog outside (0, 3600] s");
  m->watchdog_ticks = (uint64_t)(m->wall_khz * 1000.0 * seconds);
  m->K.watchdog = m->watchdog_ticks;
  return LD_OK;
}

extern "C" ld_status ld_set_debug(ld_model* m, int32_t flags) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (flags & ~LD_DEBUG_POISON) return fail(m, LD_EINVAL, "unknown debug flag");
  m->debug = flags;
  return LD_OK;
}

extern "C" ld_status ld_audit(ld_model* m) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  HIPCHK(m, hipDeviceSynchronize());
  std::vector<uint32_t> c(m->ctr_bytes / 4);
  HIPCHK(m, hipMemcpy(c.data(), m->K.ctr, m->ctr_bytes, hipMemcpyDeviceToHost));
  int err = 0;
  HIPCHK(m, hipMemcpy(&err, m->K.err, sizeof(int), hipMemcpyDeviceToHost));
  const Dims& D = m->D;
  auto at = [&](const uint32_t* p) { return (size_t)(p - m->K.ctr); };
  auto leaves = [&](size_t o) {
    uint32_t t = 0;  // (the waits add the leaves modulo 2^32 too)
    for (int lf = 0; lf < kLeaves; ++lf) t += c[o + (size_t)lf * kLeafStride];
    return t;
  };
  std::string bad;
  int nbad = 0;
  auto check = [&](const char* what, int l, int i, uint32_t got, uint32_t want) {
    if (got == want) return;
    if (nbad++ < 4) {
      char buf[128];
      snprintf(buf, sizeof buf, "%s%s[layer %d][%d] = %u, expected %u", bad.empty() ? "" : "; ",
               what, l, i, got, want);
      bad += buf;
    }
  };
  // whole-stage counters: every step that signals adds the host's totals
  const uint32_t tot[kStageCtrs] = {m->tot_qkv, m->tot_attn, m->tot_o, m->tot_gu, m->tot_d};
  static const char* names[kStageCtrs] = {"qkv", "attention", "o", "swiglu", "down"};
  for (int l = 0; l < D.L; ++l)
    for (int st = 0; st < kStageCtrs; ++st) {
      const size_t o = ((size_t)l * kStageCtrs + st) * kCtrWords;
      check(names[st], l, 0, leaves(o), tot[st]);
      check(names[st], l, 1, c[o + (size_t)kLeaves * kLeafStride], 0u);
    }
  // row-count counters: each tile-granular step adds every row once
  for (int l = 0; l < D.L; ++l) {
    for (int g = 0; g < D.nkv; ++g)
      check("qkv rows of kv group", l, g,
            leaves(at(m->K.qg_ctr) + ((size_t)l * D.nkv + g) * kCtrWords),
            m->n_tile * (uint32_t)((D.group + 2) * D.d));
    for (int ch = 0; ch < D.nhc; ++ch)
      check("swiglu rows of chunk", l, ch,
            leaves(at(m->K.hc_ctr) + ((size_t)l * D.nhc + ch) * kCtrWords),
            m->n_tile * (uint32_t)std::min(kHChunk, D.I - ch * kHChunk));
  }
  // last-arriver counters (LM head, attention splits, split K) return to zero
  for (size_t o = at(m->K.lm_ctr); o < at(m->K.qg_ctr); ++o)
    if (c[o] != 0) check("last-arriver counter word", -1, (int)(o - at(m->K.lm_ctr)), c[o], 0u);
  if (err != 0) check("device error word", -1, 0, (uint32_t)err, 0u);
  if (nbad == 0) return LD_OK;
  return fail(m, LD_EAUDIT, std::to_string(nbad) + " counter mismatches: " + bad);
}

extern "C" ld_status ld_debug_inject_stall(ld_model* m) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  m->inject_next = 1;  // next step's attention waits for one signal too many
  return LD_OK;
}

extern "C" ld_status ld_set_trace(ld_model* m, void* dev_buf, size_t bytes) {
  if (!m) return fail(nullptr, LD_EINVAL, "null model");
  if (!m->kv_ready) return fail(m, LD_ESTATE, "ld_alloc_kv first");
  const size_t need = ld_trace_bytes(&m->cfg);
  if (dev_buf && bytes < need) return fail(m, LD_ENOMEM, "trace buffer too small");
  m->K.trace = static_cast<uint64_t*>(dev_buf);
  return LD_OK;
}

extern "C" size_t ld_trace_bytes(const ld_config* cfg) {
  if (!cfg) return 0;
  return ((size_t)cfg->n_layers + 1) * 8 * 4 * 1024 * sizeof(uint64_t);
}

extern "C" ld_status ld_launch_info(const ld_model* m, int32_t* out, int32_t n) {
  if (!m || !out || n < 6) return LD_EINVAL;
  out[0] = m->n_cu;
  out[1] = m->grid_wait;
  out[2] = m->flags_ok ? m->grid_flags : 0;
  out[3] = m->grid_mega[1];
  out[4] = m->D.split_len;
  out[5] = (int32_t)m->mode;
  return LD_OK;
}
