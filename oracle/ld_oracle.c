/*
 * ld_oracle.c - CPU oracle for the small-batch Llama-style decode step.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).
 *
 * Plain, single-threaded, obviously-correct loops.  Built twice:
 *   liblo32.so : lo_real = float  (the oracle the GPU path is compared with)
 *   liblo64.so : lo_real = double (a self-check of the float build's rounding)
 * Weight and KV-cache storage is bf16 in both builds.
 *
 * See ld_oracle.h for the sources each step follows.  Inputs come from the
 * seeded generator in synth/ld_synth.h, the only code shared with the GPU
 * library.
 */
#include "ld_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "../synth/ld_synth.h"

#if defined(LO_REAL_IS_DOUBLE)
#define LO_EXP exp
#define LO_SQRT sqrt
#else
#define LO_EXP expf
#define LO_SQRT sqrtf
#endif

int32_t lo_real_bytes(void) { return (int32_t)sizeof(lo_real); }

/* ------------------------------------------------------------------ bf16 */

uint16_t lo_bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) { /* inf or nan: keep, quiet nan */
    uint16_t hi = (uint16_t)(u >> 16);
    if (u & 0x007FFFFFu) hi |= 0x0040u;
    return hi;
  }
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

float lo_bf16_widen(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ----------------------------------------------------------------- model */

typedef struct {
  uint16_t *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *wg, *wu, *wd;
} lo_layer;

struct lo_model {
  lo_config cfg;
  uint16_t* embed;      /* [V, H] */
  uint16_t* final_norm; /* [H] */
  uint16_t* lm_head;    /* [V, H]; == embed when tied */
  lo_layer* layers;
};

struct lo_kv {
  lo_config cfg;
  int32_t max_batch, max_seq;
  uint16_t* k; /* [L][B][n_kv][max_seq][d] */
  uint16_t* v;
};

static int cfg_ok(const lo_config* c) {
  if (!c) return 0;
  if (c->n_layers < 1 || c->hidden < 2 || c->n_q_heads < 1 || c->n_kv_heads < 1) return 0;
  if (c->head_dim < 2 || (c->head_dim & 1) || c->intermediate < 1 || c->vocab < 1) return 0;
  if (c->n_q_heads % c->n_kv_heads) return 0;
  if (!(c->rms_eps >= 0.0f) || !(c->rope_theta > 0.0f)) return 0;
  return 1;
}

static uint16_t* alloc_bf16(int64_t n, uint16_t fill) {
  uint16_t* p = (uint16_t*)malloc((size_t)n * sizeof(uint16_t));
  if (!p) return NULL;
  if (fill == 0) {
    memset(p, 0, (size_t)n * sizeof(uint16_t));
  } else {
    for (int64_t i = 0; i < n; ++i) p[i] = fill;
  }
  return p;
}

void lo_model_free(lo_model* m) {
  if (!m) return;
  if (m->layers) {
    for (int l = 0; l < m->cfg.n_layers; ++l) {
      lo_layer* L = &m->layers[l];
      free(L->attn_norm); free(L->wq); free(L->wk); free(L->wv); free(L->wo);
      free(L->mlp_norm); free(L->wg); free(L->wu); free(L->wd);
    }
    free(m->layers);
  }
  if (m->lm_head != m->embed) free(m->lm_head);
  free(m->embed);
  free(m->final_norm);
  free(m);
}

lo_model* lo_model_create(const lo_config* c) {
  if (!cfg_ok(c)) return NULL;
  lo_model* m = (lo_model*)calloc(1, sizeof(lo_model));
  if (!m) return NULL;
  m->cfg = *c;
  const int64_t H = c->hidden, V = c->vocab, I = c->intermediate;
  const int64_t QD = (int64_t)c->n_q_heads * c->head_dim;
  const int64_t KD = (int64_t)c->n_kv_heads * c->head_dim;
  int ok = 1;
  m->embed = alloc_bf16(V * H, 0);
  m->final_norm = alloc_bf16(H, LS_BF16_ONE);
  m->lm_head = c->tied ? m->embed : alloc_bf16(V * H, 0);
  m->layers = (lo_layer*)calloc((size_t)c->n_layers, sizeof(lo_layer));
  ok = m->embed && m->final_norm && m->lm_head && m->layers;
  for (int l = 0; ok && l < c->n_layers; ++l) {
    lo_layer* L = &m->layers[l];
    L->attn_norm = alloc_bf16(H, LS_BF16_ONE);
    L->wq = alloc_bf16(QD * H, 0);
    L->wk = alloc_bf16(KD * H, 0);
    L->wv = alloc_bf16(KD * H, 0);
    L->wo = alloc_bf16(H * QD, 0);
    L->mlp_norm = alloc_bf16(H, LS_BF16_ONE);
    L->wg = alloc_bf16(I * H, 0);
    L->wu = alloc_bf16(I * H, 0);
    L->wd = alloc_bf16(H * I, 0);
    ok = L->attn_norm && L->wq && L->wk && L->wv && L->wo && L->mlp_norm && L->wg && L->wu &&
         L->wd;
  }
  if (!ok) {
    lo_model_free(m);
    return NULL;
  }
  return m;
}

uint16_t* lo_weight(lo_model* m, int kind, int layer, int64_t* rows, int64_t* cols) {
  if (!m) return NULL;
  const lo_config* c = &m->cfg;
  const int64_t H = c->hidden, V = c->vocab, I = c->intermediate;
  const int64_t QD = (int64_t)c->n_q_heads * c->head_dim;
  const int64_t KD = (int64_t)c->n_kv_heads * c->head_dim;
  int64_t r = 0, k = 0;
  uint16_t* p = NULL;
  int per_layer = !(kind == LO_W_EMBED || kind == LO_W_FINAL_NORM || kind == LO_W_LM_HEAD);
  if (per_layer && (layer < 0 || layer >= c->n_layers)) return NULL;
  lo_layer* L = per_layer ? &m->layers[layer] : NULL;
  switch (kind) {
    case LO_W_EMBED: p = m->embed; r = V; k = H; break;
    case LO_W_FINAL_NORM: p = m->final_norm; r = 1; k = H; break;
    case LO_W_LM_HEAD: p = m->lm_head; r = V; k = H; break;
    case LO_W_ATTN_NORM: p = L->attn_norm; r = 1; k = H; break;
    case LO_W_Q: p = L->wq; r = QD; k = H; break;
    case LO_W_K: p = L->wk; r = KD; k = H; break;
    case LO_W_V: p = L->wv; r = KD; k = H; break;
    case LO_W_O: p = L->wo; r = H; k = QD; break;
    case LO_W_MLP_NORM: p = L->mlp_norm; r = 1; k = H; break;
    case LO_W_GATE: p = L->wg; r = I; k = H; break;
    case LO_W_UP: p = L->wu; r = I; k = H; break;
    case LO_W_DOWN: p = L->wd; r = H; k = I; break;
    default: return NULL;
  }
  if (rows) *rows = r;
  if (cols) *cols = k;
  return p;
}

/* Inputs only: fill from the seeded generator (logical row-major index). */
static void fill_normal(uint16_t* dst, int64_t n, uint64_t seed, uint64_t tensor, float kappa) {
  const uint64_t key = ls_key(seed, tensor);
#if defined(_OPENMP)
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; ++i) dst[i] = ls_normal_bf16(key, (uint64_t)i, kappa);
}

int lo_model_synth(lo_model* m, uint64_t seed, float w_std) {
  if (!m) return -1;
  const lo_config* c = &m->cfg;
  const float kappa = ls_kappa(w_std);
  const int64_t H = c->hidden, V = c->vocab, I = c->intermediate;
  const int64_t QD = (int64_t)c->n_q_heads * c->head_dim;
  const int64_t KD = (int64_t)c->n_kv_heads * c->head_dim;
  fill_normal(m->embed, V * H, seed, LS_T_EMBED, kappa);
  if (!c->tied) fill_normal(m->lm_head, V * H, seed, LS_T_LM_HEAD, kappa);
  for (int l = 0; l < c->n_layers; ++l) {
    lo_layer* L = &m->layers[l];
    fill_normal(L->wq, QD * H, seed, LS_T_LAYER(l, LS_K_WQ), kappa);
    fill_normal(L->wk, KD * H, seed, LS_T_LAYER(l, LS_K_WK), kappa);
    fill_normal(L->wv, KD * H, seed, LS_T_LAYER(l, LS_K_WV), kappa);
    fill_normal(L->wo, H * QD, seed, LS_T_LAYER(l, LS_K_WO), kappa);
    fill_normal(L->wg, I * H, seed, LS_T_LAYER(l, LS_K_WG), kappa);
    fill_normal(L->wu, I * H, seed, LS_T_LAYER(l, LS_K_WU), kappa);
    fill_normal(L->wd, H * I, seed, LS_T_LAYER(l, LS_K_WD), kappa);
  }
  return 0;
}

/* -------------------------------------------------------------- KV cache */

lo_kv* lo_kv_create(const lo_config* c, int32_t max_batch, int32_t max_seq) {
  if (!cfg_ok(c) || max_batch < 1 || max_seq < 1) return NULL;
  lo_kv* kv = (lo_kv*)calloc(1, sizeof(lo_kv));
  if (!kv) return NULL;
  kv->cfg = *c;
  kv->max_batch = max_batch;
  kv->max_seq = max_seq;
  const size_t n = (size_t)c->n_layers * max_batch * c->n_kv_heads * (size_t)max_seq * c->head_dim;
  kv->k = (uint16_t*)calloc(n, sizeof(uint16_t));
  kv->v = (uint16_t*)calloc(n, sizeof(uint16_t));
  if (!kv->k || !kv->v) {
    lo_kv_free(kv);
    return NULL;
  }
  return kv;
}

void lo_kv_free(lo_kv* kv) {
  if (!kv) return;
  free(kv->k);
  free(kv->v);
  free(kv);
}

static size_t kv_off(const lo_kv* kv, int layer, int seq, int h) {
  const lo_config* c = &kv->cfg;
  return ((((size_t)layer * kv->max_batch + seq) * c->n_kv_heads + h) * (size_t)kv->max_seq) *
         c->head_dim;
}

uint16_t* lo_kv_k(lo_kv* kv, int layer, int seq, int h) {
  if (!kv || layer < 0 || layer >= kv->cfg.n_layers || seq < 0 || seq >= kv->max_batch || h < 0 ||
      h >= kv->cfg.n_kv_heads)
    return NULL;
  return kv->k + kv_off(kv, layer, seq, h);
}

uint16_t* lo_kv_v(lo_kv* kv, int layer, int seq, int h) {
  if (!kv || layer < 0 || layer >= kv->cfg.n_layers || seq < 0 || seq >= kv->max_batch || h < 0 ||
      h >= kv->cfg.n_kv_heads)
    return NULL;
  return kv->v + kv_off(kv, layer, seq, h);
}

int lo_kv_synth(lo_kv* kv, uint64_t seed, float kv_std, const int32_t* prefill_len) {
  return lo_kv_synth_from(kv, seed, kv_std, prefill_len, 0);
}

int lo_kv_synth_from(lo_kv* kv, uint64_t seed, float kv_std, const int32_t* prefill_len,
                     int32_t seq0) {
  if (!kv || !prefill_len || seq0 < 0) return -1;
  const lo_config* c = &kv->cfg;
  const float kappa = ls_kappa(kv_std);
  const int d = c->head_dim;
  for (int b = 0; b < kv->max_batch; ++b)
    if (prefill_len[b] < 0 || prefill_len[b] > kv->max_seq) return -1;
  for (int l = 0; l < c->n_layers; ++l) {
    const uint64_t kk = ls_key(seed, LS_T_KCACHE(l));
    const uint64_t kvk = ls_key(seed, LS_T_VCACHE(l));
    for (int b = 0; b < kv->max_batch; ++b)
      for (int h = 0; h < c->n_kv_heads; ++h) {
        uint16_t* K = lo_kv_k(kv, l, b, h);
        uint16_t* V = lo_kv_v(kv, l, b, h);
        for (int p = 0; p < prefill_len[b]; ++p)
          for (int i = 0; i < d; ++i) {
            const uint64_t idx = ls_kv_index((uint64_t)(b + seq0), (uint64_t)c->n_kv_heads, (uint64_t)h,
                                             (uint64_t)p, (uint64_t)d, (uint64_t)i);
            K[(size_t)p * d + i] = ls_normal_bf16(kk, idx, kappa);
            V[(size_t)p * d + i] = ls_normal_bf16(kvk, idx, kappa);
          }
      }
  }
  return 0;
}

/* ------------------------------------------------------------ operations */

/* SiLU(a) = a * sigmoid(a) = a / (1 + e^-a) (Shazeer's GLU variants, cited
 * by "Deep Kernel Fusion for Transformers" for the SwiGLU first stage). */
lo_real lo_silu(lo_real a) { return a / ((lo_real)1 + LO_EXP(-a)); }

/* RMSNorm: r = 1 / sqrt(sum(x^2)/n + eps); out_j = (x_j * r) * g_j. */
void lo_rmsnorm(const lo_real* x, const uint16_t* g, int32_t n, float eps, lo_real* out) {
  lo_real ss = 0;
  for (int32_t j = 0; j < n; ++j) ss += x[j] * x[j];
  const lo_real r = (lo_real)1 / LO_SQRT(ss / (lo_real)n + (lo_real)eps);
  for (int32_t j = 0; j < n; ++j) {
    const lo_real gj = g ? (lo_real)lo_bf16_widen(g[j]) : (lo_real)1;
    out[j] = (x[j] * r) * gj;
  }
}

void lo_matvec(const uint16_t* W, int64_t rows, int64_t cols, const lo_real* x, lo_real* y) {
  for (int64_t i = 0; i < rows; ++i) {
    const uint16_t* w = W + i * cols;
    lo_real acc = 0;
    for (int64_t j = 0; j < cols; ++j) acc += (lo_real)lo_bf16_widen(w[j]) * x[j];
    y[i] = acc;
  }
}

/* Rotary embedding, rotate-half pairing: pair i (< d/2) holds (h_i, h_{i+d/2})
 * and turns by angle p * theta^(-2i/d).  Angle and its cosine and sine are
 * computed in double, then rounded to lo_real. */
void lo_rope(lo_real* h, int32_t d, int32_t p, float theta) {
  const int32_t half = d / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double inv = pow((double)theta, -2.0 * (double)i / (double)d);
    const double a = (double)p * inv;
    const lo_real c = (lo_real)cos(a), s = (lo_real)sin(a);
    const lo_real h0 = h[i], h1 = h[i + half];
    h[i] = h0 * c - h1 * s;
    h[i + half] = h0 * s + h1 * c;
  }
}

/* Max-subtracted softmax: s_t <- e^(s_t - max) / sum_u e^(s_u - max). */
void lo_softmax(lo_real* s, int32_t n) {
  if (n <= 0) return;
  lo_real m = s[0];
  for (int32_t t = 1; t < n; ++t)
    if (s[t] > m) m = s[t];
  lo_real z = 0;
  for (int32_t t = 0; t < n; ++t) {
    s[t] = LO_EXP(s[t] - m);
    z += s[t];
  }
  for (int32_t t = 0; t < n; ++t) s[t] = s[t] / z;
}

/* Scores s_t = (q . K_t) / sqrt(d), softmax over t, output sum_t w_t V_t. */
void lo_attention_head(const lo_real* q, const uint16_t* K, const uint16_t* V, int32_t len,
                       int32_t d, lo_real* out) {
  lo_real* s = (lo_real*)malloc((size_t)(len > 0 ? len : 1) * sizeof(lo_real));
  if (!s) return;
  const lo_real scale = (lo_real)1 / LO_SQRT((lo_real)d);
  for (int32_t t = 0; t < len; ++t) {
    lo_real dot = 0;
    for (int32_t i = 0; i < d; ++i) dot += q[i] * (lo_real)lo_bf16_widen(K[(size_t)t * d + i]);
    s[t] = dot * scale;
  }
  lo_softmax(s, len);
  for (int32_t i = 0; i < d; ++i) {
    lo_real acc = 0;
    for (int32_t t = 0; t < len; ++t) acc += s[t] * (lo_real)lo_bf16_widen(V[(size_t)t * d + i]);
    out[i] = acc;
  }
  free(s);
}

/* First MLP stage: Up and Gate projections, SiLU on the gate, elementwise
 * product ("Deep Kernel Fusion for Transformers", Summary). */
void lo_swiglu(const uint16_t* Wg, const uint16_t* Wu, int64_t inter, int64_t hidden,
               const lo_real* xn, lo_real* h) {
  for (int64_t i = 0; i < inter; ++i) {
    lo_real a = 0, u = 0;
    lo_matvec(Wg + i * hidden, 1, hidden, xn, &a);
    lo_matvec(Wu + i * hidden, 1, hidden, xn, &u);
    h[i] = lo_silu(a) * u;
  }
}

int32_t lo_argmax(const lo_real* v, int64_t n) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return (int32_t)best;
}

/* ------------------------------------------------------------ decode step */

static void copy_real(lo_real* dst, const lo_real* src, int64_t n) {
  if (dst) memcpy(dst, src, (size_t)n * sizeof(lo_real));
}

/* One sequence: the whole layer stack and the LM head for cache slot b. */
static int decode_seq(const lo_model* m, lo_kv* kv, int32_t b, int32_t tok, int32_t p,
                      float* logits_b, int32_t* next_b, lo_trace* trace) {
  const lo_config* c = &m->cfg;
  const int32_t H = c->hidden, d = c->head_dim, nq = c->n_q_heads, nkv = c->n_kv_heads;
  const int32_t I = c->intermediate, V = c->vocab, group = nq / nkv;
  const int64_t nbuf = (int64_t)H + 2 * (int64_t)nq * d + 2 * (int64_t)nkv * d + I + V + H + H;
  lo_real* buf = (lo_real*)malloc((size_t)nbuf * sizeof(lo_real));
  if (!buf) return -1;
  lo_real* x = buf;
  lo_real* xn = x + H;
  lo_real* q = xn + H;
  lo_real* k = q + (int64_t)nq * d;
  lo_real* v = k + (int64_t)nkv * d;
  lo_real* o = v + (int64_t)nkv * d;
  lo_real* hh = o + (int64_t)nq * d;
  lo_real* lg = hh + I;
  lo_real* tmp = lg + V;

  /* embedding row, widened */
  for (int32_t j = 0; j < H; ++j) x[j] = (lo_real)lo_bf16_widen(m->embed[(int64_t)tok * H + j]);

  for (int32_t l = 0; l < c->n_layers; ++l) {
    const lo_layer* L = &m->layers[l];
    const int tr = trace && trace->seq == b && trace->layer == l;
    /* attention block: x += Wo . attn(rope(Wq n(x)), cache + rope(Wk n(x)), cache + Wv n(x)) */
    lo_rmsnorm(x, L->attn_norm, H, c->rms_eps, xn);
    if (tr) copy_real(trace->xn, xn, H);
    lo_matvec(L->wq, (int64_t)nq * d, H, xn, q);
    lo_matvec(L->wk, (int64_t)nkv * d, H, xn, k);
    lo_matvec(L->wv, (int64_t)nkv * d, H, xn, v);
    for (int32_t hq = 0; hq < nq; ++hq) lo_rope(q + (int64_t)hq * d, d, p, c->rope_theta);
    for (int32_t hk = 0; hk < nkv; ++hk) lo_rope(k + (int64_t)hk * d, d, p, c->rope_theta);
    if (tr) {
      copy_real(trace->q, q, (int64_t)nq * d);
      copy_real(trace->k, k, (int64_t)nkv * d);
      copy_real(trace->v, v, (int64_t)nkv * d);
    }
    for (int32_t hk = 0; hk < nkv; ++hk) {
      uint16_t* Kc = lo_kv_k(kv, l, b, hk);
      uint16_t* Vc = lo_kv_v(kv, l, b, hk);
      for (int32_t i = 0; i < d; ++i) {
        Kc[(size_t)p * d + i] = lo_bf16_round((float)k[(int64_t)hk * d + i]);
        Vc[(size_t)p * d + i] = lo_bf16_round((float)v[(int64_t)hk * d + i]);
      }
    }
    for (int32_t hq = 0; hq < nq; ++hq) {
      const int32_t hk = hq / group;
      lo_attention_head(q + (int64_t)hq * d, lo_kv_k(kv, l, b, hk), lo_kv_v(kv, l, b, hk), p + 1,
                        d, o + (int64_t)hq * d);
    }
    if (tr) copy_real(trace->o, o, (int64_t)nq * d);
    lo_matvec(L->wo, H, (int64_t)nq * d, o, tmp);
    for (int32_t j = 0; j < H; ++j) x[j] = x[j] + tmp[j];
    if (tr) copy_real(trace->x_attn, x, H);

    /* MLP block: x += Wd . (silu(Wg n(x)) * (Wu n(x))) */
    lo_rmsnorm(x, L->mlp_norm, H, c->rms_eps, xn);
    if (tr) copy_real(trace->xn2, xn, H);
    lo_swiglu(L->wg, L->wu, I, H, xn, hh);
    if (tr) copy_real(trace->hh, hh, I);
    lo_matvec(L->wd, H, I, hh, tmp);
    for (int32_t j = 0; j < H; ++j) x[j] = x[j] + tmp[j];
    if (tr) copy_real(trace->x_out, x, H);
  }

  lo_rmsnorm(x, m->final_norm, H, c->rms_eps, xn);
  lo_matvec(m->lm_head, V, H, xn, lg);
  for (int32_t vv = 0; vv < V; ++vv) logits_b[vv] = (float)lg[vv];
  if (next_b) *next_b = lo_argmax(lg, V);
  free(buf);
  return 0;
}

int lo_decode_step(const lo_model* m, lo_kv* kv, const int32_t* tokens, int32_t B,
                   const int32_t* pos, float* logits, int32_t* next, lo_trace* trace) {
  if (!m || !kv || !tokens || !pos || !logits || B < 1 || B > kv->max_batch) return -1;
  const lo_config* c = &m->cfg;
  if (memcmp(c, &kv->cfg, sizeof(lo_config)) != 0) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (tokens[b] < 0 || tokens[b] >= c->vocab || pos[b] < 0 || pos[b] >= kv->max_seq) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (decode_seq(m, kv, b, tokens[b], pos[b], logits + (int64_t)b * c->vocab,
                   next ? next + b : NULL, trace) != 0)
      return -1;
  return 0;
}

int lo_decode_one(const lo_model* m, lo_kv* kv, int32_t seq, int32_t token, int32_t pos,
                  float* logits, int32_t* next) {
  if (!m || !kv || !logits || seq < 0 || seq >= kv->max_batch) return -1;
  const lo_config* c = &m->cfg;
  if (memcmp(c, &kv->cfg, sizeof(lo_config)) != 0) return -1;
  if (token < 0 || token >= c->vocab || pos < 0 || pos >= kv->max_seq) return -1;
  return decode_seq(m, kv, seq, token, pos, logits, next, NULL);
}
