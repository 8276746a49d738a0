/*
 * oracle.c -- plain CPU reference decoder.  TEST INFRASTRUCTURE ONLY: the
 * test suite, the smoke check and the benchmark's CPU-baseline leg are its
 * only users; the product path never loads it.  It shares no code with the
 * GPU library.
 *
 * The decode step it implements, in the order the MPK digest
 * (fr.news.hada.io, "Part 1. Compilateur") lists the operators of an LLM
 * computation graph: per layer RMSNorm -> Q/K/V projections -> (QK-Norm) ->
 * RoPE -> KV append -> attention -> O-projection + residual -> RMSNorm ->
 * gated MLP -> down-projection + residual; then final RMSNorm, LM head and
 * greedy argmax.  Each primitive below names the passage that defines it.
 *
 * Precision: fp32 everywhere, bf16 weights and KV cache, sequential sums in
 * ascending index.  Build with -ffp-contract=off and without -ffast-math so
 * every multiply and add is rounded separately, as written.
 */
#include "oracle.h"
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32                                                        */
/* ------------------------------------------------------------------ */
float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0; /* NaN */
  /* round to nearest, ties to even */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Linear layer y = W x (Mirage article, "Case 1: Normalization +      */
/* Linear": the MatMul that follows the norm).  Each output row is a   */
/* sequential fp32 sum over k = 0..cols-1.  Four rows are walked side  */
/* by side for instruction-level parallelism; no row's sum is split or */
/* reordered.  With n_threads > 1 disjoint row blocks go to threads,   */
/* which cannot change any result.                                     */
/* ------------------------------------------------------------------ */
static void matvec_rows(const uint16_t* W, int r0, int r1, int cols, const float* x, float* y) {
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    const uint16_t* w0 = W + (size_t)r * cols;
    const uint16_t* w1 = w0 + cols;
    const uint16_t* w2 = w1 + cols;
    const uint16_t* w3 = w2 + cols;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    for (int k = 0; k < cols; ++k) {
      float xk = x[k];
      a0 += orc_bf16_to_f32(w0[k]) * xk;
      a1 += orc_bf16_to_f32(w1[k]) * xk;
      a2 += orc_bf16_to_f32(w2[k]) * xk;
      a3 += orc_bf16_to_f32(w3[k]) * xk;
    }
    y[r] = a0; y[r + 1] = a1; y[r + 2] = a2; y[r + 3] = a3;
  }
  for (; r < r1; ++r) {
    const uint16_t* w = W + (size_t)r * cols;
    float a = 0.0f;
    for (int k = 0; k < cols; ++k) a += orc_bf16_to_f32(w[k]) * x[k];
    y[r] = a;
  }
}

void orc_matvec(const uint16_t* W, int rows, int cols, const float* x, float* y, int n_threads) {
  if (n_threads <= 1 || rows < 64) {
    matvec_rows(W, 0, rows, cols, x, y);
    return;
  }
  int nb = n_threads * 4;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
  for (int b = 0; b < nb; ++b) {
    int r0 = (int)((int64_t)rows * b / nb), r1 = (int)((int64_t)rows * (b + 1) / nb);
    matvec_rows(W, r0, r1, cols, x, y);
  }
}

/* ------------------------------------------------------------------ */
/* RMSNorm (Mirage article, "Case 1": the norm divides x by the root   */
/* mean square; the weight gamma scales each element).                 */
/*   y_i = (x_i * (1 / sqrt(mean(x^2) + eps))) * gamma_i               */
/* ------------------------------------------------------------------ */
void orc_rmsnorm(const float* x, const uint16_t* gamma, int n, float eps, float* y) {
  float ss = 0.0f;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  float r = 1.0f / sqrtf(ss / (float)n + eps);
  for (int i = 0; i < n; ++i) y[i] = (x[i] * r) * orc_bf16_to_f32(gamma[i]);
}

/* ------------------------------------------------------------------ */
/* Rotary position embedding, rotate-half pairing (i, i + d/2) with    */
/* frequency theta^(-2i/d).  Angle, cos and sin in fp64, then rounded  */
/* to fp32; the rotation itself in fp32.                               */
/* ------------------------------------------------------------------ */
void orc_rope(float* x, int d, int pos, double theta) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
    double ang = (double)pos * inv_freq;
    float c = (float)cos(ang), s = (float)sin(ang);
    float x0 = x[i], x1 = x[i + half];
    x[i] = x0 * c - x1 * s;
    x[i + half] = x0 * s + x1 * c;
  }
}

/* ------------------------------------------------------------------ */
/* Attention for one query head (Mirage article, attention example:   */
/* A = Q K, S = softmax(A), O = S V), with the usual 1/sqrt(d) scale.  */
/* Softmax subtracts the row max before exponentiating.                */
/* ------------------------------------------------------------------ */
void orc_attend(const float* q, const uint16_t* K, const uint16_t* V, int n, int d, int ld, float* out) {
  float* s = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  float scale = (float)(1.0 / sqrt((double)d));
  float m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    const uint16_t* kj = K + (size_t)j * ld;
    float dot = 0.0f;
    for (int c = 0; c < d; ++c) dot += q[c] * orc_bf16_to_f32(kj[c]);
    s[j] = dot * scale;
    if (s[j] > m) m = s[j];
  }
  float l = 0.0f;
  for (int j = 0; j < n; ++j) {
    s[j] = expf(s[j] - m);
    l += s[j];
  }
  for (int j = 0; j < n; ++j) s[j] = s[j] / l;
  for (int c = 0; c < d; ++c) {
    float o = 0.0f;
    for (int j = 0; j < n; ++j) o += s[j] * orc_bf16_to_f32(V[(size_t)j * ld + c]);
    out[c] = o;
  }
  free(s);
}

/* SiLU of the gated MLP (Mirage article, "Case 3: Gated MLP"). */
float orc_silu(float z) { return z / (1.0f + expf(-z)); }

int orc_argmax(const float* x, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i;
  return best;
}

/* ------------------------------------------------------------------ */
/* Model and sequences                                                  */
/* ------------------------------------------------------------------ */
struct orc_model {
  orc_cfg c;
  const uint16_t* const* w; /* canonical order */
  int n_w;
};

struct orc_seq {
  orc_model* m;
  int pos;
  uint16_t* K; /* [L][max_seq][Hkv*D] */
  uint16_t* V;
};

static int per_layer(const orc_cfg* c) { return 9 + (c->qk_norm ? 2 : 0); }

int orc_n_weights(const orc_cfg* c) { return 1 + c->n_layers * per_layer(c) + 2; }

int64_t orc_weight_numel(const orc_cfg* c, int i) {
  int64_t H = c->hidden, QD = (int64_t)c->n_q_heads * c->head_dim, KD = (int64_t)c->n_kv_heads * c->head_dim;
  int64_t F = c->ffn, Vv = c->vocab, D = c->head_dim;
  int n = orc_n_weights(c);
  if (i < 0 || i >= n) return -1;
  if (i == 0) return Vv * H;           /* embed */
  if (i == n - 2) return H;            /* final_norm */
  if (i == n - 1) return Vv * H;       /* lm_head */
  int j = (i - 1) % per_layer(c);
  if (!c->qk_norm && j >= 5) j += 2;   /* skip q_norm, k_norm slots */
  switch (j) {
    case 0: return H;        /* attn_norm */
    case 1: return QD * H;   /* wq */
    case 2: return KD * H;   /* wk */
    case 3: return KD * H;   /* wv */
    case 4: return H * QD;   /* wo */
    case 5: return D;        /* q_norm */
    case 6: return D;        /* k_norm */
    case 7: return H;        /* ffn_norm */
    case 8: return F * H;    /* w_gate */
    case 9: return F * H;    /* w_up */
    case 10: return H * F;   /* w_down */
  }
  return -1;
}

orc_model* orc_create(const orc_cfg* cfg, const uint16_t* const* weights, int n) {
  if (!cfg || !weights || n != orc_n_weights(cfg)) return NULL;
  if (cfg->n_q_heads % cfg->n_kv_heads != 0 || cfg->head_dim % 2 != 0) return NULL;
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  m->c = *cfg;
  m->w = weights;
  m->n_w = n;
  return m;
}

void orc_destroy(orc_model* m) { free(m); }

orc_seq* orc_seq_create(orc_model* m) {
  orc_seq* s = (orc_seq*)calloc(1, sizeof(orc_seq));
  size_t n = (size_t)m->c.n_layers * m->c.max_seq * m->c.n_kv_heads * m->c.head_dim;
  s->m = m;
  s->K = (uint16_t*)calloc(n, 2);
  s->V = (uint16_t*)calloc(n, 2);
  if (!s->K || !s->V) { free(s->K); free(s->V); free(s); return NULL; }
  return s;
}

void orc_seq_destroy(orc_seq* s) {
  if (!s) return;
  free(s->K);
  free(s->V);
  free(s);
}

int orc_seq_pos(const orc_seq* s) { return s->pos; }

int orc_seq_set_kv(orc_seq* s, int n_pos, const uint16_t* k, const uint16_t* v) {
  const orc_cfg* c = &s->m->c;
  if (n_pos < 0 || n_pos > c->max_seq) return -1;
  size_t row = (size_t)c->n_kv_heads * c->head_dim;
  for (int l = 0; l < c->n_layers; ++l) {
    memcpy(s->K + (size_t)l * c->max_seq * row, k + (size_t)l * n_pos * row, (size_t)n_pos * row * 2);
    memcpy(s->V + (size_t)l * c->max_seq * row, v + (size_t)l * n_pos * row, (size_t)n_pos * row * 2);
  }
  s->pos = n_pos;
  return 0;
}

int orc_seq_step(orc_seq* s, int token, float* logits) {
  const orc_cfg* c = &s->m->c;
  const uint16_t* const* W = s->m->w;
  const int H = c->hidden, D = c->head_dim, Hq = c->n_q_heads, Hkv = c->n_kv_heads, F = c->ffn;
  const int G = Hq / Hkv, QD = Hq * D, KD = Hkv * D, nt = c->n_threads;
  const int pos = s->pos;
  if (pos >= c->max_seq || token < 0 || token >= c->vocab) return -1;

  float* x = (float*)malloc(sizeof(float) * H);
  float* h = (float*)malloc(sizeof(float) * (H > F ? H : F));
  float* q = (float*)malloc(sizeof(float) * QD);
  float* k = (float*)malloc(sizeof(float) * KD);
  float* v = (float*)malloc(sizeof(float) * KD);
  float* o = (float*)malloc(sizeof(float) * QD);
  float* t = (float*)malloc(sizeof(float) * H);
  float* gt = (float*)malloc(sizeof(float) * F);
  float* up = (float*)malloc(sizeof(float) * F);
  float* tmp = (float*)malloc(sizeof(float) * D);

  /* embedding lookup */
  for (int i = 0; i < H; ++i) x[i] = orc_bf16_to_f32(W[0][(size_t)token * H + i]);

  const int pl = per_layer(c);
  for (int l = 0; l < c->n_layers; ++l) {
    const uint16_t* const* Lw = W + 1 + l * pl;
    const uint16_t *attn_norm = Lw[0], *wq = Lw[1], *wk = Lw[2], *wv = Lw[3], *wo = Lw[4];
    const uint16_t *q_norm = c->qk_norm ? Lw[5] : NULL, *k_norm = c->qk_norm ? Lw[6] : NULL;
    const int b = c->qk_norm ? 7 : 5;
    const uint16_t *ffn_norm = Lw[b], *wg = Lw[b + 1], *wu = Lw[b + 2], *wd = Lw[b + 3];

    /* attention sublayer */
    orc_rmsnorm(x, attn_norm, H, c->rms_eps, h);
    orc_matvec(wq, QD, H, h, q, nt);
    orc_matvec(wk, KD, H, h, k, nt);
    orc_matvec(wv, KD, H, h, v, nt);
    for (int hh = 0; hh < Hq; ++hh) {
      if (c->qk_norm) {
        orc_rmsnorm(q + hh * D, q_norm, D, c->rms_eps, tmp);
        memcpy(q + hh * D, tmp, sizeof(float) * D);
      }
      orc_rope(q + hh * D, D, pos, c->rope_theta);
    }
    for (int g = 0; g < Hkv; ++g) {
      if (c->qk_norm) {
        orc_rmsnorm(k + g * D, k_norm, D, c->rms_eps, tmp);
        memcpy(k + g * D, tmp, sizeof(float) * D);
      }
      orc_rope(k + g * D, D, pos, c->rope_theta);
    }
    uint16_t* Kl = s->K + (size_t)l * c->max_seq * KD;
    uint16_t* Vl = s->V + (size_t)l * c->max_seq * KD;
    for (int i = 0; i < KD; ++i) {
      Kl[(size_t)pos * KD + i] = orc_f32_to_bf16(k[i]);
      Vl[(size_t)pos * KD + i] = orc_f32_to_bf16(v[i]);
    }
    for (int hh = 0; hh < Hq; ++hh) {
      int g = hh / G; /* consecutive query heads share one KV head */
      orc_attend(q + hh * D, Kl + g * D, Vl + g * D, pos + 1, D, KD, o + hh * D);
    }
    orc_matvec(wo, H, QD, o, t, nt);
    for (int i = 0; i < H; ++i) x[i] = x[i] + t[i];

    /* MLP sublayer */
    orc_rmsnorm(x, ffn_norm, H, c->rms_eps, h);
    orc_matvec(wg, F, H, h, gt, nt);
    orc_matvec(wu, F, H, h, up, nt);
    for (int i = 0; i < F; ++i) gt[i] = orc_silu(gt[i]) * up[i];
    orc_matvec(wd, H, F, gt, t, nt);
    for (int i = 0; i < H; ++i) x[i] = x[i] + t[i];
  }

  if (logits) {
    const int n = orc_n_weights(c);
    orc_rmsnorm(x, W[n - 2], H, c->rms_eps, h);
    orc_matvec(W[n - 1], c->vocab, H, h, logits, nt);
  }
  s->pos = pos + 1;
  free(x); free(h); free(q); free(k); free(v); free(o); free(t); free(gt); free(up); free(tmp);
  return 0;
}
