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
 * Precision.  The decoder's stored activations are fp32: the residual
 * stream x, the raw q/k/v projections, each attention head's output o, the
 * SwiGLU output a and the logits.  Weights and the KV cache are bf16.  Every
 * operator computes its result in fp64 from those stored inputs (sums
 * sequential in ascending index) and rounds once, to fp32, where the decoder
 * stores it; the rotated key is such an fp32 value before its bf16 rounding
 * for the cache.  Build with -ffp-contract=off and without -ffast-math so
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
/* sequential fp64 sum over k = 0..cols-1; every product of a bf16     */
/* weight and an input is exact in fp64.  Four rows are walked side by */
/* side for instruction-level parallelism; no row's sum is split or    */
/* reordered.  With n_threads > 1 disjoint row blocks go to threads,   */
/* which cannot change any result.                                     */
/* ------------------------------------------------------------------ */
static void matvec_rows(const uint16_t* W, int r0, int r1, int cols, const double* x, double* y) {
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    const uint16_t* w0 = W + (size_t)r * cols;
    const uint16_t* w1 = w0 + cols;
    const uint16_t* w2 = w1 + cols;
    const uint16_t* w3 = w2 + cols;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    for (int k = 0; k < cols; ++k) {
      double xk = x[k];
      a0 += (double)orc_bf16_to_f32(w0[k]) * xk;
      a1 += (double)orc_bf16_to_f32(w1[k]) * xk;
      a2 += (double)orc_bf16_to_f32(w2[k]) * xk;
      a3 += (double)orc_bf16_to_f32(w3[k]) * xk;
    }
    y[r] = a0; y[r + 1] = a1; y[r + 2] = a2; y[r + 3] = a3;
  }
  for (; r < r1; ++r) {
    const uint16_t* w = W + (size_t)r * cols;
    double a = 0.0;
    for (int k = 0; k < cols; ++k) a += (double)orc_bf16_to_f32(w[k]) * x[k];
    y[r] = a;
  }
}

void orc_matvec(const uint16_t* W, int rows, int cols, const double* x, double* y, int n_threads) {
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
/* LoRA-adapted linear layer (Mirage article, "Case 2: LoRA + Linear"): */
/* y = W x + B (A x), taken in the concatenated form the article gives, */
/* (W|B) times (x|A x).  The low-rank projection u = A x is summed in   */
/* fp64 and materialised as fp32 (the second half of the concatenated   */
/* operand); each output row is then one sequential fp64 sum over its   */
/* concatenated row: the cols products of W with x, followed by the r   */
/* products of B with u.                                                */
/* ------------------------------------------------------------------ */
void orc_lora_linear(const uint16_t* W, const uint16_t* A, const uint16_t* B, int rows, int cols, int r,
                     const double* x, double* y, int n_threads) {
  orc_matvec(W, rows, cols, x, y, n_threads);
  if (!A || !B || r <= 0) return;
  double* ud = (double*)malloc(sizeof(double) * r);
  matvec_rows(A, 0, r, cols, x, ud);
  for (int j = 0; j < r; ++j) ud[j] = (double)(float)ud[j];
  for (int i = 0; i < rows; ++i) {
    const uint16_t* b = B + (size_t)i * r;
    double a = y[i];
    for (int j = 0; j < r; ++j) a += (double)orc_bf16_to_f32(b[j]) * ud[j];
    y[i] = a;
  }
  free(ud);
}

/* ------------------------------------------------------------------ */
/* RMSNorm (Mirage article, "Case 1": the norm divides x by the root   */
/* mean square; the weight gamma scales each element), in fp64:        */
/*   y_i = x_i * (1 / sqrt(mean(x^2) + eps)) * gamma_i                 */
/* ------------------------------------------------------------------ */
void orc_rmsnorm(const float* x, const uint16_t* gamma, int n, float eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
  double r = 1.0 / sqrt(ss / (double)n + (double)eps);
  for (int i = 0; i < n; ++i) y[i] = (double)x[i] * r * (double)orc_bf16_to_f32(gamma[i]);
}

/* ------------------------------------------------------------------ */
/* Rotary position embedding, rotate-half pairing (i, i + d/2) with    */
/* frequency theta^(-2i/d); angle, cos, sin and the rotation in fp64.  */
/* ------------------------------------------------------------------ */
void orc_rope(double* x, int d, int pos, double theta) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
    double ang = (double)pos * inv_freq;
    double c = cos(ang), s = sin(ang);
    double x0 = x[i], x1 = x[i + half];
    x[i] = x0 * c - x1 * s;
    x[i + half] = x0 * s + x1 * c;
  }
}

/* ------------------------------------------------------------------ */
/* Attention for one query head (Mirage article, attention example:   */
/* A = Q K, S = softmax(A), O = S V), with the usual 1/sqrt(d) scale.  */
/* Softmax subtracts the row max before exponentiating.  All in fp64;  */
/* the head's output is rounded once to fp32:                           */
/*   o_c = (sum_j e^{s_j - m} v_jc) / (sum_j e^{s_j - m})              */
/* ------------------------------------------------------------------ */
void orc_attend(const double* q, const uint16_t* K, const uint16_t* V, int n, int d, int ld, float* out) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double scale = 1.0 / sqrt((double)d);
  double m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    const uint16_t* kj = K + (size_t)j * ld;
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += q[c] * (double)orc_bf16_to_f32(kj[c]);
    s[j] = dot * scale;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int j = 0; j < n; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  for (int c = 0; c < d; ++c) {
    double o = 0.0;
    for (int j = 0; j < n; ++j) o += s[j] * (double)orc_bf16_to_f32(V[(size_t)j * ld + c]);
    out[c] = (float)(o / l);
  }
  free(s);
}

/* SiLU of the gated MLP (Mirage article, "Case 3: Gated MLP"), fp64. */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

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

static int n_base(const orc_cfg* c) { return 1 + c->n_layers * per_layer(c) + 2; }
enum { LORA_PER_LAYER = 14 }; /* lora_a and lora_b of q, k, v, o, gate, up, down */

int orc_n_weights(const orc_cfg* c) { return n_base(c) + (c->lora_rank > 0 ? c->n_layers * LORA_PER_LAYER : 0); }

/* input and output width of adapter target t (q, k, v, o, gate, up, down) */
static void lora_dims(const orc_cfg* c, int t, int64_t* in, int64_t* out) {
  const int64_t H = c->hidden, QD = (int64_t)c->n_q_heads * c->head_dim, KD = (int64_t)c->n_kv_heads * c->head_dim;
  const int64_t F = c->ffn;
  const int64_t ins[7] = {H, H, H, QD, H, H, F}, outs[7] = {QD, KD, KD, H, F, F, H};
  *in = ins[t];
  *out = outs[t];
}

int64_t orc_weight_numel(const orc_cfg* c, int i) {
  int64_t H = c->hidden, QD = (int64_t)c->n_q_heads * c->head_dim, KD = (int64_t)c->n_kv_heads * c->head_dim;
  int64_t F = c->ffn, Vv = c->vocab, D = c->head_dim;
  int n = n_base(c);
  if (i < 0 || i >= orc_n_weights(c)) return -1;
  if (i >= n) { /* LoRA adapters */
    const int j = (i - n) % LORA_PER_LAYER;
    int64_t in, out;
    lora_dims(c, j / 2, &in, &out);
    return (int64_t)c->lora_rank * (j % 2 ? out : in);
  }
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
  const int HF = H > F ? H : F;

  /* stored activations (fp32) */
  float* x = (float*)malloc(sizeof(float) * H);
  float* q = (float*)malloc(sizeof(float) * QD);
  float* k = (float*)malloc(sizeof(float) * KD);
  float* v = (float*)malloc(sizeof(float) * KD);
  float* o = (float*)malloc(sizeof(float) * QD);
  float* a = (float*)malloc(sizeof(float) * F);
  /* intermediates (fp64) */
  double* h = (double*)malloc(sizeof(double) * HF);
  double* y = (double*)malloc(sizeof(double) * (QD > HF ? QD : HF));
  double* gt = (double*)malloc(sizeof(double) * F);
  double* up = (double*)malloc(sizeof(double) * F);
  double* qh = (double*)malloc(sizeof(double) * QD);
  double* kh = (double*)malloc(sizeof(double) * D);

  /* embedding lookup */
  for (int i = 0; i < H; ++i) x[i] = orc_bf16_to_f32(W[0][(size_t)token * H + i]);

  const int pl = per_layer(c), r = c->lora_rank;
  for (int l = 0; l < c->n_layers; ++l) {
    const uint16_t* const* Lw = W + 1 + l * pl;
    /* adapter t of this layer: A = La[2 t], B = La[2 t + 1] (none without LoRA) */
    const uint16_t* const* La = r > 0 ? W + n_base(c) + l * LORA_PER_LAYER : NULL;
#define LA(t) (La ? La[2 * (t)] : NULL)
#define LB(t) (La ? La[2 * (t) + 1] : NULL)
    const uint16_t *attn_norm = Lw[0], *wq = Lw[1], *wk = Lw[2], *wv = Lw[3], *wo = Lw[4];
    const uint16_t *q_norm = c->qk_norm ? Lw[5] : NULL, *k_norm = c->qk_norm ? Lw[6] : NULL;
    const int b = c->qk_norm ? 7 : 5;
    const uint16_t *ffn_norm = Lw[b], *wg = Lw[b + 1], *wu = Lw[b + 2], *wd = Lw[b + 3];

    /* attention sublayer: q, k, v stored in fp32 */
    orc_rmsnorm(x, attn_norm, H, c->rms_eps, h);
    orc_lora_linear(wq, LA(0), LB(0), QD, H, r, h, y, nt);
    for (int i = 0; i < QD; ++i) q[i] = (float)y[i];
    orc_lora_linear(wk, LA(1), LB(1), KD, H, r, h, y, nt);
    for (int i = 0; i < KD; ++i) k[i] = (float)y[i];
    orc_lora_linear(wv, LA(2), LB(2), KD, H, r, h, y, nt);
    for (int i = 0; i < KD; ++i) v[i] = (float)y[i];
    /* per-head QK-norm and RoPE in fp64 */
    for (int hh = 0; hh < Hq; ++hh) {
      if (c->qk_norm) orc_rmsnorm(q + hh * D, q_norm, D, c->rms_eps, qh + hh * D);
      else for (int i = 0; i < D; ++i) qh[hh * D + i] = (double)q[hh * D + i];
      orc_rope(qh + hh * D, D, pos, c->rope_theta);
    }
    uint16_t* Kl = s->K + (size_t)l * c->max_seq * KD;
    uint16_t* Vl = s->V + (size_t)l * c->max_seq * KD;
    for (int g = 0; g < Hkv; ++g) {
      if (c->qk_norm) orc_rmsnorm(k + g * D, k_norm, D, c->rms_eps, kh);
      else for (int i = 0; i < D; ++i) kh[i] = (double)k[g * D + i];
      orc_rope(kh, D, pos, c->rope_theta);
      /* the rotated key is an fp32 value; the cache holds it, and v, in bf16 */
      for (int i = 0; i < D; ++i) {
        Kl[(size_t)pos * KD + g * D + i] = orc_f32_to_bf16((float)kh[i]);
        Vl[(size_t)pos * KD + g * D + i] = orc_f32_to_bf16(v[g * D + i]);
      }
    }
    for (int hh = 0; hh < Hq; ++hh) {
      int g = hh / G; /* consecutive query heads share one KV head */
      orc_attend(qh + hh * D, Kl + g * D, Vl + g * D, pos + 1, D, KD, o + hh * D);
    }
    for (int i = 0; i < QD; ++i) qh[i] = (double)o[i];
    orc_lora_linear(wo, LA(3), LB(3), H, QD, r, qh, y, nt);
    for (int i = 0; i < H; ++i) x[i] = (float)((double)x[i] + y[i]);

    /* MLP sublayer */
    orc_rmsnorm(x, ffn_norm, H, c->rms_eps, h);
    orc_lora_linear(wg, LA(4), LB(4), F, H, r, h, gt, nt);
    orc_lora_linear(wu, LA(5), LB(5), F, H, r, h, up, nt);
    for (int i = 0; i < F; ++i) a[i] = (float)(orc_silu(gt[i]) * up[i]);
    for (int i = 0; i < F; ++i) h[i] = (double)a[i];
    orc_lora_linear(wd, LA(6), LB(6), H, F, r, h, y, nt);
    for (int i = 0; i < H; ++i) x[i] = (float)((double)x[i] + y[i]);
#undef LA
#undef LB
  }

  if (logits) {
    const int n = n_base(c);
    double* lg = (double*)malloc(sizeof(double) * c->vocab);
    orc_rmsnorm(x, W[n - 2], H, c->rms_eps, h);
    orc_matvec(W[n - 1], c->vocab, H, h, lg, nt);
    for (int i = 0; i < c->vocab; ++i) logits[i] = (float)lg[i];
    free(lg);
  }
  s->pos = pos + 1;
  free(x); free(q); free(k); free(v); free(o); free(a);
  free(h); free(y); free(gt); free(up); free(qh); free(kh);
  return 0;
}
