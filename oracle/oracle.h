/*
 * oracle.h -- plain CPU reference decoder (TEST INFRASTRUCTURE ONLY).
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product path never calls it.
 *
 * What it computes: autoregressive greedy decode of a Llama-style decoder
 * (RMSNorm, Q/K/V projections, optional per-head QK RMSNorm, rotate-half
 * RoPE, bf16 KV cache append, grouped-query softmax attention, O-projection
 * with residual, SwiGLU MLP with residual, final norm, LM head, argmax).
 * Sources: the decode step listed by the MPK digest (fr.news.hada.io, "Part 1.
 * Compilateur" and "Part 2. Runtime": the operators a decode task graph is
 * built from); the Mirage article (iaiol.com, "Case 1: Normalization +
 * Linear" for RMSNorm, "Case 3: Gated MLP" for SwiGLU, "Case 4.1" for QK-Norm,
 * and the attention example matmul -> softmax -> matmul).
 *
 * Arithmetic: stored activations (residual stream, raw q/k/v, attention
 * output, SwiGLU output, logits) are fp32; bf16 weights are widened exactly.
 * Every operator evaluates in fp64 from its stored inputs -- dot products
 * summed sequentially in ascending index (no reassociation, built with
 * -ffp-contract=off), RMSNorm, RoPE (angles, cos, sin and rotation), softmax
 * with exp, SiLU -- and rounds once to fp32 where the result is stored.  The
 * KV cache holds the fp32 rotated key and the fp32 value rounded to bf16
 * (round to nearest even).
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;
  double rope_theta;
  int qk_norm;   /* 1: per-head RMSNorm of q and k before RoPE */
  int max_seq;   /* KV capacity in positions */
  int n_threads; /* >1 splits independent output rows across threads; results are identical */
  int lora_rank; /* r > 0: a LoRA adapter (A [r][in], B [out][r]) on every projection of every layer */
} orc_cfg;

typedef struct orc_model orc_model;
typedef struct orc_seq orc_seq;

/* Number of weight tensors in canonical order for this config.  With lora_rank > 0 the base
 * tensors are followed, per layer, by lora_a and lora_b of q, k, v, o, gate, up, down in that
 * order (14 tensors per layer). */
int orc_n_weights(const orc_cfg* cfg);
/* Element count of canonical tensor i. */
int64_t orc_weight_numel(const orc_cfg* cfg, int i);
/* weights[i]: bf16 bit patterns of canonical tensor i; the model keeps the
 * pointers (caller keeps ownership and must keep them alive). */
orc_model* orc_create(const orc_cfg* cfg, const uint16_t* const* weights, int n);
void orc_destroy(orc_model* m);

orc_seq* orc_seq_create(orc_model* m);
void orc_seq_destroy(orc_seq* s);
/* Load n_pos cached positions; k and v are bf16 [n_layers][n_pos][n_kv_heads*head_dim]
 * (keys already rotated).  Sets the position to n_pos.  Returns 0 or -1. */
int orc_seq_set_kv(orc_seq* s, int n_pos, const uint16_t* k, const uint16_t* v);
int orc_seq_pos(const orc_seq* s);
/* One decode step: consumes `token` at the current position, appends its K/V,
 * advances the position.  If logits != NULL, writes [vocab] fp32 logits.
 * Returns 0, or -1 if the cache is full / token out of range. */
int orc_seq_step(orc_seq* s, int token, float* logits);

/* ---- the primitives the decoder is made of (exported so tests can pin them) ---- */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);
/* y[r] = sum_k W[r][k] * x[k] in fp64, W bf16 [rows][cols] */
void orc_matvec(const uint16_t* W, int rows, int cols, const double* x, double* y, int n_threads);
/* y = W x + B (A x), W bf16 [rows][cols], A bf16 [r][cols], B bf16 [rows][r]: u = A x in fp64
 * stored as fp32, then each row one sequential fp64 sum over the concatenated row (W|B) against
 * (x|u).  A == NULL or B == NULL or r == 0: y = W x exactly as orc_matvec. */
void orc_lora_linear(const uint16_t* W, const uint16_t* A, const uint16_t* B, int rows, int cols, int r,
                     const double* x, double* y, int n_threads);
/* y = x * (1/sqrt(mean(x^2)+eps)) * gamma, in fp64 */
void orc_rmsnorm(const float* x, const uint16_t* gamma, int n, float eps, double* y);
/* rotate-half RoPE of one head vector of length d at position pos, in place, fp64 */
void orc_rope(double* x, int d, int pos, double theta);
/* single-head softmax attention over n cached bf16 keys/values (row stride ld),
 * evaluated in fp64; the output is rounded to fp32 */
void orc_attend(const double* q, const uint16_t* K, const uint16_t* V, int n, int d, int ld, float* out);
double orc_silu(double z);
/* index of the largest value, lowest index on ties */
int orc_argmax(const float* x, int n);

#ifdef __cplusplus
}
#endif
#endif
