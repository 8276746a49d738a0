/*
 * mk.h -- C ABI of the persistent decode megakernel library (libmk.so).
 *
 * The library runs greedy autoregressive decode of a Llama-style decoder on
 * one MI355X (gfx950) GPU.  Each decode step is lowered, once, by a host-side
 * builder to a fine-grained task graph: every operator becomes row tiles
 * ("tasks"), and tasks are joined by events that fire when a counter of
 * completed producers reaches a threshold.  This is the compiler / runtime
 * split described in the MPK digest (fr.news.hada.io, "Part 1. Compilateur"
 * and "Part 2. Runtime", "Exécution pilotée par événements").  The runtime
 * is one persistent kernel whose workgroups (one per compute unit) each walk
 * a static, pre-planned task list, the schedule being fixed ahead of time as
 * in Ada-MK (gist.science, "L'Itinéraire Pré-planifié").  A second mode
 * launches the same tasks as one kernel per operator, to measure what the
 * single persistent kernel removes.
 *
 * Conventions for every call:
 *  - Return value: MK_OK (0) or a negative MK_ERR_* code; no call throws.
 *    After a failure, mk_last_error(ctx) describes it.
 *  - A context is used by one host thread at a time.
 *  - Device pointers are HIP device addresses on the context's device;
 *    host pointers are ordinary host memory.  Ownership never transfers:
 *    the library copies what it needs and never frees caller memory.
 *  - Work is ordered on the context's stream (cfg.stream, or the null
 *    stream); calls that produce results synchronise that stream before
 *    returning.
 *  - Layouts are row-major; bf16 values are raw 16-bit patterns.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------ */
#define MK_OK 0
#define MK_ERR_INVALID_ARG (-1) /* bad pointer, size, name, shape or value */
#define MK_ERR_UNSUPPORTED (-2) /* shape or batch this build cannot tile  */
#define MK_ERR_OOM (-3)         /* device or host allocation failed       */
#define MK_ERR_HIP (-4)         /* a HIP runtime call failed              */
#define MK_ERR_CAPACITY (-5)    /* a position would exceed max_seq        */
#define MK_ERR_TIMEOUT (-6)     /* an event wait exceeded its poll budget */
#define MK_ERR_STATE (-7)       /* call out of order (e.g. no weights)    */

/* ---- execution modes ---------------------------------------------------- */
#define MK_MODE_MEGAKERNEL 0 /* one persistent cooperative launch per mk_decode */
#define MK_MODE_PER_OP 1     /* ablation: one kernel launch per operator        */

/* ---- prefill modes ---------------------------------------------------------- */
#define MK_PREFILL_PER_OP 0     /* one launch per operator per prompt token            */
#define MK_PREFILL_MEGAKERNEL 1 /* one persistent launch per sequence, chunk of tokens
                                   per step as the columns of every projection         */

/* ---- schedules ------------------------------------------------------------ */
#define MK_SCHEDULE_FROZEN 0 /* the schedule the offline search froze for this case */
#define MK_SCHEDULE_GIVEN 1  /* the schedule fields of mk_model_cfg, as given        */

/* ---- model / runtime configuration (plain data, copied by mk_create) ---- */
typedef struct mk_model_cfg {
  int32_t n_layers;   /* decoder layers L                                   */
  int32_t hidden;     /* model width H                                      */
  int32_t n_q_heads;  /* query heads Hq                                     */
  int32_t n_kv_heads; /* key/value heads Hkv (Hq % Hkv == 0)                */
  int32_t head_dim;   /* D, even, multiple of 8, <= 256                     */
  int32_t ffn;        /* SwiGLU width F                                     */
  int32_t vocab;      /* V                                                  */
  float rms_eps;      /* RMSNorm epsilon                                    */
  double rope_theta;  /* RoPE base                                          */
  int32_t qk_norm;    /* 1: per-head RMSNorm of q and k before RoPE         */
  int32_t batch;      /* B independent sequences decoded together           */
  int32_t max_seq;    /* KV capacity in positions per sequence              */
  int32_t mode;       /* MK_MODE_*                                          */
  int32_t split;      /* KV positions per attention task; 0 = default rule   */
  int32_t n_workers;  /* persistent workgroups; 0 = one per compute unit    */
  uint32_t watchdog_polls; /* max polls of one event wait; 0 = default     */
  void* stream;       /* hipStream_t the library launches on, or NULL       */
  /* Schedule of the task graph (Ada-MK, gist.science, "L'Itinéraire
   * Pré-planifié": searched offline, then fixed).  With schedule ==
   * MK_SCHEDULE_FROZEN the fields below are ignored and the builder takes
   * the entry the offline search froze for this shape, batch, worker count
   * and max_seq (csrc/schedule_table.inc), else the plain rules; split > 0
   * still overrides the split.  With MK_SCHEDULE_GIVEN they are used as
   * given, 0 in a tile count meaning the plain rule.  All must be >= 0. */
  int32_t schedule;   /* MK_SCHEDULE_*                                      */
  int32_t qkv_tiles;  /* QKV tiles per KV-head group (at most workers / Hkv) */
  int32_t wo_tiles, gu_tiles, down_tiles, lm_tiles; /* tiles per operator (<= workers) */
  int32_t rotate;     /* tile i of a layer's k-th GEMV operator (QKV 0, WO 1,
                         gate/up 2, down 3; LM head 4) runs on worker
                         (i + k * rotate) mod workers                        */
  int32_t attn_offset; /* attention task k runs on worker (k + attn_offset) mod workers */
  int32_t wo_ksplit, down_ksplit; /* batch >= 8: the O- and down-projection tiles come in
                         groups of ksplit tasks sharing a row range, each taking a part of K;
                         the last adds the others' partial sums in order.  0: the plain rule
                         (batch >= 8: the larger of 4 and 2 that is at most K / 2048 rounded up
                         and divides the tile count; batch 2 and 4: the fewest of 1, 2, 4, 8
                         parts whose fp64 staging of every sequence fits 128 KB, the next that
                         divides the tile count; batch 1, LoRA: none); 1: none; else 2, 4 or 8,
                         dividing the tile count (batch >= 8: at most K / 2048 rounded up) */
  int32_t qkv_ksplit; /* batch >= 8 only: the same for the QKV tiles of each KV-head group (the
                         parts also pass on their sums of squares for the RMSNorm scale).  0 or
                         1: none (the plain rule; a split measured slower); else 2, 4 or 8,
                         dividing the tiles per group, at most hidden / 2048 rounded up */
  /* LoRA (Mirage article, "Case 2: LoRA + Linear"): rank r of an adapter
   * on every projection of every layer (q, k, v, o, gate, up, down), each
   * y = W x + B (A x) computed as one fused GEMV over the concatenation
   * (W|B)(x|A x).  0: no adapters; else a multiple of 8 up to 64, batch
   * <= 4 (UNSUPPORTED otherwise). */
  int32_t lora_rank;
  /* How mk_prefill runs the prompt (MK_PREFILL_*).  MK_PREFILL_MEGAKERNEL
   * (Ada-MK, gist.science, "La « Flotte Hybride »" keeps prefill on a
   * conventional engine; this runs it through the same task graph
   * instead): per sequence one persistent launch; step s takes prompt
   * tokens [s C, (s + 1) C) as C columns of every GEMV -- C = 16 on the
   * matrix cores where hidden, ffn and n_q_heads * head_dim are multiples
   * of 512 and there are no adapters, else 4 -- then an append task per
   * KV-head group writes their rotated keys and values, and each token
   * attends over the cache up to its own position.  mk_prefill_noalloc
   * always runs per operator. */
  int32_t prefill;
} mk_model_cfg;

typedef struct mk_ctx mk_ctx;

/* One weight tensor in canonical form.  Names and shapes (all bf16):
 *   "embed" [V,H]; per layer l, prefix "layers.<l>.":
 *   "attn_norm" [H], "wq" [Hq*D,H], "wk" [Hkv*D,H], "wv" [Hkv*D,H],
 *   "wo" [H,Hq*D], ("q_norm" [D], "k_norm" [D] when qk_norm),
 *   "ffn_norm" [H], "w_gate" [F,H], "w_up" [F,H], "w_down" [H,F];
 *   "final_norm" [H], "lm_head" [V,H].
 * With lora_rank r > 0, also per layer "lora_a.<t>" [r,in] and
 *   "lora_b.<t>" [out,r] for t in q, k, v, o, gate, up, down (in and out
 *   being the projection's input and output widths).
 * Matrices are [out, in] row-major.  data is a host pointer, or a device
 * pointer when on_device != 0. */
typedef struct mk_tensor {
  const char* name;
  const void* data;
  int64_t numel;
  int32_t on_device;
} mk_tensor;

/* Validate cfg, build the task graph (host only) and allocate every device
 * buffer: packed weights, KV cache [L][B][Hkv][max_seq][D] bf16 (K and V),
 * activations, event flags.  *out receives the context.  With cfg.split == 0
 * the attention split is S = min(Smax, max(32, ceil(max_seq / max(1, workers /
 * (batch * n_kv_heads))))) positions, Smax = 20480 / head_dim (32768 /
 * head_dim with one query head per KV head).  Where Smax caps it and the
 * attention tasks then come to at most 3 per worker, the split shrinks to
 * max(32, ceil(max_seq / n)), n the largest split count that keeps that
 * per-worker count.  An explicit split above Smax is UNSUPPORTED.  Batch 8 and
 * 16 run the
 * projections on the matrix cores and need hidden, ffn and n_q_heads *
 * head_dim to be multiples of 512.  Errors: INVALID_ARG, UNSUPPORTED (shape
 * cannot be tiled), OOM, HIP. */
int mk_create(const mk_model_cfg* cfg, mk_ctx** out);

/* Copy and repack all weights.  Exactly the canonical set must be given,
 * each with its canonical numel, in any order.  Synchronous.  Errors:
 * INVALID_ARG (missing, duplicate, unknown or misshaped tensor), HIP. */
int mk_load_weights(mk_ctx* ctx, const mk_tensor* tensors, int n);

/* Prefill every sequence with its prompt: prompts is host int32 [B][len],
 * ids in [0, V).  Positions 0..len-2 are written to the KV cache (per
 * operator: decode steps without the LM head, one launch per operator; or
 * through the megakernel, see mk_model_cfg.prefill) and prompts[b][len-1]
 * becomes the token decode step 0 consumes at position len-1.  Resets any
 * previous state.  The prompts of all sequences have the same length: the
 * sequences share one position (a sequence of its own length is installed
 * with mk_load_kv instead).  Synchronous.  Errors: INVALID_ARG, CAPACITY
 * (len > max_seq), STATE (no weights), UNSUPPORTED (megakernel prefill
 * graph), TIMEOUT, HIP. */
int mk_prefill(mk_ctx* ctx, const int32_t* prompts, int len);

/* mk_prefill for callers that cannot allocate memory (code inside a HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, results and errors, but the forced prompt tokens are
 * staged in a static device array that the library holds for the life of
 * the process (one per device, resolved at mk_create) instead of a buffer
 * the context allocates on first use.  It calls no hipMalloc or hipFree.
 * Limit: batch * (len - 1) <= 65536 tokens; a longer prompt set returns
 * MK_ERR_CAPACITY.  Every context on a device shares the array, which
 * keeps the last call's tokens: calls that overlap on one device race. */
int mk_prefill_noalloc(mk_ctx* ctx, const int32_t* prompts, int len);

/* Install a pre-filled KV cache for sequence seq: k and v are bf16
 * [L][n_pos][Hkv*D] (keys already rotated), host memory or device memory
 * (on_device != 0).  pending is the token decode step 0 consumes at
 * position n_pos.  All sequences must hold the same n_pos before
 * mk_decode.  Synchronous.  Errors: INVALID_ARG, CAPACITY, HIP. */
int mk_load_kv(mk_ctx* ctx, int seq, int n_pos, const void* k, const void* v, int32_t pending,
               int on_device);

/* Run n_steps greedy decode steps for all B sequences.  out_tokens is a
 * device int32 [n_steps][B] buffer; out_logits a device fp32
 * [n_steps][B][V] buffer or NULL.  Step i consumes the pending token at
 * position pos+i, appends its K/V, and writes logits and the argmax
 * (lowest index on ties), which becomes the next pending token.  In
 * megakernel mode this is ONE kernel launch.  Synchronous.  Errors:
 * INVALID_ARG, CAPACITY (pos + n_steps > max_seq), STATE, TIMEOUT
 * (watchdog; state is then undefined until mk_reset), HIP. */
int mk_decode(mk_ctx* ctx, int n_steps, int32_t* out_tokens, float* out_logits);

/* Switch between MK_MODE_MEGAKERNEL and MK_MODE_PER_OP; state is kept. */
int mk_set_mode(mk_ctx* ctx, int mode);

/* Choose how the next mk_prefill runs (MK_PREFILL_PER_OP or
 * MK_PREFILL_MEGAKERNEL, as mk_model_cfg.prefill).  Errors: INVALID_ARG. */
int mk_set_prefill(mk_ctx* ctx, int prefill);

/* Current position (shared by all sequences) and, if pending != NULL,
 * host int32 [B] pending tokens. */
int mk_get_state(mk_ctx* ctx, int32_t* pos, int32_t* pending);

/* Copy the context's configuration (as given to mk_create, with the mode
 * set by mk_set_mode) into *out, so that a caller can size the buffers the
 * other calls read and write.  Errors: INVALID_ARG. */
int mk_get_config(mk_ctx* ctx, mk_model_cfg* out);

/* Canonical little-endian serialisation of the decode task graph, u32 words:
 * header 'MKG1', version 3, n_workers, split, n_splits, n_events, n_tasks,
 * n_slots; per event (id, fanin, first slot); per task in topological order
 * (index, op, layer, tile, a0, a1, wait event, its fanin, wait lag, signal
 * event, signal slot, worker, LoRA unit range la0, la1, LoRA event, split-K
 * part kp and part count kn; a part below the last signals no event).  If
 * buf is NULL or *len is too small, *len receives the size needed and
 * MK_ERR_INVALID_ARG is returned when buf is non-NULL. */
int mk_get_graph(mk_ctx* ctx, void* buf, size_t* len);

/* Build the canonical graph bytes for cfg with n_workers workgroups without
 * touching any GPU (same rules as mk_create). */
int mk_build_graph(const mk_model_cfg* cfg, int n_workers, void* buf, size_t* len);

/* The same for the megakernel prefill's graph: `chunk` prompt tokens per step
 * (virtual sequences), the decode graph's `split`, an append task (op 7) per
 * (layer, KV-head group) between QKV and attention, no LM head, and layer 0
 * waiting on the last layer of the previous step.  Host only.  Errors:
 * INVALID_ARG, UNSUPPORTED. */
int mk_build_prefill_graph(const mk_model_cfg* cfg, int n_workers, int chunk, int split, void* buf, size_t* len);

/* Reset the whole context (every sequence): positions and pending tokens to
 * zero, event slots and attention partials cleared, watchdog status cleared;
 * weights, the schedule and the KV cache memory are kept (its contents become
 * unreachable: decode reads only positions written since). */
int mk_reset(mk_ctx* ctx);

/* Measured streaming-read rate of this device: a plain kernel reads a
 * zero-filled buffer of `bytes` (rounded down to a whole number of 16-byte
 * chunks per compute unit; >= 1 MiB) `iters` times with the same 16-byte
 * non-temporal loads the GEMV tasks use; *gbps receives bytes*iters/time.
 * Context-free: allocates and frees its own buffer on the current device,
 * runs on the null stream.  Errors: INVALID_ARG, OOM, HIP. */
int mk_read_bandwidth(size_t bytes, int iters, float* gbps);

/* Same, but the kernel copies the first half of the buffer into the second
 * (bytes/2 read and bytes/2 written per pass); *gbps counts read + write
 * bytes.  Serves as the known-volume kernel for byte counters. */
int mk_copy_bandwidth(size_t bytes, int iters, float* gbps);

/* Duration in milliseconds of the last mk_decode's kernel work, measured
 * with HIP events on the context's stream around the launch(es). */
int mk_last_decode_ms(mk_ctx* ctx, float* ms);

/* Tracing (diagnostics).  mk_set_trace(ctx, step) makes the next megakernel
 * mk_decode record, for decode step `step` of that call (0-based; -1
 * disables), four device wall-clock stamps per task of every worker: task
 * start, event satisfied, inputs staged (GEMV tasks) or split partial stored
 * (attention tasks), task end; 0 where a point was not reached (e.g.
 * attention splits beyond the current length).
 * mk_get_trace copies them as uint64 [n_workers][max_list][4] into out
 * (host, *len words; with out == NULL only the sizes are returned) and
 * reports the clock rate in kHz. */
int mk_set_trace(mk_ctx* ctx, int step);
int mk_get_trace(mk_ctx* ctx, uint64_t* out, size_t* len, int32_t* n_workers, int32_t* max_list,
                 int32_t* clock_khz);

/* Canary (diagnostics): fill the context's scratch -- the activations x,
 * q/k/v, o and a, the LM-head partial maxima, the step-tagged attention
 * partials and LoRA sums -- with all-ones bytes (NaN, and tags no step
 * uses).  A correct decode writes every such value before reading it, so
 * its tokens and logits are unchanged; a read before a write shows up as
 * NaN or a wait that never ends.  Event slots, the KV cache, positions and
 * pending tokens are left alone.  Synchronous.  Errors: INVALID_ARG, HIP. */
int mk_debug_poison(mk_ctx* ctx);

/* Text of the last error on ctx (or of the last failed mk_create when ctx
 * is NULL).  Owned by the library; valid until the next call on ctx. */
const char* mk_last_error(mk_ctx* ctx);

/* Free everything; NULL is a no-op. */
void mk_destroy(mk_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
