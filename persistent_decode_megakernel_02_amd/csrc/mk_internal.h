// mk_internal.h -- records shared by the host builder/runtime and the HIP kernels.
//
// Vocabulary follows the MPK digest (fr.news.hada.io, "Part 1. Compilateur"):
// a *task* is a unit of work given to one compute unit, an *event* is a
// synchronisation point between tasks, and a task waits on at most one event
// and notifies at most one.  An event fires when every producer slot holds the
// current step's value ("Exécution pilotée par événements": counters that
// reach a threshold); here each producer owns one 32-bit slot, so firing
// needs no atomic read-modify-write on a shared counter.
#pragma once
#include <stdint.h>

namespace mk {

enum Op : uint32_t {
  OP_QKV = 1,   // norm + fused Q/K/V projection rows (one KV-head group per tile)
  OP_ATTN = 2,  // QK-norm + RoPE + KV append + split-KV attention partial (+ merge)
  OP_WO = 3,    // O-projection rows + residual
  OP_GU = 4,    // norm + gate/up row pairs + SwiGLU
  OP_DOWN = 5,  // down-projection rows + residual
  OP_LM = 6,    // final norm + LM-head rows + per-tile argmax
  OP_APPEND = 7,  // prefill: QK-norm + RoPE of a KV-head group's keys for every token of the chunk, K/V append
};

constexpr uint32_t EV_NONE = 0xffffffffu;

// One task; 32 bytes on the device.
struct TaskRec {
  uint32_t op;        // Op
  uint32_t layer;     // decoder layer (0 for OP_LM)
  uint32_t tile;      // index of the task within its operator
  uint32_t a0, a1;    // GEMV: unit range [a0, a1); ATTN: a0 = b*Hkv + g, a1 = split index
  uint32_t wait_ev;   // event waited on (EV_NONE: none)
  uint32_t wait_lag;  // 1: the event belongs to the previous decode step
  uint32_t sig_ev;    // event notified (slot sig_slot)
  uint32_t sig_slot;
  // LoRA (GEMV operators of a model with adapters): the tile also computes the adapters' A rows
  // [la0, la1) of its operator and publishes their sums as words tagged with the step and lora_ev;
  // it reads all of them before its epilogue.  lora_ev, an event whose fan-in counts the tiles
  // holding A rows, names the operator's sums (their tag); no slot of it is signalled.  EV_NONE
  // without adapters.
  uint32_t la0, la1, lora_ev;
  // split-K (O- and down-projection at batch >= 8): part kp of kn of the operator's K slices for
  // the tile's rows; parts below kn - 1 publish step-tagged partial row sums, part kn - 1 adds
  // them in order of kp and signals.  kn = 1: the whole K.
  uint32_t kp, kn;
  uint32_t pad[2];
};
static_assert(sizeof(TaskRec) == 64, "TaskRec layout");

struct EventRec {
  uint32_t fanin;  // number of producer slots
  uint32_t slot0;  // first slot in the flag array
};

struct LayerW {
  const uint16_t* wqkv;  // [(Hq + 2 Hkv) D, H], rows grouped per KV head: G q heads, k, v
  const uint16_t* wo;    // [H, Hq D]
  const uint16_t* wg;    // [F, H]
  const uint16_t* wu;    // [F, H]
  const uint16_t* wd;    // [H, F]
  const uint16_t* attn_norm;  // [H]
  const uint16_t* ffn_norm;   // [H]
  const uint16_t* q_norm;     // [D] or null
  const uint16_t* k_norm;     // [D] or null
  // LoRA B matrices [rows][r] (null without adapters); the A matrices [n][K] follow the rows of
  // their weight matrix in the arena (wqkv: A_q, A_k, A_v; wo: A_o; wg: A_gate; wu: A_up; wd: A_down)
  const uint16_t* b_qkv;  // [(Hq + 2 Hkv) D][r], rows in wqkv's order
  const uint16_t* b_o;    // [H][r]
  const uint16_t* b_g;    // [F][r]
  const uint16_t* b_u;    // [F][r]
  const uint16_t* b_d;    // [H][r]
};

// What the streaming GEMV engine (batch <= 4) reads about a task, built by the host once the
// weight arena exists.  GEMV tasks stream rows w0 + r K for r < nu, then (gate/up) the up rows
// w1 + (r - nu) K for nu <= r < R.  Their input is act [B][K] (x, o or a); the activations of K
// slices of kc elements are staged as fp64 x * gamma when f64 (operators with a norm), else as
// fp32.  Attention tasks carry only op and a1 (their split), which is what the engine needs to
// skip the ones with no work.
struct SegRec {
  const uint16_t* w0;
  const uint16_t* w1;
  const uint16_t* gamma;
  const float* act;
  uint32_t op, a1;
  uint32_t K, nu, R, kc, nsl, f64;
};
static_assert(sizeof(SegRec) == 64, "SegRec layout");

struct LmPart {
  float val;
  int32_t idx;
};

// 32 bits of a value with the sequence tag of the step that wrote it, stored
// and loaded as one 64-bit word: a reader that sees the expected tag also sees
// the bits written with it.  An fp64 value is two of these (low word, high
// word).  Tag of event ev at global step n: n * ntag + ev + 1.
struct TV {
  uint32_t bits;
  uint32_t tag;
};

// status[0]: abort flag; status[1..7]: first error record
enum : uint32_t { ST_ABORT = 0, ST_CODE = 1, ST_CU = 2, ST_TASK = 3, ST_EVENT = 4, ST_SEEN = 5, ST_WANT = 6 };
constexpr uint32_t ERR_WATCHDOG = 1;

struct KParams {
  // model shape
  int32_t L, H, Hq, Hkv, D, F, V, G, RG, QKVR, QD, B, max_seq, S, NS, qk_norm;
  int32_t lora_r;  // LoRA rank (0: no adapters)
  float eps;          // RMSNorm epsilon (an fp32 value, widened to fp64 where used)
  double attn_scale;  // 1 / sqrt(D)
  // tiling
  int32_t n_workers, n_qkv, n_wo, n_gu, n_down, n_lm;
  // LDS layout of a worker: [activation staging: xs_doubles fp64][row sums: red_doubles fp64][misc]
  int32_t xs_doubles, red_doubles;
  int32_t red_off, misc_off;  // byte offsets
  int32_t mk_ks;              // B >= 8: K slice staged per pass of the matrix-core GEMV
  // B <= 4, streaming GEMV engine: two activation regions, two row-sum buffers, two residual
  // buffers (byte offsets), their capacities, and the K slice of fp64- and fp32-staged operators
  int32_t sg_rg0, sg_rg1, sg_red, sg_red_cap, sg_xold, sg_xold_cap, sg_kc64, sg_kc32;
  // weights
  const LayerW* layers;
  const uint16_t* embed;
  const uint16_t* final_norm;
  const uint16_t* lm_head;
  const double* rope_cos;  // [max_seq][D/2]
  const double* rope_sin;
  // KV cache [L][B][Hkv][max_seq][D] bf16
  uint16_t* kc;
  uint16_t* vc;
  // activations (fp32)
  float* x;         // [B][H]
  float* qkv;       // [B][QKVR]
  float* o;         // [B][QD]
  float* a;         // [B][F]
  TV* part_ml;      // [B][Hkv][NS][G][2][2] split max and sum (fp64 as two tagged words)
  TV* part_acc;     // [B][Hkv][NS][G][D][2] split unnormalised P.V (fp64 as two tagged words)
  LmPart* lm_part;    // [B][n_lm]
  TV* lora_u;         // [4 operators][B][3 r]: the adapters' A x of the current GEMV operator (fp32, step-tagged)
  TV* kpart;          // [WO, DN, QKV][max split - 1][rows + 1][16][2]: split-K partial row sums (fp64, step-tagged)
  int32_t kpart_max;  // largest split of the graph (1: none)
  // tokens
  int32_t* pending;           // [B]
  int32_t* out_tokens;        // [n_steps][B] or null
  float* out_logits;          // [n_steps][B][V] or null
  const int32_t* force_tok;   // [n_steps][B] or null (prefill)
  // graph
  uint32_t* flags;
  const EventRec* events;
  const TaskRec* tasks;
  const uint32_t* task_cu;
  const uint32_t* list_off;
  const uint32_t* list_len;
  const uint32_t* cu_tasks;
  const uint32_t* range_start;  // [n_ranges + 1][workers]: a worker's first list position per operator instance
  const SegRec* segrec;       // per task (batch <= 4)
  uint32_t* status;
  // run
  int32_t pos0, n_steps, with_lm;
  uint32_t epoch, watchdog;  // epoch: decode steps run by this context so far (any mode, prefill included)
  uint32_t lm_skip;          // steps of epoch run without the LM head (counter-form events only)
  uint32_t ntag;             // tag period: number of events
  // per-operator launch
  int32_t op_first, op_count, op_range, step;
  // prefill graph (chunk > 0): virtual sequence b of step s is token pos0 + s chunk + b of real
  // sequence kv_seq (of kvB in the cache layout); tokens at or past pos_end are padding.
  // Decode: chunk = 0, kvB = B, and virtual sequence b is cache sequence b.
  int32_t chunk, kv_seq, kvB, pos_end;
  // optional trace of one decode step: [worker][list index][4] wall-clock stamps
  uint64_t* trace;
  int32_t trace_step, trace_stride;
};

}  // namespace mk
