// api.cpp -- the C ABI of libmk.so: context lifecycle, weight packing, KV
// installation, prefill (per operator, as in Ada-MK's split between a
// conventional prefill engine and the megakernel for decode -- gist.science,
// "La « Flotte Hybride »"), decode in either execution mode, and the graph
// export used to check the builder bit for bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "graph.h"
#include "mk_internal.h"

namespace mk {
hipError_t prepare_kernels(int B);
hipError_t launch(int kind, const KParams& P, hipStream_t st);
hipError_t launch_read_probe(const void* buf, size_t bytes, int n_wg, uint32_t* out, hipStream_t st);
hipError_t launch_copy_probe(void* buf, size_t bytes, int n_wg, hipStream_t st);
size_t lds_bytes(const KParams& P);
int max_coresident_workers(int B, size_t lds);
hipError_t noalloc_token_staging(int device, int32_t** ptr);
constexpr int kNoAllocTokens = 1 << 16;  // capacity of the static token staging array (same as in kernels.hip)
constexpr int kLdsBytes = 163840;  // one worker per compute unit takes all of its LDS
constexpr int kMiscBytes = 4096;   // per-worker scalars at the top of LDS (same size as in the kernels)
constexpr int kMkSlice = 2048;     // K slice of the matrix-core GEMV (same as in the kernels)
constexpr uint32_t kDefaultWatchdog = 1u << 22;  // ~1-2 us per poll: several seconds, far above any healthy wait
}  // namespace mk

using namespace mk;

// LDS of one worker: [activation staging, fp64][GEMV row sums, fp64][misc].  Attention tasks reuse the
// space below misc for q/k/v, rotated queries, scores and per-wave P.V sums.
struct LdsPlan {
  int xs_doubles, red_doubles, red_off, misc_off;
  int mk_ks;  // batch >= 8: K slice of the matrix-core GEMV
  // batch <= 4 (streaming GEMV engine): two activation regions, two row-sum and two residual
  // buffers, and the K slices that fit a region with fp64 and with fp32 staging
  int sg_rg0, sg_rg1, sg_red, sg_red_cap, sg_xold, sg_xold_cap, sg_kc64, sg_kc32;
};

// The megakernel prefill (MK_PREFILL_MEGAKERNEL): its own graph of `chunk` virtual sequences, its
// tables, event slots and activations; the weights and the KV cache are the context's.  Built on
// first use.
struct PrefillCtx {
  bool built = false;
  Graph g;
  LdsPlan lds{};
  EventRec* d_events = nullptr;
  TaskRec* d_tasks = nullptr;
  uint32_t *d_list_off = nullptr, *d_list_len = nullptr, *d_cu_tasks = nullptr, *d_range_start = nullptr;
  uint32_t* flags = nullptr;
  float *x = nullptr, *qkv = nullptr, *o = nullptr, *a = nullptr;
  TV *part_ml = nullptr, *part_acc = nullptr, *lora_u = nullptr;
  size_t n_part_ml = 0, n_part_acc = 0, n_lora_u = 0;
  LmPart* lm_part = nullptr;
  int32_t* force = nullptr;  // [steps][chunk] prompt tokens of one sequence, padded
  size_t force_cap = 0;
  uint32_t epoch = 0;        // steps run on this graph since the last reset
};

struct mk_ctx {
  mk_model_cfg cfg{};
  LdsPlan lds{};
  Graph g;
  PrefillCtx pf;
  hipStream_t stream = nullptr;
  int device = 0;
  std::string err;
  // device memory
  std::vector<void*> allocs;
  uint16_t* warena = nullptr;
  size_t wbytes = 0;
  std::map<std::string, std::pair<size_t, int64_t>> wslots;  // canonical name -> (offset in elems, numel) for plain tensors
  LayerW* d_layers = nullptr;
  std::vector<LayerW> h_layers;
  uint16_t *embed = nullptr, *final_norm = nullptr, *lm_head = nullptr;
  double *rope_cos = nullptr, *rope_sin = nullptr;
  uint16_t *kc = nullptr, *vc = nullptr;
  size_t kv_elems = 0;
  float *x = nullptr, *qkv = nullptr, *o = nullptr, *a = nullptr;
  TV *part_ml = nullptr, *part_acc = nullptr;
  size_t n_part_ml = 0, n_part_acc = 0;
  LmPart* lm_part = nullptr;
  TV* lora_u = nullptr;  // [4][B][3 r] adapter A x of the current GEMV operator (LoRA), step-tagged
  size_t n_lora_u = 0;
  TV* kpart = nullptr;  // split-K partial row sums (and QKV sums of squares), step-tagged
  size_t n_kpart = 0;
  int kpart_max = 1;
  int32_t* pending = nullptr;
  int32_t* force = nullptr;
  size_t force_cap = 0;
  int32_t* noalloc_tokens = nullptr;  // this device's static staging array (mk_prefill_noalloc)
  uint32_t* flags = nullptr;
  uint32_t* status = nullptr;
  EventRec* d_events = nullptr;
  TaskRec* d_tasks = nullptr;
  SegRec* d_segrec = nullptr;
  uint32_t *d_task_cu = nullptr, *d_list_off = nullptr, *d_list_len = nullptr, *d_cu_tasks = nullptr;
  uint32_t* d_range_start = nullptr;
  // state
  bool have_weights = false;
  int pos = 0;
  std::vector<int> seq_pos;
  uint32_t epoch = 0;
  uint32_t lm_skip = 0;  // steps of epoch run without the LM head (prefill)
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  float last_ms = 0.f;
  // tracing
  int trace_step = -1;
  uint64_t* trace = nullptr;
  int trace_stride = 0;
};

static std::string g_create_err;

static int fail(mk_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  else g_create_err = msg;
  return code;
}

#define HIPCHK(ctx, call)                                                                           \
  do {                                                                                              \
    hipError_t e_ = (call);                                                                         \
    if (e_ != hipSuccess) return fail(ctx, MK_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

static int dalloc(mk_ctx* c, void** p, size_t bytes) {
  bytes = (bytes + 255) & ~(size_t)255;
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) return fail(c, MK_ERR_OOM, std::string("hipMalloc(") + std::to_string(bytes) + "): " + hipGetErrorString(e));
  c->allocs.push_back(*p);
  return MK_OK;
}

static std::string validate(const mk_model_cfg& cfg) {
  if (cfg.batch != 1 && cfg.batch != 2 && cfg.batch != 4 && cfg.batch != 8 && cfg.batch != 16)
    return "batch must be 1, 2, 4, 8 or 16";
  if (cfg.n_q_heads <= 0 || cfg.n_kv_heads <= 0 || cfg.n_q_heads % cfg.n_kv_heads) return "bad head counts";
  const int G = cfg.n_q_heads / cfg.n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return "query heads per KV head must be 1, 2 or 4";
  if (cfg.head_dim != 64 && cfg.head_dim != 128) return "head_dim must be 64 or 128";
  if (cfg.mode != MK_MODE_MEGAKERNEL && cfg.mode != MK_MODE_PER_OP) return "unknown mode";
  if (!(cfg.rms_eps > 0.f) || !(cfg.rope_theta > 0.0)) return "rms_eps and rope_theta must be positive";
  if (cfg.lora_rank < 0 || cfg.lora_rank > 64 || cfg.lora_rank % 8) return "lora_rank must be 0 or a multiple of 8 up to 64";
  if (cfg.prefill != MK_PREFILL_PER_OP && cfg.prefill != MK_PREFILL_MEGAKERNEL) return "unknown prefill mode";
  return "";
}

static int plan_lds(const mk_model_cfg& cfg, const Graph& g, LdsPlan* out, std::string* why) {
  const int D = cfg.head_dim, G = cfg.n_q_heads / cfg.n_kv_heads, B = cfg.batch;
  const int S = g.split;
  const int lpp = D / 8, ppb = 512 / lpp;
  if (S > (G == 1 ? 8 : 5) * ppb) {
    *why = "split too large for head_dim (at most 20480 / head_dim, 32768 / head_dim with one query head per KV head)";
    return MK_ERR_UNSUPPORTED;
  }
  // attention: raw q/k/v, rotated q, current k/v, scores, the split's values (bf16), then
  // the P.V partial sums (4 per thread) or the merge's (m, l), weights and slice of accumulators
  // (at most G D + n_splits items)
  const int64_t merge_doubles = (int64_t)3 * G * g.n_splits + (int64_t)G * D + g.n_splits;
  const int64_t att_bytes = (int64_t)(G + 2) * D * 4 + (int64_t)G * D * 8 + 2 * D * 2 + (int64_t)G * ((S + 1) & ~1) * 8 +
                            (int64_t)S * D * 2 + std::max<int64_t>(4 * 512, merge_doubles) * 8;
  auto maxrows = [](int R, int T) { return (R + T - 1) / T; };
  // with LoRA a tile also sums up to ceil(A rows / tiles) adapter rows (row pairs at gate/up)
  const int lr = cfg.lora_rank;
  // (a split-K row tile of the O- or down-projection holds ksplit tiles' rows)
  const int worst = std::max({maxrows(cfg.hidden, g.n_wo / g.wo_ksplit) + maxrows(lr, g.n_wo),
                              (maxrows(cfg.ffn, g.n_gu) + maxrows(lr, g.n_gu)) * 2,
                              maxrows(cfg.hidden, g.n_down / g.down_ksplit) + maxrows(lr, g.n_down),
                              maxrows(cfg.vocab, g.n_lm),
                              (G + 2) * D / (g.qkv_tiles_per_group / g.qkv_ksplit) + 1 + maxrows(3 * lr, g.n_qkv)});
  LdsPlan L;
  L.mk_ks = 0;
  if (B >= 8) {
    // matrix-core GEMV: passes of up to 8 row tiles (128 rows), K staged in slices of kMkSlice elements
    // as fp32 at 16 columns (64 bytes per K element), each wave taking 1/8 of a slice
    if (cfg.hidden % 512 || cfg.ffn % 512 || (cfg.n_q_heads * D) % 512) {
      *why = "batch >= 8 needs hidden, ffn and n_q_heads * head_dim to be multiples of 512";
      return MK_ERR_UNSUPPORTED;
    }
    L.red_doubles = 128 * B;
    L.misc_off = kLdsBytes - kMiscBytes;
    L.red_off = L.misc_off - L.red_doubles * 8;
    L.mk_ks = kMkSlice;
    L.xs_doubles = L.red_off / 8;
    if ((int64_t)kMkSlice * 64 > L.red_off) {
      *why = "LDS too small for the matrix-core GEMV";
      return MK_ERR_UNSUPPORTED;
    }
  } else {
    L.red_doubles = (worst * B + 1) / 2 * 2;
    L.misc_off = kLdsBytes - kMiscBytes;
    L.red_off = L.misc_off - L.red_doubles * 8;
    L.xs_doubles = L.red_off / 8;
    // streaming engine: [region 0][region 1][residual x 2][row sums x 2][misc]
    const int resid =
        std::max(maxrows(cfg.hidden, g.n_wo / g.wo_ksplit), maxrows(cfg.hidden, g.n_down / g.down_ksplit)) * B;
    L.sg_red_cap = (worst * B + 1) / 2 * 2;
    L.sg_red = (L.misc_off - 2 * L.sg_red_cap * 8) & ~15;
    L.sg_xold_cap = (resid + 3) / 4 * 4;
    L.sg_xold = (L.sg_red - 2 * L.sg_xold_cap * 4) & ~15;
    const int rg = (L.sg_xold / 2) & ~15;
    L.sg_rg0 = 0;
    L.sg_rg1 = rg;
    L.sg_kc64 = rg / (B * 8) / 512 * 512;
    L.sg_kc32 = rg / (B * 4) / 512 * 512;
    if (L.sg_kc64 < 512) {
      *why = "a GEMV tile has too many rows for LDS at this batch (use more workers or a smaller batch)";
      return MK_ERR_UNSUPPORTED;
    }
  }
  if (att_bytes > L.misc_off) {
    *why = "attention working set exceeds LDS";
    return MK_ERR_UNSUPPORTED;
  }
  *out = L;
  return MK_OK;
}

extern "C" {

int mk_build_prefill_graph(const mk_model_cfg* cfg, int n_workers, int chunk, int split, void* buf, size_t* len) {
  if (!cfg || !len) return fail(nullptr, MK_ERR_INVALID_ARG, "null argument");
  std::string why = validate(*cfg);
  if (!why.empty()) return fail(nullptr, MK_ERR_INVALID_ARG, why);
  Graph g;
  why = build_prefill_graph(*cfg, n_workers, chunk, split, &g);
  if (!why.empty()) return fail(nullptr, MK_ERR_UNSUPPORTED, why);
  std::vector<uint8_t> bytes = serialize_graph(*cfg, g);
  const size_t need = bytes.size();
  if (!buf || *len < need) {
    *len = need;
    return buf ? fail(nullptr, MK_ERR_INVALID_ARG, "buffer too small") : MK_OK;
  }
  std::memcpy(buf, bytes.data(), need);
  *len = need;
  return MK_OK;
}

int mk_build_graph(const mk_model_cfg* cfg, int n_workers, void* buf, size_t* len) {
  if (!cfg || !len) return fail(nullptr, MK_ERR_INVALID_ARG, "null argument");
  std::string why = validate(*cfg);
  if (!why.empty()) return fail(nullptr, MK_ERR_INVALID_ARG, why);
  Graph g;
  why = build_graph(*cfg, n_workers, &g);
  if (!why.empty()) return fail(nullptr, MK_ERR_UNSUPPORTED, why);
  std::vector<uint8_t> bytes = serialize_graph(*cfg, g);
  const size_t need = bytes.size();
  if (!buf || *len < need) {
    *len = need;
    return buf ? fail(nullptr, MK_ERR_INVALID_ARG, "buffer too small") : MK_OK;
  }
  std::memcpy(buf, bytes.data(), need);
  *len = need;
  return MK_OK;
}

int mk_create(const mk_model_cfg* cfg_in, mk_ctx** out) {
  if (!cfg_in || !out) return fail(nullptr, MK_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  std::string why = validate(*cfg_in);
  if (!why.empty()) return fail(nullptr, MK_ERR_INVALID_ARG, why);
  mk_ctx* c = new mk_ctx();
  c->cfg = *cfg_in;
  const mk_model_cfg& cfg = c->cfg;
  auto bail = [&](int code) {
    g_create_err = c->err;
    mk_destroy(c);
    return code;
  };
  c->stream = (hipStream_t)cfg.stream;
  if (hipGetDevice(&c->device) != hipSuccess) return bail(fail(c, MK_ERR_HIP, "hipGetDevice failed"));
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c->device) != hipSuccess) return bail(fail(c, MK_ERR_HIP, "hipGetDeviceProperties"));
  // the static token staging array of mk_prefill_noalloc: its address on this device, resolved
  // once per device and kept for the life of the process
  if (noalloc_token_staging(c->device, &c->noalloc_tokens) != hipSuccess)
    return bail(fail(c, MK_ERR_HIP, "hipGetSymbolAddress of the static token staging array failed"));
  int nw = cfg.n_workers > 0 ? cfg.n_workers : prop.multiProcessorCount;
  if (cfg.lora_rank > 0 && cfg.batch >= 8)
    return bail(fail(c, MK_ERR_UNSUPPORTED, "LoRA adapters run on the batch <= 4 GEMV path only"));
  why = build_graph(cfg, nw, &c->g);
  if (!why.empty()) return bail(fail(c, MK_ERR_UNSUPPORTED, why));
  LdsPlan lp{};
  int rc = plan_lds(cfg, c->g, &lp, &why);
  if (rc) return bail(fail(c, rc, why));
  c->lds = lp;
  if (prepare_kernels(cfg.batch) != hipSuccess) return bail(fail(c, MK_ERR_HIP, "hipFuncSetAttribute failed"));
  {
    KParams tmp{};
    tmp.misc_off = lp.misc_off;
    const int per_cu = max_coresident_workers(cfg.batch, lds_bytes(tmp));
    if (per_cu < 1 || (int64_t)per_cu * prop.multiProcessorCount < nw)
      return bail(fail(c, MK_ERR_UNSUPPORTED, "workers cannot all be resident at once (cooperative launch)"));
  }
  const int L = cfg.n_layers, H = cfg.hidden, D = cfg.head_dim, Hq = cfg.n_q_heads, Hkv = cfg.n_kv_heads;
  const int F = cfg.ffn, V = cfg.vocab, B = cfg.batch, G = Hq / Hkv;
  const size_t QD = (size_t)Hq * D, KD = (size_t)Hkv * D, QKVR = QD + 2 * KD;

  // ---- weight arena (256-byte aligned tensors)
  size_t off = 0;
  auto take = [&](size_t elems) {
    size_t o = off;
    off += (elems * 2 + 255) / 256 * 128;  // elems of bf16, rounded to 256 bytes
    return o;
  };
  // With LoRA (rank r), each weight matrix is followed by its adapters' A rows (wqkv: A_q, A_k,
  // A_v), so that a GEMV tile streams its A rows exactly like its weight rows; the B matrices
  // [rows][r] have their own slots (b_qkv with rows in wqkv's grouped order).
  const size_t r = (size_t)cfg.lora_rank;
  std::vector<size_t> lo(L * 14);
  const size_t o_embed = take((size_t)V * H);
  for (int l = 0; l < L; ++l) {
    lo[l * 14 + 0] = take(QKVR * H + 3 * r * H);
    lo[l * 14 + 1] = take((size_t)H * QD + r * QD);
    lo[l * 14 + 2] = take((size_t)F * H + r * H);
    lo[l * 14 + 3] = take((size_t)F * H + r * H);
    lo[l * 14 + 4] = take((size_t)H * F + r * F);
    lo[l * 14 + 5] = take(H);
    lo[l * 14 + 6] = take(H);
    lo[l * 14 + 7] = take(D);
    lo[l * 14 + 8] = take(D);
    if (r) {
      lo[l * 14 + 9] = take(QKVR * r);
      lo[l * 14 + 10] = take((size_t)H * r);
      lo[l * 14 + 11] = take((size_t)F * r);
      lo[l * 14 + 12] = take((size_t)F * r);
      lo[l * 14 + 13] = take((size_t)H * r);
    }
  }
  const size_t o_fn = take(H), o_lm = take((size_t)V * H);
  c->wbytes = off * 2;
  if ((rc = dalloc(c, (void**)&c->warena, c->wbytes))) return bail(rc);
  c->embed = c->warena + o_embed;
  c->final_norm = c->warena + o_fn;
  c->lm_head = c->warena + o_lm;
  c->h_layers.resize(L);
  for (int l = 0; l < L; ++l) {
    LayerW& w = c->h_layers[l];
    const size_t* o = &lo[l * 14];
    w.wqkv = c->warena + o[0];
    w.wo = c->warena + o[1];
    w.wg = c->warena + o[2];
    w.wu = c->warena + o[3];
    w.wd = c->warena + o[4];
    w.attn_norm = c->warena + o[5];
    w.ffn_norm = c->warena + o[6];
    w.q_norm = cfg.qk_norm ? c->warena + o[7] : nullptr;
    w.k_norm = cfg.qk_norm ? c->warena + o[8] : nullptr;
    w.b_qkv = r ? c->warena + o[9] : nullptr;
    w.b_o = r ? c->warena + o[10] : nullptr;
    w.b_g = r ? c->warena + o[11] : nullptr;
    w.b_u = r ? c->warena + o[12] : nullptr;
    w.b_d = r ? c->warena + o[13] : nullptr;
    const std::string p = "layers." + std::to_string(l) + ".";
    c->wslots[p + "wo"] = {o[1], (int64_t)H * QD};
    c->wslots[p + "w_gate"] = {o[2], (int64_t)F * H};
    c->wslots[p + "w_up"] = {o[3], (int64_t)F * H};
    c->wslots[p + "w_down"] = {o[4], (int64_t)H * F};
    c->wslots[p + "attn_norm"] = {o[5], H};
    c->wslots[p + "ffn_norm"] = {o[6], H};
    if (cfg.qk_norm) {
      c->wslots[p + "q_norm"] = {o[7], D};
      c->wslots[p + "k_norm"] = {o[8], D};
    }
    if (r) {  // A rows after their weight matrix; B matrices in their own slots (b_qkv: regrouped at load)
      c->wslots[p + "lora_a.q"] = {o[0] + QKVR * H, (int64_t)(r * H)};
      c->wslots[p + "lora_a.k"] = {o[0] + QKVR * H + r * H, (int64_t)(r * H)};
      c->wslots[p + "lora_a.v"] = {o[0] + QKVR * H + 2 * r * H, (int64_t)(r * H)};
      c->wslots[p + "lora_a.o"] = {o[1] + (size_t)H * QD, (int64_t)(r * QD)};
      c->wslots[p + "lora_a.gate"] = {o[2] + (size_t)F * H, (int64_t)(r * H)};
      c->wslots[p + "lora_a.up"] = {o[3] + (size_t)F * H, (int64_t)(r * H)};
      c->wslots[p + "lora_a.down"] = {o[4] + (size_t)H * F, (int64_t)(r * F)};
      c->wslots[p + "lora_b.o"] = {o[10], (int64_t)(H * r)};
      c->wslots[p + "lora_b.gate"] = {o[11], (int64_t)(F * r)};
      c->wslots[p + "lora_b.up"] = {o[12], (int64_t)(F * r)};
      c->wslots[p + "lora_b.down"] = {o[13], (int64_t)(H * r)};
    }
  }
  c->wslots["embed"] = {o_embed, (int64_t)V * H};
  c->wslots["final_norm"] = {o_fn, H};
  c->wslots["lm_head"] = {o_lm, (int64_t)V * H};
  if ((rc = dalloc(c, (void**)&c->d_layers, sizeof(LayerW) * L))) return bail(rc);
  if (hipMemcpy(c->d_layers, c->h_layers.data(), sizeof(LayerW) * L, hipMemcpyHostToDevice) != hipSuccess)
    return bail(fail(c, MK_ERR_HIP, "layer table upload"));
  (void)G;

  // ---- RoPE tables: angle pos * theta^(-2i/D), cos and sin, all in fp64
  {
    const int half = D / 2;
    std::vector<double> hc((size_t)cfg.max_seq * half), hs(hc.size());
    for (int p = 0; p < cfg.max_seq; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * std::pow(cfg.rope_theta, -2.0 * (double)i / (double)D);
        hc[(size_t)p * half + i] = std::cos(ang);
        hs[(size_t)p * half + i] = std::sin(ang);
      }
    if ((rc = dalloc(c, (void**)&c->rope_cos, hc.size() * 8))) return bail(rc);
    if ((rc = dalloc(c, (void**)&c->rope_sin, hs.size() * 8))) return bail(rc);
    if (hipMemcpy(c->rope_cos, hc.data(), hc.size() * 8, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(c->rope_sin, hs.data(), hs.size() * 8, hipMemcpyHostToDevice) != hipSuccess)
      return bail(fail(c, MK_ERR_HIP, "rope upload"));
  }

  // ---- KV cache and activations
  c->kv_elems = (size_t)L * B * Hkv * cfg.max_seq * D;
  if ((rc = dalloc(c, (void**)&c->kc, c->kv_elems * 2))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->vc, c->kv_elems * 2))) return bail(rc);
  const int NS = c->g.n_splits;
  if ((rc = dalloc(c, (void**)&c->x, (size_t)B * H * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->qkv, (size_t)B * QKVR * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->o, (size_t)B * QD * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->a, (size_t)B * F * 4))) return bail(rc);
  c->n_part_ml = (size_t)B * Hkv * NS * G * 2 * 2;  // (max, sum), each fp64 as two tagged words
  c->n_part_acc = (size_t)B * Hkv * NS * G * D * 2;
  if ((rc = dalloc(c, (void**)&c->part_ml, c->n_part_ml * sizeof(TV)))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->part_acc, c->n_part_acc * sizeof(TV)))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->lm_part, (size_t)B * c->g.n_lm * sizeof(LmPart)))) return bail(rc);
  c->n_lora_u = (size_t)4 * B * 3 * r;
  if (r && (rc = dalloc(c, (void**)&c->lora_u, c->n_lora_u * sizeof(TV)))) return bail(rc);
  // [WO: H + 1 rows][DN: H + 1][QKV: QKVR + 1] per part below the last, 16 sequences, two words
  c->kpart_max = std::max({c->g.wo_ksplit, c->g.down_ksplit, c->g.qkv_ksplit});
  c->n_kpart = (size_t)(c->kpart_max - 1) * (2 * ((size_t)H + 1) + (size_t)QKVR + 1) * 16 * 2;
  if (c->n_kpart && (rc = dalloc(c, (void**)&c->kpart, c->n_kpart * sizeof(TV)))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->pending, (size_t)B * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->flags, (size_t)c->g.n_slots * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->status, 64))) return bail(rc);
  // ---- graph tables
  const Graph& g = c->g;
  if ((rc = dalloc(c, (void**)&c->d_events, g.events.size() * sizeof(EventRec)))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->d_tasks, g.tasks.size() * sizeof(TaskRec)))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->d_task_cu, g.task_cu.size() * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->d_list_off, g.list_off.size() * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->d_list_len, g.list_len.size() * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->d_cu_tasks, g.cu_tasks.size() * 4))) return bail(rc);
  if ((rc = dalloc(c, (void**)&c->d_range_start, g.range_start.size() * 4))) return bail(rc);
  if (hipMemcpy(c->d_range_start, g.range_start.data(), g.range_start.size() * 4, hipMemcpyHostToDevice) ||
      hipMemcpy(c->d_events, g.events.data(), g.events.size() * sizeof(EventRec), hipMemcpyHostToDevice) ||
      hipMemcpy(c->d_tasks, g.tasks.data(), g.tasks.size() * sizeof(TaskRec), hipMemcpyHostToDevice) ||
      hipMemcpy(c->d_task_cu, g.task_cu.data(), g.task_cu.size() * 4, hipMemcpyHostToDevice) ||
      hipMemcpy(c->d_list_off, g.list_off.data(), g.list_off.size() * 4, hipMemcpyHostToDevice) ||
      hipMemcpy(c->d_list_len, g.list_len.data(), g.list_len.size() * 4, hipMemcpyHostToDevice) ||
      hipMemcpy(c->d_cu_tasks, g.cu_tasks.data(), g.cu_tasks.size() * 4, hipMemcpyHostToDevice))
    return bail(fail(c, MK_ERR_HIP, "graph upload"));
  // ---- per-task records of the streaming GEMV engine (weight addresses are fixed from here on)
  {
    std::vector<SegRec> sr(g.tasks.size());
    for (size_t k = 0; k < g.tasks.size(); ++k) {
      const TaskRec& t = g.tasks[k];
      SegRec& r = sr[k];
      std::memset(&r, 0, sizeof r);
      r.op = t.op;
      r.a1 = t.a1;
      if (t.op == OP_ATTN) continue;
      const LayerW& w = c->h_layers[t.op == OP_LM ? 0 : t.layer];
      const uint16_t* W0;
      const uint16_t* W1 = nullptr;
      const uint16_t* gam = nullptr;
      int K;
      switch (t.op) {
        case OP_QKV: W0 = w.wqkv; K = H; gam = w.attn_norm; break;
        case OP_WO: W0 = w.wo; K = (int)QD; break;
        case OP_GU: W0 = w.wg; W1 = w.wu; K = H; gam = w.ffn_norm; break;
        case OP_DOWN: W0 = w.wd; K = F; break;
        default: W0 = c->lm_head; K = H; gam = c->final_norm; break;
      }
      const uint32_t nu = t.a1 - t.a0;
      r.w0 = W0 + (size_t)t.a0 * K;
      r.w1 = W1 ? W1 + (size_t)t.a0 * K : r.w0 + (size_t)nu * K;
      r.gamma = gam;
      r.act = t.op == OP_WO ? c->o : t.op == OP_DOWN ? c->a : c->x;
      r.K = (uint32_t)K;
      r.nu = nu;
      r.R = W1 ? 2 * nu : nu;
      r.f64 = gam ? 1u : 0u;
      r.kc = (uint32_t)(gam ? lp.sg_kc64 : lp.sg_kc32);
      r.nsl = r.kc ? (uint32_t)((K + r.kc - 1) / r.kc) : 0u;
    }
    if ((rc = dalloc(c, (void**)&c->d_segrec, sr.size() * sizeof(SegRec)))) return bail(rc);
    if (hipMemcpy(c->d_segrec, sr.data(), sr.size() * sizeof(SegRec), hipMemcpyHostToDevice) != hipSuccess)
      return bail(fail(c, MK_ERR_HIP, "segment records upload"));
  }
  if (hipEventCreate(&c->ev0) != hipSuccess || hipEventCreate(&c->ev1) != hipSuccess)
    return bail(fail(c, MK_ERR_HIP, "hipEventCreate"));
  c->seq_pos.assign(B, 0);
  if ((rc = mk_reset(c))) return bail(rc);
  HIPCHK(c, hipMemset(c->kc, 0, c->kv_elems * 2));
  HIPCHK(c, hipMemset(c->vc, 0, c->kv_elems * 2));
  HIPCHK(c, hipDeviceSynchronize());
  *out = c;
  return MK_OK;
}

void mk_destroy(mk_ctx* c) {
  if (!c) return;
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  else (void)hipDeviceSynchronize();
  for (void* p : c->allocs) (void)hipFree(p);
  if (c->ev0) (void)hipEventDestroy(c->ev0);
  if (c->ev1) (void)hipEventDestroy(c->ev1);
  delete c;
}

const char* mk_last_error(mk_ctx* c) { return c ? c->err.c_str() : g_create_err.c_str(); }

int mk_reset(mk_ctx* c) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "null ctx");
  HIPCHK(c, hipMemsetAsync(c->flags, 0, (size_t)c->g.n_slots * 4, c->stream));
  HIPCHK(c, hipMemsetAsync(c->part_ml, 0, c->n_part_ml * sizeof(TV), c->stream));
  HIPCHK(c, hipMemsetAsync(c->part_acc, 0, c->n_part_acc * sizeof(TV), c->stream));
  if (c->lora_u) HIPCHK(c, hipMemsetAsync(c->lora_u, 0, c->n_lora_u * sizeof(TV), c->stream));
  if (c->kpart) HIPCHK(c, hipMemsetAsync(c->kpart, 0, c->n_kpart * sizeof(TV), c->stream));
  HIPCHK(c, hipMemsetAsync(c->status, 0, 64, c->stream));
  HIPCHK(c, hipMemsetAsync(c->pending, 0, (size_t)c->cfg.batch * 4, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->pos = 0;
  std::fill(c->seq_pos.begin(), c->seq_pos.end(), 0);
  c->epoch = 0;
  c->lm_skip = 0;
  return MK_OK;
}

int mk_load_weights(mk_ctx* c, const mk_tensor* t, int n) {
  if (!c || (!t && n > 0) || n < 0) return fail(c, MK_ERR_INVALID_ARG, "null argument");
  const mk_model_cfg& cfg = c->cfg;
  const int L = cfg.n_layers, H = cfg.hidden, D = cfg.head_dim, Hq = cfg.n_q_heads, Hkv = cfg.n_kv_heads;
  const int G = Hq / Hkv;
  const size_t RG = (size_t)(G + 2) * D;
  std::map<std::string, int> seen;
  const int lr = cfg.lora_rank;
  const int expected = 1 + L * (9 + (cfg.qk_norm ? 2 : 0)) + 2 + (lr > 0 ? 14 * L : 0);
  for (int i = 0; i < n; ++i) {
    if (!t[i].name || !t[i].data) return fail(c, MK_ERR_INVALID_ARG, "tensor with null name or data");
    if (seen.count(t[i].name)) return fail(c, MK_ERR_INVALID_ARG, std::string("duplicate tensor ") + t[i].name);
    seen[t[i].name] = i;
  }
  if (n != expected) return fail(c, MK_ERR_INVALID_ARG, "expected " + std::to_string(expected) + " tensors, got " + std::to_string(n));
  for (int i = 0; i < n; ++i) {
    const std::string name = t[i].name;
    const hipMemcpyKind kind = t[i].on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
    const uint16_t* src = (const uint16_t*)t[i].data;
    auto it = c->wslots.find(name);
    if (it != c->wslots.end()) {
      if (t[i].numel != it->second.second) return fail(c, MK_ERR_INVALID_ARG, "wrong numel for " + name);
      HIPCHK(c, hipMemcpyAsync(c->warena + it->second.first, src, (size_t)t[i].numel * 2, kind, c->stream));
      continue;
    }
    // q/k/v: pack per KV-head group [G q heads | k | v]
    int l = -1;
    char which[16] = {0};
    // q/k/v weights and (LoRA) their B matrices: rows regrouped per KV-head group like wqkv
    const bool scanned = std::sscanf(name.c_str(), "layers.%d.%15s", &l, which) == 2 && l >= 0 && l < L;
    const bool is_w = scanned && (!std::strcmp(which, "wq") || !std::strcmp(which, "wk") || !std::strcmp(which, "wv"));
    const bool is_b = scanned && lr > 0 &&
                      (!std::strcmp(which, "lora_b.q") || !std::strcmp(which, "lora_b.k") || !std::strcmp(which, "lora_b.v"));
    if (is_w || is_b) {
      const char kind_c = is_w ? which[1] : which[7];  // q, k or v
      const bool isq = kind_c == 'q';
      const int nh = isq ? Hq : Hkv;
      const size_t rowlen = is_w ? (size_t)H : (size_t)lr;
      if (t[i].numel != (int64_t)nh * D * (int64_t)rowlen) return fail(c, MK_ERR_INVALID_ARG, "wrong numel for " + name);
      uint16_t* dst0 = const_cast<uint16_t*>(is_w ? c->h_layers[l].wqkv : c->h_layers[l].b_qkv);
      for (int h = 0; h < nh; ++h) {
        const int grp = isq ? h / G : h;
        const size_t row = grp * RG + (isq ? (size_t)(h % G) * D : (kind_c == 'k' ? (size_t)G * D : (size_t)(G + 1) * D));
        HIPCHK(c, hipMemcpyAsync(dst0 + row * rowlen, src + (size_t)h * D * rowlen, (size_t)D * rowlen * 2, kind,
                                 c->stream));
      }
      continue;
    }
    return fail(c, MK_ERR_INVALID_ARG, "unknown tensor " + name);
  }
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->have_weights = true;
  return MK_OK;
}

static KParams make_params(mk_ctx* c) {
  const mk_model_cfg& cfg = c->cfg;
  KParams P{};
  P.L = cfg.n_layers;
  P.H = cfg.hidden;
  P.Hq = cfg.n_q_heads;
  P.Hkv = cfg.n_kv_heads;
  P.D = cfg.head_dim;
  P.F = cfg.ffn;
  P.V = cfg.vocab;
  P.G = P.Hq / P.Hkv;
  P.RG = (P.G + 2) * P.D;
  P.QKVR = P.Hkv * P.RG;
  P.QD = P.Hq * P.D;
  P.B = cfg.batch;
  P.max_seq = cfg.max_seq;
  P.S = c->g.split;
  P.NS = c->g.n_splits;
  P.qk_norm = cfg.qk_norm;
  P.eps = cfg.rms_eps;
  P.attn_scale = 1.0 / std::sqrt((double)cfg.head_dim);
  P.n_workers = c->g.n_workers;
  P.n_qkv = c->g.n_qkv;
  P.n_wo = c->g.n_wo;
  P.n_gu = c->g.n_gu;
  P.n_down = c->g.n_down;
  P.n_lm = c->g.n_lm;
  P.xs_doubles = c->lds.xs_doubles;
  P.red_doubles = c->lds.red_doubles;
  P.red_off = c->lds.red_off;
  P.misc_off = c->lds.misc_off;
  P.mk_ks = c->lds.mk_ks;
  P.sg_rg0 = c->lds.sg_rg0;
  P.sg_rg1 = c->lds.sg_rg1;
  P.sg_red = c->lds.sg_red;
  P.sg_red_cap = c->lds.sg_red_cap;
  P.sg_xold = c->lds.sg_xold;
  P.sg_xold_cap = c->lds.sg_xold_cap;
  P.sg_kc64 = c->lds.sg_kc64;
  P.sg_kc32 = c->lds.sg_kc32;
  P.layers = c->d_layers;
  P.embed = c->embed;
  P.final_norm = c->final_norm;
  P.lm_head = c->lm_head;
  P.rope_cos = c->rope_cos;
  P.rope_sin = c->rope_sin;
  P.kc = c->kc;
  P.vc = c->vc;
  P.x = c->x;
  P.qkv = c->qkv;
  P.o = c->o;
  P.a = c->a;
  P.part_ml = c->part_ml;
  P.part_acc = c->part_acc;
  P.ntag = (uint32_t)c->g.events.size();
  P.epoch = c->epoch;
  P.lm_skip = c->lm_skip;
  P.kvB = cfg.batch;
  P.kv_seq = -1;
  P.lm_part = c->lm_part;
  P.lora_u = c->lora_u;
  P.lora_r = cfg.lora_rank;
  P.kpart = c->kpart;
  P.kpart_max = c->kpart_max;
  P.pending = c->pending;
  P.flags = c->flags;
  P.events = c->d_events;
  P.tasks = c->d_tasks;
  P.task_cu = c->d_task_cu;
  P.list_off = c->d_list_off;
  P.list_len = c->d_list_len;
  P.cu_tasks = c->d_cu_tasks;
  P.range_start = c->d_range_start;
  P.segrec = c->d_segrec;
  P.status = c->status;
  P.watchdog = cfg.watchdog_polls ? cfg.watchdog_polls : kDefaultWatchdog;
  P.with_lm = 1;
  P.trace = nullptr;
  P.trace_step = -1;
  P.trace_stride = c->trace_stride;
  return P;
}

// one decode step per operator launch (ablation mode and prefill)
static int run_per_op_steps(mk_ctx* c, KParams P, int n_steps, bool with_lm) {
  const Graph& g = c->g;
  const size_t n_ranges = g.op_ranges.size() - (with_lm ? 0 : 1);
  for (int s = 0; s < n_steps; ++s) {
    P.step = s;
    for (size_t r = 0; r < n_ranges; ++r) {
      P.op_first = (int)g.op_ranges[r].first;
      P.op_count = (int)g.op_ranges[r].count;
      P.op_range = (int)r;
      // cooperative where tasks of one launch wait on each other: attention mergers poll the other
      // splits' partials, with LoRA every GEMV tile waits for its operator's adapter rows, and the
      // last K part of a split row tile polls the other parts' sums
      const uint32_t op = g.tasks[g.op_ranges[r].first].op;
      const bool coop = op == OP_ATTN || (c->cfg.lora_rank > 0 && op != OP_LM) ||
                        (op == OP_WO && g.wo_ksplit > 1) || (op == OP_DOWN && g.down_ksplit > 1) ||
                        (op == OP_QKV && g.qkv_ksplit > 1);
      HIPCHK(c, launch(coop ? 3 : 1, P, c->stream));
    }
  }
  if (with_lm) {
    P.step = n_steps - 1;
    HIPCHK(c, launch(2, P, c->stream));
  }
  return MK_OK;
}

// Prefill shared by mk_prefill and mk_prefill_noalloc.  force: device int32 buffer of at least
// B * (len - 1) elements for the forced tokens (step-major), staged here from the host prompts.
// Allocates nothing.
static int prefill_into(mk_ctx* c, const int32_t* prompts, int len, int32_t* force) {
  const int B = c->cfg.batch;
  int rc = mk_reset(c);
  if (rc) return rc;
  const int n = len - 1;
  if (n > 0) {
    // forced token of step s, sequence b at force[s * B + b]: one strided copy per sequence
    for (int b = 0; b < B; ++b)
      HIPCHK(c, hipMemcpy2DAsync(force + b, (size_t)B * 4, prompts + (size_t)b * len, 4, 4, (size_t)n,
                                 hipMemcpyHostToDevice, c->stream));
    KParams P = make_params(c);
    P.pos0 = 0;
    P.n_steps = n;
    P.force_tok = force;
    P.with_lm = 0;
    if ((rc = run_per_op_steps(c, P, n, false))) return rc;
    c->epoch += (uint32_t)n;
    c->lm_skip += (uint32_t)n;
  }
  int32_t pend[16];
  for (int b = 0; b < B; ++b) pend[b] = prompts[(size_t)b * len + len - 1];
  HIPCHK(c, hipMemcpyAsync(c->pending, pend, (size_t)B * 4, hipMemcpyHostToDevice, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->pos = n;
  std::fill(c->seq_pos.begin(), c->seq_pos.end(), n);
  return MK_OK;
}

// ---- megakernel prefill ------------------------------------------------------------------------
// Columns per prefill step: 16 where the shape runs on the matrix-core GEMV (hidden, ffn and
// n_q_heads * head_dim multiples of 512, no LoRA), else 4 (the fp64 GEMV).
static int prefill_chunk(const mk_model_cfg& cfg) {
  const bool mfma = cfg.hidden % 512 == 0 && cfg.ffn % 512 == 0 && (cfg.n_q_heads * cfg.head_dim) % 512 == 0 &&
                    cfg.lora_rank == 0;
  return mfma ? 16 : 4;
}

static int prefill_build(mk_ctx* c) {
  PrefillCtx& f = c->pf;
  if (f.built) return MK_OK;
  const mk_model_cfg& cfg = c->cfg;
  const int C = prefill_chunk(cfg), nw = c->g.n_workers;
  std::string why = build_prefill_graph(cfg, nw, C, c->g.split, &f.g);
  if (!why.empty()) return fail(c, MK_ERR_UNSUPPORTED, "prefill graph: " + why);
  mk_model_cfg cc = cfg;
  cc.batch = C;
  int rc = plan_lds(cc, f.g, &f.lds, &why);
  if (rc) return fail(c, rc, "prefill: " + why);
  if (prepare_kernels(C) != hipSuccess) return fail(c, MK_ERR_HIP, "hipFuncSetAttribute failed");
  {
    KParams tmp{};
    tmp.misc_off = f.lds.misc_off;
    const int per_cu = max_coresident_workers(C, lds_bytes(tmp));
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, c->device) != hipSuccess) return fail(c, MK_ERR_HIP, "hipGetDeviceProperties");
    if (per_cu < 1 || (int64_t)per_cu * prop.multiProcessorCount < nw)
      return fail(c, MK_ERR_UNSUPPORTED, "prefill workers cannot all be resident at once");
  }
  const Graph& g = f.g;
  const int H = cfg.hidden, D = cfg.head_dim, Hkv = cfg.n_kv_heads, G = cfg.n_q_heads / Hkv, NS = g.n_splits;
  const size_t QD = (size_t)cfg.n_q_heads * D, QKVR = QD + 2 * (size_t)Hkv * D;
  if ((rc = dalloc(c, (void**)&f.d_events, g.events.size() * sizeof(EventRec))) ||
      (rc = dalloc(c, (void**)&f.d_tasks, g.tasks.size() * sizeof(TaskRec))) ||
      (rc = dalloc(c, (void**)&f.d_list_off, g.list_off.size() * 4)) ||
      (rc = dalloc(c, (void**)&f.d_list_len, g.list_len.size() * 4)) ||
      (rc = dalloc(c, (void**)&f.d_cu_tasks, g.cu_tasks.size() * 4)) ||
      (rc = dalloc(c, (void**)&f.d_range_start, g.range_start.size() * 4)) ||
      (rc = dalloc(c, (void**)&f.flags, (size_t)g.n_slots * 4)) ||
      (rc = dalloc(c, (void**)&f.x, (size_t)C * H * 4)) || (rc = dalloc(c, (void**)&f.qkv, (size_t)C * QKVR * 4)) ||
      (rc = dalloc(c, (void**)&f.o, (size_t)C * QD * 4)) || (rc = dalloc(c, (void**)&f.a, (size_t)C * cfg.ffn * 4)) ||
      (rc = dalloc(c, (void**)&f.part_ml, (f.n_part_ml = (size_t)C * Hkv * NS * G * 2 * 2) * sizeof(TV))) ||
      (rc = dalloc(c, (void**)&f.part_acc, (f.n_part_acc = (size_t)C * Hkv * NS * G * D * 2) * sizeof(TV))) ||
      (rc = dalloc(c, (void**)&f.lm_part, (size_t)C * g.n_lm * sizeof(LmPart))))
    return rc;
  f.n_lora_u = (size_t)4 * C * 3 * cfg.lora_rank;
  if (cfg.lora_rank && (rc = dalloc(c, (void**)&f.lora_u, f.n_lora_u * sizeof(TV)))) return rc;
  if (hipMemcpy(f.d_events, g.events.data(), g.events.size() * sizeof(EventRec), hipMemcpyHostToDevice) ||
      hipMemcpy(f.d_tasks, g.tasks.data(), g.tasks.size() * sizeof(TaskRec), hipMemcpyHostToDevice) ||
      hipMemcpy(f.d_list_off, g.list_off.data(), g.list_off.size() * 4, hipMemcpyHostToDevice) ||
      hipMemcpy(f.d_list_len, g.list_len.data(), g.list_len.size() * 4, hipMemcpyHostToDevice) ||
      hipMemcpy(f.d_cu_tasks, g.cu_tasks.data(), g.cu_tasks.size() * 4, hipMemcpyHostToDevice) ||
      hipMemcpy(f.d_range_start, g.range_start.data(), g.range_start.size() * 4, hipMemcpyHostToDevice))
    return fail(c, MK_ERR_HIP, "prefill graph upload");
  f.built = true;
  return MK_OK;
}

// Prefill through the persistent kernel: for each sequence, one launch whose step s takes prompt
// tokens [s C, (s + 1) C) as the C columns of every projection.
static int prefill_megakernel(mk_ctx* c, const int32_t* prompts, int len) {
  int rc = mk_reset(c);
  if (rc) return rc;
  if ((rc = prefill_build(c))) return rc;
  PrefillCtx& f = c->pf;
  const Graph& g = f.g;
  const int B = c->cfg.batch, C = g.chunk, n = len - 1;
  if (n > 0) {
    const int steps = (n + C - 1) / C;
    if ((size_t)steps * C > f.force_cap) {
      if ((rc = dalloc(c, (void**)&f.force, (size_t)steps * C * 4))) return rc;
      f.force_cap = (size_t)steps * C;
    }
    // a fresh start of the prefill graph's steps: event slots and step-tagged words cleared
    HIPCHK(c, hipMemsetAsync(f.flags, 0, (size_t)g.n_slots * 4, c->stream));
    HIPCHK(c, hipMemsetAsync(f.part_ml, 0, f.n_part_ml * sizeof(TV), c->stream));
    HIPCHK(c, hipMemsetAsync(f.part_acc, 0, f.n_part_acc * sizeof(TV), c->stream));
    if (f.lora_u) HIPCHK(c, hipMemsetAsync(f.lora_u, 0, f.n_lora_u * sizeof(TV), c->stream));
    f.epoch = 0;
    KParams P = make_params(c);
    P.B = C;
    P.S = g.split;
    P.NS = g.n_splits;
    P.n_qkv = g.n_qkv;
    P.n_wo = g.n_wo;
    P.n_gu = g.n_gu;
    P.n_down = g.n_down;
    P.n_lm = g.n_lm;
    P.xs_doubles = f.lds.xs_doubles;
    P.red_doubles = f.lds.red_doubles;
    P.red_off = f.lds.red_off;
    P.misc_off = f.lds.misc_off;
    P.mk_ks = f.lds.mk_ks;
    P.x = f.x;
    P.qkv = f.qkv;
    P.o = f.o;
    P.a = f.a;
    P.part_ml = f.part_ml;
    P.part_acc = f.part_acc;
    P.lm_part = f.lm_part;
    P.lora_u = f.lora_u;
    P.flags = f.flags;
    P.events = f.d_events;
    P.tasks = f.d_tasks;
    P.task_cu = nullptr;
    P.list_off = f.d_list_off;
    P.list_len = f.d_list_len;
    P.cu_tasks = f.d_cu_tasks;
    P.range_start = f.d_range_start;
    P.segrec = nullptr;
    P.ntag = (uint32_t)g.events.size();
    P.with_lm = 0;
    P.chunk = C;
    P.kvB = B;
    P.pos_end = n;
    P.pos0 = 0;
    P.n_steps = steps;
    P.force_tok = f.force;
    P.lm_skip = 0;
    std::vector<int32_t> tok((size_t)steps * C, 0);  // padding tokens: id 0, masked in the kernel
    for (int q = 0; q < B; ++q) {
      for (int i = 0; i < n; ++i) tok[i] = prompts[(size_t)q * len + i];
      HIPCHK(c, hipMemcpyAsync(f.force, tok.data(), tok.size() * 4, hipMemcpyHostToDevice, c->stream));
      P.kv_seq = q;
      P.epoch = f.epoch;
      HIPCHK(c, launch(0, P, c->stream));
      HIPCHK(c, hipStreamSynchronize(c->stream));
      f.epoch += (uint32_t)steps;
    }
    uint32_t st[8];
    HIPCHK(c, hipMemcpy(st, c->status, sizeof st, hipMemcpyDeviceToHost));
    if (st[ST_ABORT] || st[ST_CODE]) {
      char buf[256];
      std::snprintf(buf, sizeof buf, "prefill watchdog: worker %u task %u waited on event %u (slot value %u, wanted %u)",
                    st[ST_CU], st[ST_TASK], st[ST_EVENT], st[ST_SEEN], st[ST_WANT]);
      return fail(c, MK_ERR_TIMEOUT, buf);
    }
  }
  int32_t pend[16];
  for (int b = 0; b < B; ++b) pend[b] = prompts[(size_t)b * len + len - 1];
  HIPCHK(c, hipMemcpyAsync(c->pending, pend, (size_t)B * 4, hipMemcpyHostToDevice, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->pos = n;
  std::fill(c->seq_pos.begin(), c->seq_pos.end(), n);
  return MK_OK;
}

static int prefill_check(mk_ctx* c, const int32_t* prompts, int len) {
  if (!c || !prompts || len <= 0) return fail(c, MK_ERR_INVALID_ARG, "null prompts or len <= 0");
  if (!c->have_weights) return fail(c, MK_ERR_STATE, "weights not loaded");
  if (len > c->cfg.max_seq) return fail(c, MK_ERR_CAPACITY, "prompt longer than max_seq");
  for (int64_t i = 0; i < (int64_t)c->cfg.batch * len; ++i)
    if (prompts[i] < 0 || prompts[i] >= c->cfg.vocab) return fail(c, MK_ERR_INVALID_ARG, "token id out of range");
  return MK_OK;
}

int mk_prefill(mk_ctx* c, const int32_t* prompts, int len) {
  int rc = prefill_check(c, prompts, len);
  if (rc) return rc;
  if (c->cfg.prefill == MK_PREFILL_MEGAKERNEL) return prefill_megakernel(c, prompts, len);
  const size_t need = (size_t)(len - 1) * c->cfg.batch;
  if (need > c->force_cap) {
    if (c->force) {
      (void)hipFree(c->force);
      c->allocs.erase(std::find(c->allocs.begin(), c->allocs.end(), (void*)c->force));
      c->force = nullptr;
      c->force_cap = 0;
    }
    if ((rc = dalloc(c, (void**)&c->force, need * 4))) return rc;
    c->force_cap = need;
  }
  return prefill_into(c, prompts, len, c->force);
}

int mk_prefill_noalloc(mk_ctx* c, const int32_t* prompts, int len) {
  int rc = prefill_check(c, prompts, len);
  if (rc) return rc;
  const size_t need = (size_t)(len - 1) * c->cfg.batch;
  if (need > (size_t)kNoAllocTokens)
    return fail(c, MK_ERR_CAPACITY, "prompt needs " + std::to_string(need) + " staged tokens (batch * (len - 1)); "
                                    "mk_prefill_noalloc holds at most " + std::to_string(kNoAllocTokens));
  if (!c->noalloc_tokens) return fail(c, MK_ERR_STATE, "static token staging not resolved on this device");
  return prefill_into(c, prompts, len, c->noalloc_tokens);
}

int mk_load_kv(mk_ctx* c, int seq, int n_pos, const void* k, const void* v, int32_t pending, int on_device) {
  if (!c || !k || !v) return fail(c, MK_ERR_INVALID_ARG, "null argument");
  const mk_model_cfg& cfg = c->cfg;
  if (seq < 0 || seq >= cfg.batch || n_pos < 0) return fail(c, MK_ERR_INVALID_ARG, "bad seq or n_pos");
  if (n_pos >= cfg.max_seq) return fail(c, MK_ERR_CAPACITY, "n_pos must leave room for one decode step");
  if (pending < 0 || pending >= cfg.vocab) return fail(c, MK_ERR_INVALID_ARG, "pending token out of range");
  const int L = cfg.n_layers, D = cfg.head_dim, Hkv = cfg.n_kv_heads, B = cfg.batch;
  const hipMemcpyKind kind = on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  const size_t KD = (size_t)Hkv * D;
  for (int l = 0; l < L && n_pos > 0; ++l)
    for (int g = 0; g < Hkv; ++g) {
      const size_t dst = (((size_t)l * B + seq) * Hkv + g) * cfg.max_seq * D;
      const size_t src = (size_t)l * n_pos * KD + (size_t)g * D;
      HIPCHK(c, hipMemcpy2DAsync(c->kc + dst, D * 2, (const uint16_t*)k + src, KD * 2, D * 2, n_pos, kind, c->stream));
      HIPCHK(c, hipMemcpy2DAsync(c->vc + dst, D * 2, (const uint16_t*)v + src, KD * 2, D * 2, n_pos, kind, c->stream));
    }
  HIPCHK(c, hipMemcpyAsync(c->pending + seq, &pending, 4, hipMemcpyHostToDevice, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->seq_pos[seq] = n_pos;
  c->pos = n_pos;
  return MK_OK;
}

int mk_set_mode(mk_ctx* c, int mode) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "null ctx");
  if (mode != MK_MODE_MEGAKERNEL && mode != MK_MODE_PER_OP) return fail(c, MK_ERR_INVALID_ARG, "unknown mode");
  c->cfg.mode = mode;
  return MK_OK;
}

int mk_debug_poison(mk_ctx* c) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "null ctx");
  const mk_model_cfg& cfg = c->cfg;
  const size_t B = (size_t)cfg.batch, QD = (size_t)cfg.n_q_heads * cfg.head_dim;
  const size_t QKVR = QD + 2 * (size_t)cfg.n_kv_heads * cfg.head_dim;
  HIPCHK(c, hipMemsetAsync(c->x, 0xff, B * cfg.hidden * 4, c->stream));
  HIPCHK(c, hipMemsetAsync(c->qkv, 0xff, B * QKVR * 4, c->stream));
  HIPCHK(c, hipMemsetAsync(c->o, 0xff, B * QD * 4, c->stream));
  HIPCHK(c, hipMemsetAsync(c->a, 0xff, B * cfg.ffn * 4, c->stream));
  HIPCHK(c, hipMemsetAsync(c->lm_part, 0xff, B * c->g.n_lm * sizeof(LmPart), c->stream));
  HIPCHK(c, hipMemsetAsync(c->part_ml, 0xff, c->n_part_ml * sizeof(TV), c->stream));
  HIPCHK(c, hipMemsetAsync(c->part_acc, 0xff, c->n_part_acc * sizeof(TV), c->stream));
  if (c->lora_u) HIPCHK(c, hipMemsetAsync(c->lora_u, 0xff, c->n_lora_u * sizeof(TV), c->stream));
  if (c->kpart) HIPCHK(c, hipMemsetAsync(c->kpart, 0xff, c->n_kpart * sizeof(TV), c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  return MK_OK;
}

int mk_set_prefill(mk_ctx* c, int prefill) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "null ctx");
  if (prefill != MK_PREFILL_PER_OP && prefill != MK_PREFILL_MEGAKERNEL) return fail(c, MK_ERR_INVALID_ARG, "unknown prefill mode");
  c->cfg.prefill = prefill;
  return MK_OK;
}

int mk_get_config(mk_ctx* c, mk_model_cfg* out) {
  if (!c || !out) return fail(c, MK_ERR_INVALID_ARG, "null argument");
  *out = c->cfg;
  return MK_OK;
}

int mk_get_state(mk_ctx* c, int32_t* pos, int32_t* pending) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "null ctx");
  if (pos) *pos = c->pos;
  if (pending) {
    HIPCHK(c, hipMemcpyAsync(pending, c->pending, (size_t)c->cfg.batch * 4, hipMemcpyDeviceToHost, c->stream));
    HIPCHK(c, hipStreamSynchronize(c->stream));
  }
  return MK_OK;
}

int mk_decode(mk_ctx* c, int n_steps, int32_t* out_tokens, float* out_logits) {
  if (!c || n_steps <= 0 || !out_tokens) return fail(c, MK_ERR_INVALID_ARG, "null out_tokens or n_steps <= 0");
  if (!c->have_weights) return fail(c, MK_ERR_STATE, "weights not loaded");
  for (int p : c->seq_pos)
    if (p != c->pos) return fail(c, MK_ERR_STATE, "sequences hold different numbers of positions");
  if ((int64_t)c->pos + n_steps > c->cfg.max_seq) return fail(c, MK_ERR_CAPACITY, "decode would exceed max_seq");
  KParams P = make_params(c);
  P.pos0 = c->pos;
  P.n_steps = n_steps;
  P.out_tokens = out_tokens;
  P.out_logits = out_logits;
  P.epoch = c->epoch;
  P.lm_skip = c->lm_skip;
  if (c->trace && c->trace_step >= 0 && c->trace_step < n_steps && c->cfg.mode == MK_MODE_MEGAKERNEL) {
    HIPCHK(c, hipMemsetAsync(c->trace, 0, (size_t)c->g.n_workers * c->trace_stride * 4 * 8, c->stream));
    P.trace = c->trace;
    P.trace_step = c->trace_step;
  }
  HIPCHK(c, hipEventRecord(c->ev0, c->stream));
  if (c->cfg.mode == MK_MODE_MEGAKERNEL) {
    HIPCHK(c, launch(0, P, c->stream));
  } else {
    int rc = run_per_op_steps(c, P, n_steps, true);
    if (rc) return rc;
  }
  HIPCHK(c, hipEventRecord(c->ev1, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  HIPCHK(c, hipEventElapsedTime(&c->last_ms, c->ev0, c->ev1));
  uint32_t st[8];
  HIPCHK(c, hipMemcpy(st, c->status, sizeof st, hipMemcpyDeviceToHost));
  if (st[ST_ABORT] || st[ST_CODE]) {
    char buf[256];
    std::snprintf(buf, sizeof buf, "watchdog: worker %u task %u waited on event %u (slot value %u, wanted %u)",
                  st[ST_CU], st[ST_TASK], st[ST_EVENT], st[ST_SEEN], st[ST_WANT]);
    return fail(c, MK_ERR_TIMEOUT, buf);
  }
  c->pos += n_steps;
  std::fill(c->seq_pos.begin(), c->seq_pos.end(), c->pos);
  c->epoch += (uint32_t)n_steps;
  return MK_OK;
}

int mk_get_graph(mk_ctx* c, void* buf, size_t* len) {
  if (!c || !len) return fail(c, MK_ERR_INVALID_ARG, "null argument");
  std::vector<uint8_t> bytes = serialize_graph(c->cfg, c->g);
  if (!buf || *len < bytes.size()) {
    *len = bytes.size();
    return buf ? fail(c, MK_ERR_INVALID_ARG, "buffer too small") : MK_OK;
  }
  std::memcpy(buf, bytes.data(), bytes.size());
  *len = bytes.size();
  return MK_OK;
}

int mk_set_trace(mk_ctx* c, int step) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "null ctx");
  if (step >= 0 && !c->trace) {
    uint32_t mx = 0;
    for (uint32_t n : c->g.list_len) mx = std::max(mx, n);
    c->trace_stride = (int)mx;
    int rc = dalloc(c, (void**)&c->trace, (size_t)c->g.n_workers * mx * 4 * 8);
    if (rc) return rc;
    HIPCHK(c, hipMemset(c->trace, 0, (size_t)c->g.n_workers * mx * 4 * 8));
  }
  c->trace_step = step;
  return MK_OK;
}

int mk_get_trace(mk_ctx* c, uint64_t* out, size_t* len, int32_t* n_workers, int32_t* max_list, int32_t* clock_khz) {
  if (!c || !len) return fail(c, MK_ERR_INVALID_ARG, "null argument");
  if (!c->trace) return fail(c, MK_ERR_STATE, "tracing was never enabled");
  const size_t need = (size_t)c->g.n_workers * c->trace_stride * 4;
  if (n_workers) *n_workers = c->g.n_workers;
  if (max_list) *max_list = c->trace_stride;
  if (clock_khz) {
    int khz = 0;
    HIPCHK(c, hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, c->device));
    *clock_khz = khz;
  }
  if (!out) {
    *len = need;
    return MK_OK;
  }
  if (*len < need) return fail(c, MK_ERR_INVALID_ARG, "trace buffer too small");
  HIPCHK(c, hipMemcpy(out, c->trace, need * 8, hipMemcpyDeviceToHost));
  *len = need;
  return MK_OK;
}

static int stream_probe(size_t bytes, int iters, bool copy, float* gbps) {
  if (!gbps || bytes < ((size_t)1 << 20) || iters <= 0) return fail(nullptr, MK_ERR_INVALID_ARG, "bad argument");
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(nullptr, MK_ERR_HIP, "no device");
  const int n_wg = prop.multiProcessorCount;
  bytes = bytes / ((size_t)32 * n_wg) * ((size_t)32 * n_wg);
  void* buf = nullptr;
  uint32_t* out = nullptr;
  if (hipMalloc(&buf, bytes) != hipSuccess) return fail(nullptr, MK_ERR_OOM, "probe buffer");
  if (hipMalloc((void**)&out, 256) != hipSuccess) {
    (void)hipFree(buf);
    return fail(nullptr, MK_ERR_OOM, "probe buffer");
  }
  hipEvent_t e0, e1;
  int rc = MK_OK;
  if (hipMemset(buf, 0, bytes) != hipSuccess || hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    rc = fail(nullptr, MK_ERR_HIP, "probe setup");
  } else {
    auto run = [&]() {
      return copy ? launch_copy_probe(buf, bytes, n_wg, nullptr) : launch_read_probe(buf, bytes, n_wg, out, nullptr);
    };
    if (run() != hipSuccess) rc = fail(nullptr, MK_ERR_HIP, "probe launch");
    (void)hipEventRecord(e0, nullptr);
    for (int i = 0; i < iters && rc == MK_OK; ++i)
      if (run() != hipSuccess) rc = fail(nullptr, MK_ERR_HIP, "probe launch");
    (void)hipEventRecord(e1, nullptr);
    float ms = 0.f;
    if (rc == MK_OK && (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
      rc = fail(nullptr, MK_ERR_HIP, "probe timing");
    if (rc == MK_OK) *gbps = (float)((double)bytes * iters / (ms * 1e-3) / 1e9);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  (void)hipFree(out);
  (void)hipFree(buf);
  return rc;
}

int mk_read_bandwidth(size_t bytes, int iters, float* gbps) { return stream_probe(bytes, iters, false, gbps); }
int mk_copy_bandwidth(size_t bytes, int iters, float* gbps) { return stream_probe(bytes, iters, true, gbps); }

int mk_last_decode_ms(mk_ctx* c, float* ms) {
  if (!c || !ms) return fail(c, MK_ERR_INVALID_ARG, "null argument");
  *ms = c->last_ms;
  return MK_OK;
}

}  // extern "C"
