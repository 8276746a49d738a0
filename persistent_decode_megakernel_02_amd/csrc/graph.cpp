// graph.cpp -- lowers one decode step to tasks and events.
//
// This is the compiler half of the method (MPK digest, fr.news.hada.io,
// "Part 1. Compilateur"): operators become fine-grained tasks, each given to
// one compute unit, joined by events that carry data dependencies at the
// granularity the data allows (a KV-head group of Q/K/V rows feeds only the
// attention tasks of that group).  The schedule is decided here, once, and
// frozen into per-worker lists (Ada-MK, gist.science, "L'Itinéraire
// Pré-planifié"): no decision is taken while the kernel runs.
//
// Rules (the Python spec builder in the tests re-derives the same bytes):
//  * GEMV operators are tiled by output rows; tile i of T over R units covers
//    [floor(i R / T), floor((i+1) R / T)).  T = min(workers, R), except Q/K/V
//    which is tiled per KV-head group: TG = min(max(1, workers / Hkv), RG)
//    tiles per group of RG = (G + 2) D rows.  Gate/up units are row pairs.
//  * Attention tasks: one per (split s, sequence b, KV head g), enumerated
//    split-major; split s covers positions [s S, (s+1) S).
//  * Task t of an operator goes to worker (index mod workers).
//  * Topological order per layer: QKV, ATTN, WO, GU, DOWN; then LM.  Every
//    worker walks its tasks in this order, so the unfinished task with the
//    lowest index always has its inputs ready: no deadlock while all
//    workers are resident.
#include "graph.h"

#include <algorithm>
#include <cstring>

namespace mk {

namespace {
uint32_t tile_lo(uint64_t i, uint64_t R, uint64_t T) { return (uint32_t)(i * R / T); }
}  // namespace

std::string build_graph(const mk_model_cfg& c, int n_workers, Graph* out) {
  Graph g;
  if (n_workers <= 0) return "n_workers must be positive";
  if (c.n_layers <= 0 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 || c.ffn <= 0 ||
      c.vocab <= 0 || c.batch <= 0 || c.max_seq <= 0)
    return "all shape fields must be positive";
  if (c.n_q_heads % c.n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
  const int G = c.n_q_heads / c.n_kv_heads, D = c.head_dim, Hkv = c.n_kv_heads;
  if (D % 8 || D > 256 || 64 % (D / 8)) return "head_dim must be 64/8*2^k-compatible: D%8==0, D<=256, (D/8) | 64";
  if (G > 8) return "at most 8 query heads per KV head";
  if (c.hidden % 8 || c.ffn % 8) return "hidden and ffn must be multiples of 8";
  // Default split: enough splits that the (sequence, KV head, split) tasks of a
  // full cache fill the workers once, each split between 32 positions and the
  // per-task register budget (5 * 4096 / D positions, 8 * 4096 / D with one query
  // head per KV head).  Attention tasks are
  // latency-bound at short contexts, so more, shorter splits finish sooner.
  const int smax = (G == 1 ? 8 : 5) * 4096 / D;
  int S = c.split;
  if (S <= 0) {
    const int per = std::max(1, c.batch * Hkv);  // attention tasks per split
    const int ns_target = std::max(1, n_workers / per);
    S = std::min(smax, std::max(kDefaultSplit, (c.max_seq + ns_target - 1) / ns_target));
    // Capped by smax, the splits spill over into several tasks per worker.  Up to three per
    // worker, take as many (shorter) splits as keep that count: the critical worker then runs
    // the same number of shorter tasks.
    const int ns_min = (c.max_seq + smax - 1) / smax;
    if (ns_min > ns_target) {
      const int64_t per_worker = ((int64_t)ns_min * per + n_workers - 1) / n_workers;
      if (per_worker <= 3) {
        const int ns = std::max<int64_t>(ns_min, per_worker * n_workers / per);
        S = std::max(kDefaultSplit, (c.max_seq + ns - 1) / ns);
      }
    }
  }
  if (S > smax) return "split must be <= 5 * 4096 / head_dim (8 * 4096 / head_dim with one query head per KV head)";
  g.n_workers = n_workers;
  g.split = S;
  g.n_splits = (c.max_seq + S - 1) / S;
  const int RG = (G + 2) * D;
  const int TG = std::min(std::max(1, n_workers / Hkv), RG);
  g.qkv_tiles_per_group = TG;
  g.n_qkv = TG * Hkv;
  g.n_wo = std::min(n_workers, c.hidden);
  g.n_gu = std::min(n_workers, c.ffn);
  g.n_down = std::min(n_workers, c.hidden);
  g.n_lm = std::min(n_workers, c.vocab);
  if ((int64_t)g.n_qkv > n_workers) return "internal: too many QKV tiles";
  // When every attention task of a layer has a worker of its own, all of a head's splits run
  // at once and each merges a slice of the outputs, signalling its own slot; otherwise the
  // split holding the current position merges everything and signals for its (sequence, head).
  const bool dist = (int64_t)g.n_splits * c.batch * Hkv <= n_workers;

  // events: per layer [QKV group 0..Hkv-1, ATT, O, A, X], then LM
  const int per_layer = Hkv + 4;
  auto ev_qkv = [&](int l, int gg) { return (uint32_t)(l * per_layer + gg); };
  auto ev_att = [&](int l) { return (uint32_t)(l * per_layer + Hkv); };
  auto ev_o = [&](int l) { return (uint32_t)(l * per_layer + Hkv + 1); };
  auto ev_a = [&](int l) { return (uint32_t)(l * per_layer + Hkv + 2); };
  auto ev_x = [&](int l) { return (uint32_t)(l * per_layer + Hkv + 3); };
  const uint32_t ev_lm = (uint32_t)(c.n_layers * per_layer);
  g.events.resize(ev_lm + 1);
  for (int l = 0; l < c.n_layers; ++l) {
    for (int gg = 0; gg < Hkv; ++gg) g.events[ev_qkv(l, gg)].fanin = TG;
    g.events[ev_att(l)].fanin = dist ? g.n_splits * c.batch * Hkv : c.batch * Hkv;
    g.events[ev_o(l)].fanin = g.n_wo;
    g.events[ev_a(l)].fanin = g.n_gu;
    g.events[ev_x(l)].fanin = g.n_down;
  }
  g.events[ev_lm].fanin = g.n_lm;
  uint32_t slot = 0;
  for (auto& e : g.events) {
    e.slot0 = slot;
    slot += e.fanin;
  }
  g.n_slots = (int)slot;

  auto push = [&](uint32_t op, int layer, uint32_t tile, uint32_t a0, uint32_t a1, uint32_t wait_ev, uint32_t lag,
                  uint32_t sig_ev, uint32_t sig_slot, uint32_t cu) {
    TaskRec t;
    std::memset(&t, 0, sizeof t);
    t.op = op;
    t.layer = (uint32_t)layer;
    t.tile = tile;
    t.a0 = a0;
    t.a1 = a1;
    t.wait_ev = wait_ev;
    t.wait_lag = lag;
    t.sig_ev = sig_ev;
    t.sig_slot = sig_slot;
    g.tasks.push_back(t);
    g.task_cu.push_back(cu % (uint32_t)n_workers);
  };
  auto range_begin = [&]() { return (uint32_t)g.tasks.size(); };
  auto range_end = [&](uint32_t first) { g.op_ranges.push_back({first, (uint32_t)g.tasks.size() - first}); };

  for (int l = 0; l < c.n_layers; ++l) {
    const uint32_t in_ev = l == 0 ? ev_lm : ev_x(l - 1);
    const uint32_t in_lag = l == 0 ? 1u : 0u;
    uint32_t f = range_begin();
    for (int gg = 0; gg < Hkv; ++gg)
      for (int i = 0; i < TG; ++i) {
        uint32_t tile = (uint32_t)(gg * TG + i);
        uint32_t r0 = (uint32_t)(gg * RG) + tile_lo(i, RG, TG), r1 = (uint32_t)(gg * RG) + tile_lo(i + 1, RG, TG);
        push(OP_QKV, l, tile, r0, r1, in_ev, in_lag, ev_qkv(l, gg), (uint32_t)i, tile);
      }
    range_end(f);
    f = range_begin();
    uint32_t idx = 0;
    for (int s = 0; s < g.n_splits; ++s)
      for (int b = 0; b < c.batch; ++b)
        for (int gg = 0; gg < Hkv; ++gg, ++idx)
          push(OP_ATTN, l, idx, (uint32_t)(b * Hkv + gg), (uint32_t)s, ev_qkv(l, gg), 0, ev_att(l),
               dist ? idx : (uint32_t)(b * Hkv + gg), idx);
    range_end(f);
    f = range_begin();
    for (int i = 0; i < g.n_wo; ++i)
      push(OP_WO, l, i, tile_lo(i, c.hidden, g.n_wo), tile_lo(i + 1, c.hidden, g.n_wo), ev_att(l), 0, ev_o(l), i, i);
    range_end(f);
    f = range_begin();
    for (int i = 0; i < g.n_gu; ++i)
      push(OP_GU, l, i, tile_lo(i, c.ffn, g.n_gu), tile_lo(i + 1, c.ffn, g.n_gu), ev_o(l), 0, ev_a(l), i, i);
    range_end(f);
    f = range_begin();
    for (int i = 0; i < g.n_down; ++i)
      push(OP_DOWN, l, i, tile_lo(i, c.hidden, g.n_down), tile_lo(i + 1, c.hidden, g.n_down), ev_a(l), 0, ev_x(l), i,
           i);
    range_end(f);
  }
  uint32_t f = range_begin();
  for (int i = 0; i < g.n_lm; ++i)
    push(OP_LM, 0, i, tile_lo(i, c.vocab, g.n_lm), tile_lo(i + 1, c.vocab, g.n_lm), ev_x(c.n_layers - 1), 0, ev_lm, i,
         i);
  range_end(f);

  // per-worker lists in topological order
  g.list_off.assign(n_workers, 0);
  g.list_len.assign(n_workers, 0);
  for (uint32_t cu : g.task_cu) g.list_len[cu]++;
  uint32_t off = 0;
  for (int w = 0; w < n_workers; ++w) {
    g.list_off[w] = off;
    off += g.list_len[w];
  }
  g.cu_tasks.assign(g.tasks.size(), 0);
  std::vector<uint32_t> fill(n_workers, 0);
  for (uint32_t i = 0; i < g.tasks.size(); ++i) {
    uint32_t cu = g.task_cu[i];
    g.cu_tasks[g.list_off[cu] + fill[cu]++] = i;
  }
  *out = std::move(g);
  return "";
}

// Canonical bytes: little-endian u32 words.
//   header: 'MKG1', version 1, n_workers, split, n_splits, n_events, n_tasks, n_slots
//   events: id, fanin, slot0
//   tasks (topological order): topo, op, layer, tile, a0, a1, wait_ev, wait_fanin, wait_lag,
//                              sig_ev, sig_slot, worker
std::vector<uint8_t> serialize_graph(const mk_model_cfg& c, const Graph& g) {
  (void)c;
  std::vector<uint32_t> w;
  w.push_back(0x31474B4Du);
  w.push_back(1);
  w.push_back((uint32_t)g.n_workers);
  w.push_back((uint32_t)g.split);
  w.push_back((uint32_t)g.n_splits);
  w.push_back((uint32_t)g.events.size());
  w.push_back((uint32_t)g.tasks.size());
  w.push_back((uint32_t)g.n_slots);
  for (uint32_t i = 0; i < g.events.size(); ++i) {
    w.push_back(i);
    w.push_back(g.events[i].fanin);
    w.push_back(g.events[i].slot0);
  }
  for (uint32_t i = 0; i < g.tasks.size(); ++i) {
    const TaskRec& t = g.tasks[i];
    w.push_back(i);
    w.push_back(t.op);
    w.push_back(t.layer);
    w.push_back(t.tile);
    w.push_back(t.a0);
    w.push_back(t.a1);
    w.push_back(t.wait_ev);
    w.push_back(t.wait_ev == EV_NONE ? 0u : g.events[t.wait_ev].fanin);
    w.push_back(t.wait_lag);
    w.push_back(t.sig_ev);
    w.push_back(t.sig_slot);
    w.push_back(g.task_cu[i]);
  }
  std::vector<uint8_t> bytes(w.size() * 4);
  for (size_t i = 0; i < w.size(); ++i) {
    bytes[4 * i + 0] = (uint8_t)(w[i] & 0xff);
    bytes[4 * i + 1] = (uint8_t)((w[i] >> 8) & 0xff);
    bytes[4 * i + 2] = (uint8_t)((w[i] >> 16) & 0xff);
    bytes[4 * i + 3] = (uint8_t)((w[i] >> 24) & 0xff);
  }
  return bytes;
}

}  // namespace mk
