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
//  * Placement: tile i of the k-th GEMV operator of a layer (QKV 0, WO 1, GU 2,
//    DOWN 3; the LM head 4) goes to worker (i + k * rotate) mod workers, and
//    attention task k to worker (k + attn_offset) mod workers.
//  * Tile counts, the split and the placement form the schedule: either given
//    in the configuration or, by default, the one the offline search froze
//    for the shape (frozen_schedule), else the rules above with rotate =
//    attn_offset = 0.
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

#include "schedule_table.inc"

Schedule frozen_schedule(const mk_model_cfg& c, int n_workers) {
  for (const FrozenSchedule& f : kFrozenSchedules)
    if (f.L == c.n_layers && f.H == c.hidden && f.Hq == c.n_q_heads && f.Hkv == c.n_kv_heads && f.D == c.head_dim &&
        f.F == c.ffn && f.V == c.vocab && f.B == c.batch && f.workers == n_workers && c.max_seq >= f.seq_lo &&
        c.max_seq <= f.seq_hi)
      return f.s;
  return Schedule{};
}

// chunk > 0: the prefill graph (see build_prefill_graph); chunk == 0: the decode graph
static std::string build_graph_impl(const mk_model_cfg& c, int n_workers, int chunk, int chunk_split, Graph* out) {
  Graph g;
  g.chunk = chunk;
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
  Schedule sc;
  if (c.schedule == MK_SCHEDULE_GIVEN) {
    sc.qkv_tiles = c.qkv_tiles;
    sc.wo_tiles = c.wo_tiles;
    sc.gu_tiles = c.gu_tiles;
    sc.down_tiles = c.down_tiles;
    sc.lm_tiles = c.lm_tiles;
    sc.rotate = c.rotate;
    sc.attn_offset = c.attn_offset;
    sc.wo_ksplit = c.wo_ksplit;
    sc.down_ksplit = c.down_ksplit;
    sc.qkv_ksplit = c.qkv_ksplit;
  } else if (c.schedule == MK_SCHEDULE_FROZEN) {
    sc = frozen_schedule(c, n_workers);
  } else {
    return "schedule must be MK_SCHEDULE_FROZEN or MK_SCHEDULE_GIVEN";
  }
  if (c.split > 0) sc.split = c.split;
  // the prefill graph: the plain tiling, the decode graph's split, chunk virtual sequences
  if (chunk > 0) {
    sc = Schedule{};
    sc.split = chunk_split;
  }
  const int B = chunk > 0 ? chunk : c.batch;
  if (sc.qkv_tiles < 0 || sc.wo_tiles < 0 || sc.gu_tiles < 0 || sc.down_tiles < 0 || sc.lm_tiles < 0 || sc.rotate < 0 ||
      sc.attn_offset < 0 || sc.wo_ksplit < 0 || sc.down_ksplit < 0 || sc.qkv_ksplit < 0)
    return "schedule fields must be >= 0";
  if (sc.wo_tiles > n_workers || sc.gu_tiles > n_workers || sc.down_tiles > n_workers || sc.lm_tiles > n_workers)
    return "at most one tile per worker for each GEMV operator";
  int S = sc.split;
  if (S <= 0) {
    const int per = std::max(1, B * Hkv);  // attention tasks per split
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
  const int TG = std::min(sc.qkv_tiles > 0 ? sc.qkv_tiles : std::max(1, n_workers / Hkv), RG);
  g.qkv_tiles_per_group = TG;
  g.n_qkv = TG * Hkv;
  auto tiles = [&](int want, int rows) { return std::min(want > 0 ? want : n_workers, rows); };
  g.n_wo = tiles(sc.wo_tiles, c.hidden);
  g.n_gu = tiles(sc.gu_tiles, c.ffn);
  g.n_down = tiles(sc.down_tiles, c.hidden);
  g.n_lm = tiles(sc.lm_tiles, c.vocab);
  if ((int64_t)g.n_qkv > n_workers) return "QKV tiles (per group times n_kv_heads) exceed the workers";
  // split-K of the O- and down-projection (matrix-core GEMV, K in slices of 2048): the operator's
  // tiles form row tiles of ksplit consecutive tasks, part p taking slices [p nsl / ks, (p+1) nsl / ks)
  // Every tile stages the whole activation of its operator; split, a tile stages only its part of
  // K.  0 takes the plain rule (decode graph, no adapters):
  //  * batch >= 8 (matrix-core GEMV, K in slices of 2048): the larger of 4 and 2 that is at most
  //    the operator's K slices and divides its tile count;
  //  * batch 2 to 4 (fp64 GEMV): the fewest parts (1, 2, 4 or 8) whose K part, staged in fp64 for
  //    every sequence, takes at most 128 KB, so that a part stages once; the next of 2, 4, 8 that
  //    divides the tile count if that one does not (none if no such part divides it);
  //  * batch 1: none (not built: one sequence's activations fit one slice).
  const int kdim[2] = {c.n_q_heads * D, c.ffn};
  const int kslices[2] = {(kdim[0] + 2047) / 2048, (kdim[1] + 2047) / 2048};
  const bool kable = chunk == 0 && c.lora_rank == 0 && c.batch >= 2;
  auto plain_ks = [&](int want, int k, int tiles) {
    if (want > 0) return want;
    if (!kable) return 1;
    if (c.batch >= 8) {
      for (int p : {4, 2})
        if (p <= kslices[k] && tiles % p == 0) return p;
      return 1;
    }
    int p = 1;
    while (p < 8 && (int64_t)((kdim[k] + p - 1) / p) * c.batch * 8 > 131072) p *= 2;
    for (; p <= 8; p *= 2)
      if (tiles % p == 0) return p;
    return 1;
  };
  g.wo_ksplit = plain_ks(sc.wo_ksplit, 0, g.n_wo);
  g.down_ksplit = plain_ks(sc.down_ksplit, 1, g.n_down);
  // QKV (matrix-core GEMV only): the parts of a row tile stay inside one KV-head group; the
  // parts also pass on their sums of squares, for the RMSNorm scale that the last part applies.
  // The plain rule leaves it unsplit: split in two it measured slower on the 8B shape at batch 8
  // and 16 (its row tiles are short, and the partial exchange sits right before attention).
  {
    const int ksq = (c.hidden + 2047) / 2048;
    const int q = sc.qkv_ksplit == 0 ? 1 : sc.qkv_ksplit;
    if (q != 1) {
      if (!kable || c.batch < 8) return "QKV split-K needs the matrix-core GEMV (batch >= 8, decode graph)";
      if (q != 2 && q != 4 && q != 8) return "split-K must be 1, 2, 4 or 8";
      if (TG % q) return "QKV split-K must divide the QKV tiles per KV-head group";
      if (q > ksq) return "split-K larger than the operator's K slices";
    }
    g.qkv_ksplit = q;
  }
  {
    const int ks[2] = {g.wo_ksplit, g.down_ksplit}, nt[2] = {g.n_wo, g.n_down};
    for (int k = 0; k < 2; ++k) {
      if (ks[k] == 1) continue;
      if (!kable) return "split-K is for the decode graph of two or more sequences without adapters";
      if (ks[k] != 2 && ks[k] != 4 && ks[k] != 8) return "split-K must be 1, 2, 4 or 8";
      if (nt[k] % ks[k]) return "split-K must divide the operator's tile count";
      if (c.batch >= 8 && ks[k] > kslices[k]) return "split-K larger than the operator's K slices";
    }
  }
  g.rotate = sc.rotate % n_workers;
  g.attn_offset = sc.attn_offset % n_workers;
  // worker of tile i of the k-th GEMV operator of a layer, and of attention task k
  auto place = [&](int k, uint32_t i) { return (uint32_t)((i + (uint64_t)k * g.rotate) % (uint32_t)n_workers); };
  auto place_att = [&](uint32_t k) { return (uint32_t)((k + (uint64_t)g.attn_offset) % (uint32_t)n_workers); };
  // When every attention task of a layer has a worker of its own, all of a head's splits run
  // at once and each merges a slice of the outputs, signalling its own slot; otherwise the
  // split holding the current position merges everything and signals for its (sequence, head).
  // (never in the prefill graph, whose virtual sequences hold different positions in one step)
  const bool dist = chunk == 0 && (int64_t)g.n_splits * B * Hkv <= n_workers;

  // LoRA: each GEMV operator of a layer spreads the A rows (units) of its adapters over its first
  // tiles, q per tile; QKV 3r rows (A_q, A_k, A_v), WO r, GU r (A_gate, A_up row pairs), DOWN r.
  // The operator's LoRA event (fan-in: the tiles holding A rows) names the step-tagged sums the
  // holders publish; the kernel polls those tags rather than event slots.
  const int lr = c.lora_rank;
  if (lr < 0 || lr > 64 || lr % 8) return "lora_rank must be 0 or a multiple of 8 up to 64";

  // events: per layer [QKV group 0..Hkv-1, ATT, O, A, X], then LM, then (LoRA) per layer the A-row
  // events of QKV, WO, GU and DOWN
  const int per_layer = Hkv + 4;
  auto ev_qkv = [&](int l, int gg) { return (uint32_t)(l * per_layer + gg); };
  auto ev_att = [&](int l) { return (uint32_t)(l * per_layer + Hkv); };
  auto ev_o = [&](int l) { return (uint32_t)(l * per_layer + Hkv + 1); };
  auto ev_a = [&](int l) { return (uint32_t)(l * per_layer + Hkv + 2); };
  auto ev_x = [&](int l) { return (uint32_t)(l * per_layer + Hkv + 3); };
  const uint32_t ev_lm = (uint32_t)(c.n_layers * per_layer);
  auto ev_lora = [&](int l, int k) { return ev_lm + 1u + (uint32_t)(4 * l + k); };
  const int n_tiles[4] = {g.n_qkv, g.n_wo, g.n_gu, g.n_down};
  const int n_arows[4] = {3 * lr, lr, lr, lr};
  int per_tile[4] = {0, 0, 0, 0}, holders[4] = {0, 0, 0, 0};
  for (int k = 0; k < 4 && lr > 0; ++k) {
    per_tile[k] = (n_arows[k] + n_tiles[k] - 1) / n_tiles[k];
    holders[k] = (n_arows[k] + per_tile[k] - 1) / per_tile[k];
  }
  // prefill graph: an append event per (layer, KV-head group) after all others; the appending task
  // writes the group's rotated keys and values of the chunk to the cache before attention reads them
  const uint32_t ev_app0 = ev_lm + 1u + (uint32_t)(lr > 0 ? 4 * c.n_layers : 0);
  auto ev_app = [&](int l, int gg) { return ev_app0 + (uint32_t)(l * Hkv + gg); };
  g.events.resize(ev_app0 + (chunk > 0 ? Hkv * c.n_layers : 0));
  for (int l = 0; l < c.n_layers; ++l) {
    for (int gg = 0; gg < Hkv; ++gg) g.events[ev_qkv(l, gg)].fanin = TG / g.qkv_ksplit;
    g.events[ev_att(l)].fanin = dist ? g.n_splits * B * Hkv : B * Hkv;
    for (int gg = 0; gg < Hkv && chunk > 0; ++gg) g.events[ev_app(l, gg)].fanin = 1;
    g.events[ev_o(l)].fanin = g.n_wo / g.wo_ksplit;
    g.events[ev_a(l)].fanin = g.n_gu;
    g.events[ev_x(l)].fanin = g.n_down / g.down_ksplit;
  }
  g.events[ev_lm].fanin = g.n_lm;
  for (int l = 0; l < c.n_layers && lr > 0; ++l)
    for (int k = 0; k < 4; ++k) g.events[ev_lora(l, k)].fanin = holders[k];
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
    t.lora_ev = EV_NONE;
    const int k = op == OP_QKV ? 0 : op == OP_WO ? 1 : op == OP_GU ? 2 : op == OP_DOWN ? 3 : -1;
    if (lr > 0 && k >= 0) {
      t.la0 = (uint32_t)std::min<int64_t>((int64_t)tile * per_tile[k], n_arows[k]);
      t.la1 = (uint32_t)std::min<int64_t>((int64_t)(tile + 1) * per_tile[k], n_arows[k]);
      t.lora_ev = ev_lora(layer, k);
    }
    t.kp = 0;
    t.kn = 1;
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
    // layer 0 waits for the previous step's LM head (decode) or last layer (prefill: no LM head)
    const uint32_t in_ev = l == 0 ? (chunk > 0 ? ev_x(c.n_layers - 1) : ev_lm) : ev_x(l - 1);
    const uint32_t in_lag = l == 0 ? 1u : 0u;
    uint32_t f = range_begin();
    const int qks = g.qkv_ksplit, nrq = TG / qks;
    for (int gg = 0; gg < Hkv; ++gg)
      for (int i = 0; i < TG; ++i) {
        // split: row tile r = i / qks of the group, part p = i mod qks; only the last part signals
        const int r = i / qks, p = i - r * qks;
        uint32_t tile = (uint32_t)(gg * TG + i);
        uint32_t r0 = (uint32_t)(gg * RG) + tile_lo(r, RG, nrq), r1 = (uint32_t)(gg * RG) + tile_lo(r + 1, RG, nrq);
        push(OP_QKV, l, tile, r0, r1, in_ev, in_lag, p == qks - 1 ? ev_qkv(l, gg) : EV_NONE,
             p == qks - 1 ? (uint32_t)r : 0u, place(0, tile));
        g.tasks.back().kp = (uint32_t)p;
        g.tasks.back().kn = (uint32_t)qks;
      }
    range_end(f);
    if (chunk > 0) {  // prefill: one append task per KV-head group, on the worker of the group's first QKV tile
      f = range_begin();
      for (int gg = 0; gg < Hkv; ++gg)
        push(OP_APPEND, l, (uint32_t)gg, (uint32_t)gg, 0, ev_qkv(l, gg), 0, ev_app(l, gg), 0, place(0, gg * TG));
      range_end(f);
    }
    f = range_begin();
    uint32_t idx = 0;
    for (int s = 0; s < g.n_splits; ++s)
      for (int b = 0; b < B; ++b)
        for (int gg = 0; gg < Hkv; ++gg, ++idx)
          push(OP_ATTN, l, idx, (uint32_t)(b * Hkv + gg), (uint32_t)s, chunk > 0 ? ev_app(l, gg) : ev_qkv(l, gg), 0,
               ev_att(l), dist ? idx : (uint32_t)(b * Hkv + gg), place_att(idx));
    range_end(f);
    f = range_begin();
    // a split row tile: tasks r ks .. r ks + ks - 1; only its last part signals (slot r)
    auto split_tiles = [&](uint32_t op, int l_, int n, int ks, int rows, uint32_t wait, uint32_t sig, int k) {
      const int nr = n / ks;
      for (int i = 0; i < n; ++i) {
        const int r = i / ks, p = i - r * ks;
        push(op, l_, i, tile_lo(r, rows, nr), tile_lo(r + 1, rows, nr), wait, 0, p == ks - 1 ? sig : EV_NONE,
             p == ks - 1 ? (uint32_t)r : 0u, place(k, i));
        g.tasks.back().kp = (uint32_t)p;
        g.tasks.back().kn = (uint32_t)ks;
      }
    };
    split_tiles(OP_WO, l, g.n_wo, g.wo_ksplit, c.hidden, ev_att(l), ev_o(l), 1);
    range_end(f);
    f = range_begin();
    for (int i = 0; i < g.n_gu; ++i)
      push(OP_GU, l, i, tile_lo(i, c.ffn, g.n_gu), tile_lo(i + 1, c.ffn, g.n_gu), ev_o(l), 0, ev_a(l), i,
           place(2, i));
    range_end(f);
    f = range_begin();
    split_tiles(OP_DOWN, l, g.n_down, g.down_ksplit, c.hidden, ev_a(l), ev_x(l), 3);
    range_end(f);
  }
  if (chunk == 0) {  // the prefill graph has no LM head
    uint32_t f = range_begin();
    for (int i = 0; i < g.n_lm; ++i)
      push(OP_LM, 0, i, tile_lo(i, c.vocab, g.n_lm), tile_lo(i + 1, c.vocab, g.n_lm), ev_x(c.n_layers - 1), 0, ev_lm,
           i, place(4, i));
    range_end(f);
  }

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
  const size_t nr = g.op_ranges.size();
  g.range_start.assign((nr + 1) * n_workers, 0);
  for (int w = 0; w < n_workers; ++w) {
    uint32_t j = 0;
    for (size_t r = 0; r < nr; ++r) {
      while (j < g.list_len[w] && g.cu_tasks[g.list_off[w] + j] < g.op_ranges[r].first) ++j;
      g.range_start[r * n_workers + w] = j;
    }
    g.range_start[nr * n_workers + w] = g.list_len[w];
  }
  *out = std::move(g);
  return "";
}

std::string build_graph(const mk_model_cfg& c, int n_workers, Graph* out) {
  return build_graph_impl(c, n_workers, 0, 0, out);
}

std::string build_prefill_graph(const mk_model_cfg& c, int n_workers, int chunk, int split, Graph* out) {
  if (chunk <= 0 || split <= 0) return "chunk and split must be positive";
  return build_graph_impl(c, n_workers, chunk, split, out);
}

// Canonical bytes: little-endian u32 words.
//   header: 'MKG1', version 3, n_workers, split, n_splits, n_events, n_tasks, n_slots
//   events: id, fanin, slot0
//   tasks (topological order): topo, op, layer, tile, a0, a1, wait_ev, wait_fanin, wait_lag,
//                              sig_ev, sig_slot, worker, la0, la1, lora_ev, kp, kn
std::vector<uint8_t> serialize_graph(const mk_model_cfg& c, const Graph& g) {
  (void)c;
  std::vector<uint32_t> w;
  w.push_back(0x31474B4Du);
  w.push_back(3);
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
    w.push_back(t.la0);
    w.push_back(t.la1);
    w.push_back(t.lora_ev);
    w.push_back(t.kp);
    w.push_back(t.kn);
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
