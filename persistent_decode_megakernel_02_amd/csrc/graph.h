// graph.h -- host-side task-graph builder (pure C++, no GPU).
#pragma once
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {

struct Graph {
  int n_workers = 0;
  int chunk = 0;  // prefill graph: tokens per step (virtual sequences); 0: the decode graph
  int split = 0, n_splits = 0;
  int qkv_tiles_per_group = 0, n_qkv = 0, n_wo = 0, n_gu = 0, n_down = 0, n_lm = 0;
  int n_slots = 0;
  std::vector<EventRec> events;
  std::vector<TaskRec> tasks;       // global topological order of one decode step
  std::vector<uint32_t> task_cu;    // worker of each task
  std::vector<uint32_t> list_off, list_len, cu_tasks;  // per-worker ordered task lists
  struct Range { uint32_t first, count; };
  std::vector<Range> op_ranges;     // operator instances of one step, in topological order
  // [op_ranges.size() + 1][n_workers]: position in worker w's list of its first task of range r
  // (row op_ranges.size(): the list lengths), so a per-operator launch finds each worker's tasks
  std::vector<uint32_t> range_start;
  int rotate = 0, attn_offset = 0;  // placement (see build_graph)
  int wo_ksplit = 1, down_ksplit = 1;  // K parts of the O- and down-projection tiles
  int qkv_ksplit = 1;                  // K parts of the QKV tiles (within a KV-head group)
};

// The schedule choices of one graph: what the offline search varies (tile counts per operator,
// the attention split, where each operator's tasks sit on the workers).  0 in a field of
// mk_model_cfg means the frozen default for the shape (frozen_schedule).
struct Schedule {
  int split = 0;       // positions per attention task (0: the default rule)
  int qkv_tiles = 0;   // QKV tiles per KV-head group
  int wo_tiles = 0, gu_tiles = 0, down_tiles = 0, lm_tiles = 0;
  int rotate = 0;      // GEMV operator k of a layer (QKV 0, WO 1, GU 2, DOWN 3; LM 4): tile i on worker i + k rotate
  int attn_offset = 0; // attention task k on worker k + attn_offset
  int wo_ksplit = 0, down_ksplit = 0;  // K parts per row tile of WO / DOWN (batch >= 2; 0: plain rule, 1: none)
  int qkv_ksplit = 0;                  // ... of the QKV tiles of a KV-head group (batch >= 8)
};

// The search's winner for cfg's shape and batch at n_workers (all fields 0 where it has none).
Schedule frozen_schedule(const mk_model_cfg& cfg, int n_workers);

// Validate the shape and build the graph; returns "" or an error message.
std::string build_graph(const mk_model_cfg& cfg, int n_workers, Graph* g);

// The prefill graph: one step takes `chunk` consecutive prompt tokens of one sequence as the
// columns ("virtual sequences") of every GEMV, so the projections run as a skinny GEMM (on the
// matrix cores at 16 columns).  Per layer an append task per KV-head group writes the chunk's
// rotated keys and values to the cache after QKV, and the attention tasks (virtual sequence b at
// its own position) wait for it; no LM head; layer 0 of step s waits for the last layer of step
// s - 1.  The split is the decode graph's, so attention adds the same partials.
std::string build_prefill_graph(const mk_model_cfg& cfg, int n_workers, int chunk, int split, Graph* g);
std::vector<uint8_t> serialize_graph(const mk_model_cfg& cfg, const Graph& g);

constexpr int kDefaultSplit = 32;  // smallest default split (positions per attention task)

}  // namespace mk
