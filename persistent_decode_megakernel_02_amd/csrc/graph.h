// graph.h -- host-side task-graph builder (pure C++, no GPU).
#pragma once
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {

struct Graph {
  int n_workers = 0;
  int split = 0, n_splits = 0;
  int qkv_tiles_per_group = 0, n_qkv = 0, n_wo = 0, n_gu = 0, n_down = 0, n_lm = 0;
  int n_slots = 0;
  std::vector<EventRec> events;
  std::vector<TaskRec> tasks;       // global topological order of one decode step
  std::vector<uint32_t> task_cu;    // worker of each task
  std::vector<uint32_t> list_off, list_len, cu_tasks;  // per-worker ordered task lists
  struct Range { uint32_t first, count; };
  std::vector<Range> op_ranges;     // operator instances of one step, in topological order
};

// Validate the shape and build the graph; returns "" or an error message.
std::string build_graph(const mk_model_cfg& cfg, int n_workers, Graph* g);
std::vector<uint8_t> serialize_graph(const mk_model_cfg& cfg, const Graph& g);

constexpr int kDefaultSplit = 32;  // smallest default split (positions per attention task)

}  // namespace mk
