// Host-side task graph of one decode step (internal to libmk).
//
// Task/event contract from the MPK blog translation ("MPK compiler" section,
// Figure 2): one dependent event and one triggering event per task; an
// event's threshold is the number of tasks that trigger it.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mk.h"

namespace mk {

// most sequences one launch decodes; the default attention chunking is sized
// for a group of this many
constexpr int32_t kGroupCols = 4;
constexpr int32_t kMfmaCols = 16;  // sequences one launch of the matrix-core bodies handles
constexpr int32_t kMfmaRowBlock = 16;  // rows of one matrix-core row block

enum TaskType : int32_t {
  T_EMB = 0, T_QKV = 1, T_ATT = 2, T_COMB = 3, T_O = 4, T_GU = 5, T_D = 6, T_LM = 7, T_ARGMAX = 8,
  T_COUNT = 9
};

struct Task {
  int32_t type, layer, b, g, chunk, row0, row1, dep, trig, cu;
};

struct Event {
  int32_t threshold, first_dependent, n_dependents;
};

struct Graph {
  mk_model_desc desc;
  mk_graph_opts opts;  // resolved: no zero fields
  std::vector<Task> tasks;
  std::vector<Event> events;
  std::vector<std::vector<int32_t>> queues;  // per compute unit, ascending task ids
  // operator segments in global order: [begin, end) task ranges of one operator
  std::vector<std::pair<int32_t, int32_t>> ops;
};

// Returns MK_OK or an error code with *err filled.
int build_graph(const mk_model_desc& d, const mk_graph_opts* o, Graph* out, std::string* err);
std::vector<uint8_t> serialize(const Graph& g);

}  // namespace mk

struct mk_graph {
  mk::Graph g;
};
