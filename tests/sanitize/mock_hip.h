// Controls and records of the mock HIP runtime (mock_hip.cpp).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace mock {
struct LaunchLog {
  const char *name;
  uint64_t a, b, c;
};
extern LaunchLog g_last;  // the last launch
extern long g_launches;   // launches so far
void reset_failures();
void fail_event_create_at(int k);  // the k-th event create from now fails (no handle written)
void fail_event_record_at(int k);
void fail_memcpy_at(int k);
size_t live_events();
void fail_launches(bool on);       // every launcher returns an error while on
void fail_scratch(bool on);        // the static argmax array's lookup fails while on
// Graphs: the nodes of the last instantiated graph, in creation order, with
// their dependencies as node indices; kinds 0 pack, 1 wire copy, 2 combine.
struct GraphNodeLog {
  int kind;
  std::vector<uint32_t> deps;
  uint64_t n;  // elements (pack, combine) or bytes (copy)
};
extern std::vector<GraphNodeLog> g_last_graph;
extern long g_live_graphs, g_live_execs, g_graph_launches;
void fail_graph_node_at(int k);     // the k-th node added from now fails
void fail_instantiate(bool on);
void fail_new_after(long k);       // the host allocation k allocations from now throws (-1: none)
bool new_failure_pending();        // set and not yet thrown
}  // namespace mock
