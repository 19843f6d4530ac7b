// The mock HIP runtime (mock_hip/hip/hip_runtime_api.h) and stand-ins for the
// kernel launchers of libxfer's .hip files, for the sanitizer build of the
// library's host code.  Launchers record what they were asked to launch and
// touch the buffers they were given at their first and last byte, so a
// wrong size or pointer handed to a launch shows up under the sanitizers.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <set>

#include "internal.h"
#include "mock_hip.h"

namespace {
std::set<hipEvent_t> g_events;
int g_create_calls = 0;
int g_fail_create_at = -1;   // the create call (0-based) that fails, -1 none
int g_record_calls = 0;
int g_fail_record_at = -1;
int g_memcpy_calls = 0;
int g_fail_memcpy_at = -1;
bool g_fail_launches = false;
bool g_fail_scratch = false;
int g_node_calls = 0;
int g_fail_node_at = -1;
bool g_fail_instantiate = false;
long g_new_countdown = -1;  // host allocations by the code under test before one fails, -1 none
int g_new_suspended = 0;    // inside the mock runtime, whose own allocations never fail

// The mock runtime's own bookkeeping allocates; a failure injected for the
// library's host code must not land there.
struct MockBookkeeping {
  MockBookkeeping() { ++g_new_suspended; }
  ~MockBookkeeping() { --g_new_suspended; }
};

[[noreturn]] void die(const char *what) {
  std::fprintf(stderr, "mock hip: %s\n", what);
  std::abort();
}

void check_event(hipEvent_t e) {
  if (!g_events.count(e)) die("unknown or destroyed event");
}
}  // namespace

// Every scalar new of the program goes through here, so a test can make the
// k-th allocation of the library's host code fail (std::bad_alloc).
void *operator new(std::size_t n) {
  if (g_new_countdown >= 0 && g_new_suspended == 0) {
    if (g_new_countdown == 0) {
      g_new_countdown = -1;
      throw std::bad_alloc();
    }
    --g_new_countdown;
  }
  if (void *p = std::malloc(n ? n : 1)) return p;
  throw std::bad_alloc();
}
void operator delete(void *p) noexcept { std::free(p); }
void operator delete(void *p, std::size_t) noexcept { std::free(p); }

namespace mock {
LaunchLog g_last;
long g_launches = 0;

void reset_failures() {
  g_fail_create_at = g_fail_record_at = g_fail_memcpy_at = -1;
  g_create_calls = g_record_calls = g_memcpy_calls = 0;
  g_fail_launches = false;
  g_fail_scratch = false;
  g_fail_node_at = -1;
  g_node_calls = 0;
  g_fail_instantiate = false;
}
void fail_launches(bool on) { g_fail_launches = on; }
void fail_scratch(bool on) { g_fail_scratch = on; }
std::vector<GraphNodeLog> g_last_graph;
long g_live_graphs = 0, g_live_execs = 0, g_graph_launches = 0;
void fail_graph_node_at(int k) { g_node_calls = 0; g_fail_node_at = k; }
void fail_instantiate(bool on) { g_fail_instantiate = on; }
void fail_new_after(long k) { g_new_countdown = k; }
bool new_failure_pending() { return g_new_countdown >= 0; }
void fail_event_create_at(int k) { g_create_calls = 0; g_fail_create_at = k; }
void fail_event_record_at(int k) { g_record_calls = 0; g_fail_record_at = k; }
void fail_memcpy_at(int k) { g_memcpy_calls = 0; g_fail_memcpy_at = k; }
size_t live_events() { return g_events.size(); }
}  // namespace mock

extern "C" {

hipError_t hipMemcpy(void *dst, const void *src, size_t bytes, hipMemcpyKind kind) {
  if (g_memcpy_calls++ == g_fail_memcpy_at) return hipErrorOutOfMemory;
  if (kind != hipMemcpyHostToDevice) die("unexpected copy kind");
  if (bytes && (!dst || !src)) die("NULL copy operand");
  if (bytes) std::memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind kind, hipStream_t) {
  if (kind != hipMemcpyDeviceToDevice) die("unexpected async copy kind");
  if (bytes && (!dst || !src)) die("NULL copy operand");
  if (bytes) std::memmove(dst, src, bytes);
  return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t *event, unsigned) {
  MockBookkeeping bookkeeping;
  if (!event) die("NULL event slot");
  if (g_create_calls++ == g_fail_create_at) return hipErrorOutOfMemory;  // leaves *event as it was
  hipEvent_t e = reinterpret_cast<hipEvent_t>(std::malloc(16));
  g_events.insert(e);
  *event = e;
  return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t event) {
  MockBookkeeping bookkeeping;
  check_event(event);
  g_events.erase(event);
  std::free(event);
  return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t event, hipStream_t) {
  check_event(event);
  if (g_record_calls++ == g_fail_record_at) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t hipEventSynchronize(hipEvent_t event) {
  check_event(event);
  return hipSuccess;
}

hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t event, unsigned) {
  check_event(event);
  return hipSuccess;
}

}  // extern "C"

// ---- graphs: nodes are recorded with their dependencies
struct hipGraphNode {
  uint32_t index;
};
struct ihipGraph {
  std::vector<hipGraphNode *> nodes;
  std::vector<mock::GraphNodeLog> log;
};
struct hipGraphExec {
  std::vector<mock::GraphNodeLog> log;
};

namespace {
hipError_t add_logged(hipGraphNode_t *node, hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, int kind,
                      uint64_t n) {
  MockBookkeeping bookkeeping;
  if (!node || !g) die("graph node: NULL node slot or graph");
  if (n_deps && !deps) die("graph node: NULL dependencies");
  if (g_node_calls++ == g_fail_node_at) return hipErrorInvalidValue;
  mock::GraphNodeLog rec{kind, {}, n};
  for (size_t j = 0; j < n_deps; ++j) {
    if (!deps[j]) die("graph node: NULL dependency");
    bool found = false;
    for (hipGraphNode *m : g->nodes) found |= (m == deps[j]);
    if (!found) die("graph node: a dependency from another graph or unknown");
    rec.deps.push_back(deps[j]->index);
  }
  hipGraphNode *nd = new hipGraphNode{(uint32_t)g->nodes.size()};
  g->nodes.push_back(nd);
  g->log.push_back(rec);
  *node = nd;
  return hipSuccess;
}
}  // namespace

namespace mock {
hipError_t add_node_for_test(hipGraphNode_t *node, hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, int kind,
                             uint64_t n) {
  return add_logged(node, g, deps, n_deps, kind, n);
}
}  // namespace mock

extern "C" {

hipError_t hipGraphCreate(hipGraph_t *graph, unsigned) {
  MockBookkeeping bookkeeping;
  if (!graph) die("graph create: NULL slot");
  *graph = new ihipGraph;
  ++mock::g_live_graphs;
  return hipSuccess;
}

hipError_t hipGraphDestroy(hipGraph_t graph) {
  MockBookkeeping bookkeeping;
  if (!graph) die("graph destroy: NULL");
  for (hipGraphNode *n : graph->nodes) delete n;
  delete graph;
  --mock::g_live_graphs;
  return hipSuccess;
}

hipError_t hipGraphAddMemcpyNode1D(hipGraphNode_t *node, hipGraph_t graph, const hipGraphNode_t *deps, size_t n_deps,
                                   void *dst, const void *src, size_t bytes, hipMemcpyKind kind) {
  if (kind != hipMemcpyDeviceToDevice) die("graph copy: unexpected kind");
  if (bytes && (!dst || !src)) die("graph copy: NULL operand");
  if (bytes) {  // the operands must hold `bytes` bytes
    const volatile uint8_t *d = static_cast<const volatile uint8_t *>(dst);
    const volatile uint8_t *s = static_cast<const volatile uint8_t *>(src);
    (void)(d[0] ^ d[bytes - 1] ^ s[0] ^ s[bytes - 1]);
  }
  return add_logged(node, graph, deps, n_deps, 1, bytes);
}

hipError_t hipGraphAddKernelNode(hipGraphNode_t *, hipGraph_t, const hipGraphNode_t *, size_t,
                                 const hipKernelNodeParams *) {
  die("direct kernel node");
}

hipError_t hipGraphInstantiateWithFlags(hipGraphExec_t *exec, hipGraph_t graph, unsigned long long) {
  MockBookkeeping bookkeeping;
  if (!exec || !graph) die("instantiate: NULL");
  if (g_fail_instantiate) return hipErrorInvalidValue;
  *exec = new hipGraphExec{graph->log};
  mock::g_last_graph = graph->log;
  ++mock::g_live_execs;
  return hipSuccess;
}

hipError_t hipGraphLaunch(hipGraphExec_t exec, hipStream_t) {
  if (!exec) die("graph launch: NULL");
  ++mock::g_graph_launches;
  return hipSuccess;
}

hipError_t hipGraphExecDestroy(hipGraphExec_t exec) {
  MockBookkeeping bookkeeping;
  if (!exec) die("graph exec destroy: NULL");
  delete exec;
  --mock::g_live_execs;
  return hipSuccess;
}

}  // extern "C"

hipError_t hipLaunchKernel(const void *, dim3, dim3, void **, size_t, hipStream_t) { die("direct kernel launch"); }

// ---- stand-ins for the launchers defined next to the kernels
namespace {
// Read the first and the last byte of [p, p + bytes): the sanitizers flag a
// buffer that is smaller than the launch was told.
uint8_t touch(const void *p, uint64_t bytes) {
  if (!bytes) return 0;
  const volatile uint8_t *b = static_cast<const volatile uint8_t *>(p);
  return b[0] ^ b[bytes - 1];
}
hipError_t note(const char *name, uint64_t a, uint64_t b, uint64_t c) {
  if (g_fail_launches) return hipErrorInvalidValue;  // the runtime refuses the launch
  mock::g_last = mock::LaunchLog{name, a, b, c};
  ++mock::g_launches;
  return hipSuccess;
}
}  // namespace

namespace xfer {

hipError_t launch_pack(const float *src, uint64_t n, uint16_t *ring, uint64_t ring_elems, uint64_t slot0,
                       hipStream_t) {
  if (slot0 >= ring_elems) die("pack: slot outside the ring");
  touch(src, n * 4);
  touch(ring, ring_elems * 2);
  return note("pack", n, ring_elems, slot0);
}

hipError_t launch_combine(const uint16_t *a, const uint16_t *b, uint64_t n, void *out, int mode, hipStream_t) {
  touch(a, n * 2);
  touch(b, n * 2);
  touch(out, n * (mode == XFER_OUT_F32 ? 4 : 2));
  return note("combine", n, (uint64_t)mode, 0);
}

hipError_t node_pack(hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, hipGraphNode_t *node, const float *src,
                     uint64_t n, uint16_t *ring, uint64_t ring_elems, uint64_t slot0) {
  if (slot0 >= ring_elems) die("pack node: slot outside the ring");
  touch(src, n * 4);
  touch(ring, ring_elems * 2);
  return mock::add_node_for_test(node, g, deps, n_deps, 0, n);
}

hipError_t node_combine(hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, hipGraphNode_t *node,
                        const uint16_t *a, const uint16_t *b, uint64_t n, void *out, int mode) {
  touch(a, n * 2);
  touch(b, n * 2);
  touch(out, n * (mode == XFER_OUT_F32 ? 4 : 2));
  return mock::add_node_for_test(node, g, deps, n_deps, 2, n);
}

hipError_t launch_combine_f32(const float *a, const float *b, uint64_t n, void *out, int mode, hipStream_t) {
  touch(a, n * 4);
  touch(b, n * 4);
  touch(out, n * (mode == XFER_OUT_F32 ? 4 : 2));
  return note("combine_f32", n, (uint64_t)mode, 0);
}

uint32_t argmax_splits(uint32_t rows, uint32_t ncols0, uint32_t ncols1) {
  (void)ncols0;
  (void)ncols1;
  return rows > 512 ? 1 : 4;
}

uint64_t argmax_workspace_bytes(uint32_t rows, uint32_t splits) { return (uint64_t)rows * 2 * splits * 8; }

hipError_t launch_argmax(ArgmaxShard s0, ArgmaxShard s1, uint32_t rows, int mode, void *out, void *workspace,
                         uint32_t splits, hipStream_t) {
  for (const ArgmaxShard &s : {s0, s1}) touch(s.ptr, ((uint64_t)(rows - 1) * s.ld + s.ncols) * 2);
  touch(out, (uint64_t)rows * (mode == XFER_ARGMAX ? 8 : 16));
  touch(workspace, argmax_workspace_bytes(rows, splits));
  return note("argmax", rows, (uint64_t)mode, splits);
}

// The library's static argmax array: host memory of the same size here.
hipError_t argmax_scratch(void **ptr) {
  alignas(256) static uint8_t buf[kArgmaxScratchBytes];
  if (g_fail_scratch) return hipErrorInvalidValue;
  *ptr = buf;
  return hipSuccess;
}

hipError_t launch_gather(const PlanView &p, void *staging, hipStream_t) {
  touch(staging, (uint64_t)p.n_lanes * p.n_blocks * p.seg_bytes);
  touch(p.run_stride, 8);
  return note("gather", p.n_lanes, p.n_blocks, p.pieces);
}

hipError_t launch_scatter(const PlanView &p, const void *staging, hipStream_t) {
  touch(staging, (uint64_t)p.n_lanes * p.n_blocks * p.seg_bytes);
  touch(p.run_stride, 8);
  return note("scatter", p.n_lanes, p.n_blocks, p.pieces);
}

hipError_t launch_copy_descs(const xfer_desc *descs, uint64_t n_descs, uint32_t max_pieces, void *, hipStream_t) {
  touch(descs, n_descs * sizeof(xfer_desc));
  return note("copy_descs", n_descs, max_pieces, 0);
}

hipError_t launch_paged_copy(const PagesView &v, hipStream_t) {
  const uint64_t n_pages = v.units_per_page ? v.n_units / v.units_per_page : 0;
  touch(v.src_idx, n_pages * 4);
  touch(v.dst_idx, n_pages * 4);
  if (v.span == 0 || v.pieces == 0) die("paged copy: empty launch shape");
  return note("paged_copy", v.n_units, v.span, v.pieces);
}

}  // namespace xfer
