// Streamed two-rank all-reduce of the copy-engine page ("Change"): per chunk,
// pack on each rank's compute stream, copy into the peer's receive ring on
// the rank's wire stream, combine on the compute stream; R slots alternate;
// streams are ordered by events only.
//
// The schedule is produced by one generator, used both by
// xfer_allreduce2_schedule (so the ordering can be checked on the host) and by
// the executor, which issues each operation as it is generated (no host
// allocation in the call).
//
// Hazards per slot s of rank r (chunk c reuses the slot of chunk c - R):
//   send[r][s]  written by PACK r c; read by WIRE r c and COMBINE r c.
//               PACK r c waits SENT[r][s] (the wire copy of chunk c - R is
//               done); COMBINE r c - R precedes it on the same stream, except
//               for the first R chunks of a call, whose slot was last read by
//               the previous call, maybe on other streams: they also wait
//               COMBINED[r][s].
//   recv[1-r][s] written by WIRE r c; read by COMBINE 1-r c.
//               WIRE r c waits PACKED[r][s] (its input is ready) and
//               COMBINED[1-r][s] (the peer's sum of chunk c - R is done);
//               COMBINE 1-r c waits SENT[r][s].
// Events are created already recorded (complete), so the waits of the first
// R chunks of a call are satisfied at once, or wait for a previous call that
// used the same events and rings.
//
// With R >= 2 the two write-after-read waits are implied from chunk R on, so
// they are issued only for the first R chunks (each pending cross-stream wait
// costs the runtime 12-19 us of host time on MI355X).  For chunk c >= R:
//   WIRE r (c - R) -> COMBINE 1-r (c - R) -> [stream] PACK 1-r (c - R + 1)
//     -> WIRE 1-r (c - R + 1) -> COMBINE r (c - R + 1) -> [stream] PACK r c,
// so PACK r c is ordered after the copy out of its slot without its own wait
// (c - R + 1 <= c - 1), and
//   COMBINE 1-r (c - R) -> [stream] PACK 1-r (c - 1) -> WIRE 1-r (c - 1)
//     -> COMBINE r (c - 1) -> [stream] PACK r c -> WIRE r c,
// so WIRE r c is ordered after the peer's sum of the slot's previous chunk
// through its PACKED wait.  The first R chunks keep both waits: they order the
// call after the previous one, which may have used other streams.
#include <cstring>
#include <vector>

#include "internal.h"

namespace {

constexpr uint32_t kStreams = 4;  // compute 0, compute 1, wire 0, wire 1

uint32_t event_id(uint32_t kind, uint32_t rank, uint32_t slot, uint32_t R) { return (kind * 2 + rank) * R + slot; }

// Calls visit(op) for every operation in issue order.
template <typename Visit>
bool for_each_op(uint32_t n_chunks, uint32_t R, Visit &&visit) {
  for (uint32_t c = 0; c < n_chunks; ++c) {
    const uint32_t s = c % R;
    for (uint32_t r = 0; r < 2; ++r) {
      xfer_op op{};
      op.kind = XFER_OP_PACK;
      op.rank = r;
      op.chunk = c;
      op.slot = s;
      op.stream = r;
      if (c < R) {
        // The slot's previous readers may belong to the previous call, on
        // other streams: its copy out and its own combine.
        op.n_waits = 2;
        op.wait_event[0] = event_id(XFER_EV_SENT, r, s, R);
        op.wait_event[1] = event_id(XFER_EV_COMBINED, r, s, R);
      } else if (R == 1) {
        op.n_waits = 1;  // the combine of chunk c - 1 precedes it on this stream
        op.wait_event[0] = event_id(XFER_EV_SENT, r, s, R);
      }
      op.record_event = event_id(XFER_EV_PACKED, r, s, R);
      if (!visit(op)) return false;
    }
    for (uint32_t r = 0; r < 2; ++r) {
      xfer_op op{};
      op.kind = XFER_OP_WIRE;
      op.rank = r;
      op.chunk = c;
      op.slot = s;
      op.stream = 2 + r;
      const bool implied = R >= 2 && c >= R;
      op.n_waits = implied ? 1 : 2;
      op.wait_event[0] = event_id(XFER_EV_PACKED, r, s, R);
      op.wait_event[1] = implied ? 0 : event_id(XFER_EV_COMBINED, 1 - r, s, R);
      op.record_event = event_id(XFER_EV_SENT, r, s, R);
      if (!visit(op)) return false;
    }
    for (uint32_t r = 0; r < 2; ++r) {
      xfer_op op{};
      op.kind = XFER_OP_COMBINE;
      op.rank = r;
      op.chunk = c;
      op.slot = s;
      op.stream = r;
      op.n_waits = 1;
      op.wait_event[0] = event_id(XFER_EV_SENT, 1 - r, s, R);
      op.record_event = event_id(XFER_EV_COMBINED, r, s, R);
      if (!visit(op)) return false;
    }
  }
  return true;
}

// The graph form's dependencies, for every operation in issue order: the
// previous operation on its stream, and for each event it waits on, the last
// operation recorded on that event before it in the same all-reduce (a wait on
// an event not yet recorded in this all-reduce orders it after an earlier
// call, which a graph gets from the launch order of its stream instead).
// visit(op, op index, dependency indices, count).
//
// With more slots than chunks (R > n_chunks) every chunk is among the first R
// and takes slot c either way, so the edges are those of R = n_chunks; the
// operations are generated with that R, which keeps the host table of last
// recorders at 6 * min(R, n_chunks) entries (the visited event ids are then
// numbered for that R; the kinds, ranks, chunks and slots are unchanged).
// Allocates that table (the callers run inside xfer::guarded).
template <typename Visit>
bool for_each_op_deps(uint32_t n_chunks, uint32_t R, Visit &&visit) {
  const uint32_t Re = (n_chunks != 0 && R > n_chunks) ? n_chunks : R;
  int64_t last_on_stream[kStreams];
  for (uint32_t k = 0; k < kStreams; ++k) last_on_stream[k] = -1;
  std::vector<int64_t> last_record(6ull * Re, -1);
  uint64_t i = 0;
  return for_each_op(n_chunks, Re, [&](const xfer_op &op) {
    uint64_t deps[3];
    uint32_t nd = 0;
    auto add = [&](int64_t k) {
      if (k < 0) return;
      for (uint32_t j = 0; j < nd; ++j)
        if (deps[j] == (uint64_t)k) return;
      deps[nd++] = (uint64_t)k;
    };
    add(last_on_stream[op.stream]);
    for (uint32_t w = 0; w < op.n_waits; ++w) add(last_record[op.wait_event[w]]);
    if (!visit(op, i, deps, nd)) return false;
    last_on_stream[op.stream] = (int64_t)i;
    last_record[op.record_event] = (int64_t)i;
    ++i;
    return true;
  });
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

int xfer_allreduce2_graph_deps(uint32_t n_chunks, uint32_t R, uint32_t *from, uint32_t *to, size_t cap,
                               size_t *n_deps) {
  if (R == 0 || !n_deps) return XFER_E_INVAL;
  if (R > UINT32_MAX / 6 || (uint64_t)n_chunks * 6 > UINT32_MAX) return XFER_E_INVAL;
  return xfer::guarded([&]() -> int {
    size_t k = 0;
    bool room = true;
    for_each_op_deps(n_chunks, R, [&](const xfer_op &, uint64_t i, const uint64_t *deps, uint32_t nd) {
      for (uint32_t j = 0; j < nd; ++j, ++k) {
        if (k >= cap) {
          room = false;
        } else if (from && to) {
          from[k] = (uint32_t)deps[j];
          to[k] = (uint32_t)i;
        }
      }
      return true;
    });
    *n_deps = k;
    if (!room) return XFER_E_RANGE;
    if (k && (!from || !to)) return XFER_E_INVAL;
    return XFER_OK;
  });
}

uint32_t xfer_allreduce2_event_id(uint32_t kind, uint32_t rank, uint32_t slot, uint32_t R) {
  return event_id(kind, rank, slot, R);
}

int xfer_allreduce2_schedule(uint32_t n_chunks, uint32_t R, xfer_op *ops, size_t cap, size_t *n_ops) {
  if (R == 0 || !n_ops) return XFER_E_INVAL;
  const uint64_t need = 6ull * n_chunks;
  if (need > cap) return XFER_E_RANGE;
  if (need && !ops) return XFER_E_INVAL;
  size_t k = 0;
  for_each_op(n_chunks, R, [&](const xfer_op &op) {
    ops[k++] = op;
    return true;
  });
  *n_ops = k;
  return XFER_OK;
}

int xfer_events_create(hipEvent_t *events, int n) {
  if (!events || n < 0) return XFER_E_INVAL;
  // Slots start empty, so a failure releases exactly what this call created
  // (a failed create may leave its slot untouched) and leaves every slot NULL.
  for (int i = 0; i < n; ++i) events[i] = nullptr;
  auto release = [&]() {
    for (int j = 0; j < n; ++j)
      if (events[j]) {
        (void)hipEventDestroy(events[j]);
        events[j] = nullptr;
      }
    return XFER_E_DEVICE;
  };
  for (int i = 0; i < n; ++i) {
    // Recorded once and completed, so a first wait on it does not block.
    if (hipEventCreateWithFlags(&events[i], hipEventDisableTiming) != hipSuccess) {
      events[i] = nullptr;
      return release();
    }
    if (hipEventRecord(events[i], nullptr) != hipSuccess) return release();
  }
  for (int i = 0; i < n; ++i)
    if (hipEventSynchronize(events[i]) != hipSuccess) return release();
  return XFER_OK;
}

int xfer_events_destroy(hipEvent_t *events, int n) {
  if (!events || n < 0) return XFER_E_INVAL;
  int st = XFER_OK;
  for (int i = 0; i < n; ++i)
    if (events[i] && hipEventDestroy(events[i]) != hipSuccess) st = XFER_E_DEVICE;
  return st;
}

}  // extern "C"

namespace {

// Shape of one call, from the descriptor's checks.
struct Call {
  uint64_t R, n_chunks, ce, out_esize;
};

// The argument checks shared by the streamed call and the graph builder
// (streams and events are checked by the caller that needs them).
int check_desc(const xfer_allreduce2_desc *d, Call *c) {
  if (!d) return XFER_E_INVAL;
  if (d->out_mode != XFER_OUT_F32 && d->out_mode != XFER_OUT_BF16) return XFER_E_INVAL;
  if (d->chunk_bytes == 0 || d->chunk_bytes % 16) return XFER_E_INVAL;
  if (d->ring_bytes == 0 || d->ring_bytes % d->chunk_bytes) return XFER_E_INVAL;
  c->R = d->ring_bytes / d->chunk_bytes;
  if (c->R > UINT32_MAX / 6) return XFER_E_INVAL;
  c->ce = d->chunk_bytes / 2;
  c->n_chunks = 0;
  c->out_esize = d->out_mode == XFER_OUT_F32 ? 4 : 2;
  if (d->n == 0) return XFER_OK;
  if (d->n > SIZE_MAX / 4) return XFER_E_INVAL;
  c->n_chunks = d->n / c->ce + (d->n % c->ce != 0);
  if (c->n_chunks > UINT32_MAX) return XFER_E_INVAL;
  struct Buf {
    const void *p;
    uint64_t bytes;
  } bufs[8] = {{d->src[0], 4ull * d->n},         {d->src[1], 4ull * d->n},    {d->send[0], d->ring_bytes},
               {d->send[1], d->ring_bytes},      {d->recv[0], d->ring_bytes}, {d->recv[1], d->ring_bytes},
               {d->out[0], c->out_esize * d->n}, {d->out[1], c->out_esize * d->n}};
  for (int i = 0; i < 8; ++i)
    if (!bufs[i].p || !aligned16(bufs[i].p)) return XFER_E_INVAL;
  // The sources may alias each other (both read only); nothing else may share a byte.
  for (int i = 0; i < 8; ++i)
    for (int j = i + 1; j < 8; ++j) {
      if (i == 0 && j == 1) continue;
      const uintptr_t a = (uintptr_t)bufs[i].p, b = (uintptr_t)bufs[j].p;
      if (a < b + bufs[j].bytes && b < a + bufs[i].bytes) return XFER_E_INVAL;
    }
  return XFER_OK;
}

// Operands of one operation: a pack, a wire copy or a combine.
struct OpArgs {
  const float *src;   // PACK: the rank's chunk
  uint16_t *ring;     // PACK: the rank's send ring
  uint64_t len;       // elements of the chunk
  uint64_t soff;      // element offset of the slot
  const void *from;   // WIRE: send slot; COMBINE: rank 0's operand
  void *to;           // WIRE: peer's receive slot
  const uint16_t *a, *b;
  void *out;          // COMBINE: the rank's output at the chunk
};

OpArgs op_args(const xfer_allreduce2_desc *d, const Call &c, const xfer_op &op) {
  OpArgs x{};
  const uint64_t e0 = (uint64_t)op.chunk * c.ce;
  x.len = (d->n - e0 < c.ce) ? d->n - e0 : c.ce;
  x.soff = (uint64_t)op.slot * c.ce;
  const uint32_t r = op.rank;
  x.src = d->src[r] + e0;
  x.ring = d->send[r];
  x.from = d->send[r] + x.soff;
  x.to = d->recv[1 - r] + x.soff;
  // rank 0's value first on both ranks
  x.a = (r == 0) ? d->send[0] + x.soff : d->recv[1] + x.soff;
  x.b = (r == 0) ? d->recv[0] + x.soff : d->send[1] + x.soff;
  x.out = static_cast<uint8_t *>(d->out[r]) + e0 * c.out_esize;
  return x;
}

// Enqueue the work of one operation on stream st.
hipError_t issue(const xfer_allreduce2_desc *d, const Call &c, const xfer_op &op, hipStream_t st) {
  const OpArgs x = op_args(d, c, op);
  if (op.kind == XFER_OP_PACK) return xfer::launch_pack(x.src, x.len, x.ring, c.R * c.ce, x.soff, st);
  if (op.kind == XFER_OP_WIRE) return hipMemcpyAsync(x.to, x.from, x.len * 2, hipMemcpyDeviceToDevice, st);
  return xfer::launch_combine(x.a, x.b, x.len, x.out, d->out_mode, st);
}

// The same operation as a node of graph g after the given nodes.
hipError_t add_op_node(hipGraph_t g, const hipGraphNode_t *deps, size_t nd, hipGraphNode_t *node,
                       const xfer_allreduce2_desc *d, const Call &c, const xfer_op &op) {
  const OpArgs x = op_args(d, c, op);
  if (op.kind == XFER_OP_PACK) return xfer::node_pack(g, deps, nd, node, x.src, x.len, x.ring, c.R * c.ce, x.soff);
  if (op.kind == XFER_OP_WIRE)
    return hipGraphAddMemcpyNode1D(node, g, deps, nd, x.to, x.from, x.len * 2, hipMemcpyDeviceToDevice);
  return xfer::node_combine(g, deps, nd, node, x.a, x.b, x.len, x.out, d->out_mode);
}

}  // namespace

extern "C" {

int xfer_allreduce2_streamed(const xfer_allreduce2_desc *d) {
  Call c;
  const int st0 = check_desc(d, &c);
  if (st0 != XFER_OK || c.n_chunks == 0) return st0;
  // The schedule names event ids up to 6 * R - 1.
  if (!d->events || d->n_events < 6 * c.R) return XFER_E_INVAL;
  hipStream_t streams[kStreams] = {d->compute[0], d->compute[1], d->wire[0], d->wire[1]};
  hipError_t err = hipSuccess;
  for_each_op((uint32_t)c.n_chunks, (uint32_t)c.R, [&](const xfer_op &op) {
    hipStream_t st = streams[op.stream];
    for (uint32_t w = 0; w < op.n_waits; ++w)
      if ((err = hipStreamWaitEvent(st, d->events[op.wait_event[w]], 0)) != hipSuccess) return false;
    if ((err = issue(d, c, op, st)) != hipSuccess) return false;
    err = hipEventRecord(d->events[op.record_event], st);
    return err == hipSuccess;
  });
  return err == hipSuccess ? XFER_OK : XFER_E_DEVICE;
}

int xfer_allreduce2_graph_create(const xfer_allreduce2_desc *d, hipGraphExec_t *exec) {
  if (!exec) return XFER_E_INVAL;
  *exec = nullptr;
  Call c;
  const int st0 = check_desc(d, &c);
  if (st0 != XFER_OK || c.n_chunks == 0) return st0;
  if (6 * c.n_chunks > UINT32_MAX) return XFER_E_INVAL;
  // Nodes with explicit dependencies; no stream capture, and the descriptor's
  // streams and events are not used.
  return xfer::guarded([&]() -> int {
    std::vector<hipGraphNode_t> nodes(6 * c.n_chunks, nullptr);
    struct Owned {  // the graph is released on every way out, a host allocation failure included
      hipGraph_t g = nullptr;
      ~Owned() {
        if (g) (void)hipGraphDestroy(g);
      }
    } owned;
    if (hipGraphCreate(&owned.g, 0) != hipSuccess) return XFER_E_DEVICE;
    hipGraph_t g = owned.g;
    hipError_t err = hipSuccess;
    auto add = [&](const xfer_op &op, uint64_t i, const uint64_t *deps, uint32_t nd) {
      hipGraphNode_t dn[3];  // a stream predecessor and at most two event waits
      for (uint32_t j = 0; j < nd; ++j) dn[j] = nodes[deps[j]];
      err = add_op_node(g, dn, nd, &nodes[i], d, c, op);
      return err == hipSuccess;
    };
    for_each_op_deps((uint32_t)c.n_chunks, (uint32_t)c.R, add);
    hipGraphExec_t e = nullptr;
    if (err == hipSuccess) err = hipGraphInstantiateWithFlags(&e, g, 0);
    if (err != hipSuccess) return XFER_E_DEVICE;  // the executable graph keeps what it needs of g
    *exec = e;
    return XFER_OK;
  });
}

int xfer_allreduce2_graph_launch(hipGraphExec_t exec, hipStream_t stream) {
  if (!exec) return XFER_OK;
  return hipGraphLaunch(exec, stream) == hipSuccess ? XFER_OK : XFER_E_DEVICE;
}

int xfer_allreduce2_graph_destroy(hipGraphExec_t exec) {
  if (!exec) return XFER_OK;
  return hipGraphExecDestroy(exec) == hipSuccess ? XFER_OK : XFER_E_DEVICE;
}

}  // extern "C"
