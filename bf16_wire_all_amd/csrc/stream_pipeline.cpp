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

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

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

// Enqueue the work of one operation on stream st.
hipError_t issue(const xfer_allreduce2_desc *d, const Call &c, const xfer_op &op, hipStream_t st) {
  const uint64_t e0 = (uint64_t)op.chunk * c.ce;
  const uint64_t len = (d->n - e0 < c.ce) ? d->n - e0 : c.ce;
  const uint64_t soff = (uint64_t)op.slot * c.ce;  // element offset of the slot
  const uint32_t r = op.rank;
  if (op.kind == XFER_OP_PACK) return xfer::launch_pack(d->src[r] + e0, len, d->send[r], c.R * c.ce, soff, st);
  if (op.kind == XFER_OP_WIRE)
    return hipMemcpyAsync(d->recv[1 - r] + soff, d->send[r] + soff, len * 2, hipMemcpyDeviceToDevice, st);
  // rank 0's value first on both ranks
  const uint16_t *a = (r == 0) ? d->send[0] + soff : d->recv[1] + soff;
  const uint16_t *b = (r == 0) ? d->recv[0] + soff : d->send[1] + soff;
  void *o = static_cast<uint8_t *>(d->out[r]) + e0 * c.out_esize;
  return xfer::launch_combine(a, b, len, o, d->out_mode, st);
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
  // Recording the schedule by stream capture on private streams crashed the
  // host process inside this call on MI355X (ROCm 7.2) and the cause is not
  // found, so building the graph is switched off: every non-empty call is
  // refused before any runtime call.
  return XFER_E_UNSUPPORTED;
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
