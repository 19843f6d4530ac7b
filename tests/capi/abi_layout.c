/*
 * Prints the size of every struct of include/xfer.h and the offset of each of
 * its fields, as compiled by a plain C compiler, one "struct field offset"
 * line each ("struct . size" for the size).  tests/test_capi_cpu.py compares
 * them with the Python binding's ctypes and numpy layouts, and also calls a
 * few host-only entry points from C.
 */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "xfer.h"

#define SIZE(T) printf("%s . %zu\n", #T, sizeof(T))
#define FIELD(T, f) printf("%s %s %zu\n", #T, #f, offsetof(T, f))

int main(void) {
  SIZE(xfer_shard);
  FIELD(xfer_shard, ptr); FIELD(xfer_shard, ld); FIELD(xfer_shard, rows); FIELD(xfer_shard, ncols);
  FIELD(xfer_shard, col_offset);
  SIZE(xfer_max_idx);
  FIELD(xfer_max_idx, max); FIELD(xfer_max_idx, idx);
  SIZE(xfer_top2);
  FIELD(xfer_top2, top1); FIELD(xfer_top2, top2); FIELD(xfer_top2, idx); FIELD(xfer_top2, reserved);
  SIZE(xfer_run_table);
  FIELD(xfer_run_table, n_lanes); FIELD(xfer_run_table, n_blocks); FIELD(xfer_run_table, seg_bytes);
  FIELD(xfer_run_table, n_runs); FIELD(xfer_run_table, runs_per_lane); FIELD(xfer_run_table, run_base);
  FIELD(xfer_run_table, run_stride); FIELD(xfer_run_table, run_count);
  SIZE(xfer_region);
  FIELD(xfer_region, base); FIELD(xfer_region, bytes);
  SIZE(xfer_runs_plan);
  FIELD(xfer_runs_plan, dev); FIELD(xfer_runs_plan, dev_bytes); FIELD(xfer_runs_plan, n_lanes);
  FIELD(xfer_runs_plan, n_blocks); FIELD(xfer_runs_plan, seg_bytes); FIELD(xfer_runs_plan, n_runs);
  FIELD(xfer_runs_plan, span_lo); FIELD(xfer_runs_plan, span_hi); FIELD(xfer_runs_plan, is_dst);
  FIELD(xfer_runs_plan, tile_blocks); FIELD(xfer_runs_plan, n_tiles); FIELD(xfer_runs_plan, group_blocks);
  FIELD(xfer_runs_plan, n_groups); FIELD(xfer_runs_plan, pieces); FIELD(xfer_runs_plan, magic);
  FIELD(xfer_runs_plan, lanes_per_wg); FIELD(xfer_runs_plan, off_group_run); FIELD(xfer_runs_plan, off_run_start);
  FIELD(xfer_runs_plan, off_run_base); FIELD(xfer_runs_plan, off_run_stride); FIELD(xfer_runs_plan, n_spans);
  FIELD(xfer_runs_plan, reserved); FIELD(xfer_runs_plan, spans);
  SIZE(xfer_desc);
  FIELD(xfer_desc, src); FIELD(xfer_desc, dst_off); FIELD(xfer_desc, bytes);
  SIZE(xfer_descs_plan);
  FIELD(xfer_descs_plan, dev); FIELD(xfer_descs_plan, dev_bytes); FIELD(xfer_descs_plan, n_descs);
  FIELD(xfer_descs_plan, slab_bytes); FIELD(xfer_descs_plan, src_lo); FIELD(xfer_descs_plan, src_hi);
  FIELD(xfer_descs_plan, max_pieces); FIELD(xfer_descs_plan, piece_bytes); FIELD(xfer_descs_plan, magic);
  FIELD(xfer_descs_plan, reserved); FIELD(xfer_descs_plan, n_spans); FIELD(xfer_descs_plan, reserved2);
  FIELD(xfer_descs_plan, spans);
  SIZE(xfer_pages);
  FIELD(xfer_pages, indices); FIELD(xfer_pages, stride); FIELD(xfer_pages, offset);
  SIZE(xfer_pages_plan);
  FIELD(xfer_pages_plan, dev); FIELD(xfer_pages_plan, dev_bytes); FIELD(xfer_pages_plan, n_pages);
  FIELD(xfer_pages_plan, page_len); FIELD(xfer_pages_plan, src_base); FIELD(xfer_pages_plan, src_stride);
  FIELD(xfer_pages_plan, dst_base); FIELD(xfer_pages_plan, dst_stride); FIELD(xfer_pages_plan, off_src_idx);
  FIELD(xfer_pages_plan, off_dst_idx); FIELD(xfer_pages_plan, units_per_page); FIELD(xfer_pages_plan, magic);
  SIZE(xfer_op);
  FIELD(xfer_op, kind); FIELD(xfer_op, rank); FIELD(xfer_op, chunk); FIELD(xfer_op, slot); FIELD(xfer_op, stream);
  FIELD(xfer_op, n_waits); FIELD(xfer_op, wait_event); FIELD(xfer_op, record_event);
  SIZE(xfer_allreduce2_desc);
  FIELD(xfer_allreduce2_desc, src); FIELD(xfer_allreduce2_desc, send); FIELD(xfer_allreduce2_desc, recv);
  FIELD(xfer_allreduce2_desc, out); FIELD(xfer_allreduce2_desc, n); FIELD(xfer_allreduce2_desc, chunk_bytes);
  FIELD(xfer_allreduce2_desc, ring_bytes); FIELD(xfer_allreduce2_desc, out_mode);
  FIELD(xfer_allreduce2_desc, compute); FIELD(xfer_allreduce2_desc, wire); FIELD(xfer_allreduce2_desc, events);
  FIELD(xfer_allreduce2_desc, n_events);

  /* host-only calls from C: a 2-lane table encoded, the schedule and the graph's edge count */
  const uint64_t addrs[6] = {0x1000, 0x2000, 0x3000, 0x9000, 0x8000, 0x7000};
  uint32_t rpl[2], cnt[6];
  uint64_t base[6], nr = 0;
  int64_t stride[6];
  int st = xfer_runs_encode(addrs, 2, 3, 0, rpl, base, stride, cnt, 6, &nr);
  printf("call runs_encode %d %llu %u %u %lld %lld\n", st, (unsigned long long)nr, rpl[0], rpl[1],
         (long long)stride[0], (long long)stride[1]);
  xfer_op ops[18];
  size_t n_ops = 0, n_deps = 0;
  st = xfer_allreduce2_schedule(3, 2, ops, 18, &n_ops);
  printf("call schedule %d %zu %u %u\n", st, n_ops, ops[2].kind, ops[2].stream);
  st = xfer_allreduce2_graph_deps(3, 2, NULL, NULL, 0, &n_deps);
  printf("call graph_deps %d %zu\n", st, n_deps);
  printf("call status %s\n", strcmp(xfer_status_str(XFER_E_TABLE), "") ? "named" : "empty");
  return 0;
}
