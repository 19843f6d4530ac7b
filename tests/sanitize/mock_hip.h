// Controls and records of the mock HIP runtime (mock_hip.cpp).
#pragma once
#include <stddef.h>
#include <stdint.h>

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
}  // namespace mock
