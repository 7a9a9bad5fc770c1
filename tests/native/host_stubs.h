// The workspace the stand-in launchers check carved arrays against, and their counters.
#pragma once
#include <stddef.h>

namespace hoststub {
struct Workspace {
  void* base;
  size_t bytes;
};
extern Workspace g_ws;
extern int g_launches;   // launchers called
extern int g_errors;     // carved arrays outside the workspace or misaligned
void carved(const char* what, const void* p, size_t bytes, size_t align = 256);
// Arrays carved since the last call must not overlap (one array recorded twice is one array);
// clears the record.  Returns the number of overlapping pairs.
int check_disjoint();
}  // namespace hoststub
