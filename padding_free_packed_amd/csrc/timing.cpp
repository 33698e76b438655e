// Optional per-kernel timing: while enabled, every kernel launch of the library
// is bracketed by two HIP events recorded on the launch's stream (launches
// recorded into a graph under stream capture are not timed). Events come
// from a pool that grows on first use and is reused after each read.
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "kernels.h"
#include "pe.h"

namespace pe {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

constexpr size_t kMaxRecords = 4096;
bool g_on = false;
std::vector<hipEvent_t> g_pool;
size_t g_next = 0;
std::vector<Rec> g_recs;

hipEvent_t take_event() {
  if (g_next == g_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_next++];
}

}  // namespace

hipEvent_t timing_start(hipStream_t stream) {
  if (!g_on || g_recs.size() >= kMaxRecords) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  hipEvent_t e = take_event();
  if (e != nullptr && hipEventRecord(e, stream) != hipSuccess) return nullptr;
  return e;
}

void timing_stop(const char* name, hipEvent_t start, hipStream_t stream) {
  if (start == nullptr) return;
  hipEvent_t e = take_event();
  if (e == nullptr || hipEventRecord(e, stream) != hipSuccess) return;
  g_recs.push_back(Rec{name, start, e});
}

}  // namespace pe

extern "C" {

pe_status pe_timing_enable(int on) {
  pe::g_on = on != 0;
  if (!pe::g_on) {
    pe::g_recs.clear();
    pe::g_next = 0;
  }
  return PE_OK;
}

int pe_timing_read(char* names, float* ms, int max_records) {
  int n = 0;
  for (const pe::Rec& r : pe::g_recs) {
    if (n >= max_records) break;
    float t = -1.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      t = -1.f;
    if (names != nullptr) {
      std::strncpy(names + 32 * n, r.name, 31);
      names[32 * n + 31] = '\0';
    }
    if (ms != nullptr) ms[n] = t;
    ++n;
  }
  pe::g_recs.clear();
  pe::g_next = 0;
  return n;
}

}  // extern "C"
