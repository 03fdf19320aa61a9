// Opt-in kernel timing (declared in include/oft.h): a fixed list of HIP event
// pairs recorded on the launch stream around the library's kernel launches.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "oft.h"
#include "oft_launch.h"
#include "oft_prof.h"

namespace oft {
namespace {

constexpr int MAXREC = 1024;
constexpr int NAMELEN = 32;
struct Rec {
  char name[NAMELEN];
  hipEvent_t a, b;
};
std::mutex g_mu;
std::atomic<bool> g_on{false};
bool g_events = false;
int g_n = 0;
Rec g_rec[MAXREC];

}  // namespace

bool prof_on() { return g_on.load(std::memory_order_relaxed); }

int prof_begin(hipStream_t st, const char* name) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_on.load(std::memory_order_relaxed) || g_n >= MAXREC) return -1;
  Rec& r = g_rec[g_n];
  strncpy(r.name, name, NAMELEN - 1);
  r.name[NAMELEN - 1] = '\0';
  if (hipEventRecord(r.a, st) != hipSuccess) return -1;
  return g_n++;
}

void prof_end(hipStream_t st, int slot) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (slot >= 0 && slot < g_n) (void)hipEventRecord(g_rec[slot].b, st);
}

}  // namespace oft

extern "C" {

int32_t oft_prof_enable(int32_t on) {
  using namespace oft;
  std::lock_guard<std::mutex> lock(g_mu);
  if (on && !g_events) {
    for (int i = 0; i < MAXREC; ++i) {
      if (hipEventCreate(&g_rec[i].a) != hipSuccess || hipEventCreate(&g_rec[i].b) != hipSuccess) {
        set_last_hip_error(static_cast<int>(hipGetLastError()));
        return OFT_EHIP;
      }
    }
    g_events = true;
  }
  if (on) g_n = 0;  // stopping keeps the records readable
  g_on.store(on != 0, std::memory_order_relaxed);
  return OFT_OK;
}

int32_t oft_prof_count(void) {
  std::lock_guard<std::mutex> lock(oft::g_mu);
  return oft::g_n;
}

int32_t oft_prof_read(int32_t i, char* name, int32_t name_len, float* ms) {
  using namespace oft;
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (i < 0 || i >= g_n || name == nullptr || name_len < 1 || ms == nullptr) return OFT_EINVAL;
    strncpy(name, g_rec[i].name, (size_t)name_len - 1);
    name[name_len - 1] = '\0';
    a = g_rec[i].a;
    b = g_rec[i].b;
  }
  hipError_t e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  if (e != hipSuccess) {
    set_last_hip_error(static_cast<int>(e));
    return OFT_EHIP;
  }
  return OFT_OK;
}

}  // extern "C"
