// Opt-in kernel timing for measurement (oft_prof_* in oft.h).  Off by
// default: a region then costs one relaxed load.  When on, a region records
// a HIP event on its launch stream before and after the kernels it wraps.
#pragma once

#include <hip/hip_runtime.h>

namespace oft {

bool prof_on();
// slot of the new record, or -1 (recording off, list full, event error)
int prof_begin(hipStream_t st, const char* name);
void prof_end(hipStream_t st, int slot);

// RAII region around the launches of one step of a call
class ProfScope {
 public:
  ProfScope(hipStream_t st, const char* name) : st_(st), slot_(prof_on() ? prof_begin(st, name) : -1) {}
  ~ProfScope() {
    if (slot_ >= 0) prof_end(st_, slot_);
  }
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  hipStream_t st_;
  int slot_;
};

}  // namespace oft
