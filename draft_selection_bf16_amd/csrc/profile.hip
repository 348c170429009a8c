// profile.hip -- kernel timing hook of the C ABI (dflash2_profile_start /
// dflash2_profile_stop): for each launch of one armed kernel tag, a start and
// a stop event recorded by the kernel's dispatch itself (hipExtLaunchKernel),
// i.e. the kernel's own execution interval.  Host code only.
#include <string.h>

#include <vector>

#include "dflash2.h"
#include "df2_internal.h"

namespace {

struct ProfState {
  char tag[64] = "";
  bool armed = false;
  int max = 0;
  int n = 0;
  std::vector<hipEvent_t> start, stop;
};
thread_local ProfState g_prof;

}  // namespace

namespace df2 {

ProfileScope::ProfileScope(const char* tag, hipStream_t s) : on(false), start(nullptr), stop(nullptr) {
  (void)s;
  ProfState& P = g_prof;
  if (!tag || !P.armed || P.n >= P.max || strcmp(tag, P.tag) != 0) return;
  start = P.start[P.n];
  stop = P.stop[P.n];
  on = true;
}

void ProfileScope::used() { g_prof.n++; }

}  // namespace df2

extern "C" {

int dflash2_profile_start(const char* kernel, int max_launches) {
  ProfState& P = g_prof;
  if (!kernel || max_launches < 1 || strlen(kernel) >= sizeof P.tag) return DF2_ERR_SHAPE;
  while ((int)P.start.size() < max_launches) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return DF2_ERR_HIP;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return DF2_ERR_HIP;
    }
    P.start.push_back(a);
    P.stop.push_back(b);
  }
  strcpy(P.tag, kernel);
  P.max = max_launches;
  P.n = 0;
  P.armed = true;
  return DF2_OK;
}

int dflash2_profile_stop(float* ms, int max, int* n) {
  ProfState& P = g_prof;
  P.armed = false;
  int k = 0;
  for (int i = 0; i < P.n; ++i) {
    if (hipEventSynchronize(P.stop[i]) != hipSuccess) return DF2_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, P.start[i], P.stop[i]) != hipSuccess) return DF2_ERR_HIP;
    if (ms && k < max) ms[k] = t;
    ++k;
  }
  if (n) *n = k < max ? k : max;
  P.n = 0;
  return DF2_OK;
}

}  // extern "C"
