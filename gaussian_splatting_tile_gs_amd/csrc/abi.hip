// Host glue of the C ABI: status strings, the thread-local last error, camera validation and
// the optional per-kernel event timing used for measurement.
#include <cmath>
#include <cstring>
#include <vector>

#include "gs_internal.h"

namespace gs {

namespace {
thread_local std::string g_last_error;

struct TimingRec {
  const char* name;
  hipEvent_t start, stop;
};
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;
const char* g_pending_name = nullptr;
hipEvent_t g_pending_start = nullptr;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

gs_status set_error(gs_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

gs_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(GS_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
  return GS_OK;
}

bool valid_camera(const gs_camera* cam, std::string* why) {
  if (!cam) {
    *why = "camera is NULL";
    return false;
  }
  if (cam->width <= 0 || cam->height <= 0) {
    *why = "camera width/height <= 0";
    return false;
  }
  for (int i = 0; i < 16; ++i)
    if (!std::isfinite(cam->viewmat[i])) {
      *why = "non-finite viewmat";
      return false;
    }
  const float f[8] = {cam->fx, cam->fy, cam->cx, cam->cy, cam->near_plane,
                      cam->background[0], cam->background[1], cam->background[2]};
  for (float v : f)
    if (!std::isfinite(v)) {
      *why = "non-finite intrinsics, near plane or background";
      return false;
    }
  if (!(cam->fx > 0.0f) || !(cam->fy > 0.0f)) {
    *why = "fx/fy must be > 0";
    return false;
  }
  if ((cam->radius_mode != 0 && cam->radius_mode != 1) || (cam->antialiased != 0 && cam->antialiased != 1) ||
      (cam->tight_tiles != 0 && cam->tight_tiles != 1)) {
    *why = "radius_mode, antialiased and tight_tiles must be 0 or 1";
    return false;
  }
  return true;
}

void timing_begin(const char* name, hipStream_t stream) {
  if (!g_timing) return;
  g_pending_name = name;
  g_pending_start = take_event();
  if (g_pending_start) (void)hipEventRecord(g_pending_start, stream);
}

void timing_end(hipStream_t stream) {
  if (!g_timing || !g_pending_start) return;
  hipEvent_t stop = take_event();
  if (!stop) return;
  (void)hipEventRecord(stop, stream);
  g_recs.push_back({g_pending_name, g_pending_start, stop});
  g_pending_start = nullptr;
}

}  // namespace gs

using namespace gs;

extern "C" const char* gs_status_string(gs_status s) {
  switch (s) {
    case GS_OK: return "GS_OK";
    case GS_ERR_INVALID_ARG: return "GS_ERR_INVALID_ARG";
    case GS_ERR_CAPACITY: return "GS_ERR_CAPACITY";
    case GS_ERR_LIMIT: return "GS_ERR_LIMIT";
    case GS_ERR_DEVICE: return "GS_ERR_DEVICE";
  }
  return "GS_ERR_UNKNOWN";
}

extern "C" const char* gs_last_error(void) { return g_last_error.c_str(); }

extern "C" gs_status gs_timing_enable(int32_t on) {
  g_timing = on != 0;
  return GS_OK;
}

extern "C" int32_t gs_timing_collect(const char** names, float* ms, int32_t max) {
  int32_t written = 0;
  for (const TimingRec& r : g_recs) {
    float t = 0.0f;
    if (hipEventSynchronize(r.stop) == hipSuccess) (void)hipEventElapsedTime(&t, r.start, r.stop);
    if (written < max && names && ms) {
      names[written] = r.name;
      ms[written] = t;
      ++written;
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  return written;
}
