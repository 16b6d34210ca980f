// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// the C-ABI layer makes, so that layer (sparse_kv_amd/csrc/api.hip) can be
// built with the host sanitizers and driven without a GPU.  Every launcher
// records its call; nothing here touches device memory.
#include <stdint.h>
#include <string.h>

#include "kernels.hpp"

extern "C" {
int stub_launches = 0;           // launcher calls since the last reset
const void* stub_last_ptr[4];    // state pointers of the last decode / merge launch
int stub_last_S = 0;             // splits of the last decode launch (rows of the last merge)
int stub_device_count = 1;
void stub_reset(void) {
  stub_launches = 0;
  memset(stub_last_ptr, 0, sizeof stub_last_ptr);
  stub_last_S = 0;
}
}

static int current_device = 0;

hipError_t hipGetDevice(int* d) {
  if (!d) return hipErrorInvalidValue;
  *d = current_device;
  return stub_device_count > 0 ? hipSuccess : hipErrorNoDevice;
}
hipError_t hipSetDevice(int d) {
  if (d < 0 || d >= stub_device_count) return hipErrorInvalidDevice;
  current_device = d;
  return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) { return hipGetDevice(d); }
// the "device address" of a symbol is its host address here
hipError_t hipGetSymbolAddress(void** p, const void* sym) {
  if (!p || !sym) return hipErrorInvalidSymbol;
  *p = const_cast<void*>(sym);
  return hipSuccess;
}

namespace skv {

hipError_t launch_decode(const DecodeArgs& a, bool, hipStream_t) {
  ++stub_launches;
  stub_last_ptr[0] = a.m;
  stub_last_ptr[1] = a.l;
  stub_last_ptr[2] = a.o;
  stub_last_S = a.S;
  return hipSuccess;
}
hipError_t launch_merge(int32_t rows, int32_t, int32_t, const float* m, const float* l, const float* o, float* out,
                        float*, float*, hipStream_t) {
  ++stub_launches;
  stub_last_ptr[0] = m;
  stub_last_ptr[1] = l;
  stub_last_ptr[2] = o;
  stub_last_ptr[3] = out;
  stub_last_S = rows;
  return hipSuccess;
}
hipError_t launch_merge2(int32_t rows, int32_t, int32_t, int32_t, const float* m, const float* l, const float* o,
                         float* out, hipStream_t) {
  ++stub_launches;
  stub_last_ptr[0] = m;
  stub_last_ptr[1] = l;
  stub_last_ptr[2] = o;
  stub_last_ptr[3] = out;
  stub_last_S = rows;
  return hipSuccess;
}
hipError_t launch_build_centroids(const void*, const int32_t*, float*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                  hipStream_t, PagedK) {
  ++stub_launches;
  return hipSuccess;
}
hipError_t launch_update_centroids(const void*, const int32_t*, const int32_t*, float*, int32_t, int32_t, int32_t,
                                   int32_t, int32_t, int32_t, hipStream_t, PagedK) {
  ++stub_launches;
  return hipSuccess;
}
hipError_t launch_score(const void*, const float*, const int32_t*, float*, int32_t, int32_t, int32_t, int32_t,
                        int32_t, int32_t, float, hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}
hipError_t launch_topk(const float*, const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                       int32_t*, int32_t*, hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}
hipError_t launch_art(const ArtArgs&, hipStream_t, void*, size_t) {
  ++stub_launches;
  return hipSuccess;
}
size_t art_workspace_bytes(int32_t units, int32_t G, int32_t d) {
  if (units < 1 || units > kArtMcMaxUnits) return 0;
  return (size_t)units * (G > 4 ? 2 : 1) * (d == 128 ? 4096 : 2048);
}
hipError_t launch_super_centroids(const float*, const int32_t*, float*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                  hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}
hipError_t launch_two_level(const void*, const float*, const float*, const int32_t*, int32_t, int32_t, int32_t,
                            int32_t, int32_t, int32_t, float, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                            int32_t*, int32_t*, hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}
hipError_t launch_order(const float*, const int32_t*, int32_t, int32_t, int32_t, int32_t*, hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

}  // namespace skv
