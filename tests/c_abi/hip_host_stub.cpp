// Host-only stand-ins for the HIP calls of the cache storage code (kdcache.cpp), so
// that its background threads can run under ThreadSanitizer and AddressSanitizer
// on a machine without a GPU: "pinned" buffers come from malloc, "device" buffers
// are host memory, and an asynchronous copy runs at once, so an event has always
// completed when it is waited for.  Test infrastructure only; linked in place of
// the HIP runtime.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

extern "C" {

hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int) {
  *ptr = std::malloc(size ? size : 1);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipHostFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
  *event = (hipEvent_t)std::malloc(8);
  return *event ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipEventDestroy(hipEvent_t event) {
  std::free(event);
  return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}

}  // extern "C"
