// Working memory of oscar_int2_decode_attn_noalloc: a file-scope device array
// that every call on a GPU shares, so the call allocates nothing (for callers
// that cannot allocate: graph capture, tight serving loops).
//
// Layout of the array (byte offsets):
//   [0, kCounterBytes)                  per-(sequence, kv head) block counters of the
//                                       head_dim-128 attention kernel; zero between calls (the
//                                       last block of a launch resets its counter)
//   [kCounterBytes, kStaticScratchBytes)   carved per call: q records, rotated q,
//                                       partial results; nothing there must start at 0
// The counter region has a fixed place, so a call never finds another call's
// records where it expects zero counters.  It is cleared once per device, when
// the device's address of the array is first taken.
#include <mutex>

#include "common.h"

namespace oscar {

// The array itself: one copy on every GPU the library runs on, held until the
// process ends.  In host code its name is only a stand-in, never a device
// address: the device's address comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

__global__ __launch_bounds__(256) void clear_words_kernel(unsigned* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
unsigned char* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(int device, hipStream_t stream, unsigned char** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    // the caller has made `device` current; the symbol's address is that
    // device's copy of the array (the name itself is only a host stand-in)
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    const size_t words = kCounterBytes / 4;
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       static_cast<unsigned*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[device] = static_cast<unsigned char*>(p);
  }
  *ptr = g_ptr[device];
  return hipSuccess;
}

}  // namespace oscar
