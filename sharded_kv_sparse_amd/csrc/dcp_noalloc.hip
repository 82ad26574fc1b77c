// Static scratch memory of mla_sparse_decode_lse_noalloc: the decode
// entry point for callers that cannot allocate device memory.
//
// The library's scratch is one file-scope device array.  Each GPU the
// library runs on holds its own copy, for the life of the process.  Host code
// never uses the array's name as an address (on the host it only names the
// symbol): at the first call on a device, with that device current, the
// device address is looked up once with hipGetSymbolAddress and kept per
// device; kernels receive that address.
//
// Layout: the first DCP_NOALLOC_COUNTER_BYTES hold the merge's arrival
// counters, whose counts and flags must be clear when a call starts.  They
// are zero when the code object is loaded, are cleared once more by a fill
// kernel queued at the first call on each device, and every decode call
// leaves its counts and flags clear again (a generation byte advances).  The rest holds the per-block partials of the
// fused merge, which each call writes before it reads them.
#include <mutex>

#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    const long long words = kNoallocCounterBytes / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       static_cast<unsigned*>(ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dcp
