// kvq_noalloc.hip -- the library's own scratch array, for kvq_paged_decode_noalloc:
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the decode's
// split-K workspace from a fixed-size array that every GPU the library runs
// on holds for the life of the process.
//
// The array's name is only a host-side stand-in for it: the device address
// is taken once per device with hipGetSymbolAddress (with that device
// current) and used everywhere the host needs the memory.  Every call on a
// GPU shares that GPU's array and leaves its contents behind, so calls that
// overlap on one GPU race; each call clears the arrival counters its plan
// uses before the decode runs.
#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

// 64 MiB: enough for the decode of every shape this library is measured on
// (the 163840-token 576/512 slab with 128 heads needs 32.3 MiB, a batch of
// 64 with up to 131072 tokens 16.8 MiB).
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_pointer(void** p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = ptr;
  }
  *p = g_ptr[dev];
  return hipSuccess;
}

hipError_t launch_zero_words(void* p, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  zero_words_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace kvq
