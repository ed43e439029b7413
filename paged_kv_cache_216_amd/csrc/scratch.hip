// The fixed device scratch of pa_decode_noalloc (see scratch.hpp) and the
// launch that fills it from kernel arguments, so that the call needs no
// staging buffer, no allocation and no host-to-device copy.
#include "scratch.hpp"

#include <mutex>

namespace pa {
namespace {

// One copy per GPU, at its own address on each.  In host code this name is a
// stand-in, not a device address: the address comes from hipGetSymbolAddress.
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_addr[kMaxDevices] = {};

constexpr int kWordThreads = 256;

__global__ __launch_bounds__(kWordThreads) void words_kernel(int32_t* dst, InlineMeta w, int n, uint32_t* zdst,
                                                             int nz) {
  const int i = blockIdx.x * kWordThreads + threadIdx.x;
  if (i < n) dst[i] = w.w[i];
  if (i < nz) zdst[i] = 0u;
}

}  // namespace

hipError_t scratch_address(int device, char** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_addr[device] = static_cast<char*>(ptr);
  }
  *out = g_addr[device];
  return hipSuccess;
}

hipError_t launch_words(int32_t* dst, const InlineMeta& words, int n, uint32_t* zero_dst, int n_zero,
                        hipStream_t stream) {
  if (n < 0 || n > kInlineWords || n_zero < 0) return hipErrorInvalidValue;
  const int work = n > n_zero ? n : n_zero;
  if (work == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((work + kWordThreads - 1) / kWordThreads));
  hipLaunchKernelGGL(words_kernel, grid, dim3(kWordThreads), 0, stream, dst, words, n, zero_dst, n_zero);
  return hipGetLastError();
}

}  // namespace pa
