// Fixed device scratch for callers that cannot allocate device memory (code
// under graph capture, tight serving loops): pa_decode_noalloc keeps its work
// plan, the in-launch merge counters and the split-KV partials in one
// file-scope device array of kScratchBytes per GPU instead of library- or
// caller-allocated buffers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kernels.hpp"

namespace pa {

constexpr size_t kScratchBytes = size_t{32} << 20;           // per GPU, held until the process ends
constexpr size_t kScratchCounterBytes = size_t{64} << 10;     // [0, 64 KiB): merge counters
constexpr size_t kScratchPlanOffset = kScratchCounterBytes;   // [64 KiB, 1 MiB): work plan
constexpr size_t kScratchPlanBytes = (size_t{1} << 20) - kScratchCounterBytes;
constexpr size_t kScratchPartialOffset = size_t{1} << 20;     // [1 MiB, 32 MiB): split-KV partials
constexpr size_t kScratchPartialBytes = kScratchBytes - kScratchPartialOffset;

// Device address of the scratch array on `device`, which must be the current
// device.  Looked up with hipGetSymbolAddress on the first call for a device
// and kept; later calls return the kept address.
hipError_t scratch_address(int device, char** out);

// Write `n` int32 words from the kernel arguments to `dst` and zero `n_zero`
// words at `zero_dst` (one launch; n <= kInlineWords).
hipError_t launch_words(int32_t* dst, const InlineMeta& words, int n, uint32_t* zero_dst, int n_zero,
                        hipStream_t stream);

}  // namespace pa
