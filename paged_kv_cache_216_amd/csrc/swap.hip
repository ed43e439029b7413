// Block swap between the device pool and pinned host memory: the second tier
// of a KV cache that spills from GPU memory to host RAM (ranksignal.fr post
// 218, "Mettre en cache", tiers G1 / G2).  The kernel reads or writes the host
// image directly through its device-visible address, 16 bytes per thread, so
// one launch moves a whole sequence whatever its block placement.
#include "swap.hpp"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One thread per 16-byte chunk of the K and V images of all blocks.
__global__ __launch_bounds__(256) void swap_kernel(SwapParams p) {
  const long long chunks = static_cast<long long>(p.block_bytes / 16);
  const long long per_pool = chunks * p.n_blocks;
  const long long w = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (w >= 2 * per_pool) return;
  const bool is_v = w >= per_pool;
  const long long c = is_v ? w - per_pool : w;
  const int i = static_cast<int>(c / chunks);  // logical block
  const long long ci = c - static_cast<long long>(i) * chunks;
  const size_t pool_off = static_cast<size_t>(p.blocks[i]) * p.block_bytes + ci * 16;
  const size_t host_off = static_cast<size_t>(i) * p.block_bytes + ci * 16;
  char* pool = (is_v ? p.v_pool : p.k_pool) + pool_off;
  char* host = (is_v ? p.v_host : p.k_host) + host_off;
  if (p.to_host) {
    *reinterpret_cast<u32x4*>(host) = *reinterpret_cast<const u32x4*>(pool);
    return;
  }
  if (i < p.n_blocks - 1 || p.last_rows >= 16) {
    *reinterpret_cast<u32x4*>(pool) = *reinterpret_cast<const u32x4*>(host);
    return;
  }
  // last, partly filled block: only the slots of rows < last_rows, so that
  // the rest of the block keeps what it held
  if (!is_v) {
    // K: each 16-byte chunk holds one token's slice (token = chunk % 16)
    if ((ci & 15) < p.last_rows) *reinterpret_cast<u32x4*>(pool) = *reinterpret_cast<const u32x4*>(host);
    return;
  }
  // V: lines of 16 tokens of one (head, dim); byte b of the line is token b / elem_bytes
  const int pos = static_cast<int>((ci * 16) % p.line_bytes);
  for (int b = 0; b < 16; ++b)
    if ((pos + b) / p.elem_bytes < p.last_rows) pool[b] = host[b];
}

}  // namespace

hipError_t launch_swap(const SwapParams& p, hipStream_t stream) {
  if (p.n_blocks <= 0) return hipSuccess;
  const long long work = 2LL * (p.block_bytes / 16) * p.n_blocks;
  const dim3 grid(static_cast<unsigned>((work + 255) / 256));
  hipLaunchKernelGGL(swap_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
