// Block swap between the device pool and pinned host memory.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

// One sequence's blocks, in logical order, copied between the pool and a
// host image [n_blocks][block bytes] per pool (K and V each), where a block's
// bytes are the pool's own layout of that block for every kv head.
struct SwapParams {
  char* k_pool;
  char* v_pool;
  char* k_host;            // device-visible addresses of the pinned host images
  char* v_host;
  const int32_t* blocks;   // device-visible: physical block of logical block i
  int n_blocks;
  int block_bytes;         // hkv * 16 * head_dim * elem_bytes
  int line_bytes;          // bytes of one V line (16 tokens of one (head, dim)): 16 * elem_bytes
  int elem_bytes;
  int last_rows;           // host -> pool: rows of the last block to restore (1..16)
  int to_host;             // 1: pool -> host (whole blocks), 0: host -> pool
};

hipError_t launch_swap(const SwapParams& p, hipStream_t stream);

}  // namespace pa
