// gfx950 (MI355X) kernels for paged KV-cache attention.
//
//  append_kernel     applies pending block-table / length updates, copies the
//                    filled slots of shared blocks before they are written
//                    (copy-on-write), and scatters new K/V rows into their slots.
//  attn_kernel       decode / speculative-verify attention over the block table:
//                    one 64-lane wave per (sequence, partition, key/value head);
//                    QK^T and PV on the matrix cores, online softmax in fp32.
//                    Short splits (one row tile, few partitions) are merged by
//                    the wave that finishes a sequence's last partition, with
//                    device-scope stores and loads of the partials only.
//  attn_append_kernel  the append work and attn_kernel in one launch: the
//                    attention takes the rows this launch appends from k_new /
//                    v_new instead of the pool.
//  tile_kernel       many query rows per (sequence, kv head) -- chunked prefill,
//                    long verifies: four waves share each pair of blocks through
//                    an LDS ring filled by buffer loads with an LDS destination;
//                    each wave's loop is software-pipelined (the PV MFMAs of one
//                    pair run under the softmax of the next).
//  prefix_kernel     the partitions of a prefix shared by copy-on-write forks,
//                    once for the query rows of all of them (four waves per
//                    workgroup, sharing each pair through the same LDS ring).
//  attn_prefix_kernel  attention units and shared-prefix units (and a fused
//                    append) in one launch of four-wave workgroups.
//  merge_rows_kernel the merge of short splits as a launch of its own, after
//                    attn_prefix_kernel: one wave per (split, kv head, 4 rows).
//  merge_kernel      exact log-sum-exp merge of the partitions of split
//                    contexts, as a separate launch for long splits (each XCD
//                    has its own L2, so merging many partitions inside the
//                    attention launch would keep one wave busy after the rest).
//  (graph steps run attn_append_kernel with its grid padded to a batch class,
//  its counts read from the step's metadata in device memory.)
//
// The pages describe the method (16-token blocks reached through a table inside
// the attention kernel: "PagedAttention, décodage spéculatif, MoE et Blackwell",
// section 1; one fused pass that keeps scores and probabilities on chip and
// writes O once: ranksignal.fr post 218, "Les noyaux d'attention").  The tiling
// below is this library's own, built around the gfx950 16x16x32 MFMA.
#include "kernels.hpp"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlk = 16;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();

// ----------------------------------------------------------------------------
// append: table updates + copy-on-write + row scatter
// ----------------------------------------------------------------------------
constexpr int kAppendThreads = 256;

struct AppendGrid {
  int upd_blocks, cow_blocks, row_blocks;
};

__host__ __device__ inline AppendGrid append_grid(const AppendParams& p, int nthreads) {
  AppendGrid g;
  g.upd_blocks = (p.n_tab + p.n_len + nthreads - 1) / nthreads;
  g.cow_blocks = p.n_cow;
  const int chunks_per_row = p.hkv * p.head_dim * p.elem_bytes / 16;
  const long long work = static_cast<long long>(p.n_rows) * chunks_per_row;
  g.row_blocks = static_cast<int>((work + nthreads - 1) / nthreads);
  return g;
}

// Workgroup `b` (of nthreads threads) of the append work.  Table and length
// updates, copies of the filled slots of shared blocks (rows [0, off) only, so
// they never overlap the slots the copying sequence writes; when another
// sequence of the call writes into a copy's source block, the host issues the
// copies in a launch of their own first), and one 16-byte chunk of a new row
// per thread.
// E4M3 code of a float: clamp to the largest finite magnitude (448), then
// round to nearest, ties to even (the conversion instruction's rounding).
__device__ inline uint32_t fp8_pack4(float a, float b, float c, float d) {
  auto cl = [](float x) { return fminf(fmaxf(x, -448.f), 448.f); };
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
}

__device__ inline float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

template <int E>  // element bytes of the pool: 1 (E4M3, bf16 rows in), 2 or 4
__device__ inline void append_work(const AppendParams& p, const int32_t* meta, int b, int nthreads) {
  using Elem = std::conditional_t<E == 1, uint8_t, std::conditional_t<E == 2, uint16_t, uint32_t>>;
  constexpr int X = 16 / E;  // elements per 16-byte chunk of the pool
  const AppendGrid g = append_grid(p, nthreads);
  const int D = p.head_dim;
  const int nchunk = D / X;                               // chunks per (head, slot)
  const size_t page = static_cast<size_t>(D) * kBlk;      // elements per (block, head)
  const int tid = threadIdx.x;

  if (b < g.upd_blocks) {
    const int i = b * nthreads + tid;
    if (i < p.n_tab) {
      p.block_table[meta[p.tab + 2 * i]] = meta[p.tab + 2 * i + 1];
    } else if (i < p.n_tab + p.n_len) {
      const int k = i - p.n_tab;
      p.seq_len[meta[p.lens + 2 * k]] = meta[p.lens + 2 * k + 1];
    }
    return;
  }
  b -= g.upd_blocks;

  if (b < g.cow_blocks) {
    const int src = meta[p.cows + 3 * b], dst = meta[p.cows + 3 * b + 1], rows = meta[p.cows + 3 * b + 2];
    // K: 16-byte chunks (head, chunk, slot < rows)
    const u32x4* ks = reinterpret_cast<const u32x4*>(p.k_pool) + static_cast<size_t>(src) * p.hkv * nchunk * kBlk;
    u32x4* kd = reinterpret_cast<u32x4*>(p.k_pool) + static_cast<size_t>(dst) * p.hkv * nchunk * kBlk;
    const int kwork = p.hkv * nchunk * rows;
    for (int w = tid; w < kwork; w += nthreads) {
      const int t = w % rows;
      const int hc = w / rows;  // head * nchunk + chunk
      kd[hc * kBlk + t] = ks[hc * kBlk + t];
    }
    // V: elements (head, dim, slot < rows)
    const Elem* vs = reinterpret_cast<const Elem*>(p.v_pool) + static_cast<size_t>(src) * p.hkv * page;
    Elem* vd = reinterpret_cast<Elem*>(p.v_pool) + static_cast<size_t>(dst) * p.hkv * page;
    const int vwork = p.hkv * D * rows;
    for (int w = tid; w < vwork; w += nthreads) {
      const int t = w % rows;
      const int hd = w / rows;  // head * D + dim
      vd[hd * kBlk + t] = vs[hd * kBlk + t];
    }
    return;
  }
  b -= g.cow_blocks;

  if constexpr (E == 1) {
    // rows: one thread per 16 bytes (8 bf16) of one row, quantized to 8 codes
    const int per_head = D / 8;
    const int chunks_per_row = p.hkv * per_head;
    const long long w = static_cast<long long>(b) * nthreads + tid;
    if (w >= static_cast<long long>(p.n_rows) * chunks_per_row) return;
    const int row = static_cast<int>(w / chunks_per_row);
    const int c = static_cast<int>(w % chunks_per_row);
    const int h = c / per_head;
    const int cc = c % per_head;  // dims 8 cc .. 8 cc + 7
    const int slot = meta[p.slots + row];
    const u32x4 kv = reinterpret_cast<const u32x4*>(p.k_new)[static_cast<size_t>(row) * chunks_per_row + c];
    const u32x4 vv = reinterpret_cast<const u32x4*>(p.v_new)[static_cast<size_t>(row) * chunks_per_row + c];
    const float ki = p.kv_scale[2 * p.hkv + h], vi = p.kv_scale[3 * p.hkv + h];
    float kf[8], vf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kf[2 * i] = bf16_bits_to_float(kv[i] & 0xFFFFu) * ki;
      kf[2 * i + 1] = bf16_bits_to_float(kv[i] >> 16) * ki;
      vf[2 * i] = bf16_bits_to_float(vv[i] & 0xFFFFu) * vi;
      vf[2 * i + 1] = bf16_bits_to_float(vv[i] >> 16) * vi;
    }
    const int phys = slot / kBlk;
    const int t = slot % kBlk;
    // K: the 8 codes are half of 16-byte chunk cc / 2 of slot t
    uint8_t* kdst = static_cast<uint8_t*>(p.k_pool) +
                    (((static_cast<size_t>(phys) * p.hkv + h) * nchunk + cc / 2) * kBlk + t) * 16 + 8 * (cc & 1);
    *reinterpret_cast<u32x2*>(kdst) = u32x2{fp8_pack4(kf[0], kf[1], kf[2], kf[3]), fp8_pack4(kf[4], kf[5], kf[6], kf[7])};
    // V: one code per dim, kBlk bytes apart
    const uint32_t v0 = fp8_pack4(vf[0], vf[1], vf[2], vf[3]), v1 = fp8_pack4(vf[4], vf[5], vf[6], vf[7]);
    uint8_t* vdst = static_cast<uint8_t*>(p.v_pool) + (static_cast<size_t>(phys) * p.hkv + h) * page +
                    static_cast<size_t>(8 * cc) * kBlk + t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vdst[i * kBlk] = static_cast<uint8_t>(v0 >> (8 * i));
      vdst[(4 + i) * kBlk] = static_cast<uint8_t>(v1 >> (8 * i));
    }
    return;
  }
  // rows: one thread per 16-byte chunk of one row (all heads)
  const int chunks_per_row = p.hkv * nchunk;
  const long long w = static_cast<long long>(b) * nthreads + tid;
  if (w >= static_cast<long long>(p.n_rows) * chunks_per_row) return;
  const int row = static_cast<int>(w / chunks_per_row);
  const int c = static_cast<int>(w % chunks_per_row);  // head * nchunk + chunk
  const int h = c / nchunk;
  const int cc = c % nchunk;
  const int slot = meta[p.slots + row];
  // both 16-byte chunks are read before anything is stored (the stores may
  // alias the sources as far as the compiler knows, which would serialise them)
  const u32x4 kv = reinterpret_cast<const u32x4*>(p.k_new)[static_cast<size_t>(row) * chunks_per_row + c];
  const u32x4 vv = reinterpret_cast<const u32x4*>(p.v_new)[static_cast<size_t>(row) * chunks_per_row + c];
  const int phys = slot / kBlk;
  const int t = slot % kBlk;
  u32x4* kdst = reinterpret_cast<u32x4*>(p.k_pool) +
                ((static_cast<size_t>(phys) * p.hkv + h) * nchunk + cc) * kBlk + t;
  *kdst = kv;
  // V: the chunk's X consecutive dims go to X dims of the slot, kBlk apart
  Elem* vdst = reinterpret_cast<Elem*>(p.v_pool) + (static_cast<size_t>(phys) * p.hkv + h) * page +
               static_cast<size_t>(cc) * X * kBlk + t;
  const auto ve = __builtin_bit_cast(Elem __attribute__((ext_vector_type(X))), vv);
#pragma unroll
  for (int i = 0; i < X; ++i) vdst[i * kBlk] = ve[i];
}

template <int E>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendParams p, InlineMeta im) {
  append_work<E>(p, p.ext ? p.ext : im.w, blockIdx.x, kAppendThreads);
}

// ----------------------------------------------------------------------------
// attention
// ----------------------------------------------------------------------------
// Wave layout (64 lanes, col = lane % 16, grp = lane / 16):
//  * QK^T as S^T = K . Q^T with v_mfma_f32_16x16x32_{bf16,f16}: the A operand is
//    16 tokens x 32 dims of one K page, lane (col, grp) holding token col, dims
//    8*grp..8*grp+7 of the 32-dim step -- one 16-byte load, and with the K page
//    stored [D/8][16][8] the 64 lanes of a load read 1 KiB contiguous.  The B
//    operand is Q^T with query row col.  The result gives lane (col, grp) the
//    scores of query row col for tokens 4*grp..4*grp+3.
//  * That is exactly the A-operand layout of P for O = P . V, so the
//    probabilities stay in registers.  Two blocks (32 tokens) form one PV step:
//    k-slots 0..3 of a lane are tokens 4*grp.. of the first block, 4..7 the same
//    tokens of the second.  The B operand is V with dim col: with the V page
//    stored [D][16] those are 4 consecutive slots = one 8-byte load, 512 B
//    contiguous per wave.
//  * O accumulates in the C layout: lane (col, grp) holds rows 4*grp..+3, dim col
//    of each 16-dim chunk.
//  * Query rows: r = i * group + g for draft i and head g of the group; up to 16
//    rows per tile, NT tiles.  Rows beyond `rows` are zero queries, discarded.
//  * Softmax statistics live in the score layout (row = col); the row max is
//    reduced over the four lane groups with permlane16/32 swaps.  Rescale
//    factors move to the accumulator layout with a lane shuffle.

template <typename T>
struct MfmaOp;
template <>
struct MfmaOp<__bf16> {
  using type = bf16x8;
  static __device__ inline f32x4 mma(type a, type b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct MfmaOp<_Float16> {
  using type = f16x8;
  static __device__ inline f32x4 mma(type a, type b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Maximum of floats as gfx950's v_maximum3_f32 takes it: NaN-propagating, so
// no operand needs quieting first (fmaxf costs a canonicalizing v_max per
// operand in IEEE mode).  Scores of valid tokens are finite; masked ones are
// -inf before any maximum.
__device__ inline float fmax_prop(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ inline float wave_max_groups(float x) {
  // max over lanes col, col+16, col+32, col+48
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax_prop(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_prop(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float wave_sum_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline float shfl_f(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

__device__ inline int readlane(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }

// Buffer resource over one K or V page: loads at byte offsets >= `bytes`
// return zero without a memory access (word 3 is the gfx9 raw-buffer format).
__device__ inline __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// cache policy bit 1 = non-temporal
template <bool NTL>
__device__ inline u32x4 page_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, NTL ? 2 : 0));
}

template <bool NTL>
__device__ inline u32x2 page_load8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, NTL ? 2 : 0));
}

// Without shared blocks every K/V page is read once per launch, so it is
// loaded with the non-temporal hint and streams past the caches instead of
// evicting the tables and queries.  Shared (copy-on-write) blocks are read by
// several sequences and are better kept in cache.

// zero the 16-bit elements of an 8-byte V fragment whose token position >= n
__device__ inline u32x2 mask_v16(u32x2 v, int pos0, int n) {
  u32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t lo = (pos0 + 2 * w < n) ? 0x0000FFFFu : 0u;
    const uint32_t hi = (pos0 + 2 * w + 1 < n) ? 0xFFFF0000u : 0u;
    r[w] = v[w] & (lo | hi);
  }
  return r;
}

__device__ inline f32x4 mask_v32(f32x4 v, int pos0, int n) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (pos0 + e < n) ? v[e] : 0.f;
  return r;
}

template <typename T>
__device__ inline void store_elem(T* p, float v) {
  *p = static_cast<T>(v);
}

// A work unit.  `n_raw` is the sequence length as read (mirror or launch
// metadata); the bodies resolve the token range from it after their first
// loads are issued, so that those loads do not wait for the length.
struct Unit {
  int q_row, seq, n_raw, tok_begin, slot_base, nparts, part, merge;
  int row0, trows;  // this wave's query rows: [row0, row0 + trows) of the call's rows
  int clip_row;     // the last row of the workgroup: no position past what it sees is read
  int pre_row0, pre_member0, pre_rows;  // shared-prefix pass only
};

struct Range {
  int n, tok_end;
};

// (readfirstlane: the length is wave-uniform, and saying so keeps the page
// addresses derived from it in scalar registers)
__device__ inline Range resolve(const AttnParams& p, const Unit& u, int n_raw) {
  Range r;
  r.n = min(__builtin_amdgcn_readfirstlane(n_raw), p.max_blocks * kBlk);  // bounded by the table row
  // a partition covers part_tokens tokens; the last one runs to the end
  r.tok_end = (u.nparts > 1 && u.part < u.nparts - 1) ? min(r.n, u.tok_begin + p.part_tokens) : r.n;
  // causal: no row of the unit sees past the last row's position
  r.tok_end = min(r.tok_end, r.n - p.k_draft + u.clip_row / p.group + 1);
  return r;
}

// Device-scope ("sc1") float store and 16-byte load: coherent across XCDs
// without flushing or invalidating whole L2 caches.
__device__ inline void store_device(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float load_device(const float* a) {
  return __hip_atomic_load(const_cast<float*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kCacheDeviceScope = 16;  // buffer-instruction cache policy: sc1

// Merge of a split (sequence, kv head) inside the attention launch, by the
// wave that arrives last (parts <= kInlineMergeParts; one unit takes all the
// query rows of a (sequence, kv head)).
// Its partial stores are complete (vmcnt 0) before it counts itself in; the
// wave that counts the last partition reads every partition's (m, l, acc) with
// device-scope loads and writes out and lse with the same exact formula as
// merge_kernel, partitions in order:
//   M = max m_q, w_q = 2^(m_q - M), O = sum w_q acc_q / sum w_q l_q.
// Rows go in chunks of 4: lane = 16 * row + column group of D / 16 columns.
// Ordering: the partials are written with device-scope (sc1) stores, which
// go past this XCD's L2, and the writer waits for their completion before its
// atomic increment; the winner issues its device-scope loads only after its
// increment has returned the count of every other partition.  That orders
// exactly the partials, the release and acquire this protocol needs, on this
// memory system.  The C++ release / acquire orders at agent scope instead
// write back and invalidate the whole L2 of the XCD around the atomic:
// measured on MI355X, batch-256 decode 64 -> 95 us and the 70B-like decode
// 54 -> 97 us with an acq_rel increment.
// The merge of one split (sequence, kv head): RG groups of 4 rows per pass,
// each lane taking 16-byte column chunks of one row of a group, the loads of
// all RG groups' partitions issued together; partitions C at a time,
// combined with a running maximum (one chunk: M = max m_q, the weights
// 2^(m_q - M)).  Chunks past the sequence's partitions weigh 0.
// (DEV: the partials were written by other waves of this launch and are read
// at device scope; else a launch boundary lies between, and plain loads see
// them)
template <typename T, int D, int C, int RG, bool DEV>
__device__ inline void merge_rows(const AttnParams& p, const MergeUnit& mu, int kvh, int lane, int r_begin,
                                  int r_end) {
  constexpr int V = D / 64;  // 16-byte column chunks per lane
  const int P = mu.nparts;
  const int rows = r_end;  // rows past r_end repeat row r_end - 1 and are not stored
  const int base = mu.slot_base + kvh * P;
  const auto racc = page_rsrc(p.ws_acc, 0x7ffffff0);
  const int c0 = (lane & 15) * (D / 16);
  for (int r0 = r_begin; r0 < rows; r0 += 4 * RG) {
    int r[RG], rr[RG];
    float M[RG], den[RG];
    f32x4 num[RG][V];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      r[g] = r0 + 4 * g + (lane >> 4);
      rr[g] = r[g] < rows ? r[g] : rows - 1;
      M[g] = kNegInf;
      den[g] = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) num[g][v] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int q0 = 0; q0 < P; q0 += C) {
      float m[RG][C], l[RG][C];
      f32x4 a[RG][C][V];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int q = 0; q < C; ++q) {
          const int qq = min(q0 + q, P - 1);
          const size_t sl = static_cast<size_t>(base + qq) * p.rows + rr[g];
          if constexpr (DEV) {
            m[g][q] = load_device(p.ws_ml + 2 * sl);
            l[g][q] = load_device(p.ws_ml + 2 * sl + 1);
          } else {
            m[g][q] = p.ws_ml[2 * sl];
            l[g][q] = p.ws_ml[2 * sl + 1];
          }
#pragma unroll
          for (int v = 0; v < V; ++v)
            a[g][q][v] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(racc, static_cast<int>((sl * D + c0 + 4 * v) * 4), 0,
                                                             DEV ? kCacheDeviceScope : 0));
        }
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        float Mn = M[g];
#pragma unroll
        for (int q = 0; q < C; ++q) Mn = q0 + q < P ? fmaxf(Mn, m[g][q]) : Mn;
        const float mu_ = (Mn == kNegInf) ? 0.f : Mn;
        const float so = __builtin_amdgcn_exp2f(M[g] - mu_);  // 0 on the first chunk
        den[g] *= so;
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) num[g][v][e] *= so;
#pragma unroll
        for (int q = 0; q < C; ++q) {
          const float w = q0 + q < P ? __builtin_amdgcn_exp2f(m[g][q] - mu_) : 0.f;
          den[g] += w * l[g][q];
#pragma unroll
          for (int v = 0; v < V; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) num[g][v][e] += w * a[g][q][v][e];
        }
        M[g] = Mn;
      }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      if (r[g] < rows) {
        const int i = r[g] / p.group, gg = r[g] - (r[g] / p.group) * p.group;
        const size_t orow = static_cast<size_t>(mu.q_row * p.k_draft + i) * p.hq + kvh * p.group + gg;
        const float inv = 1.f / den[g];
        T* op = static_cast<T*>(p.out) + orow * D + c0;
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) store_elem(op + 4 * v + e, num[g][v][e] * inv);
        if ((lane & 15) == 0 && p.lse) p.lse[orow] = (M[g] + __builtin_amdgcn_logf(den[g])) * kLn2;
      }
    }
  }
}

// Rows [r_begin, r_end) of a split (sequence, kv head), in the shape that
// fits them.  (The same arithmetic in every shape: chunks of C = 8
// partitions, or one chunk of 4 when there are at most 4, where the chunk of
// 8 would add zero weights only.)
template <typename T, int D, bool DEV = true>
__device__ inline void merge_rows_of(const AttnParams& p, const MergeUnit& mu, int kvh, int lane, int r_begin,
                                     int r_end) {
  if (r_end - r_begin <= 4) {
    if (mu.nparts <= 4)
      merge_rows<T, D, 4, 1, DEV>(p, mu, kvh, lane, r_begin, r_end);
    else
      merge_rows<T, D, 8, 1, DEV>(p, mu, kvh, lane, r_begin, r_end);
  } else if (mu.nparts <= 4) {
    merge_rows<T, D, 4, 4, DEV>(p, mu, kvh, lane, r_begin, r_end);
  } else if (mu.nparts <= 8) {
    merge_rows<T, D, 8, 2, DEV>(p, mu, kvh, lane, r_begin, r_end);
  } else {
    merge_rows<T, D, 8, 1, DEV>(p, mu, kvh, lane, r_begin, r_end);
  }
}

// One arrival at split (merge, kvh), counted by the calling lane after its
// wave's (or workgroup's) partial stores have completed; true for the last
// arrival, which also resets the counter for the next launch.
__device__ inline bool merge_arrive(const AttnParams& p, int merge, int kvh) {
  unsigned* ctr = p.merge_ctr + merge * p.hkv + kvh;
  const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // (earlier partitions: a previous launch)
  if (old != static_cast<unsigned>(p.merges[merge].arrivals - 1)) return false;
  __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

template <typename T, int D>
__device__ inline void merge_last(const AttnParams& p, int merge, int kvh) {
  const int lane = threadIdx.x & 63;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores have completed
  bool last = false;
  if (lane == 0) last = merge_arrive(p, merge, kvh);
  if (!__builtin_amdgcn_readfirstlane(static_cast<int>(last))) return;
  // every arrival has counted itself: merge
  merge_rows_of<T, D>(p, p.merges[merge], kvh, lane, 0, p.rows);
}

// Largest amount (log2 domain) by which a score may exceed its row's
// reference maximum before the maximum moves: probabilities stay <= 256.
constexpr float kMaxSlack = 8.f;

// 16-bit element types: bf16 or f16
// E4M3 codes to bf16 (exact: every E4M3 value, subnormals included, is a
// bf16 value).  gfx950 converts two codes per instruction: the low or high
// 16-bit half of a dword (the half select must be an immediate), scale 1.
__device__ inline uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
}

__device__ inline bf16x8 fp8x8_to_bf16(u32x2 w) {
  const u32x4 r = {fp8x2_to_bf16x2(w[0], false), fp8x2_to_bf16x2(w[0], true), fp8x2_to_bf16x2(w[1], false),
                   fp8x2_to_bf16x2(w[1], true)};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ inline u32x2 fp8x4_to_bf16(uint32_t w) { return u32x2{fp8x2_to_bf16x2(w, false), fp8x2_to_bf16x2(w, true)}; }

// The bf16 bits of what an E4M3 pool stores for the bf16 value `h` (bits)
// at reciprocal scale `inv`: the append's rounding (float32 product, clamp,
// nearest even code), decoded back.
__device__ inline uint32_t fp8_requant_bf16(uint32_t h, float inv) {
  const float x = fminf(fmaxf(__uint_as_float(h << 16) * inv, -448.f), 448.f);
  const uint32_t code = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xFFu;
  return __float_as_uint(__builtin_amdgcn_cvt_f32_fp8(code, 0)) >> 16;
}

template <bool NTL>
__device__ inline uint32_t page_load4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, NTL ? 2 : 0));
}

// Q8: the pool holds E4M3 codes (T is bf16): K and V are loaded at one byte
// per element, converted exactly to bf16 in registers, and the per-head
// scales fold into the score scale (K) and the output (V).
// W > 1: the workgroup's W waves take consecutive row blocks of one unit and
// share each pair of blocks through LDS: the pair is fetched once, 16 bytes
// per thread, into one of two LDS buffers while the waves compute on the
// other.  All W waves run the same pair loop (the unit's range is the
// workgroup's), so the barriers line up.
template <typename T, int D, int NT, bool NTL, bool FUSED, bool PREFIX = false, bool Q8 = false, int W = 1,
          bool ONE_PAIR = false>
__device__ inline void attn_body16(const AttnParams& p, const Unit& u, int kvh) {
  static_assert(W == 1 || !FUSED, "LDS-shared pairs: no fused append");
  using Op = typename MfmaOp<T>::type;
  constexpr int KS = D / 32;  // QK k-steps per block
  constexpr int DC = D / 16;  // output dim chunks
  constexpr int kPageBytes = D * kBlk * (Q8 ? 1 : static_cast<int>(sizeof(T)));
  const float sl2 = Q8 ? p.scale_log2 * p.kv_scale[kvh] : p.scale_log2;  // score scale, log2 domain
  const float vsc = Q8 ? p.kv_scale[p.hkv + kvh] : 1.f;
  const int lane = threadIdx.x & 63;  // one wave; the shared-prefix pass runs several per workgroup
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rows = p.rows;
  const int G = p.group;

  using PoolElem = std::conditional_t<Q8, uint8_t, T>;
  const PoolElem* kpool = static_cast<const PoolElem*>(p.k_pool);
  const PoolElem* vpool = static_cast<const PoolElem*>(p.v_pool);
  const size_t page = static_cast<size_t>(D) * kBlk;  // elements (bytes for E4M3) per (block, head)
  const int32_t* bt = p.block_table + static_cast<size_t>(u.seq) * p.max_blocks;
  const int jb0 = u.tok_begin / kBlk;

  // ---- first loads, none of which needs the length: the queries (B operand
  // of S^T = K Q^T) and the first 64 entries of the unit's table row (entries
  // past the row read as zero, entries past the unit are never used).  Tile
  // rows past `rows` repeat the last query row: their softmax is computed and
  // dropped, and it does not touch the other rows.
  // (Shared-prefix pass: tile row r is row r % rows of member r / rows.)
  Op qop[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int q_row = u.q_row, rr;
    if constexpr (PREFIX) {
      const int r = min(u.pre_row0 + nt * 16 + col, u.pre_rows - 1);
      const int j = r / rows;
      rr = r - j * rows;
      q_row = p.pre_members[u.pre_member0 + j].q_row;
    } else {
      rr = u.row0 + min(nt * 16 + col, u.trows - 1);
    }
    const int i = rr / G, g = rr - i * G;
    const T* qp = static_cast<const T*>(p.q) + (static_cast<size_t>(q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qop[nt][s] = __builtin_bit_cast(Op, *reinterpret_cast<const u32x4*>(qp + 32 * s + 8 * grp));
  }
  const auto trow = page_rsrc(bt, p.max_blocks * 4);
  int tb_next = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(trow, (jb0 + lane) * 4, 0, 0));
  // The wait for the length goes here, below the loads above: the empty asm
  // statement is the first use of the loaded value, and the compiler moves no
  // memory access across it.
  int n_raw = u.n_raw;
  asm volatile("" : "+v"(n_raw));
  const Range rg = resolve(p, u, n_raw);
  const int n = rg.n;
  const int tok_end = rg.tok_end;
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + col;
    // a shared prefix lies before every draft's first position: no causal limit
    lim[nt] = PREFIX ? 0x7fffffff : n - p.k_draft + (u.row0 + min(r, u.trows - 1)) / G;
  }

  f32x4 acc[NT][DC];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.f;
#pragma unroll
    for (int c = 0; c < DC; ++c) acc[nt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // positions above this may be masked for some row
  const int mask_from = PREFIX ? 0x7fffffff : n - p.k_draft + u.row0 / G;
  // Rows appended by this very launch (fused append) are not read from the
  // pool, which other workgroups of the launch are writing: the pool pass stops
  // at the last pair boundary before them, and a tail step processes the
  // remaining pairs with the new rows taken from k_new / v_new -- the same
  // pairs, hence the same arithmetic, as when the append was a separate launch.
  const int pool_end = FUSED
      ? min(tok_end, u.tok_begin + max(0, (n - p.t_new - u.tok_begin) / (2 * kBlk)) * (2 * kBlk))
      : tok_end;
  const int nblk = pool_end > u.tok_begin ? (pool_end + kBlk - 1) / kBlk - jb0 : 0;

  // One pair of blocks = one PV step (K and V of 32 tokens, 16 KiB at D = 128).
  struct Frag {
    Op k0[KS], k1[KS];
    u32x2 v0[DC], v1[DC];
  };
  // E4M3 pools: a pair as loaded, one byte per element (half the registers of
  // a 16-bit pair, so two pairs stay in flight for the bytes of one), turned
  // into bf16 operands just before they are used
  struct Frag8 {
    u32x2 k0[KS], k1[KS];
    uint32_t v0[DC], v1[DC];
  };
  using LFrag = std::conditional_t<Q8, Frag8, Frag>;
  // Scores, online softmax and PV for the 32 tokens starting at pos0; tokens at
  // or beyond `end` are masked (and their V zeroed: such slots may hold anything).
  // Three stages, so that the pipelined ring loop (row tiles, shared-prefix
  // pass) can run the PV MFMAs of one pair under the softmax of the next:
  //   qk:   raw scores S^T = K Q^T of every row tile (the scale (> 0) goes into
  //         the maximum once per row and into each exponent's fused multiply-add)
  //   soft: masks, the online-softmax update of m and l, and P in the operand type
  //   pv:   O = diag(alpha) O + P V
  // Within a stage each step runs for all tiles at once: the tiles' chains are
  // independent instructions of one block, which the scheduler interleaves.
  struct Soft {
    Op pa[NT];
    float a4[NT][4];
    bool rescale[NT];
  };
  auto qk = [&](const Frag& f, float (&x)[NT][8]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        s0 = MfmaOp<T>::mma(f.k0[s], qop[nt][s], s0);
        s1 = MfmaOp<T>::mma(f.k1[s], qop[nt][s], s1);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[nt][e] = s0[e];
        x[nt][4 + e] = s1[e];
      }
    }
  };
  auto needs_mask = [&](int pos0, int end) { return (pos0 + 2 * kBlk - 1 > mask_from) || (pos0 + 2 * kBlk > end); };
  // masks, the update of m and l, and P; alpha = 2^(m_old - m_new) per row
  // tile (lane col holds row col)
  auto soft_core = [&](float (&x)[NT][8], int pos0, int end, bool need_mask, Op (&pa)[NT], float (&alpha)[NT]) {
    if (need_mask) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pos = pos0 + (e >> 2) * kBlk + 4 * grp + (e & 3);
          const bool ok = pos < end && pos <= lim[nt];
          x[nt][e] = ok ? x[nt][e] : kNegInf;
        }
    }
    float mt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mt[nt] = x[nt][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt[nt] = fmax_prop(mt[nt], x[nt][e]);
    }
    // (scaling by sl2 > 0 commutes with the maximum, rounding included)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mt[nt] = wave_max_groups(mt[nt]) * sl2;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // The reference maximum of a row moves only when a score exceeds it by
      // more than kMaxSlack (log2 units), so probabilities stay <= 2^kMaxSlack:
      // exact in real arithmetic (acc, l and m stay consistent), no precision
      // lost (bf16 and fp32 keep their relative precision at that size), and
      // the accumulator rescale becomes rare.  A first finite score always
      // sets it (-inf + slack is -inf).
      const float m_new = (mt[nt] > m_run[nt] + kMaxSlack) ? mt[nt] : m_run[nt];
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nt][e], sl2, -m_use));
        ps += pe;
        pa[nt][e] = static_cast<T>(pe);
      }
      l_run[nt] = l_run[nt] * alpha[nt] + ps;
      m_run[nt] = m_new;
    }
  };
  auto rescale_of = [&](const float (&alpha)[NT], Soft& sm) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // While no reference maximum moves, alpha is exactly 1 on every row and
      // the accumulator rescale (a multiply by 1) is skipped for the whole wave.
      sm.rescale[nt] = __builtin_amdgcn_ballot_w64(alpha[nt] != 1.f) != 0;
      // rescale factors move to the accumulator layout: lane holds rows 4*grp + jj
      if (sm.rescale[nt]) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sm.a4[nt][jj] = shfl_f(alpha[nt], 4 * grp + jj);
      }
    }
  };
  auto soft = [&](float (&x)[NT][8], int pos0, int end, bool need_mask, Soft& sm) {
    float alpha[NT];
    soft_core(x, pos0, end, need_mask, sm.pa, alpha);
    rescale_of(alpha, sm);
  };
  auto pv = [&](Frag& f, int pos0, int end, const Soft& sm) {
    if (pos0 + 2 * kBlk > end) {
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        f.v0[c] = mask_v16(f.v0[c], pos0 + 4 * grp, end);
        f.v1[c] = mask_v16(f.v1[c], pos0 + kBlk + 4 * grp, end);
      }
    }
    // O = diag(alpha) O + P V
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (sm.rescale[nt]) {
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[nt][c][jj] *= sm.a4[nt][jj];
      }
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const Op vb = __builtin_bit_cast(Op, u32x4{f.v0[c][0], f.v0[c][1], f.v1[c][0], f.v1[c][1]});
        acc[nt][c] = MfmaOp<T>::mma(sm.pa[nt], vb, acc[nt][c]);
      }
    }
  };
  // pieces of the PV step for the pipelined loop: V masked past the end, the
  // MFMAs
  auto mask_v = [&](Frag& f, int pos0, int end) {
    if (pos0 + 2 * kBlk > end) {
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        f.v0[c] = mask_v16(f.v0[c], pos0 + 4 * grp, end);
        f.v1[c] = mask_v16(f.v1[c], pos0 + kBlk + 4 * grp, end);
      }
    }
  };
  auto pv_mma = [&](const Frag& f, const Op (&pa)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const Op vb = __builtin_bit_cast(Op, u32x4{f.v0[c][0], f.v0[c][1], f.v1[c][0], f.v1[c][1]});
        acc[nt][c] = MfmaOp<T>::mma(pa[nt], vb, acc[nt][c]);
      }
  };
  auto process = [&](Frag& f, int pos0, int end) {
    const bool need_mask = needs_mask(pos0, end);
    float x[NT][8];
    qk(f, x);
    Soft sm;
    soft(x, pos0, end, need_mask, sm);
    pv(f, pos0, end, sm);
  };

  // The table row, 64 entries per chunk, one per lane; each chunk's successor
  // is requested while the chunk is processed.
  // (a do-while: the first chunk is entered whatever the length, so that
  // nothing in it waits on the length before its table entries are requested;
  // with no block in range every load below reads zero and touches no memory)
  int cb = 0;
  int tb_cur = 0, cb_cur = 0;  // the last chunk processed, kept for the tail step
  do {
    const int cnt = max(0, min(64, nblk - cb));
    const int tb = tb_next;
    tb_cur = tb;
    cb_cur = cb;
    tb_next = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(trow, (jb0 + cb + 64 + lane) * 4, 0, 0));
    const int npairs = (cnt + 1) >> 1;
    // a table entry outside the pool can only come from a host-side bug; clamp
    // it so that the bug shows as a wrong result, never as a stray access
    auto phys_at = [&](int j) { return min(max(readlane(tb, j & 63), 0), p.num_blocks - 1); };
    // Branch-free loads through bounded buffer resources: a pair past the end
    // of the unit, or the missing second block of an odd count, gets a
    // resource with no valid bytes, so its loads return zeros and touch no
    // memory.  Uniform control flow lets the compiler wait only for the pair
    // being computed.
    auto load = [&](LFrag& f, int pj) {
      const int j = 2 * pj;
      const int bytes0 = j < cnt ? kPageBytes : 0;
      const int bytes1 = j + 1 < cnt ? kPageBytes : 0;
      const int phys0 = phys_at(min(j, cnt - 1));
      const int phys1 = phys_at(min(j + 1, cnt - 1));
      const size_t off0 = (static_cast<size_t>(phys0) * p.hkv + kvh) * page;
      const size_t off1 = (static_cast<size_t>(phys1) * p.hkv + kvh) * page;
      const auto rk0 = page_rsrc(kpool + off0, bytes0), rv0 = page_rsrc(vpool + off0, bytes0);
      const auto rk1 = page_rsrc(kpool + off1, bytes1), rv1 = page_rsrc(vpool + off1, bytes1);
      if constexpr (Q8) {
        // K: 8 codes = dims 32 s + 8 grp .. + 7 of token col, half of a 16-byte chunk
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int o = ((2 * s + (grp >> 1)) * kBlk + col) * 16 + 8 * (grp & 1);
          f.k0[s] = page_load8<NTL>(rk0, o);
          f.k1[s] = page_load8<NTL>(rk1, o);
        }
        // V: 4 codes = tokens 4 grp .. + 3 of dim 16 c + col
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const int o = (16 * c + col) * kBlk + 4 * grp;
          f.v0[c] = page_load4<NTL>(rv0, o);
          f.v1[c] = page_load4<NTL>(rv1, o);
        }
      } else {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        f.k0[s] = __builtin_bit_cast(Op, page_load16<NTL>(rk0, ((4 * s + grp) * kBlk + col) * 16));
#pragma unroll
      for (int s = 0; s < KS; ++s)
        f.k1[s] = __builtin_bit_cast(Op, page_load16<NTL>(rk1, ((4 * s + grp) * kBlk + col) * 16));
#pragma unroll
      for (int c = 0; c < DC; ++c) f.v0[c] = page_load8<NTL>(rv0, ((16 * c + col) * kBlk + 4 * grp) * 2);
#pragma unroll
      for (int c = 0; c < DC; ++c) f.v1[c] = page_load8<NTL>(rv1, ((16 * c + col) * kBlk + 4 * grp) * 2);
      }
    };
    const int base_pos = (jb0 + cb) * kBlk;
    // One pair in flight per wave is enough to saturate HBM with two waves
    // per SIMD, and fewer bytes queued in the memory system shorten every
    // dependent access (measured on MI355X: 3-6 % faster than keeping two
    // pairs in flight).  Multi-tile verify waves, few and short, keep the
    // second pair in flight at one wave per SIMD.  The shared-prefix pass has
    // thousands of such waves: one pair each fits two waves per SIMD, which
    // is 13 % faster there.
    if constexpr (W > 1) {
      // pair image in LDS: [K block 0][K block 1][V block 0][V block 1], each
      // page as laid out in the pool, so fragments are read at pool offsets.
      // A ring of kRing images: pairs pj + 1 .. pj + kRing - 1 load straight
      // from the pool into LDS (buffer loads with an LDS destination, no
      // staging registers) while the waves compute on pair pj.
      constexpr int kPair = 4 * kPageBytes;
      constexpr int kPer = kPair / (16 * 64 * W);  // 16-byte chunks per thread
      constexpr int kChunksPerPage = kPageBytes / 16;
      // Four images.  (Measured on MI355X with the pipelined loop: bf16
      // prefill tiles 313-314 us with five, 308 with four, 309 with three;
      // bf16 verify 61.1-61.7 / 60.8-61.1 / 61.0-61.5 us; E4M3 prefill tiles
      // 342-343 / 338-339 / 340 us; E4M3 verify, its attention units holding
      // one pair: 60.6-61.0 with five or four.  Pages further ahead queue in
      // the memory system.)
      constexpr int kRing = 4;
      static_assert(kPer * 16 * 64 * W == kPair, "pair image must split evenly");
      static_assert(kChunksPerPage == 64 * kPer, "a wave's loads cover one page");
      static_assert(kRing >= 3 && kRing <= 5 && (kRing - 2) * kPer <= 63, "the waits below cover up to three later pairs");
      __shared__ __attribute__((aligned(16))) char lds[kRing][kPair];
      static_assert(W == 4, "one wave per page of the pair image");
      const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
      // Wave w loads page w of the image (K of the pair's first block, K of
      // its second, then their V), so it builds one buffer descriptor per
      // pair; each load instruction fills 64 consecutive 16-byte chunks of
      // that page (lane l writes chunk c0 + l: the LDS address is the wave's
      // base plus 16 l).
      const bool v_page = wave >= 2;
      const auto* wpool = v_page ? vpool : kpool;
      auto dma = [&](int pj, int b) {
        const int j = 2 * pj + (wave & 1);
        const int bytes = j < cnt ? kPageBytes : 0;
        const size_t off = (static_cast<size_t>(phys_at(min(j, cnt - 1))) * p.hkv + kvh) * page;
        const auto rs = page_rsrc(wpool + off, bytes);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int lc = 64 * k + lane;  // this lane's chunk of the page
          // V pages (16-bit): LDS chunk h * D + d holds the pool's chunk
          // (dim d, tokens 8h .. 8h + 7), so that the 16 lanes of a fragment
          // read (16 dims, one token half) sit 16 bytes apart, not 32
          const int gc = (!Q8 && v_page) ? (lc % D) * 2 + lc / D : lc;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(&lds[b][(wave * kChunksPerPage + 64 * k) * 16]), 16,
              gc * 16, 0, 0, NTL ? 2 : 0);
        }
      };
      // fragments of a pair image: K (the score operands), then V (the PV operands)
      auto lfrag_k = [&](Frag& f, int b) {
        const char* kb = lds[b];
        if constexpr (Q8) {
          // the 8-bit operands at the offsets of the pool loads, turned into bf16
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const int o = ((2 * s + (grp >> 1)) * kBlk + col) * 16 + 8 * (grp & 1);
            f.k0[s] = __builtin_bit_cast(Op, fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(kb + o)));
            f.k1[s] = __builtin_bit_cast(Op, fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(kb + kPageBytes + o)));
          }
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const int o = ((4 * s + grp) * kBlk + col) * 16;
            f.k0[s] = __builtin_bit_cast(Op, *reinterpret_cast<const u32x4*>(kb + o));
            f.k1[s] = __builtin_bit_cast(Op, *reinterpret_cast<const u32x4*>(kb + kPageBytes + o));
          }
        }
      };
      auto lfrag_v = [&](Frag& f, int b) {
        const char* vb = lds[b] + 2 * kPageBytes;
        if constexpr (Q8) {
#pragma unroll
          for (int c = 0; c < DC; ++c) {
            const int o = (16 * c + col) * kBlk + 4 * grp;
            f.v0[c] = fp8x4_to_bf16(*reinterpret_cast<const uint32_t*>(vb + o));
            f.v1[c] = fp8x4_to_bf16(*reinterpret_cast<const uint32_t*>(vb + kPageBytes + o));
          }
        } else {
#pragma unroll
          for (int c = 0; c < DC; ++c) {
            const int o = ((grp >> 1) * D + 16 * c + col) * 16 + 8 * (grp & 1);
            f.v0[c] = *reinterpret_cast<const u32x2*>(vb + o);
            f.v1[c] = *reinterpret_cast<const u32x2*>(vb + kPageBytes + o);
          }
        }
      };
      // s_waitcnt immediates (gfx9 layout: vector-memory count in bits 3:0
      // and 15:14): count <= n, the other counters not waited on
      constexpr int kNoOther = (7 << 4) | (15 << 8);
      constexpr int kWait1 = kNoOther | (kPer & 15) | ((kPer >> 4) << 14);
      constexpr int kWait2 = kNoOther | ((2 * kPer) & 15) | ((2 * kPer) >> 4 << 14);
      constexpr int kWait3 = kNoOther | ((3 * kPer) & 15) | ((3 * kPer) >> 4 << 14);
      // this wave's loads have landed but for those of the last `later` pairs issued
      auto wait_later = [&](int later) {
        if (later >= 3)
          __builtin_amdgcn_s_waitcnt(kWait3);
        else if (later == 2)
          __builtin_amdgcn_s_waitcnt(kWait2);
        else if (later == 1)
          __builtin_amdgcn_s_waitcnt(kWait1);
        else
          __builtin_amdgcn_s_waitcnt(kNoOther);
      };
      // Loads into registers (queries, table entries) complete here, before
      // the ring starts: otherwise the compiler's waits for them sit inside
      // the loop, where their counts would also cover the pairs in flight.
      __builtin_amdgcn_s_waitcnt(kNoOther);
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r)
        if (r < npairs) dma(r, r);
      // Software pipeline: the PV MFMAs of pair pj - 1 are interleaved with
      // the softmax of pair pj, which does not depend on them, so the matrix
      // core works under the softmax's vector instructions (acc sees the same
      // updates in the same order: alpha_q, then P_q V_q, for q = 0, 1, ...).
      // Pair q sits in ring slot q % kRing; its V fragments are read into
      // registers in iteration q.  At the barrier of iteration pj this wave's
      // share of pair pj has landed (only the loads of the pairs after it may
      // still run), so every wave's has, and every wave has read the image of
      // pair pj - 1, which the load of pair pj + kRing - 1 then overwrites.
      // A bare s_barrier: a fence would make the compiler wait for the later
      // pairs' loads as well.  The empty asm statement after it keeps the
      // compiler from moving the LDS reads above it.
      // The end of an iteration (softmax, PV MFMAs, the next V reads) is
      // branch-free, so that the interleaving holds; the rare steps with
      // branches (masking V past the end, rescaling acc when a reference
      // maximum moved) run at the start of the next iteration.
      Frag fv;           // V of the previous pair
      Op pp[NT];         // its P
      float ap[NT];      // its alpha (lane col: row col)
      bool rp[NT];       // whether any alpha of the tile differs from 1
      int pos_prev = 0;  // its first position
      auto finish_prev = [&]() {
        mask_v(fv, pos_prev, pool_end);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (rp[nt]) {
            float a4[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) a4[jj] = shfl_f(ap[nt], 4 * grp + jj);
#pragma unroll
            for (int c = 0; c < DC; ++c)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) acc[nt][c][jj] *= a4[jj];
          }
        }
      };
      auto step = [&](int pj, auto has_prev) {
        constexpr bool kPrev = decltype(has_prev)::value;
        const int pos0 = base_pos + 2 * pj * kBlk;
        const bool mask = needs_mask(pos0, pool_end);
        wait_later(min(npairs - 1 - pj, kRing - 2));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (pj + kRing - 1 < npairs) dma(pj + kRing - 1, (pj + kRing - 1) % kRing);
        if constexpr (kPrev) finish_prev();
        Frag fk;
        lfrag_k(fk, pj % kRing);
        float x[NT][8];
        // The score MFMAs go at a raised wave priority: while a wave issues
        // them, the other wave of its SIMD (another workgroup's) fills the
        // vector unit with its softmax.  (Measured on MI355X: prefill tiles
        // 315 -> 304 us, the verify launch 52.4 -> 51.3 us.)
        __builtin_amdgcn_s_setprio(1);
        qk(fk, x);
        __builtin_amdgcn_s_setprio(0);
        Op pa[NT];
        float alpha[NT];
        soft_core(x, pos0, pool_end, mask, pa, alpha);
        if constexpr (kPrev) {
          pv_mma(fv, pp);
          // one PV MFMA, then a few softmax instructions, and so on
#pragma unroll
          for (int i = 0; i < NT * DC; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          rp[nt] = __builtin_amdgcn_ballot_w64(alpha[nt] != 1.f) != 0;
          ap[nt] = alpha[nt];
          pp[nt] = pa[nt];
        }
        lfrag_v(fv, pj % kRing);
        pos_prev = pos0;
      };
      if (npairs > 0) step(0, std::false_type{});
      for (int pj = 1; pj < npairs; ++pj) step(pj, std::true_type{});
      if (npairs > 0) {
        finish_prev();
        pv_mma(fv, pp);
      }
      __syncthreads();  // the next table chunk refills the ring
    } else if constexpr (Q8) {
      auto run = [&](Frag8& r, int pos0) {
        Frag f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          f.k0[s] = __builtin_bit_cast(Op, fp8x8_to_bf16(r.k0[s]));
          f.k1[s] = __builtin_bit_cast(Op, fp8x8_to_bf16(r.k1[s]));
        }
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          f.v0[c] = fp8x4_to_bf16(r.v0[c]);
          f.v1[c] = fp8x4_to_bf16(r.v1[c]);
        }
        process(f, pos0, pool_end);
      };
      if constexpr (D * NT <= 256 && !ONE_PAIR) {
        Frag8 ra, rb;
        load(ra, 0);
        for (int pj = 0; pj < npairs; pj += 2) {
          load(rb, pj + 1);
          run(ra, base_pos + 2 * pj * kBlk);
          if (pj + 1 >= npairs) break;
          load(ra, pj + 2);
          run(rb, base_pos + (2 * pj + 2) * kBlk);
        }
      } else {  // wide tiles, and the launch beside the shared-prefix pass: one pair in flight
        for (int pj = 0; pj < npairs; ++pj) {
          Frag8 r;
          load(r, pj);
          run(r, base_pos + 2 * pj * kBlk);
        }
      }
    } else if constexpr (NT >= 2 && D * NT < 512 && !PREFIX && !ONE_PAIR) {
      Frag fa, fb;
      load(fa, 0);
      for (int pj = 0; pj < npairs; pj += 2) {
        load(fb, pj + 1);
        process(fa, base_pos + 2 * pj * kBlk, pool_end);
        if (pj + 1 >= npairs) break;
        load(fa, pj + 2);
        process(fb, base_pos + (2 * pj + 2) * kBlk, pool_end);
      }
    } else {
      for (int pj = 0; pj < npairs; ++pj) {
        Frag fa;
        load(fa, pj);
        process(fa, base_pos + 2 * pj * kBlk, pool_end);
      }
    }
    cb += 64;
  } while (cb < nblk);

  // Tail step of a fused append: the pairs from pool_end to the end of the
  // partition.  Old rows come from the pool (blocks holding no old row are
  // not read), the rows this launch appends ([n - t_new, n)) from
  // k_new / v_new ([n_seq * t_new][hkv][D], rows of query row q at q * t_new ..).
  if constexpr (FUSED) {
    const int old_end = n - p.t_new;
    const size_t rstride = static_cast<size_t>(p.hkv) * D;  // elements between new rows
    const T* kn = static_cast<const T*>(p.app.k_new) + (static_cast<size_t>(u.q_row) * p.t_new * p.hkv + kvh) * D;
    const uint16_t* vn =
        static_cast<const uint16_t*>(p.app.v_new) + (static_cast<size_t>(u.q_row) * p.t_new * p.hkv + kvh) * D;
#pragma unroll 1
    for (int pos0 = pool_end; pos0 < tok_end; pos0 += 2 * kBlk) {
      Frag f;
      const int blk0 = pos0 / kBlk;
      const bool old0 = blk0 * kBlk < old_end;
      const bool old1 = (blk0 + 1) * kBlk < old_end;
      // table entries: from the chunks already in registers when they hold them
      auto entry = [&](int blk) {
        const int j = blk - jb0 - cb_cur;
        const int e = j < 64 ? readlane(tb_cur, j & 63) : (j < 128 ? readlane(tb_next, j & 63) : bt[blk]);
        return min(max(e, 0), p.num_blocks - 1);
      };
      const int phys0 = old0 ? entry(blk0) : 0;
      const int phys1 = old1 ? entry(blk0 + 1) : 0;
      const size_t off0 = (static_cast<size_t>(phys0) * p.hkv + kvh) * page;
      const size_t off1 = (static_cast<size_t>(phys1) * p.hkv + kvh) * page;
      const auto rk0 = page_rsrc(kpool + off0, old0 ? kPageBytes : 0), rv0 = page_rsrc(vpool + off0, old0 ? kPageBytes : 0);
      const auto rk1 = page_rsrc(kpool + off1, old1 ? kPageBytes : 0), rv1 = page_rsrc(vpool + off1, old1 ? kPageBytes : 0);
      if constexpr (Q8) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int o = ((2 * s + (grp >> 1)) * kBlk + col) * 16 + 8 * (grp & 1);
          f.k0[s] = __builtin_bit_cast(Op, fp8x8_to_bf16(page_load8<false>(rk0, o)));
          f.k1[s] = __builtin_bit_cast(Op, fp8x8_to_bf16(page_load8<false>(rk1, o)));
        }
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const int o = (16 * c + col) * kBlk + 4 * grp;
          f.v0[c] = fp8x4_to_bf16(page_load4<false>(rv0, o));
          f.v1[c] = fp8x4_to_bf16(page_load4<false>(rv1, o));
        }
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          f.k0[s] = __builtin_bit_cast(Op, page_load16<false>(rk0, ((4 * s + grp) * kBlk + col) * 16));
          f.k1[s] = __builtin_bit_cast(Op, page_load16<false>(rk1, ((4 * s + grp) * kBlk + col) * 16));
        }
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          f.v0[c] = page_load8<false>(rv0, ((16 * c + col) * kBlk + 4 * grp) * 2);
          f.v1[c] = page_load8<false>(rv1, ((16 * c + col) * kBlk + 4 * grp) * 2);
        }
      }
      // splice in the new rows, one token at a time: the row's loads are all
      // issued before any is used, and the splice is selects only
      const int i_end = min(pos0 + 2 * kBlk, n);
#pragma unroll 1
      for (int i = max(pos0, old_end); i < i_end; ++i) {
        const int rel = i - pos0;
        const bool in0 = rel < kBlk;
        const int t = rel & 15;
        const size_t row = static_cast<size_t>(i - old_end) * rstride;
        Op x[KS];
        uint16_t nv[DC];
#pragma unroll
        for (int s = 0; s < KS; ++s) x[s] = __builtin_bit_cast(Op, *reinterpret_cast<const u32x4*>(kn + row + 32 * s + 8 * grp));
#pragma unroll
        for (int c = 0; c < DC; ++c) nv[c] = vn[row + 16 * c + col];
        if constexpr (Q8) {
          // the values the pool will hold: the append's E4M3 codes, decoded
          const float ki = p.kv_scale[2 * p.hkv + kvh], vi = p.kv_scale[3 * p.hkv + kvh];
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const u32x4 w = __builtin_bit_cast(u32x4, x[s]);
            u32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              r[e] = fp8_requant_bf16(w[e] & 0xFFFFu, ki) | (fp8_requant_bf16(w[e] >> 16, ki) << 16);
            x[s] = __builtin_bit_cast(Op, r);
          }
#pragma unroll
          for (int c = 0; c < DC; ++c) nv[c] = static_cast<uint16_t>(fp8_requant_bf16(nv[c], vi));
        }
        const bool kl = col == t;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          f.k0[s] = (kl && in0) ? x[s] : f.k0[s];
          f.k1[s] = (kl && !in0) ? x[s] : f.k1[s];
        }
        // V: lane (col, grp) holds tokens 4 grp .. 4 grp + 3 of dim 16 c + col,
        // two per 32-bit word
        const bool vl = grp == (t >> 2);
        const int word = (t & 3) >> 1;
        const int shift = (t & 1) * 16;
        const uint32_t keep = ~(0xFFFFu << shift);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const uint32_t bits = static_cast<uint32_t>(nv[c]) << shift;
#pragma unroll
          for (int wi = 0; wi < 2; ++wi) {
            const bool hit = vl && word == wi;
            f.v0[c][wi] = (hit && in0) ? ((f.v0[c][wi] & keep) | bits) : f.v0[c][wi];
            f.v1[c][wi] = (hit && !in0) ? ((f.v1[c][wi] & keep) | bits) : f.v1[c][wi];
          }
        }
      }
      process(f, pos0, tok_end);
    }
  }

  // ---- epilogue
  if constexpr (PREFIX) {
    // each row's partial goes to partition u.part of its own sequence (at
    // device scope when the members' merge runs in this launch)
    const bool dev = p.pre_in_launch != 0 && p.inline_merge != 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float l = wave_sum_groups(l_run[nt]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = u.pre_row0 + nt * 16 + 4 * grp + jj;
        if (r < u.pre_rows) {
          const int j = r / rows;
          const PrefixMember m = p.pre_members[u.pre_member0 + j];
          const int slot = m.slot_base + kvh * m.nparts + u.part;
          float* ap = p.ws_acc + (static_cast<size_t>(slot) * rows + (r - j * rows)) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) {
            const float x = acc[nt][c][jj] * vsc;  // (E4M3: the head's V scale)
            if (dev)
              store_device(ap + 16 * c + col, x);
            else
              ap[16 * c + col] = x;
          }
        }
      }
      const int r = u.pre_row0 + nt * 16 + col;
      if (grp == 0 && r < u.pre_rows) {
        const int j = r / rows;
        const PrefixMember m = p.pre_members[u.pre_member0 + j];
        const int slot = m.slot_base + kvh * m.nparts + u.part;
        float* mp = p.ws_ml + (static_cast<size_t>(slot) * rows + (r - j * rows)) * 2;
        if (dev) {
          store_device(mp, m_run[nt]);
          store_device(mp + 1, l);
        } else {
          mp[0] = m_run[nt];
          mp[1] = l;
        }
      }
    }
    if (dev && u.pre_row0 < u.pre_rows) {
      // every member whose rows this wave holds: count this arrival, and the
      // last arrival merges the member
      const int r_end = min(u.pre_row0 + 16 * NT, u.pre_rows);
      for (int j = u.pre_row0 / rows; j * rows < r_end; ++j)
        merge_last<T, D>(p, p.pre_members[u.pre_member0 + j].merge, kvh);
    }
    return;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = wave_sum_groups(l_run[nt]);
    if (u.slot_base < 0) {
      float inv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) inv[jj] = vsc / shfl_f(l, 4 * grp + jj);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = nt * 16 + 4 * grp + jj;
        if (r < u.trows) {
          const int rr = u.row0 + r;
          const int i = rr / G, g = rr - (rr / G) * G;
          T* op = static_cast<T*>(p.out) +
                  (static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) store_elem(op + 16 * c + col, acc[nt][c][jj] * inv[jj]);
        }
      }
      const int r = nt * 16 + col;
      if (p.lse && grp == 0 && r < u.trows) {
        const int rr = u.row0 + r;
        const int i = rr / G, g = rr - (rr / G) * G;
        p.lse[static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g] =
            (m_run[nt] + __builtin_amdgcn_logf(l)) * kLn2;
      }
    } else {
      // single-tile partials may be merged inside this launch: they are stored
      // at device scope (written through this XCD's L2), so that a merging
      // wave on another XCD reads them
      const int slot = u.slot_base + kvh * u.nparts + u.part;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = nt * 16 + 4 * grp + jj;
        if (r < u.trows) {
          float* ap = p.ws_acc + (static_cast<size_t>(slot) * rows + u.row0 + r) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) {
            if (p.inline_merge)
              store_device(ap + 16 * c + col, acc[nt][c][jj] * vsc);
            else
              ap[16 * c + col] = acc[nt][c][jj] * vsc;
          }
        }
      }
      const int r = nt * 16 + col;
      if (grp == 0 && r < u.trows) {
        float* mp = p.ws_ml + (static_cast<size_t>(slot) * rows + u.row0 + r) * 2;
        if (p.inline_merge) {
          store_device(mp, m_run[nt]);
          store_device(mp + 1, l);
        } else {
          mp[0] = m_run[nt];
          mp[1] = l;
        }
      }
    }
  }
  if constexpr (W == 1) {
    if (p.inline_merge && u.slot_base >= 0) merge_last<T, D>(p, u.merge, kvh);
  }
}

// fp32 elements: v_mfma_f32_16x16x4_f32 (one dim per lane per instruction)
template <int D, int NT>
__device__ inline void attn_body32(const AttnParams& p, const Unit& u, int kvh) {
  constexpr int KS = D / 16;  // 16-byte K chunks per lane per block
  constexpr int DC = D / 16;
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rows = p.rows;
  const int G = p.group;
  const Range rg = resolve(p, u, u.n_raw);
  const int n = rg.n;
  const int tok_end = rg.tok_end;

  f32x4 qv[NT][KS];
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + col;
    if (r < u.trows) {
      const int rr = u.row0 + r;
      const int i = rr / G, g = rr - (rr / G) * G;
      const float* qp = static_cast<const float*>(p.q) +
                        (static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) qv[nt][s] = *reinterpret_cast<const f32x4*>(qp + 16 * s + 4 * grp);
      lim[nt] = n - p.k_draft + i;
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qv[nt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
      lim[nt] = n - 1;
    }
  }
  f32x4 acc[NT][DC];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.f;
#pragma unroll
    for (int c = 0; c < DC; ++c) acc[nt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* kpool = static_cast<const float*>(p.k_pool);
  const float* vpool = static_cast<const float*>(p.v_pool);
  const size_t page = static_cast<size_t>(D) * kBlk;
  const int32_t* bt = p.block_table + static_cast<size_t>(u.seq) * p.max_blocks;
  const int jb0 = u.tok_begin / kBlk;
  const int nblk = (tok_end + kBlk - 1) / kBlk - jb0;
  const int mask_from = n - p.k_draft;

  for (int cb = 0; cb < nblk; cb += 64) {
    const int cnt = min(64, nblk - cb);
    const int tb = (lane < cnt) ? bt[jb0 + cb + lane] : 0;
    for (int j = 0; j < cnt; ++j) {
      const int phys = min(max(readlane(tb, j), 0), p.num_blocks - 1);
      const int pos0 = (jb0 + cb + j) * kBlk;
      const float* kp = kpool + (static_cast<size_t>(phys) * p.hkv + kvh) * page;
      const float* vp = vpool + (static_cast<size_t>(phys) * p.hkv + kvh) * page;
      f32x4 kk[KS], vv[DC];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kk[s] = *reinterpret_cast<const f32x4*>(kp + ((4 * s + grp) * kBlk + col) * 4);
#pragma unroll
      for (int c = 0; c < DC; ++c) vv[c] = *reinterpret_cast<const f32x4*>(vp + (16 * c + col) * kBlk + 4 * grp);
      if (pos0 + kBlk > n) {
#pragma unroll
        for (int c = 0; c < DC; ++c) vv[c] = mask_v32(vv[c], pos0 + 4 * grp, n);
      }
      const bool need_mask = (pos0 + kBlk - 1 > mask_from) || (pos0 + kBlk > tok_end);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kk[s][e], qv[nt][s][e], s4, 0, 0, 0);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = s4[e] * p.scale_log2;
          if (need_mask) {
            const int pos = pos0 + 4 * grp + e;
            x[e] = (pos < tok_end && pos <= lim[nt]) ? x[e] : kNegInf;
          }
        }
        float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mt = wave_max_groups(mt);
        const float m_new = fmaxf(m_run[nt], mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
        float pe[4], ps = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pe[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
          ps += pe[e];
        }
        l_run[nt] = l_run[nt] * alpha + ps;
        m_run[nt] = m_new;
        float a4[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) a4[jj] = shfl_f(alpha, 4 * grp + jj);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[nt][c][jj] *= a4[jj];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[nt][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(pe[jj], vv[c][jj], acc[nt][c], 0, 0, 0);
        }
      }
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = wave_sum_groups(l_run[nt]);
    if (u.slot_base < 0) {
      float inv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) inv[jj] = 1.f / shfl_f(l, 4 * grp + jj);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = nt * 16 + 4 * grp + jj;
        if (r < u.trows) {
          const int rr = u.row0 + r;
          const int i = rr / G, g = rr - (rr / G) * G;
          float* op = static_cast<float*>(p.out) +
                      (static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) op[16 * c + col] = acc[nt][c][jj] * inv[jj];
        }
      }
      const int r = nt * 16 + col;
      if (p.lse && grp == 0 && r < u.trows) {
        const int rr = u.row0 + r;
        const int i = rr / G, g = rr - (rr / G) * G;
        p.lse[static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g] =
            (m_run[nt] + __builtin_amdgcn_logf(l)) * kLn2;
      }
    } else {
      const int slot = u.slot_base + kvh * u.nparts + u.part;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = nt * 16 + 4 * grp + jj;
        if (r < u.trows) {
          float* ap = p.ws_acc + (static_cast<size_t>(slot) * rows + u.row0 + r) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) ap[16 * c + col] = acc[nt][c][jj];
        }
      }
      const int r = nt * 16 + col;
      if (grp == 0 && r < u.trows) {
        float* mp = p.ws_ml + (static_cast<size_t>(slot) * rows + u.row0 + r) * 2;
        mp[0] = m_run[nt];
        mp[1] = l;
      }
    }
  }
}

// One workgroup (one wave) per (work unit, key/value head).
template <typename T, int D, int NT, bool NTL, bool FUSED, bool Q8 = false, bool ONE_PAIR = false>
__device__ inline void attn_unit(const AttnParams& p, const int32_t* meta, int block) {
  const int unit = block / p.hkv;
  const int kvh = block - unit * p.hkv;
  const WorkUnit w = p.units[unit];
  Unit u;
  u.q_row = w.q_row;
  u.seq = w.seq;
  u.slot_base = w.slot_base;
  u.nparts = w.nparts;
  u.part = w.part;
  u.merge = w.merge;
  // The length travels as a vector load (then made uniform), so that the
  // bodies' first loads are issued while it is on its way instead of after it.
  if constexpr (FUSED) {
    u.n_raw = meta[p.lens_by_row + w.q_row];
  } else {
    const auto lens = page_rsrc(p.seq_len, 0x7ffffff0);
    u.n_raw = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(lens, w.seq * 4, 0, 0));
  }
  u.tok_begin = w.tok_begin;
  u.row0 = w.row0;
  u.trows = min(p.tile_rows, p.rows - w.row0);
  u.clip_row = u.row0 + u.trows - 1;
  if constexpr (std::is_same_v<T, float>)
    attn_body32<D, NT>(p, u, kvh);
  else
    attn_body16<T, D, NT, NTL, FUSED, false, Q8, 1, ONE_PAIR>(p, u, kvh);
}

template <typename T, int D, int NT, bool NTL, bool Q8 = false>
__global__ __launch_bounds__(64) void attn_kernel(AttnParams p) {
  attn_unit<T, D, NT, NTL, false, Q8>(p, nullptr, blockIdx.x);
}

// Many query rows per (sequence, kv head) -- chunked prefill, long verify --
// take workgroups of TileShape::W waves, each wave 16 * NT consecutive rows of
// the workgroup's tile, the waves sharing every pair of blocks through LDS.
template <int D>
struct TileShape {
  static constexpr int NT = D <= 128 ? 2 : 1;  // row tiles per wave
  static constexpr int W = 4;                  // waves per workgroup
  static constexpr int kRows = 16 * NT * W;    // query rows per workgroup
};

template <typename T, int D, bool NTL, bool Q8 = false>
__global__ __launch_bounds__(64 * TileShape<D>::W) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void tile_kernel(AttnParams p) {
  constexpr int NT = TileShape<D>::NT, W = TileShape<D>::W;
  const int unit = blockIdx.x / p.hkv;
  const int kvh = blockIdx.x - unit * p.hkv;
  const WorkUnit w = p.units[unit];
  const int wave = threadIdx.x >> 6;
  Unit u{};
  u.q_row = w.q_row;
  u.seq = w.seq;
  u.slot_base = w.slot_base;
  u.nparts = w.nparts;
  u.part = w.part;
  u.merge = w.merge;
  const auto lens = page_rsrc(p.seq_len, 0x7ffffff0);
  u.n_raw = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(lens, w.seq * 4, 0, 0));
  u.tok_begin = w.tok_begin;
  const int g_rows = min(p.tile_rows, p.rows - w.row0);
  u.row0 = w.row0 + wave * 16 * NT;
  // a wave past the tile's rows (trows <= 0) still loads its share of every
  // pair and meets every barrier; its queries repeat the tile's last row and
  // nothing of it is stored
  u.trows = min(16 * NT, g_rows - wave * 16 * NT);
  u.clip_row = w.row0 + g_rows - 1;
  attn_body16<T, D, NT, NTL, false, false, Q8, W>(p, u, kvh);
}

// Attention and append in one launch: workgroups past the attention grid do
// the append work (table / length updates and the scatter of the new rows).
// (two waves per SIMD for the single-tile 128-dim case: the pool pass needs
// them to keep enough loads in flight)
template <typename T, int D, int NT, bool NTL, bool Q8 = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NT == 1 && D == 128 ? 2 : 1)))
void attn_append_kernel(AttnParams p, InlineMeta im) {
  const int32_t* meta = p.app.ext ? p.app.ext : im.w;
  const int b = blockIdx.x;
  if (p.graph_units > 0) {
    // a graph step: this step's counts from its metadata; workgroups of the
    // padded grid past them have nothing to do
    const int n_grid = p.graph_units * p.hkv;
    if (b >= n_grid) {
      AppendParams a = p.app;
      a.n_tab = meta[kGraphTab];
      a.n_len = meta[kGraphLen];
      a.n_rows = meta[kGraphRows];
      a.slots = meta[kGraphSlotsAt];
      a.tab = meta[kGraphTabAt];
      a.lens = meta[kGraphLenAt];
      append_work<Q8 ? 1 : static_cast<int>(sizeof(T))>(a, meta, b - n_grid, 64);
      return;
    }
    if (b >= meta[kGraphUnits] * p.hkv) return;
    attn_unit<T, D, NT, NTL, true, Q8>(p, meta, blockIdx.x);
    return;
  }
  const int n_attn = p.n_units * p.hkv;
  if (b >= n_attn) {
    append_work<Q8 ? 1 : static_cast<int>(sizeof(T))>(p.app, meta, b - n_attn, 64);
    return;
  }
  attn_unit<T, D, NT, NTL, true, Q8>(p, meta, blockIdx.x);
}

// Shared-prefix pass: one workgroup of W waves per (prefix unit, kv head);
// wave w takes 16 * NT query rows of one group of sequences over one
// partition of their common prefix, the four waves sharing each pair of
// blocks through the LDS ring of the row tiles.  (Measured on MI355X, 64-fork
// verify with 16-bit pools: single-wave workgroups with one pair in flight
// at two waves per SIMD were best while the ring's loads were built with
// four descriptors per wave and read V with 4-way bank conflicts; with one
// page per wave and the V image reordered the ring is faster, for E4M3 pools
// too, whose pair image is half the size.)
template <int D, bool Q8 = false>
struct PrefixShape {
  static constexpr int NT = D <= 128 ? 2 : 1;            // row tiles per wave
  static constexpr int W = 4;                            // waves per workgroup
  static constexpr int kWavesPerSimd = D <= 128 ? 2 : 1;  // resident waves per SIMD
};

// Unit `unit` of the shared-prefix pass (workgroup `unit * hkv + kvh`).
template <typename T, int D, bool Q8>
__device__ inline void prefix_unit(const AttnParams& p, int block) {
  using Shape = PrefixShape<D, Q8>;
  constexpr int NT = Shape::NT;
  const int unit = block / p.hkv;
  const int kvh = block - unit * p.hkv;
  const PrefixUnit pu = p.pre_units[unit];
  // With several waves per workgroup, a wave past the group's rows still
  // loads its share of every pair and meets every barrier; its queries repeat
  // the group's last row and nothing of it is stored.  A lone wave past them
  // has nothing to do.
  const int row0 = pu.row0 + static_cast<int>(threadIdx.x >> 6) * 16 * NT;
  if (Shape::W == 1 && row0 >= pu.group_rows) return;
  Unit u{};
  u.seq = pu.seq;
  u.n_raw = pu.prefix_tokens;  // the last partition of the prefix ends at the shared positions
  u.part = pu.part;
  u.tok_begin = pu.part * p.part_tokens;
  u.nparts = 1 << 30;  // a partition never the last: tokens [tok_begin, min(prefix, tok_begin + part_tokens))
  u.slot_base = 0;
  u.pre_row0 = row0;
  u.pre_member0 = pu.member0;
  u.pre_rows = pu.group_rows;
  u.row0 = 0;
  u.trows = 1 << 24;  // no causal limit: the prefix precedes every query row
  u.clip_row = 1 << 24;
  // the prefix blocks are read by every row block of the group: cached loads
  attn_body16<T, D, NT, false, false, true, Q8, Shape::W>(p, u, kvh);
}

template <typename T, int D, bool Q8 = false>
__global__ __launch_bounds__((64 * PrefixShape<D, Q8>::W)) __attribute__((amdgpu_waves_per_eu((PrefixShape<D, Q8>::kWavesPerSimd))))
void prefix_kernel(AttnParams p) {
  prefix_unit<T, D, Q8>(p, blockIdx.x);
}

// Attention units, then the shared-prefix units, then (FUSED) the append work,
// in one launch of four-wave workgroups (16-bit pools): the pass over the
// shared prefix overlaps the members' own partitions, and the last wave to
// finish partials of a (member, kv head) merges them.  An attention workgroup
// runs four independent single-wave units (no barrier, no LDS); a prefix
// workgroup is the pass's four-wave unit.  Multi-tile units keep one pair in
// flight, so that the launch holds two waves per SIMD as the prefix pass
// needs.
constexpr int kPrefixLaunchWaves = 4;

template <typename T, int D, int NT, bool FUSED, bool Q8>
__global__ __launch_bounds__(64 * kPrefixLaunchWaves) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void attn_prefix_kernel(AttnParams p, InlineMeta im) {
  static_assert(PrefixShape<D, Q8>::W == kPrefixLaunchWaves, "prefix units are the launch's workgroups");
  const int32_t* meta = p.app.ext ? p.app.ext : im.w;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int n_attn = p.n_units * p.hkv;  // attention waves
  const int n_attn_wg = (n_attn + kPrefixLaunchWaves - 1) / kPrefixLaunchWaves;
  const int n_pre = p.n_pre_units * p.hkv;
  const int b = blockIdx.x;
  if (b < n_attn_wg) {
    const int vb = b * kPrefixLaunchWaves + wave;
    if (vb < n_attn) attn_unit<T, D, NT, false, FUSED, Q8, true>(p, meta, vb);
    return;
  }
  if (b < n_attn_wg + n_pre) {
    prefix_unit<T, D, Q8>(p, b - n_attn_wg);
    return;
  }
  if constexpr (FUSED)
    append_work<Q8 ? 1 : static_cast<int>(sizeof(T))>(p.app, meta, b - n_attn_wg - n_pre, 64 * kPrefixLaunchWaves);
}

// Exact merge of one output row of a split sequence, one 256-thread workgroup
// per (sequence, key/value head, query row):
//   M = max_p m_p,  w_p = 2^(m_p - M),  O = sum_p w_p acc_p / sum_p w_p l_p,
//   lse = (M + log2 sum_p w_p l_p) * ln 2
// The D/4 16-byte chunks of a row are spread over D/4 threads, the partitions
// over NG = 1024/D groups of such threads (partition q to group q % NG).  A
// thread requests the (m, l) pair and the row chunk of all its partitions at
// once and combines them with a running maximum; the groups are then combined
// in a fixed order through LDS, so the result is deterministic.
constexpr int kMergeThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnParams p) {
  constexpr int NC = D / 4;                 // float4 chunks per row
  constexpr int NG = kMergeThreads / NC;    // partition groups
  __shared__ f32x4 part_acc[NG][NC];
  __shared__ float part_m[NG];
  __shared__ float part_l[NG];
  const int tid = threadIdx.x;
  const int rows = p.rows;
  const int r = blockIdx.x % rows;
  const int rest = blockIdx.x / rows;
  const int kvh = rest % p.hkv;
  const MergeUnit mu = p.merges[rest / p.hkv];
  const int P = mu.nparts;
  const int base = mu.slot_base + kvh * P;
  const float* ml = p.ws_ml + (static_cast<size_t>(base) * rows + r) * 2;  // partition q at ml[q * rows * 2]
  const size_t mstride = static_cast<size_t>(rows) * 2;
  const int g = tid / NC;
  const int c = tid - g * NC;
  const f32x4* acc = reinterpret_cast<const f32x4*>(p.ws_acc + (static_cast<size_t>(base) * rows + r) * D) + c;
  const size_t astride = static_cast<size_t>(rows) * D / 4;
  float mg = kNegInf, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int q = g; q < P; q += NG) {
    const float m = ml[q * mstride];
    const float l = ml[q * mstride + 1];
    const f32x4 a = acc[q * astride];
    const float mn = fmaxf(mg, m);
    const float mu_ = (mn == kNegInf) ? 0.f : mn;  // a partition may see no token of a draft row
    const float so = __builtin_amdgcn_exp2f(mg - mu_);
    const float sn = __builtin_amdgcn_exp2f(m - mu_);
    den = den * so + l * sn;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] = num[e] * so + a[e] * sn;
    mg = mn;
  }
  part_acc[g][c] = num;
  if (c == 0) {
    part_m[g] = mg;
    part_l[g] = den;
  }
  __syncthreads();
  if (tid < NC) {
    float M = part_m[0];
#pragma unroll
    for (int k = 1; k < NG; ++k) M = fmaxf(M, part_m[k]);
    const float mu_ = (M == kNegInf) ? 0.f : M;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    float dsum = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float w = __builtin_amdgcn_exp2f(part_m[k] - mu_);
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += w * part_acc[k][tid][e];
      dsum += w * part_l[k];
    }
    const int i = r / p.group, gg = r - (r / p.group) * p.group;
    const size_t orow = static_cast<size_t>(mu.q_row * p.k_draft + i) * p.hq + kvh * p.group + gg;
    const float inv = 1.f / dsum;
    T* op = static_cast<T*>(p.out) + orow * D + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_elem(op + e, sum[e] * inv);
    if (tid == 0 && p.lse) p.lse[orow] = (M + __builtin_amdgcn_logf(dsum)) * kLn2;
  }
}

// The fused append + single-tile decode at D = 128 holds two waves per SIMD
// by its registers, eight per CU.  Its launches reserve LDS that the kernel
// does not use, so that a CU holds six (16-bit pools) or seven (E4M3): fewer
// page requests queue in the memory system, and HBM delivers more of them.
// (Measured on MI355X, batch-256 step, 16-bit: 63.9-64.5 us at eight waves
// per CU, 63.8-64.1 at seven, 63.1-63.5 at six, 64.8-65.1 at five and four;
// E4M3, whose units are more latency-bound: 46.1-46.3 at eight, 45.4-45.5 at
// seven, 46.6 at six.  The plain decode launch over 8 x 32,768 tokens loses
// at six and at seven (176 -> 180-181 us) and the 70B-like one does not
// move, so they keep eight.)
template <typename T, int D, int NT, bool Q8>
constexpr unsigned fused_decode_lds() {
  return (!std::is_same_v<T, float> && D == 128 && NT == 1) ? (Q8 ? 22528u : 24576u) : 0u;
}

template <typename T, int D, int NT, bool NTL, bool Q8>
void launch_attn_nt(const AttnParams& p, const InlineMeta& m, hipStream_t stream) {
  if constexpr (!std::is_same_v<T, float> && !NTL && (D <= 128 ? NT <= 2 : NT == 1)) {
    if (p.pre_in_launch) {
      // (app_blocks counts workgroups of the launch's size here)
      const int attn_wg = (p.n_units * p.hkv + kPrefixLaunchWaves - 1) / kPrefixLaunchWaves;
      const dim3 grid(static_cast<unsigned>(attn_wg + p.n_pre_units * p.hkv + (p.t_new > 0 ? p.app_blocks : 0)));
      const dim3 block(64 * kPrefixLaunchWaves);
      if (p.t_new > 0)
        hipLaunchKernelGGL((attn_prefix_kernel<T, D, NT, true, Q8>), grid, block, 0, stream, p, m);
      else
        hipLaunchKernelGGL((attn_prefix_kernel<T, D, NT, false, Q8>), grid, block, 0, stream, p, m);
      return;
    }
  }
  if constexpr (!std::is_same_v<T, float>) {
    if (p.t_new > 0) {
      const dim3 grid(static_cast<unsigned>(p.n_units) * p.hkv + p.app_blocks);
      constexpr unsigned lds = fused_decode_lds<T, D, NT, Q8>();
      hipLaunchKernelGGL((attn_append_kernel<T, D, NT, NTL, Q8>), grid, dim3(64), lds, stream, p, m);
      return;
    }
  }
  const dim3 grid(static_cast<unsigned>(p.n_units) * p.hkv);
  hipLaunchKernelGGL((attn_kernel<T, D, NT, NTL, Q8>), grid, dim3(64), 0, stream, p);
}

template <typename T, int D, bool NTL, bool Q8>
hipError_t launch_attn_d(const AttnParams& p, const InlineMeta& m, hipStream_t stream) {
  // no fused fp32 path
  if (std::is_same_v<T, float> && p.t_new > 0) return hipErrorInvalidValue;
  if constexpr (!std::is_same_v<T, float>) {
    if (p.tile_rows > max_rows_for_head_dim(D)) {
      if (p.tile_rows != TileShape<D>::kRows || p.t_new > 0) return hipErrorInvalidValue;
      const dim3 grid(static_cast<unsigned>(p.n_units) * p.hkv);
      hipLaunchKernelGGL((tile_kernel<T, D, NTL, Q8>), grid, dim3(64 * TileShape<D>::W), 0, stream, p);
      return hipGetLastError();
    }
  }
  const int nt = (p.tile_rows + 15) / 16;
  if (nt <= 1)
    launch_attn_nt<T, D, 1, NTL, Q8>(p, m, stream);
  else if (nt <= 2)
    launch_attn_nt<T, D, 2, NTL, Q8>(p, m, stream);
  else if constexpr (D <= 128)
    launch_attn_nt<T, D, 4, NTL, Q8>(p, m, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, bool Q8 = false>
hipError_t launch_attn_t(const AttnParams& p, const InlineMeta& m, hipStream_t stream) {
  const bool ntl = p.stream_kv != 0 && !std::is_same_v<T, float>;
  switch (p.head_dim) {
    case 64: return ntl ? launch_attn_d<T, 64, true, Q8>(p, m, stream) : launch_attn_d<T, 64, false, Q8>(p, m, stream);
    case 128:
      return ntl ? launch_attn_d<T, 128, true, Q8>(p, m, stream) : launch_attn_d<T, 128, false, Q8>(p, m, stream);
    case 256:
      return ntl ? launch_attn_d<T, 256, true, Q8>(p, m, stream) : launch_attn_d<T, 256, false, Q8>(p, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int max_rows_for_head_dim(int head_dim) { return head_dim <= 128 ? 64 : 32; }

int tile_rows_for_call(int dtype, int head_dim, int rows) {
  const int one_wave = max_rows_for_head_dim(head_dim);
  if (rows <= one_wave) return rows;
  if (dtype == kF32) return one_wave;  // fp32: single-wave tiles
  switch (head_dim) {
    case 64: return TileShape<64>::kRows;
    case 128: return TileShape<128>::kRows;
    default: return TileShape<256>::kRows;
  }
}

namespace {
template <bool Q8>
int prefix_rows_t(int head_dim) {
  switch (head_dim) {
    case 64: return 16 * PrefixShape<64, Q8>::NT * PrefixShape<64, Q8>::W;
    case 128: return 16 * PrefixShape<128, Q8>::NT * PrefixShape<128, Q8>::W;
    default: return 16 * PrefixShape<256, Q8>::NT * PrefixShape<256, Q8>::W;
  }
}

template <bool Q8>
int prefix_units_t(int head_dim) {
  switch (head_dim) {
    case 64: return 4 * PrefixShape<64, Q8>::kWavesPerSimd / PrefixShape<64, Q8>::W;
    case 128: return 4 * PrefixShape<128, Q8>::kWavesPerSimd / PrefixShape<128, Q8>::W;
    default: return 4 * PrefixShape<256, Q8>::kWavesPerSimd / PrefixShape<256, Q8>::W;
  }
}
}  // namespace

// (wider row tiles would not fit the two waves per SIMD the pass needs)
bool prefix_in_attention_launch(int dtype, int head_dim, int rows) {
  return (dtype == kBF16 || dtype == kF16 || dtype == kFP8) && rows <= (head_dim <= 128 ? 32 : 16);
}

int prefix_rows_per_unit(int dtype, int head_dim) {
  return dtype == kFP8 ? prefix_rows_t<true>(head_dim) : prefix_rows_t<false>(head_dim);
}

int prefix_units_per_cu(int dtype, int head_dim) {
  return dtype == kFP8 ? prefix_units_t<true>(head_dim) : prefix_units_t<false>(head_dim);
}

hipError_t launch_prefix(DType dt, const AttnParams& p, hipStream_t stream) {
  if (p.n_pre_units == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.n_pre_units) * p.hkv);
  auto go = [&](auto kern, int waves) {
    hipLaunchKernelGGL(kern, grid, dim3(64 * waves), 0, stream, p);
    return hipGetLastError();
  };
  switch (dt) {
    case kBF16:
      switch (p.head_dim) {
        case 64: return go(prefix_kernel<__bf16, 64>, PrefixShape<64>::W);
        case 128: return go(prefix_kernel<__bf16, 128>, PrefixShape<128>::W);
        case 256: return go(prefix_kernel<__bf16, 256>, PrefixShape<256>::W);
      }
      break;
    case kF16:
      switch (p.head_dim) {
        case 64: return go(prefix_kernel<_Float16, 64>, PrefixShape<64>::W);
        case 128: return go(prefix_kernel<_Float16, 128>, PrefixShape<128>::W);
        case 256: return go(prefix_kernel<_Float16, 256>, PrefixShape<256>::W);
      }
      break;
    case kFP8:  // E4M3 codes, bf16 queries and partials
      switch (p.head_dim) {
        case 64: return go(prefix_kernel<__bf16, 64, true>, PrefixShape<64, true>::W);
        case 128: return go(prefix_kernel<__bf16, 128, true>, PrefixShape<128, true>::W);
        case 256: return go(prefix_kernel<__bf16, 256, true>, PrefixShape<256, true>::W);
      }
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

int append_blocks64(const AppendParams& p) {
  const AppendGrid g = append_grid(p, 64);
  return g.upd_blocks + g.cow_blocks + g.row_blocks;
}

int append_blocks_prefix_launch(const AppendParams& p) {
  const AppendGrid g = append_grid(p, 64 * kPrefixLaunchWaves);
  return g.upd_blocks + g.cow_blocks + g.row_blocks;
}

int prefix_rows_per_wave(int head_dim) { return 16 * (head_dim <= 128 ? PrefixShape<128>::NT : PrefixShape<256>::NT); }

int prefix_launch_waves() { return kPrefixLaunchWaves; }

hipError_t launch_append(const AppendParams& p, const InlineMeta* meta, hipStream_t stream) {
  const AppendGrid g = append_grid(p, kAppendThreads);
  const long long blocks = static_cast<long long>(g.upd_blocks) + g.cow_blocks + g.row_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.q8)
    hipLaunchKernelGGL((append_kernel<1>), dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, stream, p,
                       *meta);
  else if (p.elem_bytes == 2)
    hipLaunchKernelGGL((append_kernel<2>), dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, stream, p,
                       *meta);
  else
    hipLaunchKernelGGL((append_kernel<4>), dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, stream, p,
                       *meta);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_merge_t(const AttnParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.n_merges) * p.hkv * p.rows);
  const dim3 block(kMergeThreads);
  switch (p.head_dim) {
    case 64: hipLaunchKernelGGL((merge_kernel<T, 64>), grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((merge_kernel<T, 128>), grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL((merge_kernel<T, 256>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Merge of split sequences with at most kInlineMergeParts partitions, as a
// launch of its own after an attention launch that does not merge (the one
// that also runs the shared-prefix units): one wave per (split sequence, kv
// head, 4 query rows), four waves per workgroup, with the in-launch merge's
// arithmetic.  Every wave's loads leave at once, instead of the merges of a
// launch's last waves running one after the other in its tail.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_rows_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const int task = static_cast<int>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int groups = (p.rows + 3) / 4;
  const int per_merge = p.hkv * groups;
  const int m = task / per_merge;
  if (m >= p.n_merges) return;
  const int rem = task - m * per_merge;
  const int kvh = rem / groups;
  const int r0 = (rem - kvh * groups) * 4;
  merge_rows_of<T, D, false>(p, p.merges[m], kvh, lane, r0, min(r0 + 4, p.rows));
}

template <typename T>
hipError_t launch_merge_rows_t(const AttnParams& p, hipStream_t stream) {
  const long long tasks = static_cast<long long>(p.n_merges) * p.hkv * ((p.rows + 3) / 4);
  const dim3 grid(static_cast<unsigned>((tasks + 3) / 4));
  switch (p.head_dim) {
    case 64: hipLaunchKernelGGL((merge_rows_kernel<T, 64>), grid, dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((merge_rows_kernel<T, 128>), grid, dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL((merge_rows_kernel<T, 256>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int merge_rows_workgroups(const AttnParams& p) {
  const long long tasks = static_cast<long long>(p.n_merges) * p.hkv * ((p.rows + 3) / 4);
  return static_cast<int>((tasks + 3) / 4);
}

hipError_t launch_merge_rows(DType dt, const AttnParams& p, hipStream_t stream) {
  if (p.n_merges == 0) return hipSuccess;
  switch (dt) {
    case kBF16:
    case kFP8: return launch_merge_rows_t<__bf16>(p, stream);
    case kF16: return launch_merge_rows_t<_Float16>(p, stream);
    case kF32: return launch_merge_rows_t<float>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(DType dt, const AttnParams& p, hipStream_t stream) {
  if (p.n_merges == 0) return hipSuccess;
  switch (dt) {
    case kBF16:
    case kFP8: return launch_merge_t<__bf16>(p, stream);
    case kF16: return launch_merge_t<_Float16>(p, stream);
    case kF32: return launch_merge_t<float>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(DType dt, const AttnParams& p, const InlineMeta* meta, hipStream_t stream) {
  if (p.n_units == 0 && (p.t_new == 0 || p.app_blocks == 0) && !(p.pre_in_launch && p.n_pre_units > 0))
    return hipSuccess;
  switch (dt) {
    case kBF16: return launch_attn_t<__bf16>(p, *meta, stream);
    case kFP8: return launch_attn_t<__bf16, true>(p, *meta, stream);
    case kF16: return launch_attn_t<_Float16>(p, *meta, stream);
    case kF32: return launch_attn_t<float>(p, *meta, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
