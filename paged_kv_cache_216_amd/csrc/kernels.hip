// gfx950 (MI355X) kernels for paged KV-cache attention.
//
//  append_kernel     applies pending block-table / length updates, copies the
//                    filled slots of shared blocks before they are written
//                    (copy-on-write), and scatters new K/V rows into their slots.
//  attn_kernel       decode / speculative-verify attention over the block table:
//                    one 64-lane wave per (sequence, partition, key/value head);
//                    QK^T and PV on the matrix cores, online softmax in fp32.
//  merge_kernel      exact log-sum-exp merge of the partitions of split
//                    contexts (a separate launch: on MI355X each XCD has its
//                    own L2, so merging inside the attention launch would need
//                    device-scope write-back/invalidate fences per partition).
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

__host__ __device__ inline AppendGrid append_grid(const AppendParams& p) {
  AppendGrid g;
  g.upd_blocks = (p.n_tab + p.n_len + kAppendThreads - 1) / kAppendThreads;
  g.cow_blocks = p.n_cow;
  const int chunks_per_row = p.hkv * p.head_dim * p.elem_bytes / 16;
  const long long work = static_cast<long long>(p.n_rows) * chunks_per_row;
  g.row_blocks = static_cast<int>((work + kAppendThreads - 1) / kAppendThreads);
  return g;
}

template <int E>  // element bytes: 2 or 4
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendParams p) {
  using Elem = std::conditional_t<E == 2, uint16_t, uint32_t>;
  constexpr int X = 16 / E;  // elements per 16-byte chunk
  const AppendGrid g = append_grid(p);
  const int D = p.head_dim;
  const int nchunk = D / X;                               // chunks per (head, slot)
  const size_t page = static_cast<size_t>(D) * kBlk;      // elements per (block, head)
  int b = blockIdx.x;

  if (b < g.upd_blocks) {
    const int i = b * kAppendThreads + threadIdx.x;
    if (i < p.n_tab) {
      p.block_table[p.tab[2 * i]] = p.tab[2 * i + 1];
    } else if (i < p.n_tab + p.n_len) {
      const int k = i - p.n_tab;
      p.seq_len[p.lens[2 * k]] = p.lens[2 * k + 1];
    }
    return;
  }
  b -= g.upd_blocks;

  if (b < g.cow_blocks) {
    const int src = p.cows[3 * b], dst = p.cows[3 * b + 1], rows = p.cows[3 * b + 2];
    // K: 16-byte chunks (head, chunk, slot < rows)
    const u32x4* ks = reinterpret_cast<const u32x4*>(p.k_pool) + static_cast<size_t>(src) * p.hkv * nchunk * kBlk;
    u32x4* kd = reinterpret_cast<u32x4*>(p.k_pool) + static_cast<size_t>(dst) * p.hkv * nchunk * kBlk;
    const int kwork = p.hkv * nchunk * rows;
    for (int w = threadIdx.x; w < kwork; w += kAppendThreads) {
      const int t = w % rows;
      const int hc = w / rows;  // head * nchunk + chunk
      kd[hc * kBlk + t] = ks[hc * kBlk + t];
    }
    // V: elements (head, dim, slot < rows)
    const Elem* vs = reinterpret_cast<const Elem*>(p.v_pool) + static_cast<size_t>(src) * p.hkv * page;
    Elem* vd = reinterpret_cast<Elem*>(p.v_pool) + static_cast<size_t>(dst) * p.hkv * page;
    const int vwork = p.hkv * D * rows;
    for (int w = threadIdx.x; w < vwork; w += kAppendThreads) {
      const int t = w % rows;
      const int hd = w / rows;  // head * D + dim
      vd[hd * kBlk + t] = vs[hd * kBlk + t];
    }
    return;
  }
  b -= g.cow_blocks;

  // rows: one thread per 16-byte chunk of one row (all heads)
  const int chunks_per_row = p.hkv * nchunk;
  const long long w = static_cast<long long>(b) * kAppendThreads + threadIdx.x;
  if (w >= static_cast<long long>(p.n_rows) * chunks_per_row) return;
  const int row = static_cast<int>(w / chunks_per_row);
  const int c = static_cast<int>(w % chunks_per_row);  // head * nchunk + chunk
  const int h = c / nchunk;
  const int cc = c % nchunk;
  const int slot = p.slots[row];
  const int phys = slot / kBlk;
  const int t = slot % kBlk;
  const u32x4 kv = reinterpret_cast<const u32x4*>(p.k_new)[static_cast<size_t>(row) * chunks_per_row + c];
  u32x4* kdst = reinterpret_cast<u32x4*>(p.k_pool) +
                ((static_cast<size_t>(phys) * p.hkv + h) * nchunk + cc) * kBlk + t;
  *kdst = kv;
  const Elem* vsrc = reinterpret_cast<const Elem*>(p.v_new) + (static_cast<size_t>(row) * chunks_per_row + c) * X;
  Elem* vdst = reinterpret_cast<Elem*>(p.v_pool) + (static_cast<size_t>(phys) * p.hkv + h) * page +
               static_cast<size_t>(cc) * X * kBlk + t;
#pragma unroll
  for (int i = 0; i < X; ++i) vdst[i * kBlk] = vsrc[i];
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

__device__ inline float wave_max_groups(float x) {
  // max over lanes col, col+16, col+32, col+48
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

// K/V pages are read once per launch: load them with the non-temporal hint so
// they stream past the caches instead of evicting the tables and queries.
template <typename V>
__device__ inline V stream_load(const V* p) {
  return __builtin_nontemporal_load(p);
}

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

// A work unit with its token range resolved against the current length.
struct Unit {
  int q_row, seq, n, tok_begin, tok_end, slot_base, nparts, part;
};

// 16-bit element types: bf16 or f16
template <typename T, int D, int NT>
__device__ inline void attn_body16(const AttnParams& p, const Unit& u, int kvh) {
  using Op = typename MfmaOp<T>::type;
  constexpr int KS = D / 32;  // QK k-steps per block
  constexpr int DC = D / 16;  // output dim chunks
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rows = p.rows;
  const int G = p.group;

  // ---- queries (B operand of S^T = K Q^T), per row tile
  Op qop[NT][KS];
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + col;
    if (r < rows) {
      const int i = r / G, g = r - (r / G) * G;
      const T* qp = static_cast<const T*>(p.q) +
                    (static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qop[nt][s] = __builtin_bit_cast(Op, *reinterpret_cast<const u32x4*>(qp + 32 * s + 8 * grp));
      lim[nt] = u.n - p.k_draft + i;
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qop[nt][s] = Op{};
      lim[nt] = u.n - 1;
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

  const T* kpool = static_cast<const T*>(p.k_pool);
  const T* vpool = static_cast<const T*>(p.v_pool);
  const size_t page = static_cast<size_t>(D) * kBlk;
  const int32_t* bt = p.block_table + static_cast<size_t>(u.seq) * p.max_blocks;
  const int jb0 = u.tok_begin / kBlk;
  const int nblk = (u.tok_end + kBlk - 1) / kBlk - jb0;
  const int mask_from = u.n - p.k_draft;  // positions above this may be masked for some row

  // One pair of blocks = one PV step.  The loads of pair j+1 are issued before
  // pair j is computed, so each wave keeps 16-32 KiB of K/V in flight (except
  // for the largest query tiles, whose accumulators need those registers).
  struct Frag {
    Op k0[KS], k1[KS];
    u32x2 v0[DC], v1[DC];
  };
  for (int cb = 0; cb < nblk; cb += 64) {
    const int cnt = min(64, nblk - cb);
    const int tb = (lane < cnt) ? bt[jb0 + cb + lane] : 0;  // this chunk of the table, one entry per lane
    const int npairs = (cnt + 1) >> 1;
    // a table entry outside the pool can only come from a host-side bug; clamp
    // it so that the bug shows as a wrong result, never as a stray access
    auto phys_at = [&](int j) { return min(max(readlane(tb, j), 0), p.num_blocks - 1); };
    // Branch-free: a pair past the end (or the missing second block of an odd
    // count) re-reads blocks already requested, which hit in cache, and every
    // position it contributes is masked.  Uniform control flow lets the
    // compiler wait only for the pair being computed.
    auto load = [&](Frag& f, int pj) {
      const int j = min(2 * pj, cnt - 1);
      const int phys0 = phys_at(j);
      const int phys1 = phys_at(min(j + 1, cnt - 1));
      const T* kp0 = kpool + (static_cast<size_t>(phys0) * p.hkv + kvh) * page;
      const T* vp0 = vpool + (static_cast<size_t>(phys0) * p.hkv + kvh) * page;
      const T* kp1 = kpool + (static_cast<size_t>(phys1) * p.hkv + kvh) * page;
      const T* vp1 = vpool + (static_cast<size_t>(phys1) * p.hkv + kvh) * page;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        f.k0[s] = __builtin_bit_cast(Op, stream_load(reinterpret_cast<const u32x4*>(kp0 + ((4 * s + grp) * kBlk + col) * 8)));
#pragma unroll
      for (int s = 0; s < KS; ++s)
        f.k1[s] = __builtin_bit_cast(Op, stream_load(reinterpret_cast<const u32x4*>(kp1 + ((4 * s + grp) * kBlk + col) * 8)));
#pragma unroll
      for (int c = 0; c < DC; ++c) f.v0[c] = stream_load(reinterpret_cast<const u32x2*>(vp0 + (16 * c + col) * kBlk + 4 * grp));
#pragma unroll
      for (int c = 0; c < DC; ++c) f.v1[c] = stream_load(reinterpret_cast<const u32x2*>(vp1 + (16 * c + col) * kBlk + 4 * grp));
    };
    auto process = [&](Frag& f, int pj) {
      const int pos0 = (jb0 + cb + 2 * pj) * kBlk;  // first token of the pair
      const bool need_mask = (pos0 + 2 * kBlk - 1 > mask_from) || (pos0 + 2 * kBlk > u.tok_end);
      Op pa[NT];
      float a4[NT][4];
      // scores and online-softmax update for every row tile (needs K only)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          s0 = MfmaOp<T>::mma(f.k0[s], qop[nt][s], s0);
          s1 = MfmaOp<T>::mma(f.k1[s], qop[nt][s], s1);
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = s0[e] * p.scale_log2;
          x[4 + e] = s1[e] * p.scale_log2;
        }
        if (need_mask) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int pos = pos0 + (e >> 2) * kBlk + 4 * grp + (e & 3);
            const bool ok = pos < u.tok_end && pos <= lim[nt];
            x[e] = ok ? x[e] : kNegInf;
          }
        }
        float mt = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, x[e]);
        mt = wave_max_groups(mt);
        const float m_new = fmaxf(m_run[nt], mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(x[e] - m_use);
          ps += pe;
          pa[nt][e] = static_cast<T>(pe);
        }
        l_run[nt] = l_run[nt] * alpha + ps;
        m_run[nt] = m_new;
        // rescale factors move to the accumulator layout: lane holds rows 4*grp + jj
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) a4[nt][jj] = shfl_f(alpha, 4 * grp + jj);
      }
      // slots past the end of the sequence may hold anything: zero their V
      if (pos0 + 2 * kBlk > u.n) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          f.v0[c] = mask_v16(f.v0[c], pos0 + 4 * grp, u.n);
          f.v1[c] = mask_v16(f.v1[c], pos0 + kBlk + 4 * grp, u.n);
        }
      }
      // O = diag(alpha) O + P V
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[nt][c][jj] *= a4[nt][jj];
          const Op vb = __builtin_bit_cast(Op, u32x4{f.v0[c][0], f.v0[c][1], f.v1[c][0], f.v1[c][1]});
          acc[nt][c] = MfmaOp<T>::mma(pa[nt], vb, acc[nt][c]);
        }
      }
    };
    if constexpr (D * NT < 512) {
      Frag fa, fb;
      load(fa, 0);
      for (int pj = 0; pj < npairs; pj += 2) {
        load(fb, min(pj + 1, npairs - 1));
        process(fa, pj);
        if (pj + 1 >= npairs) break;
        load(fa, min(pj + 2, npairs - 1));
        process(fb, pj + 1);
      }
    } else {
      // the largest query tiles leave no registers for a second pair in flight
      for (int pj = 0; pj < npairs; ++pj) {
        Frag fa;
        load(fa, pj);
        process(fa, pj);
      }
    }
  }

  // ---- epilogue
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
        if (r < rows) {
          const int i = r / G, g = r - (r / G) * G;
          T* op = static_cast<T*>(p.out) +
                  (static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) store_elem(op + 16 * c + col, acc[nt][c][jj] * inv[jj]);
        }
      }
      const int r = nt * 16 + col;
      if (p.lse && grp == 0 && r < rows) {
        const int i = r / G, g = r - (r / G) * G;
        p.lse[static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g] =
            (m_run[nt] + __builtin_amdgcn_logf(l)) * kLn2;
      }
    } else {
      const int slot = u.slot_base + kvh * u.nparts + u.part;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = nt * 16 + 4 * grp + jj;
        if (r < rows) {
          float* ap = p.ws_acc + (static_cast<size_t>(slot) * rows + r) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) ap[16 * c + col] = acc[nt][c][jj];
        }
      }
      const int r = nt * 16 + col;
      if (grp == 0 && r < rows) {
        float* mp = p.ws_ml + (static_cast<size_t>(slot) * rows + r) * 2;
        mp[0] = m_run[nt];
        mp[1] = l;
      }
    }
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

  f32x4 qv[NT][KS];
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + col;
    if (r < rows) {
      const int i = r / G, g = r - (r / G) * G;
      const float* qp = static_cast<const float*>(p.q) +
                        (static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) qv[nt][s] = *reinterpret_cast<const f32x4*>(qp + 16 * s + 4 * grp);
      lim[nt] = u.n - p.k_draft + i;
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qv[nt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
      lim[nt] = u.n - 1;
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
  const int nblk = (u.tok_end + kBlk - 1) / kBlk - jb0;
  const int mask_from = u.n - p.k_draft;

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
      if (pos0 + kBlk > u.n) {
#pragma unroll
        for (int c = 0; c < DC; ++c) vv[c] = mask_v32(vv[c], pos0 + 4 * grp, u.n);
      }
      const bool need_mask = (pos0 + kBlk - 1 > mask_from) || (pos0 + kBlk > u.tok_end);
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
            x[e] = (pos < u.tok_end && pos <= lim[nt]) ? x[e] : kNegInf;
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
        if (r < rows) {
          const int i = r / G, g = r - (r / G) * G;
          float* op = static_cast<float*>(p.out) +
                      (static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) op[16 * c + col] = acc[nt][c][jj] * inv[jj];
        }
      }
      const int r = nt * 16 + col;
      if (p.lse && grp == 0 && r < rows) {
        const int i = r / G, g = r - (r / G) * G;
        p.lse[static_cast<size_t>(u.q_row * p.k_draft + i) * p.hq + kvh * G + g] =
            (m_run[nt] + __builtin_amdgcn_logf(l)) * kLn2;
      }
    } else {
      const int slot = u.slot_base + kvh * u.nparts + u.part;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = nt * 16 + 4 * grp + jj;
        if (r < rows) {
          float* ap = p.ws_acc + (static_cast<size_t>(slot) * rows + r) * D;
#pragma unroll
          for (int c = 0; c < DC; ++c) ap[16 * c + col] = acc[nt][c][jj];
        }
      }
      const int r = nt * 16 + col;
      if (grp == 0 && r < rows) {
        float* mp = p.ws_ml + (static_cast<size_t>(slot) * rows + r) * 2;
        mp[0] = m_run[nt];
        mp[1] = l;
      }
    }
  }
}

template <typename T, int D, int NT>
__global__ __launch_bounds__(64) void attn_kernel(AttnParams p) {
  const int unit = blockIdx.x / p.hkv;
  const int kvh = blockIdx.x - unit * p.hkv;
  const WorkUnit w = p.units[unit];
  Unit u;
  u.q_row = w.q_row;
  u.seq = w.seq;
  u.slot_base = w.slot_base;
  u.nparts = w.nparts;
  u.part = w.part;
  // the length mirror is bounded by the table row the host allocated
  u.n = min(p.seq_len[w.seq], p.max_blocks * kBlk);
  u.tok_begin = w.nparts > 1 ? w.part * p.part_tokens : 0;
  u.tok_end = w.nparts > 1 ? min(u.n, u.tok_begin + p.part_tokens) : u.n;
  if constexpr (std::is_same_v<T, float>)
    attn_body32<D, NT>(p, u, kvh);
  else
    attn_body16<T, D, NT>(p, u, kvh);
}

// Exact merge of one output row of a split sequence, one 256-thread workgroup
// per (sequence, key/value head, query row):
//   M = max_p m_p,  w_p = 2^(m_p - M),  O = sum_p w_p acc_p / sum_p w_p l_p,
//   lse = (M + log2 sum_p w_p l_p) * ln 2
// The D/4 16-byte chunks of a row are spread over D/4 threads; the partitions
// over NG = 1024/D groups of such threads (partition q to group q % NG), so
// every thread has several independent loads in flight.  Groups are combined
// in a fixed order, so the result is deterministic.
constexpr int kMergeThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnParams p) {
  constexpr int NC = D / 4;                 // float4 chunks per row
  constexpr int NG = kMergeThreads / NC;    // partition groups
  __shared__ float red[kMergeThreads / 64];
  __shared__ f32x4 part_acc[NG][NC];
  __shared__ float part_den[NG];
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
  // block-wide max of m_q
  float M = kNegInf;
  for (int q = tid; q < P; q += kMergeThreads) M = fmaxf(M, ml[q * mstride]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w]);
  // weighted sums: thread (g, c) takes chunk c of partitions g, g + NG, ...
  const int g = tid / NC;
  const int c = tid - g * NC;
  const f32x4* acc = reinterpret_cast<const f32x4*>(p.ws_acc + (static_cast<size_t>(base) * rows + r) * D) + c;
  const size_t astride = static_cast<size_t>(rows) * D / 4;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll 8
  for (int q = g; q < P; q += NG) {
    const float w = __builtin_amdgcn_exp2f(ml[q * mstride] - M);
    den += w * ml[q * mstride + 1];
    const f32x4 a = acc[q * astride];
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] += w * a[e];
  }
  part_acc[g][c] = num;
  if (c == 0) part_den[g] = den;
  __syncthreads();
  if (tid < NC) {
    f32x4 sum = part_acc[0][tid];
    float dsum = part_den[0];
#pragma unroll
    for (int k = 1; k < NG; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += part_acc[k][tid][e];
      dsum += part_den[k];
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

template <typename T, int D>
hipError_t launch_attn_d(const AttnParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.n_units) * p.hkv);
  const int nt = (p.rows + 15) / 16;
  if (nt <= 1)
    hipLaunchKernelGGL((attn_kernel<T, D, 1>), grid, dim3(64), 0, stream, p);
  else if (nt <= 2)
    hipLaunchKernelGGL((attn_kernel<T, D, 2>), grid, dim3(64), 0, stream, p);
  else if constexpr (D <= 128)
    hipLaunchKernelGGL((attn_kernel<T, D, 4>), grid, dim3(64), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_t(const AttnParams& p, hipStream_t stream) {
  switch (p.head_dim) {
    case 64: return launch_attn_d<T, 64>(p, stream);
    case 128: return launch_attn_d<T, 128>(p, stream);
    case 256: return launch_attn_d<T, 256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int max_rows_for_head_dim(int head_dim) { return head_dim <= 128 ? 64 : 32; }

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const AppendGrid g = append_grid(p);
  const long long blocks = static_cast<long long>(g.upd_blocks) + g.cow_blocks + g.row_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.elem_bytes == 2)
    hipLaunchKernelGGL((append_kernel<2>), dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((append_kernel<4>), dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, stream, p);
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

hipError_t launch_merge(DType dt, const AttnParams& p, hipStream_t stream) {
  if (p.n_merges == 0) return hipSuccess;
  switch (dt) {
    case kBF16: return launch_merge_t<__bf16>(p, stream);
    case kF16: return launch_merge_t<_Float16>(p, stream);
    case kF32: return launch_merge_t<float>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(DType dt, const AttnParams& p, hipStream_t stream) {
  if (p.n_units == 0) return hipSuccess;
  switch (dt) {
    case kBF16: return launch_attn_t<__bf16>(p, stream);
    case kF16: return launch_attn_t<_Float16>(p, stream);
    case kF32: return launch_attn_t<float>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
