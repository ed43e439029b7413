// Launch interface between the C-ABI layer (pa_api.cpp) and the gfx950 kernels
// (kernels.hip).  Plain structs of device pointers and sizes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

// kFP8: pools hold E4M3 codes (one byte per element); the rows appended, the
// queries and the outputs are bf16, and each (K or V, kv head) has a scale.
enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

// Per-call int32 metadata travels inside the launch's kernel arguments when it
// fits (no copy, no host-memory reads from the GPU); larger metadata is read by
// the kernel from pinned host memory (`ext` below).
constexpr int kInlineWords = 2048;
struct InlineMeta {
  int32_t w[kInlineWords];
};

// Table updates, copy-on-write block copies and the scatter of new rows.
// Offsets are in int32 words into the call's metadata:
//   tab  [n_tab][2]  (flat table index, physical block)
//   lens [n_len][2]  (sequence, length)
//   cows [n_cow][3]  (src block, dst block, rows to copy)
//   slots[n_rows]    (physical block * 16 + slot) for row r of k_new / v_new
struct AppendParams {
  void* k_pool;
  void* v_pool;
  int32_t* block_table;
  int32_t* seq_len;
  const void* k_new;
  const void* v_new;
  const int32_t* ext;  // metadata in pinned host memory, or nullptr: inline
  int tab, lens, cows, slots;
  int n_tab, n_len, n_cow, n_rows;
  int hkv, head_dim, elem_bytes;  // elem_bytes: of the rows appended (2 for E4M3 pools)
  int q8;                         // 1: E4M3 pool, rows are quantized on the way in
  const float* kv_scale;          // E4M3: [4][hkv] k_scale, v_scale, 1/k_scale, 1/v_scale
};

// Work unit of the attention kernel, one per (sequence, partition); the
// key/value head comes from the grid.  Lengths are not part of the unit: the
// kernel reads them from the device length mirror (or, when the launch also
// appends, from the call's metadata), so a plan stays valid while sequences
// grow inside their partitions.  A partition covers [tok_begin, tok_begin +
// part_tokens); the last one runs to the end of the sequence.
struct WorkUnit {
  int32_t q_row;      // index of the sequence in q / out (0..n_seq-1)
  int32_t seq;        // row of the block table and of the length mirror
  int32_t part;       // partition index
  int32_t nparts;     // partitions of this sequence (1 = unsplit)
  int32_t slot_base;  // -1: write out/lse directly; else partial slot of kv head 0, part 0
  int32_t row0;       // first query row of the unit's tile: calls with more rows
                      // than one unit takes (tile_rows) have one unit per tile
  int32_t merge;      // split sequences: index of its MergeUnit; else -1
  int32_t tok_begin;  // first position of the partition
};

// Shared-prefix pass.  Sequences of a batch that are copy-on-write forks of
// one prefix read the same physical blocks for its first `prefix_tokens`
// tokens (a multiple of the partition length).  The pass computes those
// partitions once for the query rows of all such sequences together -- up to
// 64 rows per wave instead of one sequence's G * k_draft -- and writes each
// row's partial into the slot of its own sequence's partition; the sequence's
// later partitions and the merge are the usual ones.
struct PrefixMember {
  int32_t q_row;      // index of the sequence in q / out
  int32_t slot_base;  // its partial slot of kv head 0, part 0
  int32_t nparts;     // its partitions
  int32_t merge;      // its MergeUnit
};

struct PrefixUnit {
  int32_t seq;            // a member's table row (the prefix blocks are the same in all)
  int32_t part;           // partition of the prefix
  int32_t row0;           // first row of the group's rows (member * rows + row) for this wave
  int32_t member0;        // the group's first entry in the member array
  int32_t group_rows;     // members * rows
  int32_t prefix_tokens;  // the shared positions; the last partition ends there
  int32_t pad0, pad1;
};

// One split sequence: its partials are merged into out / lse.  With the
// in-launch merge, `arrivals` is the number of times per kv head that a wave
// of the merging launch finishes partials of this sequence (its own
// partitions, and the shared-prefix waves covering its rows when they run in
// the same launch); the wave that arrives last merges.
struct MergeUnit {
  int32_t q_row;
  int32_t slot_base;
  int32_t nparts;
  int32_t arrivals;
};

struct AttnParams {
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_len;
  int max_blocks;
  int num_blocks;     // physical blocks; table entries are clamped into range
  int part_tokens;    // partition length of split sequences (multiple of 32)
  const void* q;
  void* out;
  float* lse;
  float* ws_acc;      // [slot][R][D] unnormalised partial outputs
  float* ws_ml;       // [slot][R][2] running max (log2 domain) and sum
  const WorkUnit* units;
  const MergeUnit* merges;
  int n_units;
  int n_merges;
  int hkv, hq, group, k_draft, rows;  // rows = group * k_draft
  int tile_rows;      // query rows one unit takes (tile_rows_for_call)
  int head_dim;
  float scale_log2;   // scale * log2(e)
  int stream_kv;      // 1: no block is shared, read K/V pages with the non-temporal hint
  // Fused append (t_new > 0): this launch also appends t_new rows per sequence.
  // Attention reads the new rows from k_new / v_new ([n_seq * t_new][hkv][D],
  // row q_row * t_new + i) and the lengths after the append from the metadata
  // at `lens_by_row`; `app` (run by `app_blocks` extra workgroups) writes the
  // rows into the pool and updates the table and length mirrors.
  int t_new;
  int lens_by_row;
  int app_blocks;
  AppendParams app;
  // In-launch merge (inline_merge = 1): the last wave to finish partials of a
  // split (sequence, kv head) merges all of them; merge_ctr[merge * hkv + kvh]
  // counts the arrivals and is zero between launches.  Used when every split
  // sequence has at most kInlineMergeParts partitions and one unit takes all
  // query rows of a (sequence, kv head).
  unsigned* merge_ctr;
  int inline_merge;
  const float* kv_scale;  // E4M3 pools: [4][hkv] k_scale, v_scale, 1/k_scale, 1/v_scale
  // shared-prefix pass (launch_prefix)
  const PrefixUnit* pre_units;
  const PrefixMember* pre_members;
  int n_pre_units;
  // 1: the shared-prefix units run in the attention launch itself, after the
  // attention units; the splits are then merged by launch_merge_rows
  int pre_in_launch;
  // Graph steps (graph_units > 0, fused append + attention): the grid is
  // padded to graph_units units and the launch's append workgroups, and the
  // counts that change from step to step are read from the head of the step's
  // metadata (kGraph* words below) instead of from these parameters.
  int graph_units;
};

// Head of a graph step's metadata: the units of this step; the table
// updates, length updates and new rows of its append; where in the metadata
// its slots, table updates and length updates start.  The lengths by row
// follow the head.
constexpr int kGraphUnits = 0, kGraphTab = 1, kGraphLen = 2, kGraphRows = 3, kGraphSlotsAt = 4, kGraphTabAt = 5,
              kGraphLenAt = 6, kGraphHeader = 8;

constexpr int kInlineMergeParts = 16;

hipError_t launch_append(const AppendParams& p, const InlineMeta* meta, hipStream_t stream);
hipError_t launch_attention(DType dt, const AttnParams& p, const InlineMeta* meta, hipStream_t stream);
hipError_t launch_merge(DType dt, const AttnParams& p, hipStream_t stream);
// The merge of splits with at most kInlineMergeParts partitions, one wave per
// (split, kv head, 4 query rows), after an attention launch that runs the
// shared-prefix units and does not merge; and its workgroup count.
hipError_t launch_merge_rows(DType dt, const AttnParams& p, hipStream_t stream);
int merge_rows_workgroups(const AttnParams& p);
// The shared-prefix pass as a launch of its own, run before launch_attention
// (when pre_in_launch is 0).
hipError_t launch_prefix(DType dt, const AttnParams& p, hipStream_t stream);
// Query rows one workgroup of the shared-prefix pass takes, for a head dim.
int prefix_rows_per_unit(int dtype, int head_dim);
// Whether the shared-prefix pass can run inside the attention launch of a
// call with `rows` query rows per kv head (four-wave workgroups: the pass's
// units, and attention workgroups of four single-wave units, all fitting two
// waves per SIMD).
bool prefix_in_attention_launch(int dtype, int head_dim, int rows);
// workgroups of the shared-prefix pass one compute unit holds at once
int prefix_units_per_cu(int dtype, int head_dim);
// Workgroups of 64 threads that the append work of `p` needs.
int append_blocks64(const AppendParams& p);
// Workgroups that the append work of `p` needs in the attention launch that
// also runs the shared-prefix units (pre_in_launch: workgroups of
// prefix_launch_waves() waves, each running that many attention units).
int append_blocks_prefix_launch(const AppendParams& p);
int prefix_launch_waves();
// Query rows one wave of the shared-prefix pass takes.
int prefix_rows_per_wave(int head_dim);
// Query rows one single-wave attention unit takes at most, for a head dim.
int max_rows_for_head_dim(int head_dim);
// Query rows per unit for a call with `rows` rows per kv head: all of them when
// one wave takes them; else a multi-wave workgroup's tile (16-bit and E4M3
// pools) or a single wave's (fp32 pools).
int tile_rows_for_call(int dtype, int head_dim, int rows);

}  // namespace pa
