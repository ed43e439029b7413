// C-ABI entry points declared in include/pa.h.
//
// Host side of every device call: validate, update the block allocator,
// assemble the call's metadata (table updates, copies, slots, lengths) and
// launch the kernels.  Metadata up to 8 KiB travels inside the launch's kernel
// arguments; larger metadata (bulk appends) is written to a pinned,
// device-visible host buffer that the kernel reads directly, from a ring whose
// buffers are released by events recorded after their last reader.  The
// attention work plan (which sequence / partition each workgroup takes) lives
// in device memory and is re-uploaded only when the batch or its partition
// structure changes; lengths come from the device length mirror, or from the
// metadata when the launch itself appends.
#include "../../include/pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "block_pool.hpp"
#include "kernels.hpp"
#include "scratch.hpp"
#include "swap.hpp"

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_err(hipError_t e, const char* what) {
  return set_err(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

constexpr int kStages = 64;
constexpr int kDefaultPartition = 512;
// The library's partition length for a call with `rows` query rows per kv
// head: 512 tokens, or 8 tokens per row when that is more, so that the split
// partials (rows x (D + 2) floats per partition) stay within an eighth of the
// key/value bytes the partition reads.
int default_partition(int64_t rows) {
  const int64_t pt = std::max<int64_t>(kDefaultPartition, (8 * rows + 31) / 32 * 32);
  return static_cast<int>(std::min<int64_t>(pt, int64_t{1} << 30));
}
// query rows (group * queries per sequence) of one attention call; more than
// one unit's worth are split into row tiles
constexpr int64_t kMaxRows = int64_t{1} << 22;

struct Stage {
  int32_t* host = nullptr;  // pinned, fine-grained (the GPU reads it without caching it)
  int32_t* dev = nullptr;   // the same memory as seen by the GPU
  size_t cap = 0;           // int32 words
  hipEvent_t done = nullptr;
  bool pending = false;
};

struct ProfEvent {
  int which;
  hipEvent_t start, stop;
};

// A group of copy-on-write forks found by the shared-prefix detection:
// tokens all of them hold in the same blocks (and every query row sees), and
// how many sequences of the call it has.
struct PrefixGroup {
  int shared, members;
};

// Graph steps of one capacity class (units of the padded grid, rows appended
// per sequence): a device buffer holding the step's metadata and its plan,
// the in-launch merge counters, and the launch parameters, which point at
// them and so stay the same from step to step.
// Device buffers of one class of graph steps (units padded to a power of
// two, rows appended per sequence): the step's own words -- a header, then the
// lengths by row, the slots, the table and length updates, packed -- and, at
// fixed offsets after room for the largest such step, the plan (units, then
// merges).  `plan` is the plan last written there.
struct GraphClass {
  int32_t* buf = nullptr;
  unsigned* ctr = nullptr;
  pa::AttnParams params{};
  int units = 0, n_new = 0;
  size_t tab_cap = 0, step_words = 0, words = 0, off_units = 0, off_merges = 0;
  std::vector<int32_t> plan;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct pa_pool {
  pa::BlockPool bp;
  int num_blocks = 0, hkv = 0, head_dim = 0, dtype = 0, esize = 0;
  void* k_pool = nullptr;
  void* v_pool = nullptr;
  int32_t* block_table = nullptr;
  int32_t* seq_len = nullptr;
  bool host_only = false;
  char* scratch = nullptr;  // this device's fixed scratch (pa_decode_noalloc)
  int num_cus = 256;  // compute units of the pool's device
  int last_pt = 0, last_prefix_units = 0;  // of the last attention call
  pa_call_stats last_stats{};
  // metadata ring
  Stage stage[kStages];
  int next_stage = 0;
  // cached attention plan in device memory: WorkUnits then MergeUnits
  void* dplan = nullptr;
  size_t dplan_cap = 0;  // bytes
  bool dplan_stale = false;  // the host plan changed without an upload to dplan
  // E4M3 pools: [4][hkv] k_scale, v_scale, 1/k_scale, 1/v_scale (device; host copy)
  float* kv_scale = nullptr;
  std::vector<float> kv_scale_host;
  // partition counters of the in-launch merge, zero between launches
  unsigned* merge_ctr = nullptr;
  size_t merge_ctr_cap = 0;  // counters
  int plan_max_parts = 0;
  std::vector<int32_t> plan_key, key_scratch;
  int plan_units = 0, plan_merges = 0;
  int64_t plan_slots = 0;
  int64_t plan_prefix_tokens = 0, plan_prefix_rows = 0;  // shared-prefix pass: positions read, rows served
  // reused host scratch
  pa::BlockPool::Dirty dirty;
  std::vector<int32_t> slots;
  std::vector<pa::CowCopy> cows;
  std::vector<int32_t> cow_src;  // sorted source blocks of this call's copies
  std::vector<pa::WorkUnit> units;
  std::vector<std::pair<int, pa::WorkUnit>> tail_units;  // (tokens the unit reads, unit)
  std::vector<pa::MergeUnit> merges;
  std::vector<int> lens, parts;
  // shared-prefix pass: partitions of each sequence done by the pass (0 = none)
  // and the shared positions they cover (the sequence's own partitions start there)
  std::vector<int> pre_parts, pre_shared;
  std::vector<std::pair<int32_t, int>> pre_scratch;
  std::vector<PrefixGroup> pre_groups;
  std::vector<pa::PrefixUnit> pre_units;
  std::vector<pa::PrefixMember> pre_members;
  int plan_pre_units = 0;
  bool plan_pre_in_launch = false;
  std::vector<int32_t> ntok;
  // call metadata being assembled, and its kernel-argument copy
  std::vector<int32_t> meta;
  pa::InlineMeta inline_meta;
  // graph steps: classes by (units, rows appended per sequence), and the one
  // the last pa_graph_prepare filled
  std::map<std::pair<int, int>, GraphClass> gclass;
  GraphClass* glast = nullptr;
  // profiling
  bool prof = false;
  std::vector<ProfEvent> prof_events;
  double prof_ms[4] = {0, 0, 0, 0};
  int64_t prof_n[4] = {0, 0, 0, 0};
};

namespace {

// Take the next ring buffer with room for `words` int32 values.
int acquire_stage(pa_pool* p, size_t words, Stage** out) {
  Stage& st = p->stage[p->next_stage];
  p->next_stage = (p->next_stage + 1) % kStages;
  if (st.pending) {
    hipError_t e = hipEventSynchronize(st.done);
    if (e != hipSuccess) return hip_err(e, "hipEventSynchronize(staging)");
    st.pending = false;
  }
  if (words > st.cap) {
    const size_t cap = std::max<size_t>(words, std::max<size_t>(2 * st.cap, 4096));
    if (st.host) (void)hipHostFree(st.host);
    st.host = st.dev = nullptr;
    st.cap = 0;
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&st.host), cap * sizeof(int32_t),
                                 hipHostMallocCoherent | hipHostMallocMapped);
    if (e != hipSuccess) return hip_err(e, "hipHostMalloc(staging)");
    e = hipHostGetDevicePointer(reinterpret_cast<void**>(&st.dev), st.host, 0);
    if (e != hipSuccess) return hip_err(e, "hipHostGetDevicePointer(staging)");
    st.cap = cap;
  }
  *out = &st;
  return PA_OK;
}

// The buffer may be rewritten once the work enqueued so far on `stream` is done.
int release_stage(Stage* st, hipStream_t stream) {
  hipError_t e = hipEventRecord(st->done, stream);
  if (e != hipSuccess) return hip_err(e, "hipEventRecord(staging)");
  st->pending = true;
  return PA_OK;
}

int ensure_dplan(pa_pool* p, size_t bytes) {
  if (bytes <= p->dplan_cap) return PA_OK;
  const size_t cap = std::max(bytes, 2 * p->dplan_cap);
  hipError_t e = hipDeviceSynchronize();  // no launch may still read the old plan
  if (e != hipSuccess) return hip_err(e, "hipDeviceSynchronize");
  if (p->dplan) (void)hipFree(p->dplan);
  p->dplan = nullptr;
  p->dplan_cap = 0;
  e = hipMalloc(&p->dplan, cap);
  if (e != hipSuccess) return hip_err(e, "hipMalloc(plan)");
  p->dplan_cap = cap;
  return PA_OK;
}

void prof_begin(pa_pool* p, int which, hipStream_t s, ProfEvent* ev) {
  if (!p->prof) return;
  ev->which = which;
  (void)hipEventCreate(&ev->start);
  (void)hipEventCreate(&ev->stop);
  (void)hipEventRecord(ev->start, s);
}

void prof_end(pa_pool* p, hipStream_t s, ProfEvent* ev) {
  if (!p->prof) return;
  (void)hipEventRecord(ev->stop, s);
  p->prof_events.push_back(*ev);
}

pa::AppendParams base_append(pa_pool* p) {
  pa::AppendParams ap{};
  ap.k_pool = p->k_pool;
  ap.v_pool = p->v_pool;
  ap.block_table = p->block_table;
  ap.seq_len = p->seq_len;
  ap.hkv = p->hkv;
  ap.head_dim = p->head_dim;
  ap.elem_bytes = p->dtype == PA_FP8_E4M3 ? 2 : p->esize;  // rows appended to E4M3 pools are bf16
  ap.q8 = p->dtype == PA_FP8_E4M3 ? 1 : 0;
  ap.kv_scale = p->kv_scale;
  return ap;
}

size_t pad8(std::vector<int32_t>& w) {
  while (w.size() % 8) w.push_back(0);
  return w.size();
}

// Append the pending table / length updates to the call's metadata.
void meta_dirty(pa_pool* p, pa::AppendParams* ap) {
  const pa::BlockPool::Dirty& d = p->dirty;
  std::vector<int32_t>& w = p->meta;
  ap->tab = static_cast<int>(pad8(w));
  for (size_t i = 0; i < d.table_idx.size(); ++i) {
    w.push_back(d.table_idx[i]);
    w.push_back(d.table_val[i]);
  }
  ap->lens = static_cast<int>(pad8(w));
  for (size_t i = 0; i < d.len_seq.size(); ++i) {
    w.push_back(d.len_seq[i]);
    w.push_back(d.len_val[i]);
  }
  ap->n_tab = static_cast<int>(d.table_idx.size());
  ap->n_len = static_cast<int>(d.len_seq.size());
}

// Make the assembled metadata visible to the next launches: inline (kernel
// arguments) when it fits, else a pinned ring buffer (*st set; release it
// after the last launch that reads it).
int meta_submit(pa_pool* p, const int32_t** ext, Stage** st) {
  *st = nullptr;
  *ext = nullptr;
  const size_t n = p->meta.size();
  if (n <= static_cast<size_t>(pa::kInlineWords)) {
    std::memcpy(p->inline_meta.w, p->meta.data(), n * sizeof(int32_t));
    return PA_OK;
  }
  int rc = acquire_stage(p, n, st);
  if (rc != PA_OK) return rc;
  std::memcpy((*st)->host, p->meta.data(), n * sizeof(int32_t));
  *ext = (*st)->dev;
  return PA_OK;
}

int rows_limit(const pa_pool* p) { return pa::max_rows_for_head_dim(p->head_dim); }

// Partitions per sequence for partition length pt (0 = no split); returns the
// number of partial slots (kv heads x partitions of every split sequence).
// Partition q covers [q pt, (q + 1) pt) except the last, which runs to the
// end of the sequence.  For calls of at most one 16-row tile (merged inside
// the attention launch) the last partition absorbs a remainder of up to
// pt / 4 tokens, so no partition is a handful of tokens whose merge lands at
// the end of the launch (measured on MI355X: 70B-like decode 53.9 -> 53.4 us;
// for verify's 20-row units the longer last partitions cost 4 %).
int parts_of(int n, int pt, int rows) {
  const int slack = rows <= 16 ? pt / 4 : 0;
  return (pt > 0 && n > pt + slack) ? (n - slack + pt - 1) / pt : 1;
}

int64_t count_slots(const pa_pool* p, int n_seq) {
  int64_t slots = 0;
  for (int i = 0; i < n_seq; ++i)
    if (p->parts[i] > 1) slots += static_cast<int64_t>(p->parts[i]) * p->hkv;
  return slots;
}

int64_t count_parts(pa_pool* p, int n_seq, int pt, int rows) {
  p->parts.resize(n_seq);
  for (int i = 0; i < n_seq; ++i) p->parts[i] = parts_of(p->lens[i], pt, rows);
  return count_slots(p, n_seq);
}

// Work decomposition: one unit per (sequence, partition, tile of query rows);
// units of split sequences get consecutive partial slots (kv head major within
// a sequence), shared by the sequence's row tiles.  Units that read a whole
// partition first, then the rest by the tokens they read (causal limit
// included), most first, so the grid's tail holds the short ones.
// A split sequence that belongs to a shared-prefix group has partitions
// [0, q) from the shared-prefix pass ([j pt, min((j + 1) pt, shared))) and its
// own partitions from `shared` on.  With the in-launch merge, each merge unit
// counts the arrivals that the merging launch makes for it: its own units, and
// when the pass runs in the same launch (pre_in_launch), one per pass wave
// whose rows include the sequence's.
void make_plan(pa_pool* p, const int32_t* seq_ids, int n_seq, int pt, int rows, int group, int k_draft,
               bool pre_in_launch) {
  std::vector<pa::WorkUnit>& units = p->units;
  auto& tail = p->tail_units;
  units.clear();
  tail.clear();
  p->merges.clear();
  const int tr = pa::tile_rows_for_call(p->dtype, p->head_dim, rows);
  int64_t slots = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int parts = p->parts[i];
    const int n = p->lens[i];
    const int base = parts == 1 ? -1 : static_cast<int>(slots);
    const int merge = parts == 1 ? -1 : static_cast<int>(p->merges.size());
    const int q0 = p->pre_parts[i];  // partitions done by the shared-prefix pass
    const int own0 = q0 > 0 ? p->pre_shared[i] : 0;  // first position of the sequence's own partitions
    if (parts > 1) slots += static_cast<int64_t>(parts) * p->hkv;
    int own_units = 0;
    for (int row0 = 0; row0 < rows; row0 += tr) {
      const int last_row = std::min(rows, row0 + tr) - 1;
      const int visible = n - k_draft + last_row / group + 1;  // tokens the tile's last row sees
      if (parts == 1) {
        tail.push_back({std::min(n, visible), {i, seq_ids[i], 0, 1, -1, row0, -1, 0}});
        continue;
      }
      for (int q = q0; q < parts; ++q) {
        const int begin = own0 + (q - q0) * pt;
        const int end = q == parts - 1 ? n : begin + pt;  // the last partition runs to the end
        const int len = std::max(0, std::min(end, visible) - begin);
        const pa::WorkUnit u{i, seq_ids[i], q, parts, base, row0, merge, begin};
        ++own_units;
        if (len == pt)
          units.push_back(u);
        else
          tail.push_back({len, u});
      }
    }
    if (parts > 1) p->merges.push_back({i, base, parts, own_units});
  }
  std::sort(tail.begin(), tail.end(), [](const auto& a, const auto& b) {
    if (a.first != b.first) return a.first > b.first;
    if (a.second.q_row != b.second.q_row) return a.second.q_row < b.second.q_row;
    return a.second.part != b.second.part ? a.second.part < b.second.part : a.second.row0 < b.second.row0;
  });
  for (const auto& t : tail) units.push_back(t.second);
  p->plan_slots = slots;
  p->plan_max_parts = 0;
  for (const pa::MergeUnit& m : p->merges) p->plan_max_parts = std::max(p->plan_max_parts, m.nparts);

  // shared-prefix pass: members in batch order per group, one unit per
  // (group, prefix partition, block of rows)
  p->pre_units.clear();
  p->pre_members.clear();
  std::vector<int> merge_of(n_seq, -1);
  for (size_t m = 0; m < p->merges.size(); ++m) merge_of[p->merges[m].q_row] = static_cast<int>(m);
  const auto& pairs = p->pre_scratch;  // (group key, batch index) sorted, prefix sequences only
  const int rpw = pa::prefix_rows_per_unit(p->dtype, p->head_dim);
  p->plan_prefix_tokens = 0;
  p->plan_prefix_rows = 0;
  for (size_t a = 0; a < pairs.size();) {
    size_t b = a;
    while (b < pairs.size() && pairs[b].first == pairs[a].first) ++b;
    const int member0 = static_cast<int>(p->pre_members.size());
    for (size_t k = a; k < b; ++k) {
      const int m = merge_of[pairs[k].second];
      const pa::MergeUnit& mu = p->merges[m];
      p->pre_members.push_back({pairs[k].second, mu.slot_base, mu.nparts, m});
    }
    const int first = pairs[a].second;
    const int q_parts = p->pre_parts[first];
    const int shared = p->pre_shared[first];
    const int group_rows = static_cast<int>(b - a) * rows;
    p->plan_prefix_tokens += shared;
    p->plan_prefix_rows += group_rows;
    for (int q = 0; q < q_parts; ++q)
      for (int r0 = 0; r0 < group_rows; r0 += rpw) {
        p->pre_units.push_back({seq_ids[first], q, r0, member0, group_rows, shared, 0, 0});
        if (pre_in_launch) {
          // each wave of the unit arrives once for every member whose rows it holds
          const int wr = pa::prefix_rows_per_wave(p->head_dim);
          for (int w0 = r0; w0 < std::min(r0 + rpw, group_rows); w0 += wr) {
            const int r_end = std::min(w0 + wr, group_rows);
            for (int j = w0 / rows; j * rows < r_end; ++j) p->merges[merge_of[pairs[a + j].second]].arrivals += 1;
          }
        }
      }
    a = b;
  }
}

// Groups of copy-on-write forks in the batch whose first partitions sit in the
// same physical blocks: at least kPrefixMinGroup sequences sharing at least
// one whole partition that every query row sees (all drafts included).  Sets
// pre_parts[i] (0 for sequences outside any group) and pre_scratch (group key,
// batch index), sorted by group.
constexpr int kPrefixMinGroup = 4;

void find_prefix_groups(pa_pool* p, const int32_t* seq_ids, int n_seq, int pt, int k_draft, int rows) {
  p->pre_parts.assign(n_seq, 0);
  p->pre_shared.assign(n_seq, 0);
  p->pre_groups.clear();
  auto& pairs = p->pre_scratch;
  pairs.clear();
  if (pt <= 0 || p->dtype == PA_F32 || n_seq < kPrefixMinGroup) return;
  for (int i = 0; i < n_seq; ++i) {
    const std::vector<int32_t>& tab = p->bp.table(seq_ids[i]);
    if (p->lens[i] - k_draft >= pt && !tab.empty() && p->bp.refcount(tab[0]) > 1) pairs.push_back({tab[0], i});
  }
  std::sort(pairs.begin(), pairs.end());
  size_t out = 0;
  for (size_t a = 0; a < pairs.size();) {
    size_t b = a;
    while (b < pairs.size() && pairs[b].first == pairs[a].first) ++b;
    if (b - a >= static_cast<size_t>(kPrefixMinGroup)) {
      // tokens every member holds in the same blocks and every query row sees
      int limit = 1 << 30;
      for (size_t k = a; k < b; ++k) limit = std::min(limit, p->lens[pairs[k].second] - k_draft);
      const std::vector<int32_t>& t0 = p->bp.table(seq_ids[pairs[a].second]);
      int blocks = limit / pa::kBlock;
      for (size_t k = a + 1; k < b && blocks > 0; ++k) {
        const std::vector<int32_t>& tk = p->bp.table(seq_ids[pairs[k].second]);
        int j = 0;
        while (j < blocks && tk[j] == t0[j]) ++j;
        blocks = j;
      }
      const int shared = std::min(blocks * pa::kBlock, limit);
      // the pass takes the whole shared prefix, its last partition ending at
      // `shared` (at least one whole partition); each member's own partitions
      // start there, and it keeps at least one (its drafts lie past `shared`)
      if (shared >= pt) {
        const int q_parts = (shared + pt - 1) / pt;
        p->pre_groups.push_back({shared, static_cast<int>(b - a)});
        for (size_t k = a; k < b; ++k) {
          const int i = pairs[k].second;
          p->pre_parts[i] = q_parts;
          p->pre_shared[i] = shared;
          p->parts[i] = q_parts + parts_of(p->lens[i] - shared, pt, rows);
          pairs[out++] = pairs[k];
        }
      }
    }
    a = b;
  }
  pairs.resize(out);
}

// Partition length for a call with shared-prefix groups, when the library
// chooses it.  The pass runs one workgroup per (prefix partition, row block,
// kv head); when those exceed what the device holds at once, the last,
// partial generation costs as long as a full one.  Longer partitions (up to
// twice pt0) are then tried, and the one with the shortest critical path
// (generations x tokens per wave) is taken, the shortest on ties.  (Measured
// on MI355X, 64 forks of a 4,096-token prefix with 5 drafts: 512-token
// partitions give 2,560 waves for 2,048 slots and a 105 us step; 608 gives
// 1,920 waves and 88 us.)  When the pass shares the attention launch, that
// launch's own waves (one per sequence and kv head at least) count too:
// measured for the same workload in one launch, 512 -> 111, 768 -> 87,
// 896 -> 82, 1,024 -> 83, 1,344 -> 91 us.
int prefix_partition(const pa_pool* p, int pt0, int rows, int64_t other_waves) {
  if (p->pre_groups.empty()) return pt0;
  const int64_t rpw = pa::prefix_rows_per_unit(p->dtype, p->head_dim);
  const int64_t resident = static_cast<int64_t>(p->num_cus) * pa::prefix_units_per_cu(p->dtype, p->head_dim);
  auto waves = [&](int pt) {  // workgroups of the pass (groups with a whole partition), and the launch's others
    int64_t w = other_waves;
    for (const PrefixGroup& g : p->pre_groups)
      if (g.shared >= pt)
        w += static_cast<int64_t>((g.shared + pt - 1) / pt) *
             ((static_cast<int64_t>(g.members) * rows + rpw - 1) / rpw) * p->hkv;
    return w;
  };
  const int64_t w0 = waves(pt0);
  if (w0 <= resident) return pt0;
  // the shortest partition whose waves fit one generation, else the one with
  // the fewest generations x tokens per wave
  int best = pt0;
  int64_t best_cost = (w0 + resident - 1) / resident * pt0;
  for (int pt = pt0 + 32; pt <= 2 * pt0; pt += 32) {
    const int64_t w = waves(pt);
    if (w == other_waves) break;  // no whole partition left in any prefix
    if (w <= resident) return pt;
    const int64_t cost = (w + resident - 1) / resident * pt;
    if (cost < best_cost) {
      best = pt;
      best_cost = cost;
    }
  }
  return best;
}

// Counters for the in-launch merge: at least n, zeroed when (re)allocated.
int ensure_merge_ctr(pa_pool* p, size_t n) {
  if (n <= p->merge_ctr_cap) return PA_OK;
  const size_t cap = std::max(n, 2 * p->merge_ctr_cap);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_err(e, "hipDeviceSynchronize");
  if (p->merge_ctr) (void)hipFree(p->merge_ctr);
  p->merge_ctr = nullptr;
  p->merge_ctr_cap = 0;
  e = hipMalloc(&p->merge_ctr, cap * sizeof(unsigned));
  if (e != hipSuccess) return hip_err(e, "hipMalloc(merge counters)");
  e = hipMemset(p->merge_ctr, 0, cap * sizeof(unsigned));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_err(e, "hipMemset(merge counters)");
  p->merge_ctr_cap = cap;
  return PA_OK;
}

size_t plan_ws_bytes(const pa_pool* p, int64_t slots, int rows) {
  return static_cast<size_t>(slots) * rows * (p->head_dim + 2) * sizeof(float);
}

// Launch an update-only append kernel for the pending table / length changes.
int flush_dirty(pa_pool* p, hipStream_t stream) {
  if (!p->bp.has_dirty()) return PA_OK;
  p->bp.take_dirty(&p->dirty);
  if (p->host_only) return PA_OK;
  p->meta.clear();
  pa::AppendParams ap = base_append(p);
  meta_dirty(p, &ap);
  Stage* st = nullptr;
  int rc = meta_submit(p, &ap.ext, &st);
  if (rc != PA_OK) return rc;
  hipError_t e = pa::launch_append(ap, &p->inline_meta, stream);
  if (e != hipSuccess) return hip_err(e, "append kernel (table update)");
  return st ? release_stage(st, stream) : PA_OK;
}

// Whether a copy-on-write copy of this call reads a block that the same call
// also writes rows into.  That happens when a longer sharer copies a shared
// tail block and drops its reference, and a shorter sharer served later in the
// call then holds the block alone and writes into it directly: the copy must
// see the slots as they were before the call (the host model serves the
// sequences one after the other), but the workgroups of one launch run in no
// particular order.
bool copy_source_written(pa_pool* p) {
  if (p->cows.empty()) return false;
  std::vector<int32_t>& src = p->cow_src;
  src.clear();
  for (const pa::CowCopy& c : p->cows) src.push_back(c.src);
  std::sort(src.begin(), src.end());
  for (int32_t s : p->slots)
    if (std::binary_search(src.begin(), src.end(), s / pa::kBlock)) return true;
  return false;
}

// flush_dirty with every launch's metadata in its kernel arguments (no
// staging buffer): as many update-only launches as the pending updates need.
int flush_dirty_inline(pa_pool* p, hipStream_t stream) {
  if (!p->bp.has_dirty()) return PA_OK;
  p->bp.take_dirty(&p->dirty);
  const pa::BlockPool::Dirty& d = p->dirty;
  constexpr size_t kPer = (pa::kInlineWords - 16) / 2;  // (index, value) pairs per launch
  size_t it = 0, il = 0;
  while (it < d.table_idx.size() || il < d.len_seq.size()) {
    const size_t nt = std::min(kPer, d.table_idx.size() - it);
    const size_t nl = std::min(kPer - nt, d.len_seq.size() - il);
    std::vector<int32_t>& w = p->meta;
    w.clear();
    pa::AppendParams ap = base_append(p);
    ap.tab = 0;
    for (size_t i = it; i < it + nt; ++i) {
      w.push_back(d.table_idx[i]);
      w.push_back(d.table_val[i]);
    }
    ap.lens = static_cast<int>(pad8(w));
    for (size_t i = il; i < il + nl; ++i) {
      w.push_back(d.len_seq[i]);
      w.push_back(d.len_val[i]);
    }
    ap.n_tab = static_cast<int>(nt);
    ap.n_len = static_cast<int>(nl);
    std::memcpy(p->inline_meta.w, w.data(), w.size() * sizeof(int32_t));
    hipError_t e = pa::launch_append(ap, &p->inline_meta, stream);
    if (e != hipSuccess) return hip_err(e, "append kernel (table update)");
    it += nt;
    il += nl;
  }
  return PA_OK;
}

// Host bookkeeping for an append is done and its dirty set taken; enqueue its
// kernel (table / length updates, copies, row scatter).  When a copy's source
// block is also written by this call, the copies run in a launch of their own
// before the scatter (stream order makes the copies land first).
int launch_append_call(pa_pool* p, const void* k_new, const void* v_new, hipStream_t stream) {
  p->meta.clear();
  pa::AppendParams ap = base_append(p);
  meta_dirty(p, &ap);
  ap.cows = static_cast<int>(pad8(p->meta));
  for (const pa::CowCopy& c : p->cows) {
    p->meta.push_back(c.src);
    p->meta.push_back(c.dst);
    p->meta.push_back(c.rows);
  }
  ap.slots = static_cast<int>(pad8(p->meta));
  p->meta.insert(p->meta.end(), p->slots.begin(), p->slots.end());
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.n_cow = static_cast<int>(p->cows.size());
  ap.n_rows = static_cast<int>(p->slots.size());
  const bool copies_first = copy_source_written(p);
  Stage* st = nullptr;
  int rc = meta_submit(p, &ap.ext, &st);
  if (rc != PA_OK) return rc;
  ProfEvent ev{};
  prof_begin(p, 2, stream, &ev);
  if (copies_first) {
    // table / length updates and the copies, then the rows alone
    pa::AppendParams first = ap, rows = ap;
    first.n_rows = 0;
    rows.n_tab = rows.n_len = rows.n_cow = 0;
    hipError_t e = pa::launch_append(first, &p->inline_meta, stream);
    if (e != hipSuccess) return hip_err(e, "append kernel (copy-on-write copies)");
    e = pa::launch_append(rows, &p->inline_meta, stream);
    if (e != hipSuccess) return hip_err(e, "append kernel");
  } else {
    hipError_t e = pa::launch_append(ap, &p->inline_meta, stream);
    if (e != hipSuccess) return hip_err(e, "append kernel");
  }
  prof_end(p, stream, &ev);
  return st ? release_stage(st, stream) : PA_OK;
}

struct AppendSpec {
  int t_new;
  const void* k_new;
  const void* v_new;
};

// Attention over the current lengths; with `app`, first append app->t_new rows
// to every sequence, in the same launch when possible.
// With `noalloc` (no append): the plan, the merge counters and the partials go
// to the device's fixed scratch, all metadata travels in kernel arguments, and
// nothing is allocated; sizes past the scratch are rejected.
int attend(pa_pool* p, const int32_t* seq_ids, int n_seq, int k_draft, int num_q_heads, float scale,
           const void* q, void* out, float* lse, int partition_tokens, void* workspace, size_t ws_bytes,
           void* stream_v, const AppendSpec* app, bool noalloc = false) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (p->host_only) return set_err(PA_ERR_STATE, "host-only pool has no device memory");
  if (noalloc) {
    if (app || !p->scratch) return set_err(PA_ERR_STATE, "no device scratch for this pool");
    workspace = p->scratch + pa::kScratchPartialOffset;
    ws_bytes = pa::kScratchPartialBytes;
  }
  if (n_seq < 0) return set_err(PA_ERR_INVALID, "n_seq < 0");
  if (k_draft < 1) return set_err(PA_ERR_INVALID, "k_draft must be >= 1");
  if (num_q_heads <= 0 || num_q_heads % p->hkv != 0)
    return set_err(PA_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  if (!(scale > 0.f) || !std::isfinite(scale)) return set_err(PA_ERR_INVALID, "scale must be finite and > 0");
  const int group = num_q_heads / p->hkv;
  const int64_t rows64 = static_cast<int64_t>(group) * k_draft;
  if (rows64 > kMaxRows)
    return set_err(PA_ERR_INVALID, "(num_q_heads / num_kv_heads) * k_draft exceeds 2^22 query rows");
  const int rows = static_cast<int>(rows64);
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % 32 != 0))
    return set_err(PA_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of 32");
  if (n_seq > 0 && (!seq_ids || !q || !out)) return set_err(PA_ERR_INVALID, "seq_ids, q or out is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return set_err(PA_ERR_INVALID, "q, out and workspace must be 16-byte aligned");
  const int t_new = app ? app->t_new : 0;
  if (app && (t_new < 1 || (n_seq > 0 && (!app->k_new || !app->v_new))))
    return set_err(PA_ERR_INVALID, "n_new must be >= 1 and k_new / v_new given");
  if (app && (!aligned16(app->k_new) || !aligned16(app->v_new)))
    return set_err(PA_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  p->lens.resize(n_seq);
  for (int i = 0; i < n_seq; ++i) {
    const int s = seq_ids[i];
    if (!p->bp.live(s)) return set_err(PA_ERR_INVALID, "attention over a sequence that is not live");
    p->lens[i] = p->bp.length(s) + t_new;  // length when the attention runs
    if (p->lens[i] < std::max(1, k_draft))
      return set_err(PA_ERR_INVALID, "sequence shorter than max(1, k_draft)");
  }
  int pt = partition_tokens;
  int64_t slots;
  if (pt == 0) {
    pt = default_partition(rows);
    slots = count_parts(p, n_seq, pt, rows);
    if (slots && (!workspace || plan_ws_bytes(p, slots, rows) > ws_bytes)) {
      pt = 0;  // the workspace cannot hold the split: run unsplit
      slots = count_parts(p, n_seq, 0, rows);
    }
  } else {
    slots = count_parts(p, n_seq, pt, rows);
    if (slots && (!workspace || plan_ws_bytes(p, slots, rows) > ws_bytes))
      return set_err(PA_ERR_INVALID, noalloc ? "split partials for this partition size exceed the fixed scratch"
                                             : "workspace too small for this partition size (see pa_workspace_size)");
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  // The append: host bookkeeping first (all-or-nothing; the last check that can fail).
  bool fused = false;
  if (app) {
    p->ntok.assign(n_seq, t_new);
    const bool table_pending = p->bp.dirty_entries() > 0;
    p->slots.clear();
    p->cows.clear();
    std::string err;
    int rc = p->bp.append(seq_ids, n_seq, p->ntok.data(), &p->slots, &p->cows, &err);
    if (rc != pa::kOk) return set_err(rc, err);
    // One launch can append and attend when no copy-on-write copy has to land
    // first and no earlier table change is still on its way to the device: the
    // attention reads the table while the launch's append work writes it, which
    // is safe only for the blocks this append opens (their only valid rows are
    // the new ones, which the attention takes from k_new / v_new).
    // (a call with several row tiles appends first: each tile would splice
    // the new rows again)
    fused = p->cows.empty() && !table_pending && p->dtype != PA_F32 && rows <= rows_limit(p);
    if (!fused) {
      p->bp.take_dirty(&p->dirty);
      rc = launch_append_call(p, app->k_new, app->v_new, stream);
      if (rc != PA_OK) return rc;
    }
  }
  if (!fused) {
    int rc = noalloc ? flush_dirty_inline(p, stream) : flush_dirty(p, stream);
    if (rc != PA_OK) return rc;
  }

  // forks sharing a prefix: its partitions are computed once for all of them
  find_prefix_groups(p, seq_ids, n_seq, pt, k_draft, rows);
  if (partition_tokens == 0 && pt > 0) {
    // the launch's other waves, when the pass runs inside the attention launch
    // (workgroups of that launch run prefix_launch_waves() attention units each)
    const int64_t lw = pa::prefix_launch_waves();
    const int64_t others = (pa::prefix_in_attention_launch(p->dtype, p->head_dim, rows) && rows <= rows_limit(p))
                               ? (static_cast<int64_t>(n_seq) * p->hkv + lw - 1) / lw
                               : 0;
    const int best = prefix_partition(p, pt, rows, others);
    if (best != pt) {
      pt = best;
      count_parts(p, n_seq, pt, rows);
      find_prefix_groups(p, seq_ids, n_seq, pt, k_draft, rows);
    }
  }
  slots = count_slots(p, n_seq);
  if (slots && plan_ws_bytes(p, slots, rows) > ws_bytes) {
    // a member's own partitions start at the end of the shared prefix, which
    // can take one partition more than the plain split checked above: without
    // the room for it, no shared-prefix pass (the plain split fits: a longer
    // library-chosen partition needs no more than the default)
    p->pre_parts.assign(n_seq, 0);
    p->pre_shared.assign(n_seq, 0);
    p->pre_scratch.clear();
    p->pre_groups.clear();
    slots = count_parts(p, n_seq, pt, rows);
  }
  // Merges inside the attention launch (the last wave to finish a split
  // (sequence, kv head)'s partials merges them) when one unit takes all query
  // rows of a (sequence, kv head) and no sequence has too many partitions.
  // With shared-prefix units the pass runs in the attention launch instead,
  // and a launch of its own merges: the merges of the pass's last waves would
  // run one after the other in the launch's tail (measured on MI355X, 64-fork
  // verify: 76.6 -> 68 us).
  int max_parts = 0;
  for (int i = 0; i < n_seq; ++i) max_parts = std::max(max_parts, p->parts[i]);
  const bool merge_ok = p->dtype != PA_F32 && rows <= rows_limit(p) && max_parts <= pa::kInlineMergeParts &&
                        ws_bytes < (size_t{1} << 31);
  const bool pre_in_launch = merge_ok && !p->pre_groups.empty() && pa::prefix_in_attention_launch(p->dtype, p->head_dim, rows);
  const bool inline_merge = merge_ok && !pre_in_launch;

  // reuse the device plan when the batch, its partition structure and the
  // shared-prefix grouping are unchanged
  std::vector<int32_t>& key = p->key_scratch;
  key.assign({pt, n_seq, rows, inline_merge ? 1 : 0, pre_in_launch ? 1 : 0});
  for (int i = 0; i < n_seq; ++i) {
    key.push_back(seq_ids[i]);
    key.push_back(p->parts[i]);
    key.push_back(p->pre_parts[i]);
    key.push_back(p->pre_shared[i]);
  }
  if (key != p->plan_key) {
    make_plan(p, seq_ids, n_seq, pt, rows, group, k_draft, pre_in_launch);
    p->plan_key.swap(key);
    p->plan_units = static_cast<int>(p->units.size());
    p->plan_merges = static_cast<int>(p->merges.size());
    p->plan_pre_units = static_cast<int>(p->pre_units.size());
    p->dplan_stale = true;
  }
  const size_t w_units = 8 * p->units.size(), w_merges = 4 * p->merges.size();
  const size_t w_pre = 8 * p->pre_units.size(), w_mem = 4 * p->pre_members.size();
  const size_t plan_words = w_units + w_merges + w_pre + w_mem;
  auto plan_image = [&](int32_t* h) {
    std::memcpy(h, p->units.data(), w_units * sizeof(int32_t));
    std::memcpy(h + w_units, p->merges.data(), w_merges * sizeof(int32_t));
    std::memcpy(h + w_units + w_merges, p->pre_units.data(), w_pre * sizeof(int32_t));
    std::memcpy(h + w_units + w_merges + w_pre, p->pre_members.data(), w_mem * sizeof(int32_t));
  };
  const int32_t* dplan = nullptr;
  unsigned* merge_ctr = nullptr;
  if (noalloc) {
    // the scratch is shared by every pool on the device: the plan goes in on
    // every call, through kernel arguments, with the counters it uses zeroed
    const size_t n_ctr = p->merges.size() * static_cast<size_t>(p->hkv);
    if (plan_words * sizeof(int32_t) > pa::kScratchPlanBytes)
      return set_err(PA_ERR_INVALID, "work plan exceeds the fixed scratch (too many sequences or partitions)");
    if (n_ctr * sizeof(unsigned) > pa::kScratchCounterBytes)
      return set_err(PA_ERR_INVALID, "merge counters exceed the fixed scratch (too many split sequences)");
    int32_t* dst = reinterpret_cast<int32_t*>(p->scratch + pa::kScratchPlanOffset);
    unsigned* ctr = reinterpret_cast<unsigned*>(p->scratch);
    p->meta.resize(plan_words);
    plan_image(p->meta.data());
    size_t done = 0;
    do {
      const size_t n = std::min(plan_words - done, static_cast<size_t>(pa::kInlineWords));
      std::memcpy(p->inline_meta.w, p->meta.data() + done, n * sizeof(int32_t));
      hipError_t e = pa::launch_words(dst + done, p->inline_meta, static_cast<int>(n), ctr,
                                      done == 0 ? static_cast<int>(n_ctr) : 0, stream);
      if (e != hipSuccess) return hip_err(e, "scratch plan");
      done += n;
    } while (done < plan_words);
    dplan = dst;
    merge_ctr = ctr;
  } else {
    if (p->dplan_stale) {
      int rc = ensure_dplan(p, plan_words * sizeof(int32_t));
      if (rc != PA_OK) return rc;
      if (plan_words) {
        Stage* pst = nullptr;
        rc = acquire_stage(p, plan_words, &pst);
        if (rc != PA_OK) return rc;
        plan_image(pst->host);
        hipError_t e =
            hipMemcpyAsync(p->dplan, pst->host, plan_words * sizeof(int32_t), hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync(plan)");
        rc = release_stage(pst, stream);
        if (rc != PA_OK) return rc;
      }
      rc = ensure_merge_ctr(p, p->merges.size() * static_cast<size_t>(p->hkv));
      if (rc != PA_OK) return rc;
      p->dplan_stale = false;
    }
    dplan = static_cast<const int32_t*>(p->dplan);
    merge_ctr = p->merge_ctr;
  }

  pa::AttnParams ak{};
  ak.k_pool = p->k_pool;
  ak.v_pool = p->v_pool;
  ak.block_table = p->block_table;
  ak.seq_len = p->seq_len;
  ak.max_blocks = p->bp.max_blocks_per_seq();
  ak.num_blocks = p->num_blocks;
  ak.part_tokens = pt;
  ak.q = q;
  ak.out = out;
  ak.lse = lse;
  float* ws = static_cast<float*>(workspace);
  ak.ws_acc = ws;
  ak.ws_ml = ws ? ws + static_cast<size_t>(slots) * rows * p->head_dim : nullptr;
  ak.units = reinterpret_cast<const pa::WorkUnit*>(dplan);
  ak.merges = reinterpret_cast<const pa::MergeUnit*>(dplan + 8 * p->plan_units);
  ak.pre_units = reinterpret_cast<const pa::PrefixUnit*>(dplan + 8 * p->plan_units + 4 * p->plan_merges);
  ak.pre_members = reinterpret_cast<const pa::PrefixMember*>(dplan + 8 * p->plan_units + 4 * p->plan_merges +
                                                             8 * p->plan_pre_units);
  ak.n_pre_units = p->plan_pre_units;
  ak.n_units = p->plan_units;
  ak.n_merges = p->plan_merges;
  ak.hkv = p->hkv;
  ak.hq = num_q_heads;
  ak.group = group;
  ak.k_draft = k_draft;
  ak.rows = rows;
  ak.tile_rows = pa::tile_rows_for_call(p->dtype, p->head_dim, rows);
  ak.head_dim = p->head_dim;
  ak.scale_log2 = scale * 1.4426950408889634f;
  // Pages stream past the caches (non-temporal loads) only when one unit
  // reads each of them: no shared blocks, no shared-prefix units, and one
  // row tile per (sequence, partition).  The row tiles of a long chunk read
  // the same pages one after the other and find them in L2.
  ak.stream_kv = (p->bp.num_shared() == 0 && !pre_in_launch && ak.tile_rows >= rows) ? 1 : 0;
  ak.app = base_append(p);
  // Short splits (few partitions, one row tile) are merged inside the
  // attention launch by the last partition to finish; others by merge_kernel.
  ak.merge_ctr = merge_ctr;
  ak.kv_scale = p->kv_scale;
  ak.inline_merge = inline_merge ? 1 : 0;
  ak.pre_in_launch = pre_in_launch ? 1 : 0;
  Stage* st = nullptr;
  if (fused) {
    // metadata: this append's table / length updates, the new rows' slots, and
    // the length of every query row after the append
    p->bp.take_dirty(&p->dirty);
    p->meta.clear();
    meta_dirty(p, &ak.app);
    ak.app.slots = static_cast<int>(pad8(p->meta));
    p->meta.insert(p->meta.end(), p->slots.begin(), p->slots.end());
    ak.lens_by_row = static_cast<int>(pad8(p->meta));
    p->meta.insert(p->meta.end(), p->lens.begin(), p->lens.end());
    ak.app.k_new = app->k_new;
    ak.app.v_new = app->v_new;
    ak.app.n_rows = static_cast<int>(p->slots.size());
    ak.t_new = t_new;
    ak.app_blocks = pre_in_launch ? pa::append_blocks_prefix_launch(ak.app) : pa::append_blocks64(ak.app);
    int rc = meta_submit(p, &ak.app.ext, &st);
    if (rc != PA_OK) return rc;
  }
  const pa::DType dt = static_cast<pa::DType>(p->dtype);
  if (ak.n_pre_units > 0 && !pre_in_launch) {
    ProfEvent ev{};
    if (!noalloc) prof_begin(p, 3, stream, &ev);
    hipError_t e = pa::launch_prefix(dt, ak, stream);
    if (e != hipSuccess) return hip_err(e, "shared-prefix kernel");
    if (!noalloc) prof_end(p, stream, &ev);
  }
  if (ak.n_units > 0 || fused || (pre_in_launch && ak.n_pre_units > 0)) {
    ProfEvent ev{};
    if (!noalloc) prof_begin(p, 0, stream, &ev);
    hipError_t e = pa::launch_attention(dt, ak, &p->inline_meta, stream);
    if (e != hipSuccess) return hip_err(e, "attention kernel");
    if (!noalloc) prof_end(p, stream, &ev);
  }
  if (ak.n_merges > 0 && !ak.inline_merge) {
    ProfEvent ev{};
    if (!noalloc) prof_begin(p, 1, stream, &ev);
    hipError_t e = pre_in_launch ? pa::launch_merge_rows(dt, ak, stream) : pa::launch_merge(dt, ak, stream);
    if (e != hipSuccess) return hip_err(e, "merge kernel");
    if (!noalloc) prof_end(p, stream, &ev);
  }
  p->last_pt = slots > 0 ? pt : 0;
  p->last_prefix_units = ak.n_pre_units * p->hkv;
  pa_call_stats& cs = p->last_stats;
  cs.partition_tokens = p->last_pt;
  cs.prefix_workgroups = p->last_prefix_units;
  cs.attention_workgroups = ak.n_units * p->hkv;
  cs.append_workgroups = fused ? ak.app_blocks : 0;
  cs.merge_workgroups = (ak.n_merges > 0 && !ak.inline_merge)
                            ? (pre_in_launch ? pa::merge_rows_workgroups(ak) : ak.n_merges * p->hkv * rows)
                            : 0;
  cs.prefix_kv_tokens = ak.n_pre_units > 0 ? p->plan_prefix_tokens : 0;
  cs.prefix_query_rows = ak.n_pre_units > 0 ? p->plan_prefix_rows : 0;
  cs.partial_rows = p->plan_slots * rows;
  return st ? release_stage(st, stream) : PA_OK;
}

// The classes graph steps are padded to: units rounded up to a power of two,
// at least 16.
int graph_class_units(int units) {
  int c = 16;
  while (c < units) c *= 2;
  return c;
}

int ensure_graph_class(pa_pool* p, int units, int n_new, GraphClass** out) {
  GraphClass& g = p->gclass[{units, n_new}];
  if (!g.buf) {
    g.units = units;
    g.n_new = n_new;
    const size_t c = static_cast<size_t>(units);
    // table entries a sequence's append can open: one per 16 rows, plus one
    g.tab_cap = c * (static_cast<size_t>(n_new) / pa::kBlock + 2);
    // header, lengths by row, slots, table updates, length updates
    g.step_words = pa::kGraphHeader + c + c * n_new + 2 * g.tab_cap + 2 * c;
    g.off_units = (g.step_words + 7) / 8 * 8;
    g.off_merges = g.off_units + 8 * c;
    g.words = g.off_merges + 4 * c;
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&g.buf), g.words * sizeof(int32_t));
    if (e == hipSuccess) e = hipMalloc(&g.ctr, c * p->hkv * sizeof(unsigned));
    if (e == hipSuccess) e = hipMemset(g.ctr, 0, c * p->hkv * sizeof(unsigned));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      if (g.buf) (void)hipFree(g.buf);
      if (g.ctr) (void)hipFree(g.ctr);
      p->gclass.erase({units, n_new});
      return hip_err(e, "graph step buffers");
    }
  }
  *out = &g;
  return PA_OK;
}

// Host side of a graph step (pa_graph_prepare): the append's bookkeeping and
// any work that cannot be replayed (pending table changes, copy-on-write
// copies) run eagerly on the stream; the step's metadata and plan go into its
// class's buffer by one copy on the stream; the launch parameters, which only
// point at that buffer, are kept for pa_graph_launch.
int graph_prepare(pa_pool* p, const int32_t* seq_ids, int n_seq, int n_new, const void* k_new, const void* v_new,
                  int num_q_heads, float scale, const void* q, void* out, float* lse, int partition_tokens,
                  void* workspace, size_t ws_bytes, void* stream_v, int* class_units) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (p->host_only) return set_err(PA_ERR_STATE, "host-only pool has no device memory");
  if (p->dtype == PA_F32) return set_err(PA_ERR_STATE, "graph steps take 16-bit or E4M3 pools");
  if (n_seq < 1 || n_new < 1) return set_err(PA_ERR_INVALID, "n_seq and n_new must be >= 1");
  if (!seq_ids || !q || !out || !k_new || !v_new) return set_err(PA_ERR_INVALID, "NULL argument");
  if (num_q_heads <= 0 || num_q_heads % p->hkv != 0)
    return set_err(PA_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  if (!(scale > 0.f) || !std::isfinite(scale)) return set_err(PA_ERR_INVALID, "scale must be finite and > 0");
  const int group = num_q_heads / p->hkv;
  const int64_t rows64 = static_cast<int64_t>(group) * n_new;
  if (rows64 > rows_limit(p))
    return set_err(PA_ERR_STATE, "graph steps take calls whose query rows per kv head fit one unit");
  const int rows = static_cast<int>(rows64);
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % 32 != 0))
    return set_err(PA_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of 32");
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace) || !aligned16(k_new) || !aligned16(v_new))
    return set_err(PA_ERR_INVALID, "q, out, workspace, k_new and v_new must be 16-byte aligned");
  if (ws_bytes >= (size_t{1} << 31)) return set_err(PA_ERR_INVALID, "workspace of 2 GiB or more");
  p->lens.resize(n_seq);
  for (int i = 0; i < n_seq; ++i) {
    if (!p->bp.live(seq_ids[i])) return set_err(PA_ERR_INVALID, "attention over a sequence that is not live");
    p->lens[i] = p->bp.length(seq_ids[i]) + n_new;
  }
  // the same partition length every step: the library's default (or the
  // caller's), and the workspace must hold its partials
  const int pt = partition_tokens ? partition_tokens : default_partition(rows);
  const int64_t slots = count_parts(p, n_seq, pt, rows);
  if (slots && (!workspace || plan_ws_bytes(p, slots, rows) > ws_bytes))
    return set_err(PA_ERR_INVALID, "graph steps need a workspace that holds this step's split partials");
  int max_parts = 0;
  for (int i = 0; i < n_seq; ++i) max_parts = std::max(max_parts, p->parts[i]);
  if (max_parts > pa::kInlineMergeParts)
    return set_err(PA_ERR_STATE, "graph steps merge inside the launch: a sequence has too many partitions");
  p->pre_parts.assign(n_seq, 0);  // no shared-prefix pass in graph steps
  p->pre_shared.assign(n_seq, 0);
  p->pre_scratch.clear();
  p->pre_groups.clear();
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  // Earlier table changes reach the device first, eagerly (the attention
  // reads the table while the step's append work writes it).  Earlier length
  // changes (truncations) ride in the step's metadata, as in a fused eager
  // call, when its class has room for them beside the step's own.
  int64_t units_est = 0;
  for (int i = 0; i < n_seq; ++i) units_est += p->parts[i];
  const int cls = graph_class_units(static_cast<int>(std::min<int64_t>(units_est, int64_t{1} << 29)));
  // the class's buffers first: nothing after the append's bookkeeping may fail
  // but a launch
  GraphClass* g = nullptr;
  int rc = ensure_graph_class(p, cls, n_new, &g);
  if (rc != PA_OK) return rc;
  if (p->bp.dirty_entries() > 0 || p->bp.dirty_lens() + static_cast<size_t>(n_seq) > static_cast<size_t>(cls)) {
    rc = flush_dirty(p, stream);
    if (rc != PA_OK) return rc;
  }
  p->ntok.assign(n_seq, n_new);
  p->slots.clear();
  p->cows.clear();
  std::string err;
  rc = p->bp.append(seq_ids, n_seq, p->ntok.data(), &p->slots, &p->cows, &err);
  if (rc != pa::kOk) return set_err(rc, err);
  // an append with copies runs eagerly, whole; the replay's append part then
  // has nothing to do (its attention still takes the new rows from k_new / v_new)
  const bool eager_append = !p->cows.empty();
  p->bp.take_dirty(&p->dirty);
  if (eager_append) {
    rc = launch_append_call(p, k_new, v_new, stream);
    if (rc != PA_OK) return rc;
  }
  make_plan(p, seq_ids, n_seq, pt, rows, group, n_new, false);
  p->plan_key.clear();  // the pool's own plan cache no longer matches its host plan
  const int units = static_cast<int>(p->units.size());
  const pa::BlockPool::Dirty& d = p->dirty;
  const size_t n_tab = eager_append ? 0 : d.table_idx.size();
  const size_t n_len = eager_append ? 0 : d.len_seq.size();
  const size_t n_rows = eager_append ? 0 : p->slots.size();
  // (the append opens at most n_new / 16 + 1 blocks per sequence, the class
  // holds n_new / 16 + 2; the lengths were bounded above)
  if (n_tab > g->tab_cap || n_len > static_cast<size_t>(g->units) || units != units_est ||
      pa::kGraphHeader + n_seq + n_rows + 2 * (n_tab + n_len) > g->step_words)
    return set_err(PA_ERR_STATE, "graph step: internal capacity check failed");

  // The step's own words, written by small kernels on the stream (their
  // arguments carry them: no copy engine, no host memory read by the GPU).
  std::vector<int32_t>& w = p->meta;
  const size_t at_slots = pa::kGraphHeader + static_cast<size_t>(n_seq);
  const size_t at_tab = at_slots + n_rows, at_len = at_tab + 2 * n_tab, n_words = at_len + 2 * n_len;
  w.assign(n_words, 0);
  w[pa::kGraphUnits] = units;
  w[pa::kGraphTab] = static_cast<int32_t>(n_tab);
  w[pa::kGraphLen] = static_cast<int32_t>(n_len);
  w[pa::kGraphRows] = static_cast<int32_t>(n_rows);
  w[pa::kGraphSlotsAt] = static_cast<int32_t>(at_slots);
  w[pa::kGraphTabAt] = static_cast<int32_t>(at_tab);
  w[pa::kGraphLenAt] = static_cast<int32_t>(at_len);
  for (int i = 0; i < n_seq; ++i) w[pa::kGraphHeader + i] = p->lens[i];
  for (size_t r = 0; r < n_rows; ++r) w[at_slots + r] = p->slots[r];
  for (size_t i = 0; i < n_tab; ++i) {
    w[at_tab + 2 * i] = d.table_idx[i];
    w[at_tab + 2 * i + 1] = d.table_val[i];
  }
  for (size_t i = 0; i < n_len; ++i) {
    w[at_len + 2 * i] = d.len_seq[i];
    w[at_len + 2 * i + 1] = d.len_val[i];
  }
  auto put = [&](size_t dst, const int32_t* src, size_t n) -> int {
    for (size_t done = 0; done < n; done += pa::kInlineWords) {
      const size_t k = std::min<size_t>(pa::kInlineWords, n - done);
      std::memcpy(p->inline_meta.w, src + done, k * sizeof(int32_t));
      hipError_t e = pa::launch_words(g->buf + dst + done, p->inline_meta, static_cast<int>(k), nullptr, 0, stream);
      if (e != hipSuccess) return hip_err(e, "graph step words");
    }
    return PA_OK;
  };
  rc = put(0, w.data(), n_words);
  if (rc != PA_OK) return rc;
  // the plan, when it differs from the one the buffer holds (it stays the same
  // while no sequence of the batch crosses a partition boundary)
  const size_t unit_words = 8 * p->units.size(), merge_words = 4 * p->merges.size();
  const int32_t* uw = reinterpret_cast<const int32_t*>(p->units.data());
  const int32_t* mw = reinterpret_cast<const int32_t*>(p->merges.data());
  if (g->plan.size() != unit_words + merge_words || !std::equal(uw, uw + unit_words, g->plan.data()) ||
      !std::equal(mw, mw + merge_words, g->plan.data() + unit_words)) {
    g->plan.assign(uw, uw + unit_words);
    g->plan.insert(g->plan.end(), mw, mw + merge_words);
    rc = put(g->off_units, uw, unit_words);
    if (rc == PA_OK) rc = put(g->off_merges, mw, merge_words);
    if (rc != PA_OK) {
      g->plan.clear();
      return rc;
    }
  }

  // launch parameters: the padded grid, pointers into the class's buffer
  const int32_t* buf = g->buf;
  pa::AttnParams& ak = g->params;
  ak = pa::AttnParams{};
  ak.k_pool = p->k_pool;
  ak.v_pool = p->v_pool;
  ak.block_table = p->block_table;
  ak.seq_len = p->seq_len;
  ak.max_blocks = p->bp.max_blocks_per_seq();
  ak.num_blocks = p->num_blocks;
  ak.part_tokens = pt;
  ak.q = q;
  ak.out = out;
  ak.lse = lse;
  float* ws = static_cast<float*>(workspace);
  ak.ws_acc = ws;
  // the (m, l) pairs after every partial row the workspace can hold
  const int64_t ws_slots = ws ? static_cast<int64_t>(ws_bytes / (sizeof(float) * (p->head_dim + 2) * rows)) : 0;
  ak.ws_ml = ws ? ws + static_cast<size_t>(ws_slots) * rows * p->head_dim : nullptr;
  ak.units = reinterpret_cast<const pa::WorkUnit*>(buf + g->off_units);
  ak.merges = reinterpret_cast<const pa::MergeUnit*>(buf + g->off_merges);
  ak.n_units = g->units;
  ak.hkv = p->hkv;
  ak.hq = num_q_heads;
  ak.group = group;
  ak.k_draft = n_new;
  ak.rows = rows;
  ak.tile_rows = pa::tile_rows_for_call(p->dtype, p->head_dim, rows);
  ak.head_dim = p->head_dim;
  ak.scale_log2 = scale * 1.4426950408889634f;
  ak.stream_kv = 1;  // (a hint only: shared blocks are read correctly either way)
  ak.t_new = n_new;
  ak.lens_by_row = pa::kGraphHeader;
  ak.merge_ctr = g->ctr;
  ak.inline_merge = 1;
  ak.kv_scale = p->kv_scale;
  ak.graph_units = g->units;
  ak.app = base_append(p);
  ak.app.ext = buf;  // (the offsets of the append's words come from the step's header)
  ak.app.k_new = k_new;
  ak.app.v_new = v_new;
  // the grid's append part: what the class's largest append needs
  {
    pa::AppendParams cap = ak.app;
    cap.n_tab = static_cast<int>(g->tab_cap);
    cap.n_len = g->units;
    cap.n_rows = g->units * n_new;
    ak.app_blocks = pa::append_blocks64(cap);
  }
  p->glast = g;
  p->last_pt = slots > 0 ? pt : 0;
  p->last_prefix_units = 0;
  pa_call_stats& cs = p->last_stats;
  cs = pa_call_stats{};
  cs.partition_tokens = p->last_pt;
  cs.attention_workgroups = units * p->hkv;
  cs.append_workgroups = ak.app_blocks;
  cs.partial_rows = slots * rows;
  if (class_units) *class_units = g->units;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_NOMEM: return "out of free blocks";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_STATE: return "operation not possible in this state";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_err.c_str(); }

int pa_create_pool(pa_pool** out, int num_blocks, int block_size, int num_kv_heads, int head_dim,
                   int dtype, void* k_pool, void* v_pool, int32_t* block_table_dev,
                   int32_t* seq_len_dev, int max_seqs, int max_blocks_per_seq,
                   const int32_t* free_order) {
  if (!out) return set_err(PA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (block_size != pa::kBlock) return set_err(PA_ERR_INVALID, "block_size must be 16");
  if (num_kv_heads <= 0) return set_err(PA_ERR_INVALID, "num_kv_heads must be positive");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return set_err(PA_ERR_INVALID, "head_dim must be 64, 128 or 256");
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16 && dtype != PA_FP8_E4M3)
    return set_err(PA_ERR_INVALID, "unknown dtype");
  const int ndev = (k_pool != nullptr) + (v_pool != nullptr) + (block_table_dev != nullptr) + (seq_len_dev != nullptr);
  if (ndev != 0 && ndev != 4)
    return set_err(PA_ERR_INVALID, "give all four device pointers, or none for a host-only pool");
  if (ndev == 4 && (!aligned16(k_pool) || !aligned16(v_pool)))
    return set_err(PA_ERR_INVALID, "k_pool and v_pool must be 16-byte aligned");
  pa_pool* p = new (std::nothrow) pa_pool();
  if (!p) return set_err(PA_ERR_INVALID, "out of host memory");
  std::string err;
  int rc = p->bp.init(num_blocks, max_seqs, max_blocks_per_seq, free_order, &err);
  if (rc != pa::kOk) {
    delete p;
    return set_err(rc, err);
  }
  p->num_blocks = num_blocks;
  p->hkv = num_kv_heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->esize = dtype == PA_F32 ? 4 : (dtype == PA_FP8_E4M3 ? 1 : 2);
  p->k_pool = k_pool;
  p->v_pool = v_pool;
  p->block_table = block_table_dev;
  p->seq_len = seq_len_dev;
  p->host_only = (ndev == 0);
  if (!p->host_only) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      p->num_cus = cus;
    // the device's fixed scratch (pa_decode_noalloc), looked up once per device
    hipError_t se = pa::scratch_address(dev, &p->scratch);
    if (se != hipSuccess) {
      pa_destroy_pool(p);
      return hip_err(se, "hipGetSymbolAddress(scratch)");
    }
    for (Stage& st : p->stage) {
      hipError_t e = hipEventCreateWithFlags(&st.done, hipEventDisableTiming);
      if (e != hipSuccess) {
        pa_destroy_pool(p);
        return hip_err(e, "hipEventCreate");
      }
    }
  }
  if (dtype == PA_FP8_E4M3) {
    p->kv_scale_host.assign(4 * static_cast<size_t>(num_kv_heads), 1.0f);
    if (!p->host_only) {
      const size_t bytes = p->kv_scale_host.size() * sizeof(float);
      hipError_t e = hipMalloc(&p->kv_scale, bytes);
      if (e == hipSuccess) e = hipMemcpy(p->kv_scale, p->kv_scale_host.data(), bytes, hipMemcpyHostToDevice);
      if (e != hipSuccess) {
        pa_destroy_pool(p);
        return hip_err(e, "E4M3 scales");
      }
    }
  }
  *out = p;
  return PA_OK;
}

int pa_destroy_pool(pa_pool* p) {
  if (!p) return PA_OK;
  for (Stage& st : p->stage) {
    if (st.pending) (void)hipEventSynchronize(st.done);
    if (st.done) (void)hipEventDestroy(st.done);
    if (st.host) (void)hipHostFree(st.host);
  }
  for (ProfEvent& ev : p->prof_events) {
    (void)hipEventDestroy(ev.start);
    (void)hipEventDestroy(ev.stop);
  }
  if (p->dplan || p->merge_ctr || p->kv_scale || !p->gclass.empty()) (void)hipDeviceSynchronize();
  for (auto& kv : p->gclass) {
    if (kv.second.buf) (void)hipFree(kv.second.buf);
    if (kv.second.ctr) (void)hipFree(kv.second.ctr);
  }
  if (p->dplan) (void)hipFree(p->dplan);
  if (p->merge_ctr) (void)hipFree(p->merge_ctr);
  if (p->kv_scale) (void)hipFree(p->kv_scale);
  delete p;
  return PA_OK;
}

int pa_alloc_blocks(pa_pool* p, int seq_id, int parent_seq, int shared_tokens) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  std::string err;
  int rc = p->bp.alloc(seq_id, parent_seq, shared_tokens, &err);
  return rc == pa::kOk ? PA_OK : set_err(rc, err);
}

int pa_swap_bytes(const pa_pool* p, int n_tokens, size_t* bytes) {
  if (!p || !bytes) return set_err(PA_ERR_INVALID, "NULL argument");
  if (n_tokens < 0) return set_err(PA_ERR_INVALID, "n_tokens < 0");
  const size_t blocks = (static_cast<size_t>(n_tokens) + 15) / 16;
  *bytes = blocks * p->hkv * 16 * p->head_dim * p->esize;
  return PA_OK;
}

namespace {

// Device-visible address of a pinned host buffer.
int host_dev_ptr(const void* host, char** out) {
  void* d = nullptr;
  hipError_t e = hipHostGetDevicePointer(&d, const_cast<void*>(host), 0);
  if (e != hipSuccess || !d) {
    (void)hipGetLastError();
    return set_err(PA_ERR_INVALID, "host buffer is not pinned host memory");
  }
  *out = static_cast<char*>(d);
  return PA_OK;
}

// Copy the blocks of `table` between the pool and the host images on `stream`.
int swap_blocks(pa_pool* p, const std::vector<int32_t>& table, char* k_host, char* v_host, int last_rows,
                bool to_host, hipStream_t stream) {
  if (table.empty()) return PA_OK;
  Stage* st = nullptr;
  int rc = acquire_stage(p, table.size(), &st);
  if (rc != PA_OK) return rc;
  std::memcpy(st->host, table.data(), table.size() * sizeof(int32_t));
  pa::SwapParams sp{};
  sp.k_pool = static_cast<char*>(p->k_pool);
  sp.v_pool = static_cast<char*>(p->v_pool);
  sp.k_host = k_host;
  sp.v_host = v_host;
  sp.blocks = st->dev;
  sp.n_blocks = static_cast<int>(table.size());
  sp.block_bytes = p->hkv * 16 * p->head_dim * p->esize;
  sp.line_bytes = 16 * p->esize;
  sp.elem_bytes = p->esize;
  sp.last_rows = last_rows;
  sp.to_host = to_host ? 1 : 0;
  hipError_t e = pa::launch_swap(sp, stream);
  if (e != hipSuccess) return hip_err(e, "swap kernel");
  return release_stage(st, stream);
}

}  // namespace

int pa_swap_out(pa_pool* p, int seq_id, void* k_host, void* v_host, size_t bytes, int* length, void* stream_v) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (p->host_only) return set_err(PA_ERR_STATE, "host-only pool has no device memory");
  if (!p->bp.live(seq_id)) return set_err(PA_ERR_INVALID, "swap out of a sequence that is not live");
  const int n = p->bp.length(seq_id);
  size_t need = 0;
  pa_swap_bytes(p, n, &need);
  if (bytes < need) return set_err(PA_ERR_INVALID, "host buffers too small (see pa_swap_bytes)");
  char *kd = nullptr, *vd = nullptr;
  if (need > 0) {
    int rc = host_dev_ptr(k_host, &kd);
    if (rc == PA_OK) rc = host_dev_ptr(v_host, &vd);
    if (rc != PA_OK) return rc;
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  const std::vector<int32_t> table = p->bp.table(seq_id);
  int rc = swap_blocks(p, table, kd, vd, 16, true, stream);
  if (rc != PA_OK) return rc;
  std::string err;
  rc = p->bp.free_seq(seq_id, &err);
  if (rc != pa::kOk) return set_err(rc, err);
  if (length) *length = n;
  return PA_OK;
}

int pa_swap_in(pa_pool* p, int seq_id, int length, const void* k_host, const void* v_host, size_t bytes,
               void* stream_v) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (p->host_only) return set_err(PA_ERR_STATE, "host-only pool has no device memory");
  if (length < 0) return set_err(PA_ERR_INVALID, "length < 0");
  size_t need = 0;
  pa_swap_bytes(p, length, &need);
  if (bytes < need) return set_err(PA_ERR_INVALID, "host buffers too small (see pa_swap_bytes)");
  char *kd = nullptr, *vd = nullptr;
  if (need > 0) {
    int rc = host_dev_ptr(k_host, &kd);
    if (rc == PA_OK) rc = host_dev_ptr(v_host, &vd);
    if (rc != PA_OK) return rc;
  }
  std::string err;
  int rc = p->bp.alloc(seq_id, -1, 0, &err);
  if (rc != pa::kOk) return set_err(rc, err);
  // the blocks are taken exactly as an append of `length` rows would take them
  p->slots.clear();
  p->cows.clear();
  rc = p->bp.append(&seq_id, 1, &length, &p->slots, &p->cows, &err);
  if (rc != pa::kOk) {
    std::string ignore;
    p->bp.free_seq(seq_id, &ignore);
    return set_err(rc, err);
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  rc = flush_dirty(p, stream);
  if (rc != PA_OK) return rc;
  const int last = length % 16 == 0 ? 16 : length % 16;
  return swap_blocks(p, p->bp.table(seq_id), kd, vd, last, false, stream);
}

int pa_prefix_insert(pa_pool* p, int seq_id, const int32_t* tokens, int n_tokens, int* n_new) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  std::string err;
  int rc = p->bp.prefix_insert(seq_id, tokens, n_tokens, n_new, &err);
  return rc == pa::kOk ? PA_OK : set_err(rc, err);
}

int pa_prefix_match(const pa_pool* p, const int32_t* tokens, int n_tokens, int* n_matched) {
  if (!p || !n_matched) return set_err(PA_ERR_INVALID, "NULL argument");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return set_err(PA_ERR_INVALID, "bad token array");
  *n_matched = p->bp.prefix_match(tokens, n_tokens);
  return PA_OK;
}

int pa_alloc_from_prefix(pa_pool* p, int seq_id, const int32_t* tokens, int n_tokens, int* n_matched) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  std::string err;
  int rc = p->bp.alloc_from_prefix(seq_id, tokens, n_tokens, n_matched, &err);
  return rc == pa::kOk ? PA_OK : set_err(rc, err);
}

int pa_prefix_evict(pa_pool* p, int max_entries, int* n_evicted) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  std::string err;
  int rc = p->bp.prefix_evict(max_entries, n_evicted, &err);
  return rc == pa::kOk ? PA_OK : set_err(rc, err);
}

int pa_prefix_entries(const pa_pool* p, int* n) {
  if (!p || !n) return set_err(PA_ERR_INVALID, "NULL argument");
  *n = p->bp.prefix_entries();
  return PA_OK;
}

int pa_set_kv_scales(pa_pool* p, const float* k_scale, const float* v_scale) {
  if (!p || !k_scale || !v_scale) return set_err(PA_ERR_INVALID, "NULL argument");
  if (p->dtype != PA_FP8_E4M3) return set_err(PA_ERR_STATE, "scales belong to PA_FP8_E4M3 pools");
  const int h = p->hkv;
  for (int i = 0; i < h; ++i)
    if (!(k_scale[i] > 0.f) || !(v_scale[i] > 0.f) || !std::isfinite(k_scale[i]) || !std::isfinite(v_scale[i]))
      return set_err(PA_ERR_INVALID, "scales must be finite and > 0");
  std::vector<float> next(4 * static_cast<size_t>(h));
  for (int i = 0; i < h; ++i) {
    next[i] = k_scale[i];
    next[h + i] = v_scale[i];
    next[2 * h + i] = 1.0f / k_scale[i];
    next[3 * h + i] = 1.0f / v_scale[i];
  }
  if (p->kv_scale) {
    // the stream work already enqueued may still read the old scales
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(p->kv_scale, next.data(), next.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_err(e, "E4M3 scales");
  }
  p->kv_scale_host.swap(next);
  return PA_OK;
}

int pa_append_kv(pa_pool* p, const int32_t* seq_ids, int n_seq, const int32_t* n_tok,
                 const void* k_new, const void* v_new, void* stream_v) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  int64_t total = 0;
  for (int i = 0; i < n_seq && n_tok; ++i) total += std::max(0, n_tok[i]);
  if (!p->host_only && total > 0 && (!k_new || !v_new))
    return set_err(PA_ERR_INVALID, "k_new / v_new are NULL");
  if (!p->host_only && total > 0 && (!aligned16(k_new) || !aligned16(v_new)))
    return set_err(PA_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  if (total > INT32_MAX / 2) return set_err(PA_ERR_INVALID, "too many rows in one append");
  p->slots.clear();
  p->cows.clear();
  std::string err;
  int rc = p->bp.append(seq_ids, n_seq, n_tok, &p->slots, &p->cows, &err);
  if (rc != pa::kOk) return set_err(rc, err);
  p->bp.take_dirty(&p->dirty);
  if (p->host_only) return PA_OK;
  return launch_append_call(p, k_new, v_new, static_cast<hipStream_t>(stream_v));
}

int pa_decode(pa_pool* p, const int32_t* seq_ids, int n_seq, int num_q_heads, float scale,
              const void* q, void* out, float* lse, int partition_tokens, void* workspace,
              size_t ws_bytes, void* stream) {
  return attend(p, seq_ids, n_seq, 1, num_q_heads, scale, q, out, lse, partition_tokens, workspace,
                ws_bytes, stream, nullptr);
}

int pa_decode_noalloc(pa_pool* p, const int32_t* seq_ids, int n_seq, int num_q_heads, float scale, const void* q,
                      void* out, float* lse, int partition_tokens, void* stream) {
  return attend(p, seq_ids, n_seq, 1, num_q_heads, scale, q, out, lse, partition_tokens, nullptr, 0, stream,
                nullptr, true);
}

int pa_verify(pa_pool* p, const int32_t* seq_ids, int n_seq, int k_draft, int num_q_heads, float scale,
              const void* q, void* out, float* lse, int partition_tokens, void* workspace,
              size_t ws_bytes, void* stream) {
  return attend(p, seq_ids, n_seq, k_draft, num_q_heads, scale, q, out, lse, partition_tokens, workspace,
                ws_bytes, stream, nullptr);
}

int pa_prefill(pa_pool* p, const int32_t* seq_ids, int n_seq, int n_new, int num_q_heads, float scale,
               const void* q, void* out, float* lse, int partition_tokens, void* workspace, size_t ws_bytes,
               void* stream) {
  return attend(p, seq_ids, n_seq, n_new, num_q_heads, scale, q, out, lse, partition_tokens, workspace,
                ws_bytes, stream, nullptr);
}

int pa_append_attend(pa_pool* p, const int32_t* seq_ids, int n_seq, int n_new, const void* k_new,
                     const void* v_new, int num_q_heads, float scale, const void* q, void* out, float* lse,
                     int partition_tokens, void* workspace, size_t ws_bytes, void* stream) {
  const AppendSpec app{n_new, k_new, v_new};
  return attend(p, seq_ids, n_seq, n_new, num_q_heads, scale, q, out, lse, partition_tokens, workspace,
                ws_bytes, stream, &app);
}

int pa_graph_prepare(pa_pool* p, const int32_t* seq_ids, int n_seq, int n_new, const void* k_new, const void* v_new,
                     int num_q_heads, float scale, const void* q, void* out, float* lse, int partition_tokens,
                     void* workspace, size_t ws_bytes, void* stream, int* class_units) {
  return graph_prepare(p, seq_ids, n_seq, n_new, k_new, v_new, num_q_heads, scale, q, out, lse, partition_tokens,
                       workspace, ws_bytes, stream, class_units);
}

int pa_graph_launch(pa_pool* p, void* stream) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (!p->glast) return set_err(PA_ERR_STATE, "no graph step prepared");
  const pa::DType dt = static_cast<pa::DType>(p->dtype);
  hipError_t e = pa::launch_attention(dt, p->glast->params, &p->inline_meta, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_err(e, "attention kernel (graph step)");
  return PA_OK;
}

int pa_truncate(pa_pool* p, int seq_id, int new_len) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  std::string err;
  int rc = p->bp.truncate(seq_id, new_len, &err);
  return rc == pa::kOk ? PA_OK : set_err(rc, err);
}

int pa_truncate_batch(pa_pool* p, const int32_t* seq_ids, int n_seq, const int32_t* new_lens) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (n_seq < 0 || (n_seq > 0 && (!seq_ids || !new_lens))) return set_err(PA_ERR_INVALID, "bad arrays");
  std::vector<int32_t> seen(seq_ids, seq_ids + n_seq);
  for (int i = 0; i < n_seq; ++i) {
    if (!p->bp.live(seq_ids[i])) return set_err(PA_ERR_INVALID, "sequence is not live");
    if (new_lens[i] < 0 || new_lens[i] > p->bp.length(seq_ids[i]))
      return set_err(PA_ERR_INVALID, "new_len outside [0, length]");
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return set_err(PA_ERR_INVALID, "sequence repeated in one truncate");
  std::string err;
  for (int i = 0; i < n_seq; ++i) p->bp.truncate(seq_ids[i], new_lens[i], &err);
  return PA_OK;
}

int pa_free_seq(pa_pool* p, int seq_id) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  std::string err;
  int rc = p->bp.free_seq(seq_id, &err);
  return rc == pa::kOk ? PA_OK : set_err(rc, err);
}

int pa_sync_tables(pa_pool* p, void* stream_v) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  return flush_dirty(p, static_cast<hipStream_t>(stream_v));
}

int pa_workspace_size(const pa_pool* p, int n_seq, int num_q_heads, int k_draft, int max_tokens,
                      int partition_tokens, size_t* bytes) {
  if (!p || !bytes) return set_err(PA_ERR_INVALID, "pool or bytes is NULL");
  if (n_seq < 0 || k_draft < 1 || max_tokens < 0 || num_q_heads <= 0 || num_q_heads % p->hkv)
    return set_err(PA_ERR_INVALID, "bad sizes");
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % 32))
    return set_err(PA_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of 32");
  const int64_t rows = static_cast<int64_t>(num_q_heads / p->hkv) * k_draft;
  const int pt = partition_tokens == 0 ? default_partition(rows) : partition_tokens;
  // (one partition more than the plain split: a shared-prefix member's own
  // partitions start where its shared prefix ends)
  const int64_t parts = max_tokens > pt ? (max_tokens + pt - 1) / pt + 1 : 0;
  *bytes = static_cast<size_t>(n_seq) * parts * p->hkv * rows * (p->head_dim + 2) * sizeof(float);
  return PA_OK;
}

int pa_get_block_table(const pa_pool* p, int seq_id, int32_t* out, int cap, int* n_blocks, int* len) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (!p->bp.live(seq_id)) return set_err(PA_ERR_INVALID, "sequence is not live");
  const std::vector<int32_t>& t = p->bp.table(seq_id);
  if (n_blocks) *n_blocks = static_cast<int>(t.size());
  if (len) *len = p->bp.length(seq_id);
  if (out) {
    if (cap < static_cast<int>(t.size())) return set_err(PA_ERR_INVALID, "cap too small");
    std::copy(t.begin(), t.end(), out);
  }
  return PA_OK;
}

int pa_get_refcount(const pa_pool* p, int block_id, int* rc) {
  if (!p || !rc) return set_err(PA_ERR_INVALID, "NULL argument");
  if (block_id < 0 || block_id >= p->bp.num_blocks()) return set_err(PA_ERR_INVALID, "block id out of range");
  *rc = p->bp.refcount(block_id);
  return PA_OK;
}

int pa_num_free_blocks(const pa_pool* p, int* n) {
  if (!p || !n) return set_err(PA_ERR_INVALID, "NULL argument");
  *n = p->bp.num_free();
  return PA_OK;
}

int pa_last_partition(const pa_pool* p, int* partition_tokens, int* prefix_units) {
  if (!p || !partition_tokens || !prefix_units) return set_err(PA_ERR_INVALID, "NULL argument");
  *partition_tokens = p->last_pt;
  *prefix_units = p->last_prefix_units;
  return PA_OK;
}

int pa_last_call_stats(const pa_pool* p, pa_call_stats* out) {
  if (!p || !out) return set_err(PA_ERR_INVALID, "NULL argument");
  *out = p->last_stats;
  return PA_OK;
}

int pa_get_free_list(const pa_pool* p, int32_t* out, int cap, int* n) {
  if (!p || !n) return set_err(PA_ERR_INVALID, "NULL argument");
  const std::deque<int32_t>& f = p->bp.free_list();
  *n = static_cast<int>(f.size());
  if (out) {
    if (cap < *n) return set_err(PA_ERR_INVALID, "cap too small");
    std::copy(f.begin(), f.end(), out);
  }
  return PA_OK;
}

int pa_profile_enable(pa_pool* p, int on) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  p->prof = on != 0;
  return PA_OK;
}

int pa_profile_read(pa_pool* p, int which, double* total_ms, int64_t* launches) {
  if (!p || which < 0 || which > 3) return set_err(PA_ERR_INVALID, "bad arguments");
  for (ProfEvent& ev : p->prof_events) {
    hipError_t e = hipEventSynchronize(ev.stop);
    if (e != hipSuccess) return hip_err(e, "hipEventSynchronize(profile)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ev.start, ev.stop);
    if (e != hipSuccess) return hip_err(e, "hipEventElapsedTime");
    p->prof_ms[ev.which] += ms;
    p->prof_n[ev.which] += 1;
    (void)hipEventDestroy(ev.start);
    (void)hipEventDestroy(ev.stop);
  }
  p->prof_events.clear();
  if (total_ms) *total_ms = p->prof_ms[which];
  if (launches) *launches = p->prof_n[which];
  p->prof_ms[which] = 0;
  p->prof_n[which] = 0;
  return PA_OK;
}

}  // extern "C"
