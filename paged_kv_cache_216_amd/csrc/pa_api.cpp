// C-ABI entry points declared in include/pa.h.  Host-side validation, the block
// allocator, packing of per-call metadata into one pinned buffer, a single
// host-to-device copy of it, and the kernel launches.
#include "../../include/pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <vector>

#include "block_pool.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_err(hipError_t e, const char* what) {
  return set_err(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

constexpr int kStages = 4;
constexpr int kDefaultPartition = 512;

struct Stage {
  int32_t* host = nullptr;  // pinned
  size_t cap = 0;           // bytes
  hipEvent_t done = nullptr;
  bool pending = false;
};

struct ProfEvent {
  int which;
  hipEvent_t start, stop;
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
  // metadata buffers
  int32_t* dmeta = nullptr;
  size_t dmeta_cap = 0;
  Stage stage[kStages];
  int next_stage = 0;
  // profiling
  bool prof = false;
  std::vector<ProfEvent> prof_events;
  double prof_ms[3] = {0, 0, 0};
  int64_t prof_n[3] = {0, 0, 0};
};

namespace {

// Grow-only buffers.  A larger device buffer is only swapped in after the
// device is idle, so in-flight kernels never read freed memory.
int ensure_capacity(pa_pool* p, Stage& st, size_t bytes) {
  if (bytes > p->dmeta_cap) {
    size_t cap = std::max<size_t>(bytes, 2 * p->dmeta_cap);
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_err(e, "hipDeviceSynchronize");
    if (p->dmeta) hipFree(p->dmeta);
    p->dmeta = nullptr;
    p->dmeta_cap = 0;
    e = hipMalloc(&p->dmeta, cap);
    if (e != hipSuccess) return hip_err(e, "hipMalloc(metadata)");
    p->dmeta_cap = cap;
  }
  if (bytes > st.cap) {
    size_t cap = std::max<size_t>(bytes, 2 * st.cap);
    if (st.host) hipHostFree(st.host);
    st.host = nullptr;
    st.cap = 0;
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&st.host), cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_err(e, "hipHostMalloc(staging)");
    st.cap = cap;
  }
  return PA_OK;
}

// Copy `words` to the device metadata buffer on `stream`.
int upload(pa_pool* p, const std::vector<int32_t>& words, hipStream_t stream) {
  if (words.empty()) return PA_OK;
  Stage& st = p->stage[p->next_stage];
  p->next_stage = (p->next_stage + 1) % kStages;
  if (st.pending) {
    hipError_t e = hipEventSynchronize(st.done);
    if (e != hipSuccess) return hip_err(e, "hipEventSynchronize(staging)");
    st.pending = false;
  }
  const size_t bytes = words.size() * sizeof(int32_t);
  int rc = ensure_capacity(p, st, bytes);
  if (rc != PA_OK) return rc;
  std::memcpy(st.host, words.data(), bytes);
  hipError_t e = hipMemcpyAsync(p->dmeta, st.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync(metadata)");
  e = hipEventRecord(st.done, stream);
  if (e != hipSuccess) return hip_err(e, "hipEventRecord(staging)");
  st.pending = true;
  return PA_OK;
}

// Section offsets are kept at multiples of 8 words (32 bytes).
size_t pad8(std::vector<int32_t>& w) {
  while (w.size() % 8) w.push_back(0);
  return w.size();
}

void prof_begin(pa_pool* p, int which, hipStream_t s, ProfEvent* ev) {
  if (!p->prof) return;
  ev->which = which;
  hipEventCreate(&ev->start);
  hipEventCreate(&ev->stop);
  hipEventRecord(ev->start, s);
}

void prof_end(pa_pool* p, hipStream_t s, ProfEvent* ev) {
  if (!p->prof) return;
  hipEventRecord(ev->stop, s);
  p->prof_events.push_back(*ev);
}

// Pending table / length updates, appended to `w`; counts returned.
void pack_dirty(pa_pool* p, std::vector<int32_t>& w, int* n_tab, int* n_len, size_t* tab_off,
                size_t* len_off) {
  pa::BlockPool::Dirty d;
  p->bp.take_dirty(&d);
  *tab_off = pad8(w);
  for (size_t i = 0; i < d.table_idx.size(); ++i) {
    w.push_back(d.table_idx[i]);
    w.push_back(d.table_val[i]);
  }
  *len_off = pad8(w);
  for (size_t i = 0; i < d.len_seq.size(); ++i) {
    w.push_back(d.len_seq[i]);
    w.push_back(d.len_val[i]);
  }
  *n_tab = static_cast<int>(d.table_idx.size());
  *n_len = static_cast<int>(d.len_seq.size());
}

pa::AppendParams base_append(pa_pool* p) {
  pa::AppendParams ap{};
  ap.k_pool = p->k_pool;
  ap.v_pool = p->v_pool;
  ap.block_table = p->block_table;
  ap.seq_len = p->seq_len;
  ap.hkv = p->hkv;
  ap.head_dim = p->head_dim;
  ap.elem_bytes = p->esize;
  return ap;
}

int rows_limit(const pa_pool* p) { return pa::max_rows_for_head_dim(p->head_dim); }

// Work decomposition shared by pa_decode / pa_verify / pa_workspace_size.
struct Plan {
  std::vector<pa::WorkUnit> units;
  std::vector<pa::MergeUnit> merges;
  int64_t slots = 0;
};

void make_plan(const pa_pool* p, const int32_t* seq_ids, const int* lens, int n_seq, int pt, Plan* out) {
  out->units.clear();
  out->merges.clear();
  out->slots = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int n = lens[i];
    const int parts = (pt > 0 && n > pt) ? (n + pt - 1) / pt : 1;
    if (parts == 1) {
      out->units.push_back({i, seq_ids[i], n, 0, n, -1, 1, 0});
      continue;
    }
    const int base = static_cast<int>(out->slots);
    out->slots += static_cast<int64_t>(parts) * p->hkv;
    for (int q = 0; q < parts; ++q)
      out->units.push_back({i, seq_ids[i], n, q * pt, std::min(n, (q + 1) * pt), base, parts, q});
    out->merges.push_back({i, base, parts, 0});
  }
  // longest units first, so the tail of the grid holds the short ones
  std::stable_sort(out->units.begin(), out->units.end(), [](const pa::WorkUnit& a, const pa::WorkUnit& b) {
    return (a.tok_end - a.tok_begin) > (b.tok_end - b.tok_begin);
  });
}

size_t plan_ws_bytes(const pa_pool* p, int64_t slots, int rows) {
  return static_cast<size_t>(slots) * rows * (p->head_dim + 2) * sizeof(float);
}

int attend(pa_pool* p, const int32_t* seq_ids, int n_seq, int k_draft, int num_q_heads, float scale,
           const void* q, void* out, float* lse, int partition_tokens, void* workspace, size_t ws_bytes,
           void* stream_v) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  if (p->host_only) return set_err(PA_ERR_STATE, "host-only pool has no device memory");
  if (n_seq < 0) return set_err(PA_ERR_INVALID, "n_seq < 0");
  if (k_draft < 1) return set_err(PA_ERR_INVALID, "k_draft must be >= 1");
  if (num_q_heads <= 0 || num_q_heads % p->hkv != 0)
    return set_err(PA_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / p->hkv;
  const int64_t rows64 = static_cast<int64_t>(group) * k_draft;
  if (rows64 > rows_limit(p))
    return set_err(PA_ERR_INVALID, "(num_q_heads / num_kv_heads) * k_draft exceeds the supported rows");
  const int rows = static_cast<int>(rows64);
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % 32 != 0))
    return set_err(PA_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of 32");
  if (n_seq > 0 && (!seq_ids || !q || !out)) return set_err(PA_ERR_INVALID, "seq_ids, q or out is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return set_err(PA_ERR_INVALID, "q, out and workspace must be 16-byte aligned");
  std::vector<int> lens(n_seq);
  int max_len = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int s = seq_ids[i];
    if (!p->bp.live(s)) return set_err(PA_ERR_INVALID, "attention over a sequence that is not live");
    lens[i] = p->bp.length(s);
    if (lens[i] < std::max(1, k_draft))
      return set_err(PA_ERR_INVALID, "sequence shorter than max(1, k_draft)");
    max_len = std::max(max_len, lens[i]);
  }
  int pt = partition_tokens;
  Plan plan;
  if (pt == 0) {
    pt = kDefaultPartition;
    make_plan(p, seq_ids, lens.data(), n_seq, pt, &plan);
    if (plan_ws_bytes(p, plan.slots, rows) > ws_bytes || (plan.slots && !workspace)) {
      pt = 0;  // the workspace cannot hold the split: run unsplit
      make_plan(p, seq_ids, lens.data(), n_seq, 0, &plan);
    }
  } else {
    make_plan(p, seq_ids, lens.data(), n_seq, pt, &plan);
    if (plan.slots && (!workspace || plan_ws_bytes(p, plan.slots, rows) > ws_bytes))
      return set_err(PA_ERR_INVALID, "workspace too small for this partition size (see pa_workspace_size)");
  }
  if (plan.slots * rows * static_cast<int64_t>(p->head_dim) > INT32_MAX * 4LL)
    return set_err(PA_ERR_INVALID, "too many split partials");
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  std::vector<int32_t> w;
  int n_tab = 0, n_len = 0;
  size_t tab_off = 0, len_off = 0;
  pack_dirty(p, w, &n_tab, &n_len, &tab_off, &len_off);
  const size_t unit_off = pad8(w);
  for (const pa::WorkUnit& u : plan.units) {
    const int32_t* x = reinterpret_cast<const int32_t*>(&u);
    w.insert(w.end(), x, x + 8);
  }
  const size_t merge_off = pad8(w);
  for (const pa::MergeUnit& m : plan.merges) {
    const int32_t* x = reinterpret_cast<const int32_t*>(&m);
    w.insert(w.end(), x, x + 4);
  }
  pad8(w);
  int rc = upload(p, w, stream);
  if (rc != PA_OK) return rc;

  if (n_tab + n_len > 0) {
    pa::AppendParams ap = base_append(p);
    ap.tab = p->dmeta + tab_off;
    ap.lens = p->dmeta + len_off;
    ap.n_tab = n_tab;
    ap.n_len = n_len;
    hipError_t e = pa::launch_append(ap, stream);
    if (e != hipSuccess) return hip_err(e, "append kernel (table update)");
  }
  if (plan.units.empty()) return PA_OK;

  pa::AttnParams ak{};
  ak.k_pool = p->k_pool;
  ak.v_pool = p->v_pool;
  ak.block_table = p->block_table;
  ak.max_blocks = p->bp.max_blocks_per_seq();
  ak.num_blocks = p->num_blocks;
  ak.q = q;
  ak.out = out;
  ak.lse = lse;
  float* ws = static_cast<float*>(workspace);
  ak.ws_acc = ws;
  ak.ws_ml = ws ? ws + static_cast<size_t>(plan.slots) * rows * p->head_dim : nullptr;
  ak.units = reinterpret_cast<const pa::WorkUnit*>(p->dmeta + unit_off);
  ak.merges = reinterpret_cast<const pa::MergeUnit*>(p->dmeta + merge_off);
  ak.n_units = static_cast<int>(plan.units.size());
  ak.n_merges = static_cast<int>(plan.merges.size());
  ak.hkv = p->hkv;
  ak.hq = num_q_heads;
  ak.group = group;
  ak.k_draft = k_draft;
  ak.rows = rows;
  ak.head_dim = p->head_dim;
  ak.scale_log2 = scale * 1.4426950408889634f;
  const pa::DType dt = static_cast<pa::DType>(p->dtype);
  ProfEvent ev{};
  prof_begin(p, 0, stream, &ev);
  hipError_t e = pa::launch_attention(dt, ak, stream);
  if (e != hipSuccess) return hip_err(e, "attention kernel");
  prof_end(p, stream, &ev);
  if (!plan.merges.empty()) {
    ProfEvent ev2{};
    prof_begin(p, 1, stream, &ev2);
    e = pa::launch_merge(dt, ak, stream);
    if (e != hipSuccess) return hip_err(e, "merge kernel");
    prof_end(p, stream, &ev2);
  }
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
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return set_err(PA_ERR_INVALID, "unknown dtype");
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
  p->esize = dtype == PA_F32 ? 4 : 2;
  p->k_pool = k_pool;
  p->v_pool = v_pool;
  p->block_table = block_table_dev;
  p->seq_len = seq_len_dev;
  p->host_only = (ndev == 0);
  if (!p->host_only) {
    for (Stage& st : p->stage) {
      hipError_t e = hipEventCreateWithFlags(&st.done, hipEventDisableTiming);
      if (e != hipSuccess) {
        pa_destroy_pool(p);
        return hip_err(e, "hipEventCreate");
      }
    }
  }
  *out = p;
  return PA_OK;
}

int pa_destroy_pool(pa_pool* p) {
  if (!p) return PA_OK;
  for (Stage& st : p->stage) {
    if (st.pending) hipEventSynchronize(st.done);
    if (st.done) hipEventDestroy(st.done);
    if (st.host) hipHostFree(st.host);
  }
  for (ProfEvent& ev : p->prof_events) {
    hipEventDestroy(ev.start);
    hipEventDestroy(ev.stop);
  }
  if (p->dmeta) {
    hipDeviceSynchronize();
    hipFree(p->dmeta);
  }
  delete p;
  return PA_OK;
}

int pa_alloc_blocks(pa_pool* p, int seq_id, int parent_seq, int shared_tokens) {
  if (!p) return set_err(PA_ERR_INVALID, "pool is NULL");
  std::string err;
  int rc = p->bp.alloc(seq_id, parent_seq, shared_tokens, &err);
  return rc == pa::kOk ? PA_OK : set_err(rc, err);
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
  std::vector<int32_t> slots;
  std::vector<pa::CowCopy> cows;
  slots.reserve(static_cast<size_t>(total));
  std::string err;
  int rc = p->bp.append(seq_ids, n_seq, n_tok, &slots, &cows, &err);
  if (rc != pa::kOk) return set_err(rc, err);
  if (p->host_only) {
    pa::BlockPool::Dirty d;
    p->bp.take_dirty(&d);
    return PA_OK;
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  std::vector<int32_t> w;
  w.reserve(slots.size() + 64);
  int n_tab = 0, n_len = 0;
  size_t tab_off = 0, len_off = 0;
  pack_dirty(p, w, &n_tab, &n_len, &tab_off, &len_off);
  const size_t cow_off = pad8(w);
  for (const pa::CowCopy& c : cows) {
    w.push_back(c.src);
    w.push_back(c.dst);
    w.push_back(c.rows);
  }
  const size_t slot_off = pad8(w);
  w.insert(w.end(), slots.begin(), slots.end());
  pad8(w);
  rc = upload(p, w, stream);
  if (rc != PA_OK) return rc;
  pa::AppendParams ap = base_append(p);
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.tab = p->dmeta + tab_off;
  ap.lens = p->dmeta + len_off;
  ap.cows = p->dmeta + cow_off;
  ap.slots = p->dmeta + slot_off;
  ap.n_tab = n_tab;
  ap.n_len = n_len;
  ap.n_cow = static_cast<int>(cows.size());
  ap.n_rows = static_cast<int>(slots.size());
  ProfEvent ev{};
  prof_begin(p, 2, stream, &ev);
  hipError_t e = pa::launch_append(ap, stream);
  if (e != hipSuccess) return hip_err(e, "append kernel");
  prof_end(p, stream, &ev);
  return PA_OK;
}

int pa_decode(pa_pool* p, const int32_t* seq_ids, int n_seq, int num_q_heads, float scale,
              const void* q, void* out, float* lse, int partition_tokens, void* workspace,
              size_t ws_bytes, void* stream) {
  return attend(p, seq_ids, n_seq, 1, num_q_heads, scale, q, out, lse, partition_tokens, workspace,
                ws_bytes, stream);
}

int pa_verify(pa_pool* p, const int32_t* seq_ids, int n_seq, int k_draft, int num_q_heads, float scale,
              const void* q, void* out, float* lse, int partition_tokens, void* workspace,
              size_t ws_bytes, void* stream) {
  return attend(p, seq_ids, n_seq, k_draft, num_q_heads, scale, q, out, lse, partition_tokens, workspace,
                ws_bytes, stream);
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
  std::vector<int32_t> seen;
  seen.reserve(n_seq);
  for (int i = 0; i < n_seq; ++i) {
    if (!p->bp.live(seq_ids[i])) return set_err(PA_ERR_INVALID, "sequence is not live");
    if (new_lens[i] < 0 || new_lens[i] > p->bp.length(seq_ids[i]))
      return set_err(PA_ERR_INVALID, "new_len outside [0, length]");
    seen.push_back(seq_ids[i]);
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
  if (p->host_only) {
    pa::BlockPool::Dirty d;
    p->bp.take_dirty(&d);
    return PA_OK;
  }
  if (!p->bp.has_dirty()) return PA_OK;
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  std::vector<int32_t> w;
  int n_tab = 0, n_len = 0;
  size_t tab_off = 0, len_off = 0;
  pack_dirty(p, w, &n_tab, &n_len, &tab_off, &len_off);
  pad8(w);
  int rc = upload(p, w, stream);
  if (rc != PA_OK) return rc;
  pa::AppendParams ap = base_append(p);
  ap.tab = p->dmeta + tab_off;
  ap.lens = p->dmeta + len_off;
  ap.n_tab = n_tab;
  ap.n_len = n_len;
  hipError_t e = pa::launch_append(ap, stream);
  return e == hipSuccess ? PA_OK : hip_err(e, "append kernel (table update)");
}

int pa_workspace_size(const pa_pool* p, int n_seq, int num_q_heads, int k_draft, int max_tokens,
                      int partition_tokens, size_t* bytes) {
  if (!p || !bytes) return set_err(PA_ERR_INVALID, "pool or bytes is NULL");
  if (n_seq < 0 || k_draft < 1 || max_tokens < 0 || num_q_heads <= 0 || num_q_heads % p->hkv)
    return set_err(PA_ERR_INVALID, "bad sizes");
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % 32))
    return set_err(PA_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of 32");
  const int pt = partition_tokens == 0 ? kDefaultPartition : partition_tokens;
  const int64_t parts = max_tokens > pt ? (max_tokens + pt - 1) / pt : 0;
  const int64_t rows = static_cast<int64_t>(num_q_heads / p->hkv) * k_draft;
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
  if (!p || which < 0 || which > 2) return set_err(PA_ERR_INVALID, "bad arguments");
  for (ProfEvent& ev : p->prof_events) {
    hipError_t e = hipEventSynchronize(ev.stop);
    if (e != hipSuccess) return hip_err(e, "hipEventSynchronize(profile)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ev.start, ev.stop);
    if (e != hipSuccess) return hip_err(e, "hipEventElapsedTime");
    p->prof_ms[ev.which] += ms;
    p->prof_n[ev.which] += 1;
    hipEventDestroy(ev.start);
    hipEventDestroy(ev.stop);
  }
  p->prof_events.clear();
  if (total_ms) *total_ms = p->prof_ms[which];
  if (launches) *launches = p->prof_n[which];
  p->prof_ms[which] = 0;
  p->prof_n[which] = 0;
  return PA_OK;
}

}  // extern "C"
