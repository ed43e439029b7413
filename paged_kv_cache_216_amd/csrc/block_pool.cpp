// Host-side block allocator; the rules are stated in block_pool.hpp.
#include "block_pool.hpp"

#include <algorithm>

namespace pa {

namespace {
int fail(std::string* err, int code, const char* msg) {
  if (err) *err = msg;
  return code;
}
}  // namespace

int BlockPool::init(int num_blocks, int max_seqs, int max_blocks_per_seq,
                    const int32_t* free_order, std::string* err) {
  if (num_blocks <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0)
    return fail(err, kInvalid, "num_blocks, max_seqs and max_blocks_per_seq must be positive");
  if (static_cast<int64_t>(max_seqs) * max_blocks_per_seq > INT32_MAX)
    return fail(err, kInvalid, "max_seqs * max_blocks_per_seq exceeds int32");
  std::vector<char> seen(num_blocks, 0);
  free_.clear();
  for (int i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b])
      return fail(err, kInvalid, "free_order must be a permutation of 0..num_blocks-1");
    seen[b] = 1;
    free_.push_back(b);
  }
  num_blocks_ = num_blocks;
  max_seqs_ = max_seqs;
  max_blocks_ = max_blocks_per_seq;
  rc_.assign(num_blocks, 0);
  tables_.assign(max_seqs, {});
  len_.assign(max_seqs, -1);
  entry_flag_.assign(static_cast<size_t>(max_seqs) * max_blocks_per_seq, 0);
  len_flag_.assign(max_seqs, 0);
  seen_flag_.assign(max_seqs, 0);
  dirty_entry_list_.clear();
  dirty_len_list_.clear();
  num_shared_ = 0;
  rc_delta_.assign(num_blocks, 0);
  touched_.clear();
  pentries_.clear();
  pfree_ids_.clear();
  pindex_.clear();
  pleaves_.clear();
  pclock_ = 0;
  porder_ = 0;
  return kOk;
}

int32_t BlockPool::pop() {
  int32_t b = free_.front();
  free_.pop_front();
  rc_[b] = 1;
  return b;
}

void BlockPool::release(int32_t b) {
  const int32_t rc = --rc_[b];
  if (rc == 1) --num_shared_;
  if (rc == 0) free_.push_back(b);
}

int BlockPool::alloc(int seq, int parent, int shared_tokens, std::string* err) {
  if (seq < 0 || seq >= max_seqs_) return fail(err, kInvalid, "seq id out of range");
  if (len_[seq] >= 0) return fail(err, kInvalid, "seq id already live");
  if (parent < 0) {
    if (shared_tokens != 0) return fail(err, kInvalid, "shared_tokens needs a parent");
    tables_[seq].clear();
    len_[seq] = 0;
    mark_len(seq);
    return kOk;
  }
  if (!live(parent)) return fail(err, kInvalid, "parent sequence is not live");
  if (shared_tokens < 0 || shared_tokens > len_[parent])
    return fail(err, kInvalid, "shared_tokens outside [0, parent length]");
  const int nb = (shared_tokens + kBlock - 1) / kBlock;
  const std::vector<int32_t>& pt = tables_[parent];
  tables_[seq].assign(pt.begin(), pt.begin() + nb);
  for (int j = 0; j < nb; ++j) {
    if (++rc_[pt[j]] == 2) ++num_shared_;
    mark_entry(seq, j);
  }
  len_[seq] = shared_tokens;
  mark_len(seq);
  return kOk;
}

int BlockPool::append(const int32_t* seqs, int n_seq, const int32_t* n_tok,
                      std::vector<int32_t>* slots, std::vector<CowCopy>* cows,
                      std::string* err) {
  if (n_seq < 0) return fail(err, kInvalid, "n_seq < 0");
  if (n_seq > 0 && (!seqs || !n_tok)) return fail(err, kInvalid, "seq_ids / n_tok are NULL");
  // Validate everything first and count the blocks the call needs, following
  // reference counts as earlier sequences of the same call copy shared tails.
  int64_t need = 0;
  int bad = kOk;
  const char* why = nullptr;
  int i = 0;
  for (; i < n_seq; ++i) {
    const int s = seqs[i];
    if (!live(s)) { bad = kInvalid; why = "append to a sequence that is not live"; break; }
    if (seen_flag_[s]) { bad = kInvalid; why = "sequence repeated in one append"; break; }
    seen_flag_[s] = 1;
    if (n_tok[i] < 0) { ++i; bad = kInvalid; why = "negative token count"; break; }
    const int64_t len = len_[s];
    if (len + n_tok[i] > static_cast<int64_t>(max_blocks_) * kBlock) {
      ++i;
      bad = kInvalid;
      why = "sequence would exceed max_blocks_per_seq";
      break;
    }
    if (n_tok[i] == 0) continue;
    if (len % kBlock != 0) {
      const int32_t tail = tables_[s].back();
      if (rc_[tail] + rc_delta_[tail] > 1) {
        ++need;
        if (rc_delta_[tail] == 0) touched_.push_back(tail);
        --rc_delta_[tail];
      }
    }
    // blocks that start inside [len, len + n): positions p with p % 16 == 0
    const int64_t first = (len + kBlock - 1) / kBlock;
    const int64_t last = (len + n_tok[i] - 1) / kBlock;
    need += last - first + 1;
  }
  // clear the scratch marks whatever the outcome
  for (int k = 0; k < std::min(i, n_seq); ++k)
    if (seqs[k] >= 0 && seqs[k] < max_seqs_) seen_flag_[seqs[k]] = 0;
  for (int32_t b : touched_) rc_delta_[b] = 0;
  touched_.clear();
  if (bad != kOk) return fail(err, bad, why);
  if (need > static_cast<int64_t>(free_.size()))
    return fail(err, kNoMem, "not enough free blocks for this append");

  for (int i = 0; i < n_seq; ++i) {
    const int s = seqs[i];
    std::vector<int32_t>& tab = tables_[s];
    for (int k = 0; k < n_tok[i]; ++k) {
      const int t = len_[s];
      const int off = t % kBlock;
      if (off == 0) {
        tab.push_back(pop());
        mark_entry(s, static_cast<int>(tab.size()) - 1);
      } else if (rc_[tab.back()] > 1) {
        const int32_t old = tab.back();
        const int32_t fresh = pop();
        cows->push_back({old, fresh, off});
        release(old);
        tab.back() = fresh;
        mark_entry(s, static_cast<int>(tab.size()) - 1);
      }
      slots->push_back(tab.back() * kBlock + off);
      len_[s] = t + 1;
    }
    if (n_tok[i] > 0) mark_len(s);
  }
  return kOk;
}

int BlockPool::truncate(int seq, int new_len, std::string* err) {
  if (!live(seq)) return fail(err, kInvalid, "sequence is not live");
  if (new_len < 0 || new_len > len_[seq]) return fail(err, kInvalid, "new_len outside [0, length]");
  const size_t keep = static_cast<size_t>((new_len + kBlock - 1) / kBlock);
  std::vector<int32_t>& tab = tables_[seq];
  for (size_t j = keep; j < tab.size(); ++j) release(tab[j]);
  tab.resize(keep);
  len_[seq] = new_len;
  mark_len(seq);
  return kOk;
}

int BlockPool::free_seq(int seq, std::string* err) {
  int rc = truncate(seq, 0, err);
  if (rc != kOk) return rc;
  len_[seq] = -1;
  mark_len(seq);
  return kOk;
}

// ---- prefix cache -----------------------------------------------------------

namespace {

uint64_t prefix_key(int32_t parent, const int32_t* tok) {
  uint64_t h = 1469598103934665603ull;  // FNV-1a, 64 bits
  auto mix = [&h](uint32_t v) {
    for (int b = 0; b < 4; ++b) {
      h ^= (v >> (8 * b)) & 0xFFu;
      h *= 1099511628211ull;
    }
  };
  mix(static_cast<uint32_t>(parent));
  for (int i = 0; i < kBlock; ++i) mix(static_cast<uint32_t>(tok[i]));
  return h;
}

}  // namespace

int32_t BlockPool::prefix_find(int32_t parent, const int32_t* tok) const {
  const auto range = pindex_.equal_range(prefix_key(parent, tok));
  for (auto it = range.first; it != range.second; ++it) {
    const PrefixEntry& e = pentries_[it->second];
    if (e.parent == parent && std::equal(tok, tok + kBlock, e.tok)) return it->second;
  }
  return -1;
}

void BlockPool::prefix_touch(int32_t id, uint64_t clock) {
  PrefixEntry& e = pentries_[id];
  if (e.children == 0) {
    pleaves_.erase({e.last, e.order, id});
    pleaves_.insert({clock, e.order, id});
  }
  e.last = clock;
}

int BlockPool::prefix_insert(int seq, const int32_t* tokens, int n_tokens, int* n_new, std::string* err) {
  if (!live(seq)) return fail(err, kInvalid, "prefix insert from a sequence that is not live");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(err, kInvalid, "bad token array");
  const int nb = std::min(n_tokens, len_[seq]) / kBlock;
  const std::vector<int32_t>& tab = tables_[seq];
  const uint64_t clock = ++pclock_;
  int added = 0;
  int32_t parent = -1;
  for (int j = 0; j < nb; ++j) {
    const int32_t* tok = tokens + j * kBlock;
    int32_t id = prefix_find(parent, tok);
    if (id < 0) {
      if (pfree_ids_.empty()) {
        id = static_cast<int32_t>(pentries_.size());
        pentries_.emplace_back();
      } else {
        id = pfree_ids_.back();
        pfree_ids_.pop_back();
      }
      PrefixEntry& e = pentries_[id];
      e.parent = parent;
      e.block = tab[j];
      e.children = 0;
      e.last = clock;
      e.order = porder_++;
      std::copy(tok, tok + kBlock, e.tok);
      pindex_.insert({prefix_key(parent, tok), id});
      pleaves_.insert({clock, e.order, id});
      if (parent >= 0) {
        PrefixEntry& pe = pentries_[parent];
        if (pe.children++ == 0) pleaves_.erase({pe.last, pe.order, parent});
      }
      if (++rc_[e.block] == 2) ++num_shared_;
      ++added;
    } else {
      prefix_touch(id, clock);
    }
    parent = id;
  }
  if (n_new) *n_new = added;
  return kOk;
}

int BlockPool::prefix_match(const int32_t* tokens, int n_tokens) const {
  if (n_tokens <= 0 || !tokens) return 0;
  int m = 0;
  int32_t parent = -1;
  while ((m + 1) * kBlock <= n_tokens && m < max_blocks_) {
    const int32_t id = prefix_find(parent, tokens + m * kBlock);
    if (id < 0) break;
    parent = id;
    ++m;
  }
  return m * kBlock;
}

int BlockPool::alloc_from_prefix(int seq, const int32_t* tokens, int n_tokens, int* n_matched,
                                 std::string* err) {
  if (seq < 0 || seq >= max_seqs_) return fail(err, kInvalid, "seq id out of range");
  if (len_[seq] >= 0) return fail(err, kInvalid, "seq id already live");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(err, kInvalid, "bad token array");
  const int m = prefix_match(tokens, n_tokens);
  const uint64_t clock = ++pclock_;
  tables_[seq].clear();
  int32_t parent = -1;
  for (int j = 0; j < m / kBlock; ++j) {
    const int32_t id = prefix_find(parent, tokens + j * kBlock);
    prefix_touch(id, clock);
    const int32_t b = pentries_[id].block;
    tables_[seq].push_back(b);
    if (++rc_[b] == 2) ++num_shared_;
    mark_entry(seq, j);
    parent = id;
  }
  len_[seq] = m;
  mark_len(seq);
  if (n_matched) *n_matched = m;
  return kOk;
}

int BlockPool::prefix_evict(int max_entries, int* n_evicted, std::string* err) {
  if (max_entries < 0) return fail(err, kInvalid, "max_entries < 0");
  int done = 0;
  while (done < max_entries && !pleaves_.empty()) {
    const int32_t id = std::get<2>(*pleaves_.begin());
    pleaves_.erase(pleaves_.begin());
    PrefixEntry& e = pentries_[id];
    const auto range = pindex_.equal_range(prefix_key(e.parent, e.tok));
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == id) {
        pindex_.erase(it);
        break;
      }
    release(e.block);
    if (e.parent >= 0) {
      PrefixEntry& pe = pentries_[e.parent];
      if (--pe.children == 0) pleaves_.insert({pe.last, pe.order, e.parent});
    }
    pfree_ids_.push_back(id);
    ++done;
  }
  if (n_evicted) *n_evicted = done;
  return kOk;
}

void BlockPool::take_dirty(Dirty* out) {
  out->table_idx.clear();
  out->table_val.clear();
  out->len_seq.clear();
  out->len_val.clear();
  for (int32_t f : dirty_entry_list_) {
    entry_flag_[f] = 0;
    const int s = f / max_blocks_;
    const int j = f % max_blocks_;
    if (len_[s] < 0 || j >= static_cast<int>(tables_[s].size())) continue;  // no longer used
    out->table_idx.push_back(f);
    out->table_val.push_back(tables_[s][j]);
  }
  for (int32_t s : dirty_len_list_) {
    len_flag_[s] = 0;
    out->len_seq.push_back(s);
    out->len_val.push_back(len_[s] < 0 ? 0 : len_[s]);
  }
  dirty_entry_list_.clear();
  dirty_len_list_.clear();
}

}  // namespace pa
