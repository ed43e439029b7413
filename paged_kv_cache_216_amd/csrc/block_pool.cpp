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
