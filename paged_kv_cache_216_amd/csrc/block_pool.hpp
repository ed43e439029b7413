// Host-side block allocator for the paged KV cache: free deque, per-block
// reference counts, per-sequence block tables and lengths, copy-on-write
// decisions, and the list of device-table entries that changed.
//
// Rules (the pages fix the first three; the rest is this library's reading):
//  - fixed 16-token blocks placed anywhere, reached through a per-sequence table
//    ("PagedAttention, décodage spéculatif, MoE et Blackwell", section 1);
//  - only the blocks a sequence needs are taken (kenji.blog
//    "llm-inference-optimization-kv-cache", section 4.2);
//  - sequences from one prompt share blocks, copied on write (same sections);
//  - free list = deque in a caller-given order, pop front, push back on release
//    in increasing logical order; copy is lazy, on the first write into a block
//    referenced more than once, and takes the slots already filled; sequences of
//    one append are served in call order, token by token; an append that cannot
//    get all the blocks it needs changes nothing.
#pragma once

#include <cstdint>
#include <deque>
#include <set>
#include <string>
#include <tuple>
#include <unordered_map>
#include <vector>

namespace pa {

constexpr int kBlock = 16;

enum Status : int { kOk = 0, kInvalid = -1, kNoMem = -2, kHip = -3, kState = -4 };

struct CowCopy {
  int32_t src;
  int32_t dst;
  int32_t rows;  // slots [0, rows) are copied
};

class BlockPool {
 public:
  int init(int num_blocks, int max_seqs, int max_blocks_per_seq, const int32_t* free_order,
           std::string* err);

  int alloc(int seq, int parent, int shared_tokens, std::string* err);
  // On success appends one slot (phys * 16 + offset) per row, in call order, to
  // *slots, and the copies to perform before the rows are written to *cows.
  int append(const int32_t* seqs, int n_seq, const int32_t* n_tok, std::vector<int32_t>* slots,
             std::vector<CowCopy>* cows, std::string* err);
  int truncate(int seq, int new_len, std::string* err);
  int free_seq(int seq, std::string* err);

  // Prefix cache: whole blocks registered under the token ids of the prompt up
  // to the end of the block (a chain of (parent entry, 16 tokens) keys), each
  // holding one reference on its block.  Reuse runs from the first block to the
  // first block whose tokens differ ("Mettre en cache" on the ranksignal.fr
  // page).  Inserts and reuses tick a clock; eviction drops entries no other
  // entry extends, least recently used first, ties to the oldest entry.
  int prefix_insert(int seq, const int32_t* tokens, int n_tokens, int* n_new, std::string* err);
  int prefix_match(const int32_t* tokens, int n_tokens) const;  // matched tokens
  int alloc_from_prefix(int seq, const int32_t* tokens, int n_tokens, int* n_matched, std::string* err);
  int prefix_evict(int max_entries, int* n_evicted, std::string* err);
  int prefix_entries() const { return static_cast<int>(pindex_.size()); }

  bool live(int seq) const { return seq >= 0 && seq < max_seqs_ && len_[seq] >= 0; }
  int length(int seq) const { return len_[seq]; }
  const std::vector<int32_t>& table(int seq) const { return tables_[seq]; }
  int refcount(int block) const { return rc_[block]; }
  int num_free() const { return static_cast<int>(free_.size()); }
  // blocks referenced by more than one sequence
  int num_shared() const { return num_shared_; }
  const std::deque<int32_t>& free_list() const { return free_; }
  int num_blocks() const { return num_blocks_; }
  int max_seqs() const { return max_seqs_; }
  int max_blocks_per_seq() const { return max_blocks_; }

  // Device-mirror bookkeeping: table entries (seq * max_blocks + j) and
  // sequences whose device copy is stale.  take_dirty() returns them and clears
  // the marks.  Flags plus lists keep marking and collecting O(1) per item.
  struct Dirty {
    std::vector<int32_t> table_idx;    // flat indices into the device table
    std::vector<int32_t> table_val;    // their current values
    std::vector<int32_t> len_seq;      // sequences whose length changed
    std::vector<int32_t> len_val;      // current length (0 if not live)
  };
  bool has_dirty() const { return !dirty_entry_list_.empty() || !dirty_len_list_.empty(); }
  void take_dirty(Dirty* out);
  size_t dirty_entries() const { return dirty_entry_list_.size(); }
  size_t dirty_lens() const { return dirty_len_list_.size(); }

 private:
  int32_t pop();
  void release(int32_t b);
  void mark_entry(int seq, int j) {
    const int32_t f = seq * max_blocks_ + j;
    if (!entry_flag_[f]) {
      entry_flag_[f] = 1;
      dirty_entry_list_.push_back(f);
    }
  }
  void mark_len(int seq) {
    if (!len_flag_[seq]) {
      len_flag_[seq] = 1;
      dirty_len_list_.push_back(seq);
    }
  }

  int num_blocks_ = 0;
  int max_seqs_ = 0;
  int max_blocks_ = 0;
  std::deque<int32_t> free_;
  std::vector<int32_t> rc_;
  std::vector<std::vector<int32_t>> tables_;
  std::vector<int32_t> len_;  // -1 = not live
  std::vector<uint8_t> entry_flag_, len_flag_, seen_flag_;
  std::vector<int32_t> dirty_entry_list_, dirty_len_list_;
  std::vector<int32_t> rc_delta_, touched_;
  int num_shared_ = 0;

  struct PrefixEntry {
    int32_t parent;    // entry of the previous block, -1 for a prompt's first block
    int32_t block;
    int32_t children;  // entries that extend this one
    uint64_t last;     // clock of the last insert / reuse through it
    int64_t order;     // registration order
    int32_t tok[kBlock];
  };
  int32_t prefix_find(int32_t parent, const int32_t* tok) const;
  void prefix_touch(int32_t id, uint64_t clock);
  std::vector<PrefixEntry> pentries_;
  std::vector<int32_t> pfree_ids_;                      // reusable entry slots
  std::unordered_multimap<uint64_t, int32_t> pindex_;   // key hash -> entry
  std::set<std::tuple<uint64_t, int64_t, int32_t>> pleaves_;  // (last, order, entry) of leaves
  uint64_t pclock_ = 0;
  int64_t porder_ = 0;
};

}  // namespace pa
