// Replays a call trace on a host-only pool through the C ABI (include/pa.h)
// and prints every call's status (and value), then the allocator state.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitized.py, which compares the output with the oracle's
// block-pool and prefix-cache models on the same trace.
//
// Input, one call per line:
//   pool NB MAX_SEQS MAX_BLOCKS N f_0 .. f_{N-1}   (free order; N = 0: identity)
//   alloc SEQ PARENT SHARED
//   append K s_1 .. s_K n_1 .. n_K
//   truncate SEQ LEN
//   truncate_batch K s_1 .. s_K l_1 .. l_K
//   free SEQ
//   pinsert SEQ N t_1 .. t_N          pmatch N t_1 .. t_N
//   palloc SEQ N t_1 .. t_N           pevict K
//   dump
// Output: "s STATUS [VALUE]" per call; dump prints "free ...", "rc ...",
// "seq S LEN b_0 ..." for live sequences and "entries E".
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pa.h"

namespace {

std::vector<int32_t> read_ints(std::istringstream& in, int n) {
  std::vector<int32_t> v(static_cast<size_t>(n > 0 ? n : 0));
  for (auto& x : v) in >> x;
  return v;
}

void dump(pa_pool* p, int num_blocks, int max_seqs, int max_blocks) {
  int n = 0;
  pa_get_free_list(p, nullptr, 0, &n);
  std::vector<int32_t> f(static_cast<size_t>(n) + 1);
  pa_get_free_list(p, f.data(), n, &n);
  std::printf("free");
  for (int i = 0; i < n; ++i) std::printf(" %d", f[i]);
  std::printf("\nrc");
  for (int b = 0; b < num_blocks; ++b) {
    int rc = 0;
    pa_get_refcount(p, b, &rc);
    std::printf(" %d", rc);
  }
  std::printf("\n");
  std::vector<int32_t> tab(static_cast<size_t>(max_blocks) + 1);
  for (int s = 0; s < max_seqs; ++s) {
    int nb = 0, len = 0;
    if (pa_get_block_table(p, s, tab.data(), max_blocks, &nb, &len) != PA_OK) continue;
    std::printf("seq %d %d", s, len);
    for (int j = 0; j < nb; ++j) std::printf(" %d", tab[j]);
    std::printf("\n");
  }
  int e = 0;
  pa_prefix_entries(p, &e);
  std::printf("entries %d\n", e);
}

}  // namespace

int main() {
  pa_pool* pool = nullptr;
  int num_blocks = 0, max_seqs = 0, max_blocks = 0;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    if (!(in >> op)) continue;
    if (op == "pool") {
      int n = 0;
      in >> num_blocks >> max_seqs >> max_blocks >> n;
      const std::vector<int32_t> order = read_ints(in, n);
      if (pool) pa_destroy_pool(pool);
      pool = nullptr;
      const int rc = pa_create_pool(&pool, num_blocks, 16, 1, 64, PA_BF16, nullptr, nullptr, nullptr, nullptr,
                                    max_seqs, max_blocks, n ? order.data() : nullptr);
      std::printf("s %d\n", rc);
    } else if (op == "alloc") {
      int s = 0, parent = 0, shared = 0;
      in >> s >> parent >> shared;
      std::printf("s %d\n", pa_alloc_blocks(pool, s, parent, shared));
    } else if (op == "append") {
      int k = 0;
      in >> k;
      const std::vector<int32_t> seqs = read_ints(in, k), ntok = read_ints(in, k);
      std::printf("s %d\n", pa_append_kv(pool, seqs.data(), k, ntok.data(), nullptr, nullptr, nullptr));
    } else if (op == "truncate") {
      int s = 0, len = 0;
      in >> s >> len;
      std::printf("s %d\n", pa_truncate(pool, s, len));
    } else if (op == "truncate_batch") {
      int k = 0;
      in >> k;
      const std::vector<int32_t> seqs = read_ints(in, k), lens = read_ints(in, k);
      std::printf("s %d\n", pa_truncate_batch(pool, seqs.data(), k, lens.data()));
    } else if (op == "free") {
      int s = 0;
      in >> s;
      std::printf("s %d\n", pa_free_seq(pool, s));
    } else if (op == "pinsert" || op == "palloc") {
      int s = 0, n = 0, out = -1;
      in >> s >> n;
      const std::vector<int32_t> t = read_ints(in, n);
      const int rc = op == "pinsert" ? pa_prefix_insert(pool, s, t.data(), n, &out)
                                     : pa_alloc_from_prefix(pool, s, t.data(), n, &out);
      std::printf("s %d %d\n", rc, rc == PA_OK ? out : -1);
    } else if (op == "pmatch") {
      int n = 0, out = -1;
      in >> n;
      const std::vector<int32_t> t = read_ints(in, n);
      const int rc = pa_prefix_match(pool, t.data(), n, &out);
      std::printf("s %d %d\n", rc, rc == PA_OK ? out : -1);
    } else if (op == "pevict") {
      int k = 0, out = -1;
      in >> k;
      const int rc = pa_prefix_evict(pool, k, &out);
      std::printf("s %d %d\n", rc, rc == PA_OK ? out : -1);
    } else if (op == "dump") {
      dump(pool, num_blocks, max_seqs, max_blocks);
    } else {
      std::fprintf(stderr, "unknown op %s\n", op.c_str());
      return 2;
    }
  }
  if (pool) pa_destroy_pool(pool);
  return 0;
}
