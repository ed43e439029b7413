"""CPU oracle for paged KV-cache attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 numpy code that states what the GPU path
must compute.  Only the tests, the smoke check and the bench's CPU-baseline leg
may import it.  It shares no code with the GPU package (``paged_kv_cache_216_amd``)
and imports nothing from it; the product path never calls it.

Modules
  numerics    decode stored element bits (fp32 / fp16 / bf16) to float64
  layout      where row (block, head, slot) of K and V lives in the physical pool
  allocator   block pool model: free deque, reference counts, block tables,
              copy-on-write, and the pool bytes an append must produce
  attention   gather through the block table + textbook softmax attention
              (decode and causal K-draft verify), with log-sum-exp
  accounting  the byte formulas the pages print (KV size, fragmentation,
              bandwidth-bound decode ceiling)

Source pages (cited by title and section):
  [P1] "PagedAttention, décodage spéculatif, MoE et Blackwell", section 1
  [P2] kenji.blog "llm-inference-optimization-kv-cache" (first heading:
       "Introduction : le « mur invisible » de l'inférence des LLM"),
       sections 2.3, 3.1, 3.2, 4, 4.1, 4.2, 5.2
  [P3] "CUDA Graphs, modèles de raisonnement et service désagrégé", section 3
  [P4] ranksignal.fr post 218, "Les noyaux d'attention : lire et écrire moins"
       and "Spéculer : plusieurs tokens par passe"

Parity status: every function here is pinned by tests in tests/test_oracle_*.py
against closed forms, invariants, a library attention routine and brute force.
Nothing is "parity unpinned" except the exact floating-point rounding order of
the GPU kernels, which the stated tolerances cover.
"""
