/*
 * pa.h — paged KV-cache attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * What the library does, and where the pages define it:
 *   - Each sequence's key/value cache is cut into fixed blocks of 16 tokens that
 *     may sit anywhere in one physical pool; a per-sequence block table maps
 *     logical blocks to physical ones and is resolved inside the attention
 *     kernel ("PagedAttention, décodage spéculatif, MoE et Blackwell", section 1;
 *     kenji.blog "llm-inference-optimization-kv-cache", section 4.1).
 *   - Sequences that derive from the same prompt share physical blocks, copied
 *     only when written (same page, section 1; kenji.blog page, section 4.2).
 *   - A decode step stores the new token's K and V rows in the cache, then the
 *     token's query attends over the whole cache (kenji.blog page, section 3.1
 *     and its data-flow graph), a step bound by memory bandwidth because it
 *     reads the entire cache ("CUDA Graphs, modèles de raisonnement et service
 *     désagrégé", section 3 table).
 *   - Speculative verify: K draft tokens are checked in one pass; after a
 *     rejection the cache is cut back to the accepted prefix (kenji.blog page,
 *     section 5.2; ranksignal.fr post 218, "Spéculer").
 *
 * Conventions for every function:
 *   - Return PA_OK (0) or a negative pa_status.  No C++ exception crosses the ABI.
 *     On any error the pool is left unchanged.  pa_last_error() gives a message
 *     for the calling thread's most recent failure.
 *   - "host" pointers are CPU memory read during the call only; "device"
 *     pointers are GPU memory owned by the caller, which must stay valid until
 *     the work enqueued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is asynchronous on that stream.  Calls on one pool must be
 *     ordered: issue them from one thread, on one stream (or synchronise).
 *   - A pool is not thread-safe.
 *
 * Physical layout (caller allocates; bit patterns are the contract):
 *   element size e = 4 (PA_F32), 2 (PA_F16, PA_BF16) or 1 (PA_FP8_E4M3);
 *   X = 16 / e
 *   K pool: [num_blocks][num_kv_heads][head_dim / X][16][X]
 *   V pool: [num_blocks][num_kv_heads][head_dim][16]
 *   so one (block, head) K or V page is 16 * head_dim * e contiguous bytes,
 *   K stored in 16-byte chunks of X consecutive dims, slot-minor; V stored
 *   dim-major with the 16 slots of one dim contiguous.
 *   block_table_dev: int32 [max_seqs][max_blocks_per_seq]; entries
 *   [0, ceil(len/16)) of a live sequence hold its physical blocks, others are
 *   unspecified.  seq_len_dev: int32 [max_seqs], the length of each live
 *   sequence, 0 for others.  Both mirrors are brought up to date by every
 *   device call (pa_append_kv, pa_decode, pa_verify, pa_sync_tables).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_pool pa_pool;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1, /* bad argument or unknown / duplicate sequence            */
  PA_ERR_NOMEM = -2,   /* not enough free blocks (nothing was changed)            */
  PA_ERR_HIP = -3,     /* a HIP runtime call or kernel launch failed              */
  PA_ERR_STATE = -4    /* call not possible in this pool's state (e.g. host-only) */
} pa_status;

/* PA_FP8_E4M3: the pools hold one-byte E4M3 codes (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; no infinities; largest finite value 448),
 * one scale per (K or V, kv head) (pa_set_kv_scales).  Rows appended, queries
 * and outputs are bf16.  The stored code of an element x of key/value head h
 * is E4M3(x * r) with r = 1.0f / scale[h] in float32: the product is rounded
 * to float32, clamped to [-448, 448] and rounded to the nearest code, ties to
 * the even code; the attention uses decode(code) * scale[h], in fp32.  An
 * 8-bit cache halves the bytes a decode step reads while the softmax stays at
 * full precision (ranksignal.fr post 218, "Quantifier"). */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Create a pool over caller-owned device memory: the physical pool of
 * fixed-size blocks that every sequence's cache is cut into, each block placed
 * anywhere in it ("PagedAttention, décodage spéculatif, MoE et Blackwell",
 * section 1; kenji.blog "llm-inference-optimization-kv-cache", section 4.1).
 *   num_blocks      physical blocks in k_pool / v_pool (> 0)
 *   block_size      tokens per block; must be 16
 *   num_kv_heads    key/value heads per block (> 0)
 *   head_dim        64, 128 or 256
 *   dtype           pa_dtype of K, V, Q and outputs
 *   k_pool, v_pool  device, sized as in the layout above
 *   block_table_dev device int32 [max_seqs * max_blocks_per_seq]
 *   seq_len_dev     device int32 [max_seqs]
 *   free_order      host int32 [num_blocks], a permutation of 0..num_blocks-1
 *                   giving the order in which blocks are handed out; NULL
 *                   means 0, 1, 2, ...
 * If all four device pointers are NULL the pool is host-only: it keeps the
 * block tables but enqueues no device work (pa_append_kv then takes NULL rows;
 * pa_decode / pa_verify return PA_ERR_STATE).
 * The library allocates, for the pool's lifetime, a ring of pinned host
 * buffers that the kernels read per-call metadata from, and three small
 * device buffers: the attention work plan, the counters of the in-launch
 * merge (zero between launches), and the E4M3 scales once set; it never
 * allocates pool memory.  The plan and the counters grow (a device-wide
 * synchronisation) when a call needs more than any call before. */
int pa_create_pool(pa_pool** out, int num_blocks, int block_size, int num_kv_heads,
                   int head_dim, int dtype, void* k_pool, void* v_pool,
                   int32_t* block_table_dev, int32_t* seq_len_dev, int max_seqs,
                   int max_blocks_per_seq, const int32_t* free_order);

/* Waits for the pool's outstanding metadata copies, then frees the library's
 * own buffers.  Caller memory is not touched.  NULL is accepted. */
int pa_destroy_pool(pa_pool* pool);

/* Start sequence seq_id (0 <= seq_id < max_seqs, not live), holding no
 * block until its first append: only the blocks a sequence needs are taken
 * (kenji.blog "llm-inference-optimization-kv-cache", section 4.2).  With
 * parent_seq >= 0 (live, != seq_id) the new sequence shares the parent's first
 * ceil(shared_tokens / 16) blocks (reference counts + 1) and starts with
 * length shared_tokens (0 <= shared_tokens <= parent length): copy-on-write
 * fork: sequences derived from one prompt point at the same physical blocks
 * and a block is copied only when written ("PagedAttention, décodage
 * spéculatif, MoE et Blackwell", section 1; kenji.blog page, section 4.2).
 * With parent_seq < 0, shared_tokens must be 0.  Host-side only; the device
 * table rows are written by the next device call.  Errors: PA_ERR_INVALID
 * for an id out of range or live, a parent not live or shared_tokens out of
 * range; nothing changes. */
int pa_alloc_blocks(pa_pool* pool, int seq_id, int parent_seq, int shared_tokens);

/* Block swap to host memory.  When GPU memory runs short, a KV cache can move
 * blocks to slower tiers and bring them back when needed; host RAM is the
 * tier after GPU memory (ranksignal.fr post 218, "Mettre en cache", tiers
 * G1 and G2).  The host images are caller-owned pinned host memory
 * (hipHostMalloc, or a pinned torch tensor), one for K and one for V, each
 * [ceil(length / 16)][num_kv_heads x 16 x head_dim elements]: every block in
 * the pool's own layout, in logical order.  pa_swap_bytes gives the bytes of
 * one image for n_tokens tokens.  The copies run on `stream` (one kernel
 * reading or writing the host images over the bus); the host images must stay
 * valid, and work on other streams must wait for `stream`, until they finish.
 *
 * pa_swap_out: copy live sequence seq_id's blocks into the images, then end
 *   the sequence as pa_free_seq does (its blocks lose one reference; shared
 *   blocks stay with their other holders).  *length (may be NULL) = its
 *   length, which pa_swap_in takes back.
 * pa_swap_in: start seq_id (in range, not live) with `length` rows taken from
 *   the images: the blocks are popped from the free list as an append of
 *   `length` rows would pop them (PA_ERR_NOMEM, changing nothing, if there are
 *   too few); slots past `length` in the last block are not written.
 * Errors: PA_ERR_INVALID for bad ids, short or unpinned buffers;
 * PA_ERR_STATE for host-only pools. */
int pa_swap_bytes(const pa_pool* pool, int n_tokens, size_t* bytes);
int pa_swap_out(pa_pool* pool, int seq_id, void* k_host, void* v_host, size_t bytes, int* length,
                void* stream);
int pa_swap_in(pa_pool* pool, int seq_id, int length, const void* k_host, const void* v_host, size_t bytes,
               void* stream);

/* Prefix cache.  A later prompt that starts with the same tokens as an earlier
 * one can reuse that prompt's cached K/V instead of recomputing it; the reuse
 * runs from the first token up to the first token that differs, never past it
 * (ranksignal.fr post 218, "Mettre en cache"; blocks shared copy-on-write:
 * "PagedAttention, décodage spéculatif, MoE et Blackwell", section 1).  Here
 * the unit of reuse is a whole 16-token block: block j is reused when tokens
 * [0, 16 (j + 1)) all agree.  tokens are host int32 token ids, caller-defined;
 * the library trusts that they name the rows the sequence holds.  Host-side
 * only: device tables are written by the next device call.
 *
 * pa_prefix_insert: register the full blocks among the first
 *   min(n_tokens, length) tokens of live sequence seq_id that are not
 *   registered yet; each one gains a reference held by the cache (so it
 *   outlives the sequence).  *n_new (may be NULL) = blocks newly registered.
 * pa_prefix_match: *n_matched = tokens (a multiple of 16) at the start of
 *   tokens[0, n_tokens) held by registered blocks.  Changes nothing.
 * pa_alloc_from_prefix: start sequence seq_id (in range, not live) sharing the
 *   matched blocks (one more reference each), with length *n_matched (may be
 *   NULL); the caller appends the rest of the prompt.  A later write into a
 *   reused block is copied first, as for any shared block.
 * pa_prefix_evict: drop up to max_entries entries, one at a time, always one
 *   that no other entry extends, least recently used first (inserts and
 *   reuses mark the entries they pass), ties to the oldest; blocks left
 *   unreferenced go to the back of the free list.  *n_evicted may be NULL.
 *   The library never evicts by itself: on PA_ERR_NOMEM the caller may evict
 *   and retry.
 * pa_prefix_entries: *n = registered blocks. */
int pa_prefix_insert(pa_pool* pool, int seq_id, const int32_t* tokens, int n_tokens, int* n_new);
int pa_prefix_match(const pa_pool* pool, const int32_t* tokens, int n_tokens, int* n_matched);
int pa_alloc_from_prefix(pa_pool* pool, int seq_id, const int32_t* tokens, int n_tokens, int* n_matched);
int pa_prefix_evict(pa_pool* pool, int max_entries, int* n_evicted);
int pa_prefix_entries(const pa_pool* pool, int* n);

/* Scales of a PA_FP8_E4M3 pool, one per kv head: host float arrays
 * [num_kv_heads], finite and > 0 (default 1.0).  Codes already stored are
 * not rewritten: set the scales before the first append.  Synchronous.
 * PA_ERR_STATE for pools of other dtypes. */
int pa_set_kv_scales(pa_pool* pool, const float* k_scale, const float* v_scale);

/* Append n_tok[i] new K/V rows to sequence seq_ids[i], i = 0..n_seq-1: the
 * key and value of every new token are stored in the cache, so that later
 * steps read them instead of recomputing them (kenji.blog
 * "llm-inference-optimization-kv-cache", section 3.1 and its data-flow graph);
 * a sequence takes a new block only when its last one is full (same page,
 * section 4.2).
 *   seq_ids, n_tok  host int32 [n_seq]; sequences live and distinct;
 *                   n_tok[i] >= 0; length + n_tok[i] <= 16 * max_blocks_per_seq
 *   k_new, v_new    device [sum(n_tok)][num_kv_heads][head_dim] in dtype, rows
 *                   packed in call order
 * Blocks are taken from the front of the free list, sequence by sequence,
 * token by token.  Writing into a block that other sequences still reference
 * first copies its filled slots into a fresh block (copy-on-write).  Fails
 * with PA_ERR_NOMEM, changing nothing, if the free list cannot cover the
 * call.  Stored bytes are bit-exact copies of the input rows. */
int pa_append_kv(pa_pool* pool, const int32_t* seq_ids, int n_seq, const int32_t* n_tok,
                 const void* k_new, const void* v_new, void* stream);

/* One query token per sequence attends over all of its cached tokens.
 *   seq_ids      host int32 [n_seq]; live, length >= 1 (repeats allowed)
 *   num_q_heads  multiple of num_kv_heads; query head h reads key/value head
 *                h / (num_q_heads / num_kv_heads)
 *   scale        multiplies q.k before the softmax (typically 1/sqrt(head_dim));
 *                finite and > 0, else PA_ERR_INVALID (the same for every
 *                attention call below)
 *   q, out       device [n_seq][num_q_heads][head_dim] in dtype
 *   lse          device float [n_seq][num_q_heads] (natural-log log-sum-exp of
 *                the scaled scores) or NULL
 *   partition_tokens  0 = library choice (512 tokens, or 8 per query row
 *                of a kv head when that is more; for calls with shared
 *                prefixes (below) a longer one, up to twice that, when it
 *                lets the shared-prefix launch run in fewer rounds of
 *                resident workgroups -- never more workspace than the
 *                default needs); otherwise a positive
 *                multiple of 32: contexts longer than this are cut into
 *                partitions processed in parallel and merged exactly by their
 *                log-sum-exp; a value >= the longest context disables the
 *                split.  Partition q covers [q * pt, (q + 1) * pt) and the last
 *                one runs to the end of the sequence; when the call has at most
 *                16 query rows per kv head, a context of up to 1.25 * pt tokens
 *                stays unsplit and the last partition absorbs a remainder of
 *                up to pt / 4 tokens (so no partition is a handful of tokens)
 *   workspace    device scratch for split partials, ws_bytes long (see
 *                pa_workspace_size); may be NULL when no sequence is split.
 *                With partition_tokens = 0 the library only splits when the
 *                workspace is large enough.
 * Shared prefixes: when at least 4 sequences of the call are copy-on-write
 * forks that hold at least one whole partition in the same physical blocks
 * (positions every query row sees), the whole shared prefix is computed once
 * for the query rows of all of them -- inside the attention launch, followed
 * by a launch that merges the splits, when one unit takes all query rows of a
 * (sequence, kv head) and no sequence has more than 16 partitions; else in a
 * launch before the attention launch -- so the shared blocks are read once
 * per call instead of once per sequence (blocks
 * shared by sequences of one prompt: "PagedAttention, décodage spéculatif,
 * MoE et Blackwell", section 1; kenji.blog page, section 4.2; reusing the KV
 * cache of a common prefix: ranksignal.fr post 218, "Mettre en cache").
 * Needs the split (a workspace) and a 16-bit or E4M3 pool.  Results equal the
 * per-sequence computation up to floating-point summation order.
 * Softmax and accumulation are fp32; out is rounded to dtype (nearest even).
 * Graph capture: engines replay a recorded launch sequence instead of
 * launching kernel by kernel ("CUDA Graphs, modèles de raisonnement et service
 * désagrégé", section 1).  A pa_decode / pa_verify call can be captured into
 * a HIP graph on `stream` when it runs unsplit (workspace NULL), the same call
 * (same sequences, num_q_heads, k_draft) has run once before so that its work
 * plan is on the device, and the device tables are current (pa_sync_tables).
 * Each replay then reads the lengths and block tables current at replay time,
 * so appends made eagerly between replays are seen.  The pool holds one work
 * plan: an attention call with other sequences between the capture and a
 * replay invalidates the graph.  Calls that append (pa_append_kv,
 * pa_append_attend) pass their rows and slots as launch arguments and cannot
 * be replayed. */
int pa_decode(pa_pool* pool, const int32_t* seq_ids, int n_seq, int num_q_heads, float scale,
              const void* q, void* out, float* lse, int partition_tokens, void* workspace,
              size_t ws_bytes, void* stream);

/* pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as pa_decode (bitwise), without the workspace: the
 * work plan, the in-launch merge counters and the split partials live in a
 * fixed device array of 32 MiB per GPU, [0, 64 KiB) counters, [64 KiB,
 * 1 MiB) plan, [1 MiB, 32 MiB) partials, that the library holds on every GPU
 * it runs on until the process ends.  The call allocates nothing (no
 * hipMalloc, no pinned staging, no profiling events) and copies nothing from
 * the host: the plan and pending table updates travel in kernel arguments.
 * partition_tokens = 0 splits only when the partials fit the array; an
 * explicit partition whose partials do not fit, a plan past 960 KiB or more
 * than 16,384 (split sequence, kv head) merge counters return PA_ERR_INVALID
 * before any launch.  Every call on one GPU shares that GPU's array (it keeps
 * the last call's contents; the counters a call uses are zeroed by the call):
 * calls that overlap on one GPU -- on different streams, or from different
 * pools on different streams -- race, and must be ordered by the caller. */
int pa_decode_noalloc(pa_pool* pool, const int32_t* seq_ids, int n_seq, int num_q_heads, float scale,
                      const void* q, void* out, float* lse, int partition_tokens, void* stream);

/* Speculative verify: the last k_draft rows of each sequence are draft tokens
 * (already appended) and draft i (0-based) attends to positions
 * [0, length - k_draft + i], its own row included (speculative decoding:
 * "PagedAttention, décodage spéculatif, MoE et Blackwell", section 1;
 * kenji.blog "llm-inference-optimization-kv-cache", section 5.2; ranksignal.fr
 * post 218, "Spéculer").
 *   q, out  device [n_seq][k_draft][num_q_heads][head_dim]
 *   lse     device float [n_seq][k_draft][num_q_heads] or NULL
 * Lengths must be >= k_draft; (num_q_heads / num_kv_heads) * k_draft is at
 * most 2^22.  A unit of work takes at most 64 query rows (32 when head_dim is
 * 256); calls with more run one unit per tile of rows, and each tile reads
 * only the positions its last row sees.  Other arguments as pa_decode.
 * k_draft = 1 is exactly pa_decode. */
int pa_verify(pa_pool* pool, const int32_t* seq_ids, int n_seq, int k_draft, int num_q_heads,
              float scale, const void* q, void* out, float* lse, int partition_tokens,
              void* workspace, size_t ws_bytes, void* stream);

/* Chunked prefill: the last n_new rows of each sequence are a chunk of its
 * prompt (already appended, e.g. with pa_append_kv), and chunk token i
 * (0-based) attends to positions [0, length - n_new + i].  Long prompts are
 * split into such chunks so that their attention can run between decode steps
 * (ranksignal.fr post 218, "Les noyaux d'attention", chunked prefill).  The
 * computation is exactly
 * pa_verify with k_draft = n_new; q, out, lse, limits and errors as there.  */
int pa_prefill(pa_pool* pool, const int32_t* seq_ids, int n_seq, int n_new, int num_q_heads,
               float scale, const void* q, void* out, float* lse, int partition_tokens,
               void* workspace, size_t ws_bytes, void* stream);

/* pa_append_kv of n_new rows to each listed sequence followed by pa_verify
 * with k_draft = n_new (n_new = 1: pa_decode), issued as one kernel launch
 * when possible: the launch writes the rows into the pool while the attention
 * takes the new rows straight from k_new / v_new.  Results are identical to
 * the two separate calls.  Falls back to two launches (same results) when a
 * write needs a copy-on-write copy first, when earlier table changes are still
 * pending, when (num_q_heads / num_kv_heads) * n_new is more than one unit's
 * rows (see pa_verify), or for PA_F32 pools.  With PA_FP8_E4M3 pools the
 * attention takes the new rows as the codes the append stores, decoded. 
 *   seq_ids  host int32 [n_seq]; live and distinct
 *   k_new, v_new  device [n_seq * n_new][num_kv_heads][head_dim], rows of
 *            sequence i at i * n_new .. i * n_new + n_new - 1
 *   q, out   device [n_seq][n_new][num_q_heads][head_dim]; lse [n_seq][n_new][num_q_heads] or NULL
 * Other arguments and errors as pa_append_kv and pa_verify; nothing changes
 * on error. */
int pa_append_attend(pa_pool* pool, const int32_t* seq_ids, int n_seq, int n_new, const void* k_new,
                     const void* v_new, int num_q_heads, float scale, const void* q, void* out, float* lse,
                     int partition_tokens, void* workspace, size_t ws_bytes, void* stream);

/* Graph steps.  Serving engines record a step's kernel launches once and
 * replay the recording every step instead of launching kernel by kernel,
 * padding each batch to a few fixed size classes and updating the data the
 * recording points at in place between replays ("CUDA Graphs, modèles de
 * raisonnement et service désagrégé", section 1).  A graph step is the step
 * of pa_append_attend (append n_new rows to each sequence, then attend) split
 * in two:
 *
 * pa_graph_prepare: the step's host bookkeeping and everything that cannot be
 *   replayed, eagerly on `stream` -- pending table changes, and the whole
 *   append when it needs copy-on-write copies -- then small kernels on
 *   `stream` write the step's metadata (lengths, slots of the new rows, table
 *   and length updates) and, when it changed, its work plan into a buffer that
 *   the library keeps for the step's class (allocated on the class's first
 *   prepare).  The
 *   class is the number of work units rounded up to a power of two (at least
 *   16), with n_new: *class_units (may be NULL) returns it.  Arguments as
 *   pa_append_attend, with these limits: 16-bit or E4M3 pools; (num_q_heads /
 *   num_kv_heads) * n_new within one unit's rows (64, 32 at head_dim 256); the
 *   partition is partition_tokens or the library's default, every step, and the
 *   workspace must hold the step's partials (PA_ERR_INVALID otherwise); at most
 *   16 partitions per sequence (PA_ERR_STATE otherwise); no shared-prefix pass.
 *   Results are bitwise those of pa_append_attend with the same partition
 *   (the appended rows too).  On error nothing changes.
 * pa_graph_launch: enqueue the attention + append launch of the last prepared
 *   step on `stream`: one kernel, whose grid is padded to the class (its
 *   workgroups past the step's units and rows have nothing to do) and whose
 *   arguments point only at the class's buffer, the pool and the caller's
 *   buffers.  It can be captured into a HIP graph; a replay after a later
 *   pa_graph_prepare of the same class runs that step.  Replays use the
 *   buffers (q, out, lse, k_new, v_new, workspace) and the scale given to the
 *   prepare before the capture: pass the same ones to every prepare of a
 *   class.  PA_ERR_STATE before any prepare.
 * Ordering: the device's table and length mirrors receive the step's updates
 * only when its launch (or replay) runs, so run it on `stream` after each
 * prepare, before any other call on the pool; replaying an older step after a
 * newer prepare of the same class runs the newer one. */
int pa_graph_prepare(pa_pool* pool, const int32_t* seq_ids, int n_seq, int n_new, const void* k_new,
                     const void* v_new, int num_q_heads, float scale, const void* q, void* out, float* lse,
                     int partition_tokens, void* workspace, size_t ws_bytes, void* stream, int* class_units);
int pa_graph_launch(pa_pool* pool, void* stream);

/* Cut sequence seq_id back to new_len tokens (0 <= new_len <= length), e.g. to
 * drop rejected drafts: after a rejection, generation resumes from the first
 * wrong draft, so the cache keeps only the accepted prefix (kenji.blog
 * "llm-inference-optimization-kv-cache", section 5.2; ranksignal.fr post 218,
 * "Spéculer").  Blocks past ceil(new_len / 16) lose one reference and go to
 * the back of the free list, in logical order, when unreferenced.  Host-side
 * only; PA_ERR_INVALID (nothing changes) for a sequence not live or new_len
 * out of range. */
int pa_truncate(pa_pool* pool, int seq_id, int new_len);

/* pa_truncate for n_seq sequences in one call (host int32 arrays
 * seq_ids[n_seq], new_lens[n_seq]), e.g. rolling a whole batch back to its
 * accepted drafts.  All arguments are checked first; on error nothing changes. */
int pa_truncate_batch(pa_pool* pool, const int32_t* seq_ids, int n_seq, const int32_t* new_lens);

/* End sequence seq_id: pa_truncate to 0, then the id becomes free; its blocks
 * go back to the pool for other sequences, which is what keeps the waste of
 * paging to the unused slots of each sequence's last block (kenji.blog
 * "llm-inference-optimization-kv-cache", section 4.2).  Host-side only;
 * PA_ERR_INVALID for a sequence not live. */
int pa_free_seq(pa_pool* pool, int seq_id);

/* Enqueue the pending block-table / length updates on `stream` now. */
int pa_sync_tables(pa_pool* pool, void* stream);

/* Bytes of workspace that pa_decode / pa_verify need for n_seq sequences of
 * at most max_tokens tokens each with this partition_tokens (0 = the library's
 * choice) and k_draft queries per sequence (1 for decode).  0 if nothing splits.
 * The workspace holds the split-KV partials: each partition of a long context
 * is attended separately, its unnormalised output and (max, sum) kept in
 * fp32, and the partitions are merged exactly by log-sum-exp -- this
 * library's way of running one pass over a long cache in parallel while the
 * scores and probabilities stay on chip and the output is written once
 * (ranksignal.fr post 218, "Les noyaux d'attention").  The figure is an upper
 * bound: it counts ceil(max_tokens / partition_tokens) + 1 partitions per
 * sequence, at least what any call of those sizes uses (a shared-prefix
 * member's own partitions start where the shared prefix ends, which can take
 * one more; a library-chosen partition for shared prefixes is longer, never
 * shorter).  Host-side only; PA_ERR_INVALID for bad sizes. */
int pa_workspace_size(const pa_pool* pool, int n_seq, int num_q_heads, int k_draft,
                      int max_tokens, int partition_tokens, size_t* bytes);

/* Host copies of the allocator state (for tests and schedulers). */
int pa_get_block_table(const pa_pool* pool, int seq_id, int32_t* out, int cap, int* n_blocks,
                       int* len);
int pa_get_refcount(const pa_pool* pool, int block_id, int* rc);
int pa_num_free_blocks(const pa_pool* pool, int* n);
/* The free list, front first (out may be NULL to query the count). */
int pa_get_free_list(const pa_pool* pool, int32_t* out, int cap, int* n);
/* The split-KV partition length (tokens) the pool's last successful
 * pa_decode / pa_verify / pa_prefill / pa_append_attend call used -- the
 * library's choice when it was given 0 -- and the number of shared-prefix
 * workgroups that call launched; *partition_tokens = 0 when nothing was
 * split (and before the first call). */
int pa_last_partition(const pa_pool* pool, int* partition_tokens, int* prefix_units);

/* What the pool's last successful attention call (pa_decode, pa_verify,
 * pa_prefill, pa_append_attend, pa_decode_noalloc) launched, for measurement:
 * the split length as pa_last_partition, the workgroups of each launch, the
 * key/value positions the shared-prefix pass read (per kv head, each group's
 * shared positions once) and the query rows it served (per kv head, summed
 * over groups), and the split partial rows written (all kv heads; each row
 * is head_dim + 2 floats, read again by the merge).  All zero before the
 * first call. */
typedef struct pa_call_stats {
  int32_t partition_tokens;
  int32_t prefix_workgroups;     /* shared-prefix units, in their own launch or the attention launch (0: none) */
  int32_t attention_workgroups;  /* attention units of the attention launch (units x kv heads) */
  int32_t append_workgroups;     /* append workgroups inside that launch (fused append) */
  int32_t merge_workgroups;      /* separate merge launch (0: none, or merged inside) */
  int32_t reserved;
  int64_t prefix_kv_tokens;
  int64_t prefix_query_rows;
  int64_t partial_rows;
} pa_call_stats;
int pa_last_call_stats(const pa_pool* pool, pa_call_stats* out);

const char* pa_strerror(int status);
const char* pa_last_error(void);

/* Timing of the attention kernels: when enabled, HIP events are recorded on the
 * call's stream around each attention-kernel launch.  pa_profile_read
 * synchronises those events and returns the summed elapsed milliseconds and
 * the number of launches since the last read (then resets).
 * which: 0 = attention kernel (decode / verify), 1 = split merge kernel,
 *        2 = append kernel, 3 = shared-prefix kernel. */
int pa_profile_enable(pa_pool* pool, int on);
int pa_profile_read(pa_pool* pool, int which, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
