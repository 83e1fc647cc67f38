/*
 * pkv.h -- paged KV cache write and paged attention for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels. Every data pointer is a DEVICE
 * pointer owned by the caller; descriptor structs are HOST pointers read
 * during the call. The library allocates nothing, keeps no state between
 * calls, never synchronises and never reads device memory on the host: each
 * entry point validates its scalar arguments, enqueues kernels on `stream`
 * (a hipStream_t; NULL is the null stream) and returns. Buffers must stay alive
 * until that work completes. Every entry point returns a pkv_status; on error
 * nothing is enqueued and pkv_last_error() names the offending argument.
 *
 * Sources for what is computed (page titles as they appear on the pages):
 *  [MV]  "Build a Mini vLLM: Paged KV Cache and Continuous Batching From
 *        Scratch": section 2 "The paged KV cache" (block pool, per-sequence
 *        block table, append_slot -> (table[pos // BLOCK], pos % BLOCK));
 *        section 3 "PagedAttention" (gather K/V through the table in logical
 *        order, GQA by repeating KV heads onto query heads, softmax(q.k/sqrt(hd)),
 *        weighted sum of V); section 4 (prefill writes every token's K/V into
 *        its slot and attends with a causal -inf mask; decode writes one token
 *        per sequence, then attends).
 *  [D16] "Day 16: the paged KV cache, real K/V through scattered blocks":
 *        "What I added today" (per-layer flat pool
 *        [num_blocks * block_size, num_kv_heads, head_dim], each token at the
 *        flat slot its table assigns); "What I learned" items 1-3 (one table
 *        shared by all layers; write = scatter; read = gather).
 *  [NV]  "nano-vLLM": "How it works" (pool [blocks, 16, kv_heads, hd]; write
 *        at table[n // 16], slot n % 16; short tables padded with the dummy
 *        block 0; query heads grouped onto their shared K/V head; masked
 *        attention), "Where the time went" (a real kernel reads the blocks in
 *        place instead of gathering a copy).
 *
 * Layouts (all row-major, contiguous, element type `dtype`):
 *   pool:   k_pool, v_pool  [num_blocks, block_size, num_kv_heads, head_dim]
 *           (one pair per layer; a layered pool is passed as a per-layer
 *           pointer). Flat slot s = block * block_size + offset addresses
 *           row s of the [num_blocks * block_size, num_kv_heads, head_dim] view.
 *   k, v:   [num_tokens, num_kv_heads, head_dim]
 *   q, out: [num_seqs, num_q_heads, head_dim]            (decode)
 *           [total_q_rows, num_q_heads, head_dim]        (prefill, packed)
 *   block_tables: int32 [num_seqs, max_blocks_per_seq]; entries past a
 *           sequence's last block are never read (pad them with 0).
 *   context_lens, slot_mapping, first_pos, cu_*: int32.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * The context length of a sequence counts the token being decoded: write the
 * new K/V first, then attend ([MV] section 4).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                          */
  PKV_ERR_DTYPE = 2,       /* dtype is not PKV_F32 or PKV_BF16                    */
  PKV_ERR_SHAPE = 3,       /* sizes inconsistent or negative                      */
  PKV_ERR_UNSUPPORTED = 4, /* valid but outside the compiled set (head_dim,
                              group size, block size)                             */
  PKV_ERR_WORKSPACE = 5,   /* decode workspace missing or too small              */
  PKV_ERR_HIP = 6,         /* the HIP runtime rejected a launch                   */
  PKV_ERR_ALIGN = 7,       /* a pointer is not 16-byte aligned where required     */
  PKV_ERR_CAPACITY = 8     /* a planned pool cannot hold one request of the
                              required length                                    */
} pkv_status;

typedef enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* One layer's pool pair. block_size is a power of two in [1, 256];
 * num_blocks * block_size < 2^31. */
typedef struct pkv_pool_desc {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pkv_dtype */
} pkv_pool_desc;

/* ---------------------------------------------------------------------------
 * pkv_slot_mapping -- flat slot of every token a write will place.
 * [MV] section 2 (append_slot), [D16] "What I added today" (flat slot),
 * [NV] "How it works" (table[n // 16], slot n % 16).
 *
 * Segment w (0 <= w < num_segments) places tokens cu_tokens[w] ..
 * cu_tokens[w+1]-1 at consecutive logical positions first_pos[w], ... of the
 * sequence whose table is row w of `tables` ([num_segments, max_blocks_per_seq]).
 * Output: slot_mapping[t] = tables[w][p / block_size] * block_size
 * + p % block_size, or -1 when p < 0, p / block_size >= max_blocks_per_seq,
 * or the table entry is outside [0, num_blocks). Tokens past num_tokens are
 * not written. Device pointers: tables, first_pos, cu_tokens (num_segments+1
 * entries, non-decreasing, starting at 0), slot_mapping (num_tokens entries).
 * One table per decode step serves every layer ([D16] "What I learned" 1-2),
 * so a caller builds this once per step and passes it to each layer's write.
 * ------------------------------------------------------------------------- */
pkv_status pkv_slot_mapping(const int32_t* tables, int32_t max_blocks_per_seq,
                            int32_t num_segments, const int32_t* first_pos,
                            const int32_t* cu_tokens, int32_t num_tokens,
                            int32_t block_size, int32_t num_blocks,
                            int32_t* slot_mapping, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_write -- scatter new K/V rows into the pool ([D16] "What I learned"
 * item 3: write is a scatter, pool[slots] = k; [MV] section 4).
 *
 * For each t < num_tokens with 0 <= slot_mapping[t] < num_blocks*block_size:
 * row slot_mapping[t] of k_pool (v_pool) receives row t of k (v), copied bit
 * for bit. Other slots are skipped (nothing written). Slots must be distinct
 * within a call; if not, one of the duplicates' rows lands (unspecified which).
 * k, v, k_pool, v_pool: dtype of `pool`; any alignment of the element size
 * (16-byte aligned rows take the vector path).
 * ------------------------------------------------------------------------- */
pkv_status pkv_write(const void* k, const void* v, const int32_t* slot_mapping,
                     int32_t num_tokens, void* k_pool, void* v_pool,
                     const pkv_pool_desc* pool, void* stream);

/* ---------------------------------------------------------------------------
 * Paged decode attention ([MV] section 3; [NV] "How it works"), reading each
 * sequence's blocks in place (no gathered copy).
 *
 * out[s][h] = sum_p softmax_p(scale * q[s][h] . K_s[p]) V_s[p][...] over
 * positions p < context_lens[s], where K_s[p] (V_s[p]) is row
 * block_tables[s][p / block_size] * block_size + p % block_size of k_pool
 * (v_pool), KV head h / (num_q_heads / num_kv_heads). Accumulation is fp32;
 * a bf16 result is rounded to nearest even.
 *
 * Sequences are cut into pieces of `partition` tokens (a multiple of the
 * block size and of the decode tile, which is 2 to 64 tokens by row size: 8
 * at bf16 head_dim 128, 32 at bf16 head_dim 64; 0 picks one from the sizes,
 * see pkv_decode_partition). With at most 1024 sequences, a power-of-two
 * partition and pieces of at least 128 KiB of K and V (smaller ones finish
 * before a schedule pays) the cut is finer: each context gets full pieces of
 * `partition` tokens; a rest shorter than half of it joins the last full
 * piece, a longer one becomes one tail piece of its own (shorter than a
 * partition); the launch runs all full pieces first, then
 * the tail pieces, longer ones first (near-equal pieces keep every workgroup
 * stream of the GPU equally loaded and the last pieces short). When every
 * context fits one piece, the sequences run longest first (32 length
 * classes), their ranks dealt over the passes in which the CUs take the grid
 * so that the lengths each CU serves add up to near the mean. With
 * partition 0, when a tile lies within one block and the contexts are long
 * (num_seqs * num_kv_heads * max_context_len rows of K and V average at least
 * 256 KiB over two workgroups per CU), pkv_decode and pkv_decode_step cut
 * instead each KV head's sequences, laid end to end (each non-empty one
 * preceded by 128 tokens that stand for a piece's fixed cost), into one
 * range per workgroup, two workgroups per CU, each range at least the
 * automatic partition long (the half of the workgroups that reach their CU
 * first take ranges 9/64 longer than the rest); a workgroup runs the parts
 * of every sequence its range touches, one after another (pkv_decode_schedule tells which cut a
 * call uses). Each piece of
 * a sequence with more than one yields a partial (running max m in log2
 * units, exp-sum l, unnormalised o) in `workspace`;
 * the last workgroup of a (sequence, KV head) to finish merges them in the
 * same launch, counted by one int32 per (sequence, KV head) in a fixed
 * 256 KiB area at the start of the workspace (with more than 65536 such
 * pairs a second kernel merges instead). Sequences with a single piece are
 * written directly.
 * workspace (device) must hold pkv_decode_workspace_bytes(...) bytes; it may
 * be NULL when that is 0. Its first 256 KiB must be zero before the first
 * call that uses it (a zero-filled buffer); every call leaves them zero and
 * writes partials only after them, so one buffer of the largest size serves
 * calls of any size. Calls that share a workspace must not overlap (run
 * them in stream order).
 *
 * context_lens[s] is clamped to [0, min(max_context_len,
 * max_blocks_per_seq * block_size)]; a sequence of length 0 gets zeros.
 * max_context_len must not exceed max_blocks_per_seq * block_size.
 * A needed table entry outside [0, num_blocks) removes that block's tokens
 * from the softmax (no out-of-bounds read). Slots of a block past the
 * sequence's length may hold anything (NaN included): they are masked by
 * selection, never multiplied in ([NV] "Correctness"). Non-finite values in q
 * or in the rows a sequence owns are not handled: the affected output rows
 * are unspecified (no access leaves its bounds).
 * q, out, k_pool, v_pool must be 16-byte aligned.
 * Compiled set: head_dim in {16, 32, 64, 128, 256}; num_q_heads / num_kv_heads
 * in 1..8; block_size a power of two <= 256.
 * ------------------------------------------------------------------------- */
int32_t pkv_decode_partition(int32_t num_seqs, int32_t max_context_len,
                             const pkv_pool_desc* pool);

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition,
                                  const pkv_pool_desc* pool);

/* Which cut pkv_decode and pkv_decode_step use for these sizes (the
 * two-phase entry points never use stream-K ranges): PKV_SCHED_GRID (one
 * workgroup per split of `partition` tokens of every sequence),
 * PKV_SCHED_PIECES (the piece schedule), PKV_SCHED_LONGEST_FIRST (one piece
 * per sequence, longest first), PKV_SCHED_STREAM_K (ranges of the laid-end-
 * to-end sequences); -1 when the sizes are invalid (see pkv_last_error). */
#define PKV_SCHED_GRID 0
#define PKV_SCHED_PIECES 1
#define PKV_SCHED_LONGEST_FIRST 2
#define PKV_SCHED_STREAM_K 3
int32_t pkv_decode_schedule(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                            int32_t partition, const pkv_pool_desc* pool);

pkv_status pkv_decode(const void* q, int32_t num_seqs, int32_t num_q_heads,
                      const void* k_pool, const void* v_pool,
                      const pkv_pool_desc* pool, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, int32_t partition,
                      void* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* The two phases of pkv_decode, for callers that time or schedule them
 * separately: every piece's partial, then a second kernel that merges them.
 * Call both, in this order, with identical arguments. They leave the counter
 * words of the workspace untouched, and their result is bit-identical to
 * pkv_decode's. */
pkv_status pkv_decode_partials(const void* q, int32_t num_seqs, int32_t num_q_heads,
                               const void* k_pool, const void* v_pool,
                               const pkv_pool_desc* pool,
                               const int32_t* block_tables,
                               int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len,
                               float scale, int32_t partition, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

pkv_status pkv_decode_reduce(const void* q, int32_t num_seqs, int32_t num_q_heads,
                             const void* k_pool, const void* v_pool,
                             const pkv_pool_desc* pool, const int32_t* block_tables,
                             int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len,
                             float scale, int32_t partition, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_decode_step -- one decode step with the KV write fused in ([MV] section
 * 4, decode_step: the new token's K/V is written into its slot, then the
 * sequence attends over all its positions; [D16] "What I learned" item 2).
 *
 * k_new, v_new: device [num_seqs, num_kv_heads, head_dim], dtype of the pool:
 * the new token of sequence s, at position context_lens[s] - 1 (the length
 * counts the new token). Its rows are written into slot
 * block_tables[s][p / block_size] * block_size + p % block_size of k_pool /
 * v_pool (skipped when that table entry is outside [0, num_blocks), as
 * pkv_write skips an out-of-range slot), and the attention reads position p
 * from k_new / v_new directly. The result and the pool contents are
 * bit-identical to pkv_slot_mapping + pkv_write + pkv_decode with the same
 * partition; the two launches of the separate write are saved. A sequence of
 * length 0 writes nothing and gets zeros. Slots written must be distinct
 * across sequences (as for pkv_write). Other arguments, the workspace and the
 * errors are those of pkv_decode; k_new and v_new must be 16-byte aligned.
 *
 * One launch: the fused write, every piece, and the merge of the pieces in
 * the same launch (workspace counters as for pkv_decode).
 * pkv_decode_step_partials is its first phase (the fused write and the
 * partials, counters untouched); pkv_decode_reduce with the same arguments
 * completes it.
 * ------------------------------------------------------------------------- */
pkv_status pkv_decode_step(const void* q, const void* k_new, const void* v_new,
                           int32_t num_seqs, int32_t num_q_heads, void* k_pool,
                           void* v_pool, const pkv_pool_desc* pool,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len,
                           float scale, int32_t partition, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);

pkv_status pkv_decode_step_partials(const void* q, const void* k_new, const void* v_new,
                                    int32_t num_seqs, int32_t num_q_heads, void* k_pool,
                                    void* v_pool, const pkv_pool_desc* pool,
                                    const int32_t* block_tables,
                                    int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    float scale, int32_t partition, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_decode_step_noalloc -- pkv_decode_step without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Same computation, kernels, partition choice and result bits as
 * pkv_decode_step with the same arguments; the split partials and merge
 * counters live in a fixed device array of PKV_NOALLOC_SCRATCH_BYTES bytes
 * inside the library (one per GPU, held until the process ends) instead of a
 * passed workspace. Nothing is allocated and nothing is freed: the first call
 * on a device looks up that device's copy of the array and clears its counter
 * words with one small kernel on `stream`; every call leaves them zero.
 * A call whose plan needs more than PKV_NOALLOC_SCRATCH_BYTES of scratch
 * (pkv_decode_workspace_bytes with the same sizes) returns PKV_ERR_WORKSPACE
 * before anything is enqueued; use pkv_decode_step with a workspace then.
 * All calls of one process on one GPU share that GPU's array, so two calls
 * that may run at the same time on one GPU (on two streams, from two threads)
 * race and give wrong results: run them in stream order. (Each process has
 * its own array.) Arguments and other errors are those of pkv_decode_step.
 * ------------------------------------------------------------------------- */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

pkv_status pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                   int32_t num_seqs, int32_t num_q_heads, void* k_pool,
                                   void* v_pool, const pkv_pool_desc* pool,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   float scale, int32_t partition, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_decode_shared -- paged decode for groups of sequences whose block tables
 * begin with the same blocks (a shared prompt: [NV] "Prefix caching", where
 * later users reuse the first user's full prompt blocks; [NV] "Where the time
 * went", where per-user gathers read a 500-token shared prompt once per user
 * and step; [NV] "Next steps" item 3, reading shared blocks once; [MV] "Key
 * Takeaways" item 6, prefix sharing).
 *
 * The result is that of pkv_decode with the same arguments (same definition;
 * only the summation order differs). Group i holds the consecutive sequences
 * group_start[i] .. group_start[i+1]-1 and shares its first prefix_lens[i]
 * tokens, rounded down to whole blocks and capped at max_prefix_len and the
 * table reach; call that P_i. The caller guarantees that the first P_i /
 * block_size table entries of every member are the same blocks (the kernels
 * read them from the group's first member). Each member s attends its
 * positions 0 .. min(ctx_s, P_i) - 1 through a shared pass that reads every
 * shared K/V row once for all members and heads of the group (matrix cores,
 * fp32 accumulation; bf16 probabilities are rounded to bf16 for the PV
 * product, as in pkv_prefill), and its positions min(ctx_s, P_i) .. ctx_s - 1
 * through the decode kernel; the split partials of both are merged as in
 * pkv_decode.
 *
 * group_start: device int32 [num_groups + 1], non-decreasing, group_start[0]
 *   == 0, group_start[num_groups] == num_seqs (values are clamped into
 *   [0, num_seqs]; sequences outside every group are not valid input).
 * prefix_lens: device int32 [num_groups], tokens.
 * max_group_size >= the member count of every group; max_prefix_len >= every
 *   prefix_lens[i] (and <= max_context_len); max_tail_len >= ctx_s - min(ctx_s,
 *   P_i) for every s, or < 0 for max_context_len (positions past that bound
 *   are not attended). partition: tokens per tail split (0 = auto from
 *   max_tail_len), as in pkv_decode. With partition 0 and tails long enough
 *   (the stream-K rule of pkv_decode with max_tail_len as the longest
 *   context), the tails are laid end to end per KV head and cut into
 *   stream-K ranges as in pkv_decode, each non-empty tail charged 256
 *   tokens; otherwise each tail is cut into splits of `partition` tokens.
 * workspace: pkv_decode_shared_workspace_bytes(...) bytes (device, 16-byte
 *   aligned); 0 when no shared pass and no split is needed. Its counter
 *   area (the first 256 KiB) must be zero before the first call, as for
 *   pkv_decode; the
 *   tail launch merges the shared and tail partials, so a call is two launches
 *   (shared pass, tails + merge).
 * With num_groups == 0, max_prefix_len < block_size, a shape the shared
 * pass does not compile (it covers bf16 and fp32 pools, head_dim 64 and 128,
 * group size 1..8), or when the reads the shared pass could save at most,
 * (num_seqs - num_groups) * max_prefix_len * 2 * num_kv_heads * head_dim *
 * itemsize bytes, are below 64 MiB (one launch of plain decode is then
 * faster than the extra shared-pass launch; the environment variable
 * PKV_SHARED_MIN_SAVED_BYTES, read at each call, sets another bound, 0 for
 * always), the call is exactly pkv_decode. Errors are those of
 * pkv_decode, plus PKV_ERR_SHAPE for inconsistent group sizes and
 * PKV_ERR_NULL for a NULL group_start / prefix_lens when num_groups > 0.
 * ------------------------------------------------------------------------- */
size_t pkv_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t max_context_len, int32_t num_groups,
                                         int32_t max_group_size, int32_t max_prefix_len,
                                         int32_t max_tail_len, int32_t partition,
                                         const pkv_pool_desc* pool);

pkv_status pkv_decode_shared(const void* q, int32_t num_seqs, int32_t num_q_heads,
                             const void* k_pool, const void* v_pool,
                             const pkv_pool_desc* pool, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, const int32_t* group_start,
                             const int32_t* prefix_lens, int32_t num_groups,
                             int32_t max_group_size, int32_t max_prefix_len,
                             int32_t max_tail_len, float scale, int32_t partition, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_prefill -- causal attention of a chunk of query rows over the pool
 * ([MV] section 4: each query sees the keys at its own and earlier positions;
 * softmax of the scaled scores, weighted sum of V).
 *
 * Sequence s owns packed query rows cu_q[s] .. cu_q[s+1]-1 (n_s rows). Row i
 * sits at absolute position a = context_lens[s] - n_s + i and attends the
 * sequence's positions 0..a through its block table (its own K/V must already
 * be in the pool: write, then attend). Rows with a < 0 are zero.
 * cu_q: device int32 [num_seqs+1], non-decreasing from 0, cu_q[num_seqs] ==
 * total_q_rows; max_q_len >= every n_s. Pools with head_dim 64 or 128 and at
 * most 2048 table entries per sequence in reach (min(max_context_len,
 * max_blocks_per_seq * block_size) / block_size) use matrix cores: bf16 pools
 * bf16 products with fp32 accumulation, probabilities rounded to bf16 for the
 * PV product; fp32 pools fp32 products throughout. Other cases run each row as
 * a one-split decode.
 * ------------------------------------------------------------------------- */
pkv_status pkv_prefill(const void* q, const int32_t* cu_q, int32_t num_seqs,
                       int32_t num_q_heads, int32_t max_q_len, int32_t total_q_rows,
                       const void* k_pool, const void* v_pool,
                       const pkv_pool_desc* pool, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t max_context_len, float scale, void* out,
                       void* stream);

/* ---------------------------------------------------------------------------
 * pkv_validate -- debug check of the index data a write or a decode uses.
 * The path's kernels never check device indices against each other (that
 * would need a synchronisation): a write skips slots outside the pool and
 * keeps one of several rows sent to one slot, a decode or prefill leaves the
 * tokens of an invalid table entry out of the softmax and clamps a context to
 * the table's reach. Each token is written once ([MV] section 4) and a table
 * maps a sequence's blocks into the pool ([NV] "How it works"), so any of
 * these is a caller error this call makes visible. It writes five int32
 * counters to report (device memory, overwritten):
 *   report[0]  slots < 0 (pkv_slot_mapping gives -1 for a position past the
 *              table or through an invalid entry; padding rows may use it)
 *   report[1]  slots >= num_blocks * block_size
 *   report[2]  duplicate slots: tokens of this call whose slot another token
 *              also names (k tokens on one slot count k - 1)
 *   report[3]  table entries outside [0, num_blocks) among the blocks
 *              0 .. ceil(ctx / block_size) - 1 a sequence needs
 *   report[4]  context lengths < 0 or > max_blocks_per_seq * block_size
 * Slots are checked when slot_mapping is non-NULL and num_tokens > 0; tables
 * when block_tables is non-NULL and num_seqs > 0 (context_lens is then
 * required). Checking slots needs `workspace`: pkv_validate_workspace_bytes()
 * bytes (one bit per pool slot), 4-byte aligned, zero on entry; the call
 * leaves it zero again, so one buffer serves every call in stream order.
 * Device pointers: slot_mapping, block_tables, context_lens, workspace,
 * report. Up to four launches on `stream`, nothing allocated; read report
 * after synchronising. Errors: PKV_ERR_NULL (report, or context_lens when
 * tables are checked), PKV_ERR_SHAPE, PKV_ERR_UNSUPPORTED (block size),
 * PKV_ERR_WORKSPACE.
 * ------------------------------------------------------------------------- */
size_t pkv_validate_workspace_bytes(int32_t num_blocks, int32_t block_size);

pkv_status pkv_validate(const int32_t* slot_mapping, int32_t num_tokens,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                        int32_t block_size, void* workspace, size_t workspace_bytes,
                        int32_t* report, void* stream);

/* ---------------------------------------------------------------------------
 * Pool sizing ([D38] "Why it matters"; host arithmetic, no device access).
 *
 * pkv_block_bytes: bytes of one block of a layered pool, K and V for every
 * layer and KV head: 2 * num_layers * block_size * num_kv_heads * head_dim *
 * itemsize (512 KiB for Llama-3.2-1B at block 16 in bf16; use the KV head
 * count, not the attention head count). Returns 0 if an argument is < 1 and
 * -1 (pkv_last_error() says why) if the product does not fit in int64.
 *
 * pkv_plan_pool: the number of blocks a device holds after the weights are
 * resident,
 *   budget = free_bytes - (1 - utilization) * total_bytes - activation_bytes,
 *   *num_blocks = floor(budget / block_bytes),
 * where free_bytes is what the driver reports free with the weights loaded,
 * utilization the fraction of the whole device the server may use, and
 * activation_bytes the transient reserve of the largest forward. Also
 * *requests_at_max_len = floor(*num_blocks / ceil(max_model_len / block_size))
 * (full-length requests the pool holds, not clamped by any slot count).
 * Returns PKV_ERR_CAPACITY, and still fills both outputs, when the pool holds
 * less than one request of max_model_len tokens ([D38]: a pool that cannot
 * hold one request refuses everything); pkv_last_error() then names the
 * longest length it could serve. PKV_ERR_SHAPE for negative sizes, a
 * utilization outside (0, 1], block_bytes < 1 or block_size < 1.
 * ------------------------------------------------------------------------- */
int64_t pkv_block_bytes(int32_t num_layers, int32_t block_size, int32_t num_kv_heads,
                        int32_t head_dim, int32_t itemsize);

pkv_status pkv_plan_pool(int64_t free_bytes, int64_t total_bytes, double utilization,
                         int64_t activation_bytes, int64_t block_bytes, int32_t block_size,
                         int32_t max_model_len, int64_t* num_blocks,
                         int64_t* requests_at_max_len);

/* Human-readable name of a status. Never NULL. */
const char* pkv_status_string(pkv_status status);

/* Message of the last failed call on this thread ("" if none). */
const char* pkv_last_error(void);

/* PKV_ABI_VERSION of the built library. */
int32_t pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
