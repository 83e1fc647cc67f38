// Host entry points of the C ABI declared in include/pkv.h: argument checks,
// work sizing and kernel launches on the caller's stream. No allocation, no
// synchronisation, no device reads.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "pkv_internal.h"

namespace pkv {

namespace {
thread_local char g_err[512] = "";

constexpr int kMaxPartition = 8192;   // tokens per split (bounds the LDS table slice)
constexpr int kMaxSplits = 4096;      // splits per sequence (bounds the merge kernel's LDS)
constexpr int64_t kSchedMinPieceBytes = 128 << 10;   // K+V bytes of a piece worth a lookup
// Longest-first ranks dealt over the passes in which the CUs take the grid
// (DecodeArgs::lpt_pass): Llama-3.2-1B shape, 192 sequences (768 workgroups,
// three passes of 64 sequences), 7 interleaved rounds on one box: 4 length
// classes in grid order 82.0 us, 32 classes 81.2, 32 classes with every
// second pass reversed 79.8, with the last three passes balanced 78.6 us.
constexpr bool kLptDealPasses = true;
// Stream-K ranges (DecodeArgs::sched_sk): two workgroups per CU, so that
// every CU holds two equal ranges; a piece is charged 128 tokens of cost;
// used when, at the largest contexts, a range would average at least 256 KiB
// of K/V. Measured on the LLaMA-2-70B layer step (A/B on one box, 5 interleaved
// rounds): 134.5 us with the piece schedule, 128.3 with equal ranges, 124.5
// with the 128-token charge (64: 125.4, 256: 125.6, 512: 133.8); with equal
// ranges, one workgroup per CU 175, 1.5: 156, 2.5: 152, 3: 144 us. Its TP=8
// shard (86 MB, 1 KV head): 28.6 us against 30.5 with 256-token pieces.
// Head_dim 128, 8 query heads per KV head, log-uniform contexts up to 8,192,
// block tables rotated past the last-level cache (ranges / pieces, us): at
// 64 MiB of K/V at the largest contexts, 22.6 / 21.4; at 128 MiB, 25.5 / 25.3,
// 25.3 / 23.8, 23.7 / 23.7 and, at a uniform 4,096, 33.8 / 40.4; at 256 MiB,
// 29.3 / 31.4 and 33.5 / 39.3; at 384-512 MiB, 6.3-8.1 us less.
// The first-dispatched half of a head's ranges is 9/64 longer than the mean:
// the older of a CU's two workgroups streams faster, and with equal ranges it
// ended ~15 us before the other (per-workgroup ends from the traced build).
// Measured on the same step (7 and 9 interleaved rounds on two boxes): equal
// ranges 124.5 / 123.4 us; 4/64: 122.8; 5/64: 121.8; 7/64: 120.4; 8/64:
// 119.2 / 121.1; 9/64: 119.6; 10/64: 119.7 / 120.1; 12/64: 118.8 / 123.2 (the
// spread grows); 16/64: 126.7; 20/64: 129.8.
constexpr int kSkWgPerCu = 2;
constexpr int kSkAlphaTokens = 128;
// Shared-prefix tails on stream-K ranges: each tail piece also merges the
// shared pass's partials (16 on the LLaMA-2-70B layer with a 4096-token
// prompt, 64 users): a charge of 256 tokens per tail. Measured on that case
// (3 rounds on one box, the whole call with its shared pass): 128 tokens
// 148.7-148.9 us, 256: 144.4-144.9, 512: 148.3-148.5.
constexpr int kSkTailAlphaTokens = 256;
constexpr int kSkFirstExtra64 = 9;
constexpr int64_t kSkMinWgBytes = 1 << 18;
// Merge counters: a fixed area at the start of every workspace, so that calls
// of any size sharing one buffer never write partials where another counts.
// Launches with more (sequence, KV head) pairs merge in a second kernel.
constexpr size_t kMergeCounters = 65536;
constexpr size_t kCounterBytes = kMergeCounters * sizeof(int32_t);   // 256 KiB

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int dtype_bytes(int dtype) { return dtype == PKV_F32 ? 4 : 2; }

pkv_status check_pool(const pkv_pool_desc* pool) {
  if (!pool) {
    set_error("pool descriptor is NULL");
    return PKV_ERR_NULL;
  }
  if (pool->dtype != PKV_F32 && pool->dtype != PKV_BF16) {
    set_error("pool dtype %d is not PKV_F32 (0) or PKV_BF16 (1)", pool->dtype);
    return PKV_ERR_DTYPE;
  }
  if (pool->num_blocks < 1 || pool->num_kv_heads < 1 || pool->head_dim < 1) {
    set_error("pool sizes must be positive (num_blocks %d, num_kv_heads %d, head_dim %d)",
              pool->num_blocks, pool->num_kv_heads, pool->head_dim);
    return PKV_ERR_SHAPE;
  }
  if (!is_pow2(pool->block_size) || pool->block_size > 256) {
    set_error("block_size %d must be a power of two in [1, 256]", pool->block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if ((int64_t)pool->num_blocks * pool->block_size > INT32_MAX) {
    set_error("num_blocks * block_size = %lld exceeds int32 slots",
              (long long)pool->num_blocks * pool->block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  return PKV_OK;
}

struct DecodePlan {
  int rep = 0;
  int partition = 0;
  int splits = 0;       // partial slots per (sequence, head)
  int sched_q = 0;      // small piece of the piece schedule (0: plain split grid)
  int sched_align = 0;
  bool sched_lpt = false;   // one piece per sequence, longest-first
  int lpt_pass = 0;         // longest-first ranks dealt in passes of this many sequences
  int sched_sk = 0;         // > 0: stream-K ranges, workgroups per KV head
  int sk_min_units = 0;
  int sk_alpha = 0;
  int sk_first_extra = 0;
  int pair_rep = 0;         // > 0: KV heads read in pairs (real group size)
  pkv_pool_desc view{};     // the pool as the kernels read it
  size_t ws_ml_offset = 0;   // partial (m, l) pairs, after the counter area
  size_t ws_o_offset = 0;    // partial o rows
  size_t ws_bytes = 0;
};

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// The merge counter area, then partials [S, Hq, J] (m, l), then o.
void plan_workspace(int32_t num_seqs, int32_t num_q_heads, const pkv_pool_desc* pool, int J,
                    DecodePlan* plan) {
  const size_t rows = (size_t)num_seqs * num_q_heads * J;
  plan->ws_ml_offset = kCounterBytes;
  plan->ws_o_offset = plan->ws_ml_offset + round256(rows * 2 * sizeof(float));
  plan->ws_bytes = plan->ws_o_offset + round256(rows * (size_t)pool->head_dim * sizeof(float));
}

int align_tokens(const pkv_pool_desc* pool) {
  const int tile = decode_tile_tokens(pool->head_dim * dtype_bytes(pool->dtype));
  return tile > pool->block_size ? tile : pool->block_size;
}

int auto_partition(int num_seqs, int max_ctx, const pkv_pool_desc* pool) {
  const int cus = num_cus();
  const int align = align_tokens(pool);
  const int whole = ((std::max(max_ctx, 1) + align - 1) / align) * align;   // one split covers all
  const int cap = (kMaxPartition / align) * align;
  if (max_ctx <= 0 || num_seqs <= 0) return align;
  // With at least four (sequence, KV head) units per CU there is enough
  // parallelism without splitting. Otherwise split so that, with lengths
  // spread up to max_ctx, there are about 8 split workgroups per CU. Each
  // split workgroup costs a prologue and, with the merge in the launch, a
  // counted partial; measured on the LLaMA-2-70B-layer workload: 1024-token
  // splits 150 us, 512-token 172 us, 2048-token 164 us.
  const double units = (double)num_seqs * pool->num_kv_heads;
  int part;
  if (units >= 4.0 * cus) {
    part = whole;
  } else {
    const double p = units * (double)max_ctx / (16.0 * cus);
    part = 256;
    while (part < p && part < cap) part <<= 1;
  }
  part = ((part + align - 1) / align) * align;
  if (part > cap) part = cap;
  if (part > whole) part = whole;
  if (part < align) part = align;
  return part;
}

// Adjacent KV heads read as one: bf16 rows of 64 dims (128 bytes) pair into
// 256-byte rows, a layout the pool already has ([.., Hkv, 64] is
// [.., Hkv / 2, 128]), when there are at least four (sequence, KV head) pairs
// per CU: pairing halves the workgroups. Measured on Llama-3.2-1B's shape:
// 192 sequences (1536 pairs) 82.5 us paired against 98.4 us; 8 sequences of
// 2048 tokens (64 pairs) 16.0 us against 14.8 us.
bool pair_heads(const pkv_pool_desc* pool, int num_seqs, int rep) {
  return pool->dtype == PKV_BF16 && pool->head_dim == 64 && pool->num_kv_heads % 2 == 0 &&
         rep <= 4 && (double)num_seqs * pool->num_kv_heads >= 4.0 * num_cus();
}

pkv_status plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                       int32_t max_ctx, int32_t partition, const pkv_pool_desc* pool,
                       DecodePlan* plan, bool allow_sched = true, bool allow_pair = true,
                       bool allow_sk = false) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_q_heads < 1 || max_ctx < 0 || max_blocks < 1) {
    set_error("bad sizes: num_seqs %d, num_q_heads %d, max_context_len %d, "
              "max_blocks_per_seq %d", num_seqs, num_q_heads, max_ctx, max_blocks);
    return PKV_ERR_SHAPE;
  }
  if (num_q_heads % pool->num_kv_heads != 0) {
    set_error("num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
              pool->num_kv_heads);
    return PKV_ERR_SHAPE;
  }
  if ((int64_t)max_ctx > (int64_t)max_blocks * pool->block_size) {
    set_error("max_context_len %d exceeds max_blocks_per_seq * block_size = %lld", max_ctx,
              (long long)max_blocks * pool->block_size);
    return PKV_ERR_SHAPE;
  }
  const int rep = num_q_heads / pool->num_kv_heads;
  if (!decode_supported(pool->dtype, pool->head_dim, rep)) {
    set_error("head_dim %d with group size %d is not compiled (head_dim 16/32/64/128/256, "
              "group 1..8)", pool->head_dim, rep);
    return PKV_ERR_UNSUPPORTED;
  }
  plan->view = *pool;
  plan->pair_rep = 0;
  if (allow_pair && pair_heads(pool, num_seqs, rep)) {
    plan->pair_rep = rep;
    plan->view.num_kv_heads /= 2;
    plan->view.head_dim *= 2;
  }
  // the stricter of the two alignments, so that whether a partition is valid
  // does not depend on whether this launch pairs its heads
  const int align = std::max(align_tokens(&plan->view), align_tokens(pool));
  int part = partition;
  if (part == 0) {
    // from the real heads: a multiple of their (coarser) alignment
    part = auto_partition(num_seqs, max_ctx, pool);
  } else if (part < 0 || part % align != 0 || part > kMaxPartition) {
    set_error("partition %d must be a positive multiple of %d and at most %d", part, align,
              kMaxPartition);
    return PKV_ERR_SHAPE;
  }
  const int splits = max_ctx > 0 ? (max_ctx + part - 1) / part : 1;
  if (num_seqs > 65535 || splits > kMaxSplits) {
    set_error("num_seqs %d exceeds 65535 or split count %d exceeds %d (raise partition)",
              num_seqs, splits, kMaxSplits);
    return PKV_ERR_UNSUPPORTED;
  }
  plan->rep = plan->pair_rep ? 2 * rep : rep;
  plan->partition = part;
  plan->splits = splits;
  plan->sched_q = 0;
  // The schedule's lookup adds one dependent round trip to every workgroup;
  // it pays where a piece streams long enough to hide it. Measured on
  // Llama-3.2-1B's shape with 8 sequences of 2048 tokens (64 KiB pieces):
  // 13.5 us per call on the plain grid against 14.9 with the lookup.
  const int64_t row_bytes = 2 * (int64_t)plan->view.head_dim * dtype_bytes(pool->dtype);
  const bool sched_pieces = allow_sched && (int64_t)part * row_bytes >= kSchedMinPieceBytes;
  if (splits > 1 && sched_pieces && num_seqs <= kSchedMaxSeqs && is_pow2(part) &&
      is_pow2(align)) {
    // piece schedule: full pieces of `part` tokens; a rest under half a
    // piece joins the last full piece, a longer one is one tail piece of its
    // own (tail pieces of at most `part` tokens). Measured on the
    // LLaMA-2-70B-layer workload (1024-token pieces, A/B on one box, 9
    // interleaved rounds): 135.0 us against 136.2 with tails of at most half
    // a piece (two tail pieces for a long rest); its TP=8 shard (256-token
    // pieces) 30.6 against 31.1 us. Earlier kernels: tails of about 256
    // tokens 141 us, 128 150 us, none (every rest joined) 149 us.
    const int q = std::max(align, part);   // powers of two: a multiple of align
    const int64_t J = (int64_t)max_ctx / part + (part - 1 + q - 1) / q;
    if (J <= kMaxSplits && max_piece(part, q) <= kMaxPartition) {
      plan->sched_q = q;
      plan->sched_align = align;
      plan->splits = (int)J;
    }
  }
  // single-piece plans: the sequences in longest-first order (the piece is
  // the longest context)
  plan->sched_lpt = plan->splits == 1 && allow_sched && num_seqs <= kSchedMaxSeqs &&
                    (int64_t)max_ctx * row_bytes >= kSchedMinPieceBytes;
  {
    const int hv = plan->view.num_kv_heads;   // the grid's x extent
    plan->lpt_pass = plan->sched_lpt && kLptDealPasses && num_cus() % hv == 0 ? num_cus() / hv : 0;
  }
  // Stream-K ranges in place of the pieces, for an automatic partition of a
  // launch that merges in place, when the kernel reads block ids uniformly
  // (a tile within one block), its rows are unpaired and of 256 bytes or more
  // (the compiled stream-K variants) and the ranges are long. The partition is the
  // least range (a bound on the partial slots a sequence can need).
  plan->sched_sk = plan->sk_min_units = plan->sk_alpha = plan->sk_first_extra = 0;
  const int A = plan->view.block_size;
  const int heads = plan->view.num_kv_heads;
  const int64_t wgs = (int64_t)kSkWgPerCu * num_cus();
  const int64_t units = ((int64_t)max_ctx + A - 1) / A;
  const int alpha = std::max(1, kSkAlphaTokens / A);
  if (allow_sk && partition == 0 && plan->sched_q > 0 && A >= align && wgs >= heads &&
      plan->pair_rep == 0 && plan->view.head_dim * dtype_bytes(pool->dtype) >= 256 &&
      (int64_t)num_seqs * heads <= (int64_t)kMergeCounters &&
      (int64_t)num_seqs * (units + alpha) < (1ll << 30) &&
      (int64_t)num_seqs * heads * max_ctx * row_bytes >= kSkMinWgBytes * wgs) {
    const int mu = std::max(1, part / A);
    const int64_t J = (units + mu - 1) / mu + 1;
    if (J <= kMaxSplits) {
      plan->sched_sk = (int)(wgs / heads);
      plan->sk_min_units = mu;
      plan->sk_alpha = alpha;
      plan->sk_first_extra = kSkFirstExtra64;
      plan->sched_q = 0;
      plan->sched_align = A;
      plan->splits = (int)J;
    }
  }
  plan->ws_ml_offset = plan->ws_o_offset = plan->ws_bytes = 0;
  if (plan->splits > 1) plan_workspace(num_seqs, num_q_heads, &plan->view, plan->splits, plan);
  return PKV_OK;
}

enum class Phase { kBoth, kPartials, kReduce };

// Caller's description of the shared-prefix groups (pkv_decode_shared).
struct SharedIn {
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int32_t num_groups, max_group, max_prefix, max_tail;
};

// Least K/V bytes a shared pass must be able to save for pkv_decode_shared to
// run it (environment PKV_SHARED_MIN_SAVED_BYTES overrides; 0 always runs
// it). Measured: 30 users of a 500-token prompt at the SmolLM2-135M shape
// save at most 22 MB per call and ran 15.6 us plain against 21.3 us shared;
// 64 users of a 4096-token prompt at the LLaMA-2-70B layer shape save 1.06 GB
// and ran 294 us plain against 166 us shared.
constexpr int64_t kSharedMinSavedBytes = 64ll << 20;
int64_t shared_min_saved_bytes() {
  const char* e = getenv("PKV_SHARED_MIN_SAVED_BYTES");
  if (!e || !*e) return kSharedMinSavedBytes;
  char* end = nullptr;
  const long long v = strtoll(e, &end, 10);
  return (end && *end == '\0' && v >= 0) ? (int64_t)v : kSharedMinSavedBytes;
}

// Shared-prefix plan: the tail splits (partition from the longest tail), then
// the shared pass's key splits, sized for about one workgroup per CU.
// sd->group_start stays NULL when the shared pass is not used (no groups, a
// prefix shorter than a block, or a shape the matrix-core pass does not
// compile); the plan is then plain decode.
pkv_status plan_shared(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                       int32_t max_ctx, const SharedIn& in, int32_t partition,
                       const pkv_pool_desc* pool, DecodePlan* plan, SharedDesc* sd,
                       bool allow_sk = true) {
  *sd = SharedDesc{};
  pkv_status st = plan_decode(num_seqs, num_q_heads, max_blocks, max_ctx, partition, pool, plan);
  if (st != PKV_OK) return st;
  if (in.num_groups < 0 || in.num_groups > std::max(num_seqs, 0) || in.max_prefix < 0 ||
      in.max_prefix > max_ctx || in.max_tail > max_ctx ||
      (in.num_groups > 0 && (in.max_group < 1 || in.max_group > num_seqs))) {
    set_error("bad shared-prefix sizes: num_groups %d, max_group_size %d, max_prefix_len %d, "
              "max_tail_len %d (num_seqs %d, max_context_len %d)", in.num_groups, in.max_group,
              in.max_prefix, in.max_tail, num_seqs, max_ctx);
    return PKV_ERR_SHAPE;
  }
  const int bs = pool->block_size;
  if (in.num_groups == 0 || in.max_prefix < bs ||
      !shared_pass_supported(pool->dtype, pool->head_dim, num_q_heads / pool->num_kv_heads))
    return PKV_OK;
  // The shared pass is a launch of its own; it pays only when the reads it
  // saves cover it. At most every member but one per group skips the prompt:
  // (num_seqs - num_groups) * max_prefix rows of K and V.
  const int64_t saved = (int64_t)(num_seqs - in.num_groups) * in.max_prefix * 2 *
                        pool->num_kv_heads * pool->head_dim * dtype_bytes(pool->dtype);
  if (saved < shared_min_saved_bytes()) return PKV_OK;
  // The tails: stream-K ranges over the laid-end-to-end tails when they are
  // long enough (the only schedule that knows tails), else the plain grid.
  const int tail = in.max_tail < 0 ? max_ctx : in.max_tail;
  st = plan_decode(num_seqs, num_q_heads, max_blocks, tail, partition, pool, plan, true, false,
                   allow_sk);
  if (st == PKV_OK && plan->sched_sk == 0)
    st = plan_decode(num_seqs, num_q_heads, max_blocks, tail, partition, pool, plan, false, false);
  if (st != PKV_OK) return st;
  // a tail's piece also merges the shared pass's partials: a larger charge
  if (plan->sched_sk > 0) plan->sk_alpha = std::max(1, kSkTailAlphaTokens / plan->sched_align);
  const int64_t align = std::max(kSharedAlign, bs);
  const int64_t row_tiles = ((int64_t)in.max_group * plan->rep + kSharedRows - 1) / kSharedRows;
  const int64_t base = (int64_t)in.num_groups * pool->num_kv_heads * row_tiles;
  const int64_t max_ks = (in.max_prefix + align - 1) / align;
  const int64_t cus = num_cus();
  // key splits for about one shared-pass workgroup per CU: fewer splits leave
  // each tail fewer partials to merge. LLaMA-2-70B layer, 64 users of a
  // 4096-token prompt (3 rounds on one box, whole call): 4 splits (half a
  // workgroup per CU) 143.2-143.6 us, 6: 139.2-139.7, 8: 137.9-138.5, 16:
  // 144.4-145.1, 32: 159.4-160.2.
  const int64_t nks = std::min(std::max<int64_t>((cus + base - 1) / base, 1), max_ks);
  int64_t pp = ((in.max_prefix + nks - 1) / nks + align - 1) / align * align;
  pp = std::min(pp, (int64_t)kSharedMaxTbl * bs / align * align);
  const int64_t jp = (in.max_prefix + pp - 1) / pp;
  const int64_t J = jp + plan->splits;
  if (J > kMaxSplits) {
    set_error("shared prefix: %lld splits per sequence exceed %d (raise partition)",
              (long long)J, kMaxSplits);
    return PKV_ERR_UNSUPPORTED;
  }
  plan->splits = (int)J;
  plan_workspace(num_seqs, num_q_heads, pool, (int)J, plan);
  sd->group_start = in.group_start;
  sd->prefix_lens = in.prefix_lens;
  sd->num_groups = in.num_groups;
  sd->max_prefix = in.max_prefix;
  sd->prefix_part = (int)pp;
  sd->prefix_slots = (int)jp;
  return PKV_OK;
}

pkv_status decode_impl(Phase phase, const void* q, int32_t num_seqs, int32_t num_q_heads,
                       const void* k_pool, const void* v_pool, const pkv_pool_desc* pool,
                       const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t max_ctx, float scale,
                       int32_t partition, void* out, void* workspace, size_t workspace_bytes,
                       void* stream, const void* k_new = nullptr, const void* v_new = nullptr,
                       const SharedIn* shared = nullptr) {
  DecodePlan plan;
  SharedDesc sd{};
  pkv_status st = shared ? plan_shared(num_seqs, num_q_heads, max_blocks, max_ctx, *shared,
                                       partition, pool, &plan, &sd)
                         : plan_decode(num_seqs, num_q_heads, max_blocks, max_ctx, partition,
                                       pool, &plan, true, true, phase == Phase::kBoth);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (shared && shared->num_groups > 0 && (!shared->group_start || !shared->prefix_lens)) {
    set_error("group_start %p or prefix_lens %p is NULL", (const void*)shared->group_start,
              (const void*)shared->prefix_lens);
    return PKV_ERR_NULL;
  }
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) {
    set_error("NULL pointer among q %p, k_pool %p, v_pool %p, block_tables %p, "
              "context_lens %p, out %p", q, k_pool, v_pool, (const void*)block_tables,
              (const void*)context_lens, out);
    return PKV_ERR_NULL;
  }
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool)) {
    set_error("q, out, k_pool and v_pool must be 16-byte aligned");
    return PKV_ERR_ALIGN;
  }
  if (!std::isfinite(scale)) {
    set_error("scale must be finite");
    return PKV_ERR_SHAPE;
  }
  if (plan.ws_bytes > 0) {
    if (!workspace) {
      set_error("workspace is NULL but %zu bytes are needed", plan.ws_bytes);
      return PKV_ERR_WORKSPACE;
    }
    if (workspace_bytes < plan.ws_bytes) {
      set_error("workspace has %zu bytes, %zu needed", workspace_bytes, plan.ws_bytes);
      return PKV_ERR_WORKSPACE;
    }
    if (!aligned16(workspace)) {
      set_error("workspace must be 16-byte aligned");
      return PKV_ERR_ALIGN;
    }
  }
  DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = block_tables;
  a.ctx_lens = context_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.ws_ml = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_ml_offset) : nullptr;
  a.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_o_offset) : nullptr;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  const pkv_pool_desc& view = plan.view;   // paired heads: half the heads, twice the dims
  a.num_kv_heads = view.num_kv_heads;
  a.num_blocks = pool->num_blocks;
  a.block_shift = ilog2(pool->block_size);
  a.max_blocks = max_blocks;
  a.max_ctx = max_ctx;
  a.pair_rep = plan.pair_rep;
  a.partition = plan.partition;
  a.num_splits = plan.splits;
  a.sched_q = plan.sched_q;
  a.sched_align = plan.sched_align;
  a.sched_lpt = plan.sched_lpt;
  a.lpt_pass = plan.lpt_pass;
  a.sched_sk = plan.sched_sk;
  a.sk_min_units = plan.sk_min_units;
  a.sk_alpha = plan.sk_alpha;
  a.sk_first_extra = plan.sk_first_extra;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.cu_q = nullptr;
  a.total_q = 0;
  a.k_new = k_new;
  a.v_new = v_new;
  a.sh = sd;
  // One launch merges its own partials unless the caller runs the phases
  // apart or there are more (sequence, KV head) pairs than counters.
  const bool in_launch = phase == Phase::kBoth && plan.ws_bytes &&
                         (size_t)num_seqs * view.num_kv_heads <= kMergeCounters;
  a.counters = in_launch ? reinterpret_cast<int32_t*>(ws) : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (sd.group_start && phase != Phase::kReduce) {
    PrefillArgs p{};
    p.q = q;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.tables = block_tables;
    p.ctx_lens = context_lens;
    p.out = out;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = pool->num_kv_heads;
    p.num_blocks = pool->num_blocks;
    p.block_shift = a.block_shift;
    p.max_blocks = max_blocks;
    p.max_ctx = max_ctx;
    p.scale_log2 = a.scale_log2;
    p.sh = sd;
    p.ws_ml = a.ws_ml;
    p.ws_o = a.ws_o;
    p.num_slots = plan.splits;
    p.max_group = shared->max_group;
    st = launch_shared_pass(p, pool->dtype, pool->head_dim, plan.rep, s);
    if (st != PKV_OK) return st;
  }
  if (phase != Phase::kReduce) {
    st = launch_decode_partials(a, view.dtype, view.head_dim, plan.rep, s);
    if (st != PKV_OK) return st;
  }
  if (phase == Phase::kReduce || (phase == Phase::kBoth && plan.ws_bytes && !in_launch)) {
    st = launch_decode_reduce(a, view.dtype, view.head_dim, s);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

// Scratch of pkv_decode_step_noalloc: a fixed device array (each GPU holds
// its own copy), laid out like a decode workspace (merge counters, then
// partials). Host code never passes the array's name to a kernel (on the host
// it names a stand-in, not device memory): it uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_noalloc_ptr.
constexpr size_t kNoallocScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes > kCounterBytes, "scratch holds the counter area");
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_noalloc_ptr[kMaxDevices];
std::mutex g_noalloc_mu;

// Device address of the current device's scratch array. The first call on a
// device (with that device current) looks it up and clears the counter words
// with a kernel on `st` (a kernel rather than a memset, so that a call under
// graph capture records no memset node); every decode leaves them zero.
pkv_status noalloc_scratch(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("no usable current device (%s, device %d)", hipGetErrorString(e), dev);
    return PKV_ERR_HIP;
  }
  void* p = g_noalloc_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    p = g_noalloc_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        set_error("hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
        return PKV_ERR_HIP;
      }
      hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, st,
                         static_cast<uint32_t*>(p), (uint32_t)(kCounterBytes / 4));
      const pkv_status ls = launch_status("zero_words_kernel");
      if (ls != PKV_OK) return ls;
      g_noalloc_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}

}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int num_cus() {
  static std::atomic<int> cached[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();   // leave no error behind for a later launch check
    return kDefaultCUs;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    n = kDefaultCUs;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

pkv_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s launch failed: %s", what, hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

pkv_status pkv_slot_mapping(const int32_t* tables, int32_t max_blocks_per_seq,
                            int32_t num_segments, const int32_t* first_pos,
                            const int32_t* cu_tokens, int32_t num_tokens, int32_t block_size,
                            int32_t num_blocks, int32_t* slot_mapping, void* stream) {
  if (num_segments < 0 || num_tokens < 0 || max_blocks_per_seq < 1 || num_blocks < 1) {
    set_error("bad sizes: num_segments %d, num_tokens %d, max_blocks_per_seq %d, "
              "num_blocks %d", num_segments, num_tokens, max_blocks_per_seq, num_blocks);
    return PKV_ERR_SHAPE;
  }
  if (!is_pow2(block_size) || block_size > 256) {
    set_error("block_size %d must be a power of two in [1, 256]", block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if ((int64_t)num_blocks * block_size > INT32_MAX) {
    set_error("num_blocks * block_size exceeds int32 slots");
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_segments == 0 || num_tokens == 0) return PKV_OK;
  if (!tables || !first_pos || !cu_tokens || !slot_mapping) {
    set_error("NULL pointer among tables, first_pos, cu_tokens, slot_mapping");
    return PKV_ERR_NULL;
  }
  SlotArgs a;
  a.tables = tables;
  a.first_pos = first_pos;
  a.cu = cu_tokens;
  a.slots = slot_mapping;
  a.max_blocks = max_blocks_per_seq;
  a.num_segments = num_segments;
  a.num_tokens = num_tokens;
  a.block_shift = ilog2(block_size);
  a.num_blocks = num_blocks;
  launch_slot_mapping(a, reinterpret_cast<hipStream_t>(stream));
  return launch_status("slot_mapping_kernel");
}

pkv_status pkv_write(const void* k, const void* v, const int32_t* slot_mapping,
                     int32_t num_tokens, void* k_pool, void* v_pool, const pkv_pool_desc* pool,
                     void* stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) {
    set_error("num_tokens %d is negative", num_tokens);
    return PKV_ERR_SHAPE;
  }
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) {
    set_error("NULL pointer among k %p, v %p, slot_mapping %p, k_pool %p, v_pool %p", k, v,
              (const void*)slot_mapping, k_pool, v_pool);
    return PKV_ERR_NULL;
  }
  const int isz = dtype_bytes(pool->dtype);
  const int64_t row_bytes = (int64_t)pool->num_kv_heads * pool->head_dim * isz;
  if (row_bytes > INT32_MAX / 2) {
    set_error("row of %lld bytes is too large", (long long)row_bytes);
    return PKV_ERR_UNSUPPORTED;
  }
  const uintptr_t any = (uintptr_t)k | (uintptr_t)v | (uintptr_t)k_pool | (uintptr_t)v_pool;
  if (any % (uintptr_t)isz) {
    set_error("k, v, k_pool, v_pool must be aligned to the element size (%d)", isz);
    return PKV_ERR_ALIGN;
  }
  const bool vec16 = (row_bytes % 16 == 0) && (any % 16 == 0);
  WriteArgs a;
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.slots = slot_mapping;
  a.k_pool = static_cast<uint8_t*>(k_pool);
  a.v_pool = static_cast<uint8_t*>(v_pool);
  a.pool_slots = (int64_t)pool->num_blocks * pool->block_size;
  a.num_tokens = num_tokens;
  a.row_bytes = (int32_t)row_bytes;
  launch_write(a, vec16, isz, reinterpret_cast<hipStream_t>(stream));
  return launch_status("write_kernel");
}

int32_t pkv_decode_partition(int32_t num_seqs, int32_t max_context_len,
                             const pkv_pool_desc* pool) {
  if (check_pool(pool) != PKV_OK) return 0;
  return auto_partition(num_seqs, max_context_len, pool);
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition,
                                  const pkv_pool_desc* pool) {
  if (!pool) return 0;
  DecodePlan plan;
  const int32_t maxb = pool->block_size > 0
                           ? (max_context_len + pool->block_size - 1) / pool->block_size
                           : 1;
  if (plan_decode(num_seqs, num_q_heads, maxb > 0 ? maxb : 1, max_context_len, partition,
                  pool, &plan) != PKV_OK)
    return 0;
  // one size for every entry point: the in-launch plan may use stream-K ranges
  DecodePlan in_launch;
  if (plan_decode(num_seqs, num_q_heads, maxb > 0 ? maxb : 1, max_context_len, partition,
                  pool, &in_launch, true, true, true) != PKV_OK)
    return 0;
  return std::max(plan.ws_bytes, in_launch.ws_bytes);
}

int32_t pkv_decode_schedule(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                            int32_t partition, const pkv_pool_desc* pool) {
  if (!pool) return -1;
  DecodePlan plan;
  const int32_t maxb = pool->block_size > 0
                           ? (max_context_len + pool->block_size - 1) / pool->block_size
                           : 1;
  if (plan_decode(num_seqs, num_q_heads, maxb > 0 ? maxb : 1, max_context_len, partition,
                  pool, &plan, true, true, true) != PKV_OK)
    return -1;
  if (plan.sched_sk > 0) return PKV_SCHED_STREAM_K;
  if (plan.sched_q > 0) return PKV_SCHED_PIECES;
  if (plan.sched_lpt) return PKV_SCHED_LONGEST_FIRST;
  return PKV_SCHED_GRID;
}

pkv_status pkv_decode(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_pool,
                      const void* v_pool, const pkv_pool_desc* pool,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t max_context_len, float scale,
                      int32_t partition, void* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_impl(Phase::kBoth, q, num_seqs, num_q_heads, k_pool, v_pool, pool, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, scale, partition, out,
                     workspace, workspace_bytes, stream);
}

pkv_status pkv_decode_partials(const void* q, int32_t num_seqs, int32_t num_q_heads,
                               const void* k_pool, const void* v_pool,
                               const pkv_pool_desc* pool, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, float scale, int32_t partition,
                               void* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode_impl(Phase::kPartials, q, num_seqs, num_q_heads, k_pool, v_pool, pool,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     partition, out, workspace, workspace_bytes, stream);
}

pkv_status pkv_decode_reduce(const void* q, int32_t num_seqs, int32_t num_q_heads,
                             const void* k_pool, const void* v_pool, const pkv_pool_desc* pool,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len, float scale,
                             int32_t partition, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_impl(Phase::kReduce, q, num_seqs, num_q_heads, k_pool, v_pool, pool,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     partition, out, workspace, workspace_bytes, stream);
}

namespace {
pkv_status check_step(const void* k_new, const void* v_new) {
  if (!k_new || !v_new) {
    set_error("k_new and v_new must not be NULL");
    return PKV_ERR_NULL;
  }
  if (!aligned16(k_new) || !aligned16(v_new)) {
    set_error("k_new and v_new must be 16-byte aligned");
    return PKV_ERR_ALIGN;
  }
  return PKV_OK;
}
}  // namespace

pkv_status pkv_decode_step(const void* q, const void* k_new, const void* v_new,
                           int32_t num_seqs, int32_t num_q_heads, void* k_pool, void* v_pool,
                           const pkv_pool_desc* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, float scale, int32_t partition, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0) {
    const pkv_status st = check_step(k_new, v_new);
    if (st != PKV_OK) return st;
  }
  return decode_impl(Phase::kBoth, q, num_seqs, num_q_heads, k_pool, v_pool, pool, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, scale, partition, out,
                     workspace, workspace_bytes, stream, k_new, v_new);
}

pkv_status pkv_decode_step_partials(const void* q, const void* k_new, const void* v_new,
                                    int32_t num_seqs, int32_t num_q_heads, void* k_pool,
                                    void* v_pool, const pkv_pool_desc* pool,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    float scale, int32_t partition, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (num_seqs > 0) {
    const pkv_status st = check_step(k_new, v_new);
    if (st != PKV_OK) return st;
  }
  return decode_impl(Phase::kPartials, q, num_seqs, num_q_heads, k_pool, v_pool, pool,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     partition, out, workspace, workspace_bytes, stream, k_new, v_new);
}

pkv_status pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                   int32_t num_seqs, int32_t num_q_heads, void* k_pool,
                                   void* v_pool, const pkv_pool_desc* pool,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   float scale, int32_t partition, void* out, void* stream) {
  if (num_seqs > 0) {
    const pkv_status st = check_step(k_new, v_new);
    if (st != PKV_OK) return st;
  }
  // the size check comes before any device call
  DecodePlan plan;
  pkv_status st = plan_decode(num_seqs, num_q_heads, max_blocks_per_seq, max_context_len,
                              partition, pool, &plan, true, true, true);
  if (st != PKV_OK) return st;
  if (plan.ws_bytes > kNoallocScratchBytes) {
    set_error("this decode step needs %zu bytes of scratch; the library's fixed area holds "
              "%zu (call pkv_decode_step with a workspace)", plan.ws_bytes,
              kNoallocScratchBytes);
    return PKV_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (plan.ws_bytes > 0 && num_seqs > 0) {
    st = noalloc_scratch(reinterpret_cast<hipStream_t>(stream), &ws);
    if (st != PKV_OK) return st;
  }
  return decode_impl(Phase::kBoth, q, num_seqs, num_q_heads, k_pool, v_pool, pool, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, scale, partition, out,
                     ws, ws ? kNoallocScratchBytes : 0, stream, k_new, v_new);
}

size_t pkv_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t max_context_len, int32_t num_groups,
                                         int32_t max_group_size, int32_t max_prefix_len,
                                         int32_t max_tail_len, int32_t partition,
                                         const pkv_pool_desc* pool) {
  if (!pool) return 0;
  DecodePlan plan;
  SharedDesc sd;
  const int32_t maxb = pool->block_size > 0
                           ? (max_context_len + pool->block_size - 1) / pool->block_size
                           : 1;
  const SharedIn in{nullptr, nullptr, num_groups, max_group_size, max_prefix_len, max_tail_len};
  if (plan_shared(num_seqs, num_q_heads, maxb > 0 ? maxb : 1, max_context_len, in, partition,
                  pool, &plan, &sd) != PKV_OK)
    return 0;
  return plan.ws_bytes;
}

pkv_status pkv_decode_shared(const void* q, int32_t num_seqs, int32_t num_q_heads,
                             const void* k_pool, const void* v_pool, const pkv_pool_desc* pool,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len,
                             const int32_t* group_start, const int32_t* prefix_lens,
                             int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len,
                             int32_t max_tail_len, float scale, int32_t partition, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const SharedIn in{group_start, prefix_lens, num_groups, max_group_size, max_prefix_len,
                    max_tail_len};
  return decode_impl(Phase::kBoth, q, num_seqs, num_q_heads, k_pool, v_pool, pool, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, scale, partition, out,
                     workspace, workspace_bytes, stream, nullptr, nullptr, &in);
}

pkv_status pkv_prefill(const void* q, const int32_t* cu_q, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_q_len, int32_t total_q_rows, const void* k_pool,
                       const void* v_pool, const pkv_pool_desc* pool,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t max_context_len, float scale,
                       void* out, void* stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_q_heads < 1 || max_q_len < 0 || total_q_rows < 0 ||
      max_blocks_per_seq < 1 || max_context_len < 0) {
    set_error("bad sizes: num_seqs %d, num_q_heads %d, max_q_len %d, total_q_rows %d, "
              "max_blocks_per_seq %d, max_context_len %d", num_seqs, num_q_heads, max_q_len,
              total_q_rows, max_blocks_per_seq, max_context_len);
    return PKV_ERR_SHAPE;
  }
  if (num_q_heads % pool->num_kv_heads != 0) {
    set_error("num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
              pool->num_kv_heads);
    return PKV_ERR_SHAPE;
  }
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * pool->block_size) {
    set_error("max_context_len %d exceeds max_blocks_per_seq * block_size", max_context_len);
    return PKV_ERR_SHAPE;
  }
  const int rep = num_q_heads / pool->num_kv_heads;
  if (!prefill_supported(pool->dtype, pool->head_dim, rep)) {
    set_error("prefill: head_dim %d with group size %d is not compiled", pool->head_dim, rep);
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0 || total_q_rows == 0 || max_q_len == 0) return PKV_OK;
  if (!q || !cu_q || !k_pool || !v_pool || !block_tables || !context_lens || !out) {
    set_error("NULL pointer among q, cu_q, k_pool, v_pool, block_tables, context_lens, out");
    return PKV_ERR_NULL;
  }
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool)) {
    set_error("q, out, k_pool and v_pool must be 16-byte aligned");
    return PKV_ERR_ALIGN;
  }
  if (!std::isfinite(scale)) {
    set_error("scale must be finite");
    return PKV_ERR_SHAPE;
  }
  if (num_seqs > 65535) {
    set_error("num_seqs %d exceeds 65535", num_seqs);
    return PKV_ERR_UNSUPPORTED;
  }
  PrefillArgs a{};
  a.q = q;
  a.cu_q = cu_q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = block_tables;
  a.ctx_lens = context_lens;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_blocks = pool->num_blocks;
  a.block_shift = ilog2(pool->block_size);
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.max_q_len = max_q_len;
  a.total_q = total_q_rows;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return launch_prefill(a, pool->dtype, pool->head_dim, rep,
                        reinterpret_cast<hipStream_t>(stream));
}

size_t pkv_validate_workspace_bytes(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1) return 0;
  const int64_t slots = (int64_t)num_blocks * block_size;
  return (size_t)((slots + 31) / 32) * 4;
}

pkv_status pkv_validate(const int32_t* slot_mapping, int32_t num_tokens,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                        int32_t block_size, void* workspace, size_t workspace_bytes,
                        int32_t* report, void* stream) {
  if (!report) {
    set_error("report must not be NULL");
    return PKV_ERR_NULL;
  }
  if (num_tokens < 0 || num_seqs < 0 || num_blocks < 1) {
    set_error("bad sizes: num_tokens %d, num_seqs %d, num_blocks %d", num_tokens, num_seqs,
              num_blocks);
    return PKV_ERR_SHAPE;
  }
  if (!is_pow2(block_size) || block_size > 256) {
    set_error("block_size %d must be a power of two in [1, 256]", block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if ((int64_t)num_blocks * block_size > INT32_MAX) {
    set_error("num_blocks * block_size exceeds int32 slots");
    return PKV_ERR_UNSUPPORTED;
  }
  const bool slots = slot_mapping && num_tokens > 0;
  const bool tables = block_tables && num_seqs > 0;
  if (num_seqs > 0 && block_tables && (!context_lens || max_blocks_per_seq < 1)) {
    set_error("checking tables needs context_lens and max_blocks_per_seq >= 1");
    return context_lens ? PKV_ERR_SHAPE : PKV_ERR_NULL;
  }
  if (slots) {
    const size_t need = pkv_validate_workspace_bytes(num_blocks, block_size);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 3)) {
      set_error("checking slots needs a zeroed, 4-byte aligned workspace of %zu bytes "
                "(got %zu)", need, workspace_bytes);
      return PKV_ERR_WORKSPACE;
    }
  }
  ValidateArgs a;
  a.slots = slot_mapping;
  a.tables = block_tables;
  a.ctx_lens = context_lens;
  a.bits = static_cast<uint32_t*>(workspace);
  a.report = report;
  a.pool_slots = (int64_t)num_blocks * block_size;
  a.num_tokens = slots ? num_tokens : 0;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = tables ? num_seqs : 0;
  a.block_shift = ilog2(block_size);
  a.num_blocks = num_blocks;
  launch_validate(a, reinterpret_cast<hipStream_t>(stream));
  return launch_status("validate kernels");
}

int64_t pkv_block_bytes(int32_t num_layers, int32_t block_size, int32_t num_kv_heads,
                        int32_t head_dim, int32_t itemsize) {
  if (num_layers < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1 || itemsize < 1)
    return 0;
  int64_t bytes = 2;
  for (const int32_t f : {num_layers, block_size, num_kv_heads, head_dim, itemsize})
    if (__builtin_mul_overflow(bytes, (int64_t)f, &bytes)) {
      set_error("block bytes 2 * %d * %d * %d * %d * %d exceed int64", num_layers, block_size,
                num_kv_heads, head_dim, itemsize);
      return -1;
    }
  return bytes;
}

pkv_status pkv_plan_pool(int64_t free_bytes, int64_t total_bytes, double utilization,
                         int64_t activation_bytes, int64_t block_bytes, int32_t block_size,
                         int32_t max_model_len, int64_t* num_blocks,
                         int64_t* requests_at_max_len) {
  if (!num_blocks || !requests_at_max_len) {
    set_error("num_blocks and requests_at_max_len must not be NULL");
    return PKV_ERR_NULL;
  }
  if (free_bytes < 0 || total_bytes < 0 || activation_bytes < 0 || block_bytes < 1 ||
      block_size < 1 || max_model_len < 0 || !(utilization > 0.0 && utilization <= 1.0)) {
    set_error("bad sizes: free %lld, total %lld, utilization %g, activation %lld, block_bytes "
              "%lld, block_size %d, max_model_len %d", (long long)free_bytes,
              (long long)total_bytes, utilization, (long long)activation_bytes,
              (long long)block_bytes, block_size, max_model_len);
    return PKV_ERR_SHAPE;
  }
  // reserve = (1 - utilization) * total, rounded up to whole bytes
  const long double reserve = (1.0L - (long double)utilization) * (long double)total_bytes;
  const long double budget = (long double)free_bytes - reserve - (long double)activation_bytes;
  const long double q = budget > 0 ? budget / (long double)block_bytes : 0.0L;
  const int64_t blocks = q >= (long double)INT64_MAX ? INT64_MAX : (int64_t)q;
  const int64_t per_req = ((int64_t)max_model_len + block_size - 1) / block_size;
  *num_blocks = blocks;
  *requests_at_max_len = per_req > 0 ? blocks / per_req : 0;
  if (per_req > blocks) {
    set_error("a pool of %lld blocks cannot hold one request of %d tokens (%lld blocks); the "
              "longest it could serve is %lld tokens", (long long)blocks, max_model_len,
              (long long)per_req, (long long)(blocks * block_size));
    return PKV_ERR_CAPACITY;
  }
  return PKV_OK;
}

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_NULL: return "PKV_ERR_NULL";
    case PKV_ERR_DTYPE: return "PKV_ERR_DTYPE";
    case PKV_ERR_SHAPE: return "PKV_ERR_SHAPE";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_ALIGN: return "PKV_ERR_ALIGN";
    case PKV_ERR_CAPACITY: return "PKV_ERR_CAPACITY";
  }
  return "PKV_ERR_UNKNOWN";
}

const char* pkv_last_error(void) { return g_err; }

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

}  // extern "C"
