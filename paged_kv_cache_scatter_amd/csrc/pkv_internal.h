// Internal declarations shared by the host entry points and the kernel files.
// Device helpers here are written for gfx950 (wave64, CDNA DPP controls).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);   // records the thread-local message
pkv_status launch_status(const char* what);  // hipGetLastError -> status

// Compute units of the current device, looked up once per device with
// hipDeviceGetAttribute (the planners size their split counts and head pairing
// to it, so a device partitioned into fewer CUs gets its own plan). When no
// device is visible (a planning-only call on a host without a GPU) it is
// kDefaultCUs, MI355X's 256 (8 XCDs x 32).
constexpr int kDefaultCUs = 256;
int num_cus();

struct SlotArgs {
  const int32_t* tables;
  const int32_t* first_pos;
  const int32_t* cu;
  int32_t* slots;
  int32_t max_blocks, num_segments, num_tokens, block_shift, num_blocks;
};
void launch_slot_mapping(const SlotArgs& a, hipStream_t st);

struct WriteArgs {
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* slots;
  uint8_t* k_pool;
  uint8_t* v_pool;
  int64_t pool_slots;
  int32_t num_tokens;
  int32_t row_bytes;
};
void launch_write(const WriteArgs& a, bool vec16, int elem_bytes, hipStream_t st);

constexpr int kValidateFields = 5;
struct ValidateArgs {
  const int32_t* slots;
  const int32_t* tables;
  const int32_t* ctx_lens;
  uint32_t* bits;        // one bit per pool slot, zero on entry and on exit
  int32_t* report;       // kValidateFields counters
  int64_t pool_slots;
  int32_t num_tokens, max_blocks, num_seqs, block_shift, num_blocks;
};
void launch_validate(const ValidateArgs& a, hipStream_t st);

// Shared-prefix decode: groups of consecutive sequences whose block tables
// begin with the same blocks. Group i holds sequences group_start[i] ..
// group_start[i+1]-1 and shares its first prefix_lens[i] tokens (rounded down
// to whole blocks, capped by max_prefix and the table reach). A shared pass
// attends each group's shared tokens once for all its members and leaves its
// partials in workspace slots 0 .. prefix_slots-1 of every (sequence, head);
// the decode kernel covers the rest of each context from the prefix boundary
// into the following slots; the merge kernel combines both.
struct SharedDesc {
  const int32_t* group_start;   // nullptr: no sharing
  const int32_t* prefix_lens;
  int32_t num_groups;
  int32_t max_prefix;           // tokens
  int32_t prefix_part;          // tokens per shared-pass split
  int32_t prefix_slots;         // slots per (sequence, head) given to the shared pass
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* ctx_lens;
  void* out;
  float* ws_ml;       // [S, Hq, J, 2]  (m in log2 units, l)
  float* ws_o;        // [S, Hq, J, hd]
  int32_t num_seqs, num_q_heads, num_kv_heads, num_blocks;
  int32_t block_shift, max_blocks, max_ctx, partition, num_splits;
  float scale_log2;   // scale * log2(e)
  // Prefill rows: when cu_q is set, q/out hold total_q packed rows and row r of
  // sequence s (n_s rows) attends positions 0 .. ctx_s - n_s + (r - cu_q[s]).
  const int32_t* cu_q;
  int32_t total_q;
  // Fused decode step: when k_new is set, the new token of sequence s (rows
  // k_new/v_new[s] : [Hkv, hd]) sits at position ctx_s - 1; the workgroup of the
  // sequence's last split writes its head's rows into the pool slot and every
  // read of that position takes them from k_new/v_new.
  const void* k_new;
  const void* v_new;
  SharedDesc sh;
  // In-launch merge: when set, every workgroup of a sequence with more than
  // one partial counts itself in counters[s * Hkv + g] after writing its
  // partial; the last one merges the sequence's partials for KV head g and
  // sets the counter back to zero. Must be zero when the launch starts.
  int32_t* counters;
  // Piece schedule (sched_q > 0; no shared prefix, no prefill rows, at most
  // kSchedMaxSeqs sequences): each sequence's context is cut into pieces by
  // piece_counts; the grid's (y, z) plane enumerates all large pieces, then
  // all tail pieces, so that every workgroup stream is made of near-equal
  // pieces, the last ones short, and no empty workgroup precedes a live one.
  // Each workgroup derives its piece from context_lens by a workgroup scan.
  int32_t sched_q;       // small piece (tokens); partition and sched_q are powers of two
  int32_t sched_align;   // piece starts are multiples of it (a power of two)
  // Longest-first order for single-piece plans (at most kSchedMaxSeqs
  // sequences): the grid's (y, z) plane enumerates the sequences by length
  // class, longest class first (kLenClasses classes of the length range).
  // lpt_pass > 0: ranks are dealt in passes of lpt_pass sequences (the
  // workgroups one round of the CUs takes), every second pass reversed.
  int32_t sched_lpt;
  int32_t lpt_pass;
  // Stream-K ranges (sched_sk > 0: workgroups per KV head; no shared prefix,
  // no prefill rows, in-launch merge, a uniform-id kernel, at most
  // kSchedMaxSeqs sequences): each KV head's sequences are laid end to end
  // as one stream of sched_align-token units, every non-empty sequence
  // preceded by sk_alpha units that stand for the fixed cost of a piece
  // (they hold no tokens). The stream is cut into sched_sk ranges of at
  // least sk_min_units units, the first half of them sk_first_extra / 64
  // longer than the mean and the rest sharing what is left; workgroup i of
  // a head runs, one after another, the pieces of every sequence its range
  // touches. Piece k of a sequence is its part in the k-th range it touches
  // (its partial slot k).
  int32_t sched_sk;
  int32_t sk_min_units;
  int32_t sk_alpha;
  int32_t sk_first_extra;
  // Paired KV heads (> 0: the group size of the real heads): the pool is read
  // as num_kv_heads virtual heads of two adjacent real heads each (rows of
  // 2 * head_dim, the same bytes), a workgroup serving both groups' query
  // heads. Each query head takes its dot products over its own head's half
  // only; q and out keep the real head_dim, the workspace the virtual one.
  int32_t pair_rep;
};
constexpr int kLenClasses = 32;
constexpr int kSchedMaxSeqs = 1024;   // 4 sequences per thread of the scan

// Pieces of a context of L tokens under the piece schedule (P large, Q small
// piece, starts aligned to A; all three powers of two with A <= Q <= P and
// Q >= P / 2, given as log2: lp, lq, la): full pieces of P tokens, the last
// of which also takes a rest shorter than Q / 2; a longer rest, or a context
// shorter than P, is cut into tail = ceil(rest / Q) (1 or 2) pieces of
// `base` tokens (a multiple of A), the last taking what is left. An empty
// context is one empty tail piece. Tail pieces of at least 3/4 Q are "long":
// the schedule runs them before the short ones.
struct PieceCounts {
  int big, tail, base, nlong;
};
__host__ __device__ inline bool long_tail(int len, int lq) { return 4 * len >= (3 << lq); }
__host__ __device__ inline PieceCounts piece_counts(int L, int lp, int lq, int la) {
  PieceCounts c;
  c.big = L >> lp;
  const int r = L - (c.big << lp);
  if (c.big > 0 && 2 * r < (1 << lq)) {
    c.tail = 0;
    c.base = 0;
    c.nlong = 0;
  } else {
    c.tail = (r + (1 << lq) - 1) >> lq;
    c.tail = c.tail < 1 ? 1 : c.tail;
    c.base = ((r >> (c.tail - 1)) >> la) << la;
    if (c.base == 0) c.tail = 1;
    const int last = r - (c.tail - 1) * c.base;
    c.nlong = (long_tail(c.base, lq) ? c.tail - 1 : 0) + (long_tail(last, lq) ? 1 : 0);
  }
  return c;
}
// Longest piece the schedule makes (bounds the per-lane path's table slice).
__host__ __device__ inline int max_piece(int P, int Q) { return P + Q / 2; }
constexpr int kRowGridZ = 32768;   // rows per grid z-extent in prefill-row launches
// Token tile per wave for a row of `row_bytes` (K or V of one KV head).
int decode_tile_tokens(int row_bytes);
// Returns false if (dtype, head_dim, rep) is not compiled.
bool decode_supported(int dtype, int head_dim, int rep);
pkv_status launch_decode_partials(const DecodeArgs& a, int dtype, int head_dim, int rep,
                                  hipStream_t st);
pkv_status launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim,
                                hipStream_t st);

struct PrefillArgs {
  const void* q;
  const int32_t* cu_q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* ctx_lens;
  void* out;
  int32_t num_seqs, num_q_heads, num_kv_heads, num_blocks;
  int32_t block_shift, max_blocks, max_ctx, max_q_len, total_q;
  float scale_log2;
  // shared pass (sh.group_start set): partials go to the workspace, J slots
  // per (sequence, head); q/out rows are sequences, cu_q is unused
  SharedDesc sh;
  float* ws_ml;
  float* ws_o;
  int32_t num_slots;
  int32_t max_group;   // members of the largest group
};
bool prefill_supported(int dtype, int head_dim, int rep);
pkv_status launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int rep,
                          hipStream_t st);
// Shared pass of the shared-prefix decode (matrix cores).
bool shared_pass_supported(int dtype, int head_dim, int rep);
constexpr int kSharedAlign = 64;      // shared-pass split granularity (keys per LDS tile)
constexpr int kSharedMaxTbl = 2048;   // table entries one shared-pass split may span
constexpr int kSharedRows = 128;      // (member, head) rows per shared-pass workgroup
pkv_status launch_shared_pass(const PrefillArgs& a, int dtype, int head_dim, int rep,
                              hipStream_t st);

}  // namespace pkv

// ---------------------------------------------------------------- device side
namespace pkv {
namespace dev {

// DPP controls (GCN/CDNA encoding).
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowRor = 0x120;       // + n (1..15): rotate right within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float swz_xor16(float x) {
  // ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

__device__ __forceinline__ float xor32(float x) {
  return __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, x), 32));
}

// x (op) x of lane i ^ 16, and of lane i ^ 32, in VALU cross-lane moves:
// v_permlane16_swap / v_permlane32_swap of x with x leave rows 0 and 2
// (lanes 0-31) in one result and rows 1 and 3 (lanes 32-63) in the other, so
// one op joins each lane's row (half) with its partner's. The sum is the same
// in both lanes of a pair (addition commutes). The two results are taken out
// of the returned vector as scalars before any bit cast (a bit cast of a
// vector element reads the vector's first element).
template <bool MAX>
__device__ __forceinline__ float join16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  const float a = __uint_as_float(r0), b = __uint_as_float(r1);
  return MAX ? fmaxf(a, b) : a + b;
}
template <bool MAX>
__device__ __forceinline__ float join32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  const float a = __uint_as_float(r0), b = __uint_as_float(r1);
  return MAX ? fmaxf(a, b) : a + b;
}

// Sum over aligned groups of W consecutive lanes; every lane gets its group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (W >= 2) x += dpp<kQuadXor1>(x);
  if constexpr (W >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (W >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (W >= 16) x += dpp<kRowMirror>(x);
  if constexpr (W >= 32) x = join16<false>(x);
  if constexpr (W >= 64) x = join32<false>(x);
  return x;
}

// Sum over lanes that are congruent modulo STRIDE (STRIDE a power of two);
// every lane gets the sum of its residue class.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
  if constexpr (STRIDE <= 1) x += dpp<kRowRor + 1>(x);
  if constexpr (STRIDE <= 2) x += dpp<kRowRor + 2>(x);
  if constexpr (STRIDE <= 4) x += dpp<kRowRor + 4>(x);
  if constexpr (STRIDE <= 8) x += dpp<kRowRor + 8>(x);
  if constexpr (STRIDE <= 16) x = join16<false>(x);
  if constexpr (STRIDE <= 32) x = join32<false>(x);
  return x;
}

// Max over aligned groups of W lanes (W in {1..64}); every lane gets the max.
template <int W>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (W >= 2) x = fmaxf(x, dpp<kQuadXor1>(x));
  if constexpr (W >= 4) x = fmaxf(x, dpp<kQuadXor2>(x));
  if constexpr (W >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if constexpr (W >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  if constexpr (W >= 32) x = join16<true>(x);
  if constexpr (W >= 64) x = join32<true>(x);
  return x;
}

// Group of sequence s: the last i with group_start[i] <= s (0 if none).
__device__ __forceinline__ int group_of(const SharedDesc& d, int s) {
  int lo = 0, hi = d.num_groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (d.group_start[mid] <= s) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Shared tokens of group i: whole blocks, within [0, min(max_prefix, lim)].
__device__ __forceinline__ int shared_len(const SharedDesc& d, int i, int lim, int bshift) {
  int p = d.prefix_lens[i];
  p = p < 0 ? 0 : p;
  p = p > d.max_prefix ? d.max_prefix : p;
  p = p > lim ? lim : p;
  return (p >> bshift) << bshift;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 bits <-> fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs packed in 32-bit words, fp32 sum.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Direct-to-LDS staging: global_load_lds_dwordx4 writes lane i's 16 bytes
// at LDS address M0 + 16*i, without passing through registers. The LDS
// address is an M0 operand of the asm ("{m0}"), so the compiler writes M0
// itself and knows the statement reads it; the s_nop covers the wait state
// between that write and the load. The compiler does not see the LDS writes,
// so the waits on them are explicit. (The compiler builtin for these loads
// was measured slower: it tail-merges loads into 64-bit per-lane addresses and
// changes the waits; 94.2 against 82.0 us on the 192-sequence Llama-3.2-1B
// decode.)
// NT: non-temporal hint, for rows read once in a stream larger than the
// caches (the decode's K/V rows).
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(gaddr), "{m0}"(lds) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gaddr), "{m0}"(lds) : "memory");
}
template <bool NT = false>
__device__ __forceinline__ void dma16s(const char* sbase, uint32_t voff, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// The same for one 4-byte word per lane (lane i -> M0 + 4*i).
__device__ __forceinline__ void dma4(const void* gaddr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gaddr), "{m0}"(lds) : "memory");
}
// Device-coherent (agent-scope) store and loads of fp32 partials, read back
// in the same launch by a workgroup that may run on another XCD: the store is
// written through the XCD's L2, the loads are not served from a stale L2
// line (the in-launch merge of the decode kernel states what it relies on).
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_agent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
// The merge counter's add: returns the count before this workgroup's.
__device__ __forceinline__ int count_agent(int* p) {
  return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

}  // namespace dev
}  // namespace pkv
