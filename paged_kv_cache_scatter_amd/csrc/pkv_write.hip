// Slot mapping and the KV write (scatter) for gfx950.
//
// Slot of a token: "Build a Mini vLLM" section 2 (append_slot gives
// (table[pos // BLOCK], pos % BLOCK)), "Day 16: the paged KV cache, real K/V
// through scattered blocks" "What I added today" (a flat slot per token),
// "nano-vLLM" "How it works" (block table[n // 16], slot n % 16).
// Write: "Day 16" "What I learned" item 3 (pool[slots] = k, a scatter).
//
// The write moves each token's contiguous [num_kv_heads, head_dim] row (K and
// V) into its slot with one 16-byte vector copy per lane; consecutive lanes
// cover consecutive chunks of a row, so both the read of the new rows and the
// write into the pool are fully coalesced.
#include <algorithm>

#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ void __launch_bounds__(256) slot_mapping_kernel(SlotArgs a) {
  const int w = blockIdx.x;
  const int begin = a.cu[w];
  int end = a.cu[w + 1];
  if (end > a.num_tokens) end = a.num_tokens;
  const int first = a.first_pos[w];
  const int* row = a.tables + (size_t)w * a.max_blocks;
  const int bmask = (1 << a.block_shift) - 1;
  for (int t = begin + (int)threadIdx.x; t < end; t += 256) {
    if (t < 0) continue;
    const int pos = first + (t - begin);
    int slot = -1;
    if (pos >= 0) {
      const int bi = pos >> a.block_shift;
      if (bi < a.max_blocks) {
        const int blk = row[bi];
        if ((unsigned)blk < (unsigned)a.num_blocks) slot = (blk << a.block_shift) | (pos & bmask);
      }
    }
    a.slots[t] = slot;
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One thread per CHUNK-byte piece of a token row; blockIdx.y selects K (0) or V (1).
// Both sides are streamed with nontemporal hints: the new rows are read once,
// and the pool rows are not read again by this launch (a bulk write of
// 32,768 token rows of 2 KB runs 3.7% faster with them than without: 49.3
// against 51.1 us).
template <typename CHUNK>
__global__ void __launch_bounds__(256) write_kernel(WriteArgs a) {
  const int cpr = a.row_bytes / (int)sizeof(CHUNK);   // chunks per row
  const int64_t total = (int64_t)a.num_tokens * cpr;
  const CHUNK* src = reinterpret_cast<const CHUNK*>(blockIdx.y == 0 ? a.k : a.v);
  CHUNK* dst = reinterpret_cast<CHUNK*>(blockIdx.y == 0 ? a.k_pool : a.v_pool);
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int t = (int)(i / cpr);
    const int c = (int)(i - (int64_t)t * cpr);
    const int slot = a.slots[t];
    if (slot >= 0 && (int64_t)slot < a.pool_slots)
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + i),
                                  dst + (int64_t)slot * cpr + c);
  }
}

// Index checks for debugging ("Build a Mini vLLM" section 4: each token is
// written once; "nano-vLLM" "How it works": a table maps a sequence's blocks
// into the pool). The kernels of the path never check device indices against
// each other (that would need a synchronisation); these count what they would
// silently skip or mask. report: [0] negative slots, [1] slots past the pool,
// [2] duplicate slots, [3] invalid table entries a sequence needs, [4] context
// lengths outside the table's reach.
__global__ void __launch_bounds__(64) validate_zero_kernel(int32_t* report) {
  if (threadIdx.x < kValidateFields) report[threadIdx.x] = 0;
}

// One bit per pool slot: the first token to set a slot's bit owns it, every
// later one is a duplicate (k tokens on one slot count k - 1 in any order).
__global__ void __launch_bounds__(256) validate_slots_kernel(const int32_t* slots, int n,
                                                             int64_t pool_slots, uint32_t* bits,
                                                             int32_t* report) {
  int neg = 0, past = 0, dup = 0;
  const int stride = gridDim.x * 256;
  for (int t = blockIdx.x * 256 + threadIdx.x; t < n; t += stride) {
    const int s = slots[t];
    if (s < 0) {
      ++neg;
    } else if ((int64_t)s >= pool_slots) {
      ++past;
    } else {
      const uint32_t bit = 1u << (s & 31);
      if (atomicOr(bits + (s >> 5), bit) & bit) ++dup;
    }
  }
  if (neg) atomicAdd(report + 0, neg);
  if (past) atomicAdd(report + 1, past);
  if (dup) atomicAdd(report + 2, dup);
}

// Leaves the bitmap zero again (runs after validate_slots_kernel in stream order).
__global__ void __launch_bounds__(256) validate_clear_kernel(const int32_t* slots, int n,
                                                             int64_t pool_slots, uint32_t* bits) {
  const int stride = gridDim.x * 256;
  for (int t = blockIdx.x * 256 + threadIdx.x; t < n; t += stride) {
    const int s = slots[t];
    if (s >= 0 && (int64_t)s < pool_slots) atomicAnd(bits + (s >> 5), ~(1u << (s & 31)));
  }
}

// One workgroup per sequence: the entries of blocks 0 .. ceil(ctx / bs) - 1
// (within the table row) must name pool blocks.
__global__ void __launch_bounds__(256) validate_tables_kernel(const int32_t* tables,
                                                              int max_blocks,
                                                              const int32_t* ctx_lens,
                                                              int num_seqs, int block_shift,
                                                              int num_blocks, int32_t* report) {
  const int64_t reach = (int64_t)max_blocks << block_shift;
  for (int s = blockIdx.x; s < num_seqs; s += gridDim.x) {
    const int c = ctx_lens[s];
    if (threadIdx.x == 0 && (c < 0 || (int64_t)c > reach)) atomicAdd(report + 4, 1);
    const int64_t cc = c < 0 ? 0 : ((int64_t)c > reach ? reach : c);
    const int nb = (int)((cc + (1 << block_shift) - 1) >> block_shift);
    const int32_t* row = tables + (size_t)s * max_blocks;
    int bad = 0;
    for (int i = threadIdx.x; i < nb; i += 256) bad += (unsigned)row[i] >= (unsigned)num_blocks;
    if (bad) atomicAdd(report + 3, bad);
  }
}

}  // namespace

void launch_validate(const ValidateArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(validate_zero_kernel, dim3(1), dim3(64), 0, st, a.report);
  if (a.num_tokens > 0) {
    const int blocks = (int)std::min<int64_t>(((int64_t)a.num_tokens + 255) / 256, 4096);
    hipLaunchKernelGGL(validate_slots_kernel, dim3(blocks), dim3(256), 0, st, a.slots,
                       a.num_tokens, a.pool_slots, a.bits, a.report);
    hipLaunchKernelGGL(validate_clear_kernel, dim3(blocks), dim3(256), 0, st, a.slots,
                       a.num_tokens, a.pool_slots, a.bits);
  }
  if (a.num_seqs > 0) {
    const int blocks = std::min(a.num_seqs, 65535);
    hipLaunchKernelGGL(validate_tables_kernel, dim3(blocks), dim3(256), 0, st, a.tables,
                       a.max_blocks, a.ctx_lens, a.num_seqs, a.block_shift, a.num_blocks,
                       a.report);
  }
}

void launch_slot_mapping(const SlotArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(a.num_segments), dim3(256), 0, st, a);
}

void launch_write(const WriteArgs& a, bool vec16, int elem_bytes, hipStream_t st) {
  const int chunk = vec16 ? 16 : elem_bytes;
  const int64_t total = (int64_t)a.num_tokens * (a.row_bytes / chunk);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65535LL * 8) blocks = 65535LL * 8;   // grid-stride beyond this
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks, 2);
  if (vec16)
    hipLaunchKernelGGL(write_kernel<u32x4>, grid, dim3(256), 0, st, a);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(write_kernel<uint32_t>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(write_kernel<uint16_t>, grid, dim3(256), 0, st, a);
}

}  // namespace pkv
