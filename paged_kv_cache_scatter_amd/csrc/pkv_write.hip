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

// One thread per CHUNK-byte piece of a token row; blockIdx.y selects K (0) or V (1).
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
      dst[(int64_t)slot * cpr + c] = src[(int64_t)t * cpr + c];
  }
}

}  // namespace

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
    hipLaunchKernelGGL(write_kernel<uint4>, grid, dim3(256), 0, st, a);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(write_kernel<uint32_t>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(write_kernel<uint16_t>, grid, dim3(256), 0, st, a);
}

}  // namespace pkv
