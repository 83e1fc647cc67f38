// Causal attention of packed query rows over the paged pool ("Build a Mini
// vLLM" section 4: scores + full((T,T), -inf).triu(1), softmax, weighted V),
// for a chunk of rows that ends at each sequence's last position.
//
// Row path: each query row is run as its own decode problem whose context is
// the row's causal prefix (positions 0 .. ctx - n + i), on the decode kernel
// with one split. It reads each row's prefix separately, so it is meant for
// fp32 data and short chunks; it also covers every (dtype, head_dim, group)
// the decode kernel supports.
#include "pkv_internal.h"

namespace pkv {

namespace {
constexpr int kMaxRowTableEntries = 4096;   // LDS slice of the table per row
}

bool prefill_supported(int dtype, int head_dim, int rep) {
  return decode_supported(dtype, head_dim, rep);
}

pkv_status launch_prefill(const PrefillArgs& p, int dtype, int head_dim, int rep,
                          hipStream_t st) {
  const int isz = dtype == PKV_F32 ? 4 : 2;
  const int tile = decode_tile_tokens(head_dim * isz);
  const int bs = 1 << p.block_shift;
  const int align = tile > bs ? tile : bs;
  const int lim = p.max_ctx < (p.max_blocks << p.block_shift) ? p.max_ctx
                                                               : (p.max_blocks << p.block_shift);
  int part = ((lim > 0 ? lim : 1) + align - 1) / align * align;
  if ((part >> p.block_shift) + 1 > kMaxRowTableEntries) {
    set_error("prefill: max_context_len %d is longer than the row path supports (%d tokens)",
              p.max_ctx, (kMaxRowTableEntries - 1) << p.block_shift);
    return PKV_ERR_UNSUPPORTED;
  }
  DecodeArgs a;
  a.q = p.q;
  a.k_pool = p.k_pool;
  a.v_pool = p.v_pool;
  a.tables = p.tables;
  a.ctx_lens = p.ctx_lens;
  a.out = p.out;
  a.ws_ml = nullptr;
  a.ws_o = nullptr;
  a.num_seqs = p.num_seqs;
  a.num_q_heads = p.num_q_heads;
  a.num_kv_heads = p.num_kv_heads;
  a.num_blocks = p.num_blocks;
  a.block_shift = p.block_shift;
  a.max_blocks = p.max_blocks;
  a.max_ctx = p.max_ctx;
  a.partition = part;
  a.num_splits = 1;
  a.scale_log2 = p.scale_log2;
  a.cu_q = p.cu_q;
  a.total_q = p.total_q;
  return launch_decode_partials(a, dtype, head_dim, rep, st);
}

}  // namespace pkv
