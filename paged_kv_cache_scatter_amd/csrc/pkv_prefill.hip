// Causal attention of packed query rows over the paged pool ("Build a Mini
// vLLM" section 4: scores + full((T,T), -inf).triu(1), softmax, weighted V),
// for a chunk of rows that ends at each sequence's last position.
//
// Two paths:
//
// Matrix-core path (bf16 pools, head_dim 64 or 128). One workgroup (4 waves)
// per (sequence, KV head g, tile of query positions). The tile's rows are the
// (position, head-of-group) pairs, REP heads per position, so every K/V row
// staged in LDS serves the whole GQA group. Each wave owns NBLK blocks of 16
// rows. Per tile of KT keys:
//   S^T = K . Q^T   v_mfma_f32_16x16x32_bf16, K rows from LDS as the A operand,
//                   the wave's Q rows resident in registers as the B operand.
//                   The transposed product leaves lane l holding 16 scores of
//                   query row l%16, which is the B-operand layout the PV
//                   product needs, so probabilities never leave registers.
//   softmax         online max/sum in the log2 domain; the row max is joined
//                   across the four 16-lane groups; the row sum stays per lane
//                   and is joined once at the end.
//   O^T += V^T.P^T  V^T fragments come from ds_read_b64_tr_b16 transposing
//                   reads; the keys of a 32-key step are taken in the order the
//                   score layout produced them (the same permutation on both
//                   operands leaves the sum unchanged).
// K/V tiles are filled by global_load_lds_dwordx4 (double-buffered, one
// barrier per tile), with a per-row XOR swizzle of 16-byte chunks so that both
// the 16-row K reads and the transposing V reads hit distinct LDS banks. Keys
// past the tile's last visible position, and keys of invalid table entries,
// are loaded from a zero row, so masked V rows contribute exactly 0. Workgroups
// are numbered so that all tiles of one (sequence, KV head) run on one XCD and
// share its L2.
//
// Row path (everything else: fp32 pools, other head sizes, very long tables):
// each query row is run as its own decode problem whose context is the row's
// causal prefix (positions 0 .. ctx - n + i), on the decode kernel with one
// split. It re-reads each row's prefix.
#include "pkv_internal.h"

namespace pkv {

namespace {
using namespace dev;

constexpr int kMaxRowTableEntries = 4096;   // LDS slice of the table per row

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int KT = 64;                      // keys per LDS tile
constexpr int NBLK = 2;                     // 16-row blocks per wave
constexpr int kRows = kWaves * NBLK * 16;   // query rows per workgroup
constexpr int kMaxTbl = 2048;               // table entries staged in LDS
constexpr int kXcds = 8;

// 512 zero bytes: the source of masked K/V rows (any head_dim up to 256 bf16).
__device__ __attribute__((aligned(16))) unsigned char g_zero_row[512];

template <int HD>
struct MG {
  static constexpr int ROWB = HD * 2;              // bytes of one K or V row
  static constexpr int NC = ROWB / 16;             // 16-byte chunks per row
  static constexpr int RPB = 256 / ROWB;           // rows per 256-byte bank line
  static constexpr int TILEB = KT * ROWB;          // bytes of a K (or V) tile
  static constexpr int LOADS = TILEB / 1024 / kWaves;   // DMA ops per wave per tile
  static constexpr int KK = HD / 32;               // k-steps of the QK product
  static constexpr int DB = HD / 16;               // 16-dim blocks of O
  static constexpr int STAGE = 2 * TILEB;          // K tile then V tile
  static constexpr int LDS = 2 * STAGE + kMaxTbl * 4;
  static_assert(LOADS >= 1 && LOADS * kWaves * 1024 == TILEB, "tile split");
  static_assert(NC == 8 || NC == 16, "head_dim 64 or 128");
};

// Physical 16-byte chunk of logical chunk c in tile row r. For the 16 rows a
// K read touches, the chunks are distinct; for the 8 rows of each half-wave of
// a transposing V read (two adjacent logical chunks), the 16 chunks are too.
template <int HD>
__device__ __forceinline__ int swz(int r) {
  using G = MG<HD>;
  const int t = r / G::RPB;
  return ((t & (G::NC / 2 - 1)) << 1) | ((t / (G::NC / 2)) & 1);
}

template <int HD>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * MG<HD>::ROWB + ((c ^ swz<HD>(r)) << 4);
}

template <int HD, int REP>
__global__ __launch_bounds__(kThreads, 2) void prefill_mfma_kernel(PrefillArgs a,
                                                                   int tiles_per_seq,
                                                                   int num_units) {
  using G = MG<HD>;
  constexpr int QTP = kRows / REP;   // query positions per workgroup
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int bid = blockIdx.x;
  const int per_xcd = gridDim.x / kXcds;
  const int unit = (bid % kXcds) * per_xcd + bid / kXcds;
  if (unit >= num_units) return;
  const int qt = unit % tiles_per_seq;
  const int g = (unit / tiles_per_seq) % a.num_kv_heads;
  const int s = unit / tiles_per_seq / a.num_kv_heads;

  const int cu0 = a.cu_q[s];
  const int n = a.cu_q[s + 1] - cu0;
  const int p0 = qt * QTP;
  if (p0 >= n) return;
  const int bshift = a.block_shift;
  const int lim = min(a.max_ctx, a.max_blocks << bshift);
  int c = a.ctx_lens[s];
  c = c < 0 ? 0 : (c > lim ? lim : c);
  const int pend = min(n, p0 + QTP);
  const int a_min = c - n + p0;          // position of the tile's first query
  const int a_max = c - n + pend - 1;    // position of its last; keys 0..a_max

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = l & 15;
  const int grp = l >> 4;

  // ---- this lane's query rows: row (w, nb, l16) of the tile
  int arow[NBLK];
  int qrow[NBLK];    // packed q/out row, or -1
  int qhead[NBLK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    const int r = (w * NBLK + nb) * 16 + l16;
    const int i = p0 + r / REP;
    const bool ok = r < QTP * REP && i < n;
    qrow[nb] = ok ? cu0 + i : -1;
    qhead[nb] = g * REP + r % REP;
    arow[nb] = ok ? c - n + i : -1;
  }

  const int nkeys = a_max + 1;
  if (nkeys <= 0) {   // every row precedes position 0: zeros
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      if (qrow[nb] < 0) continue;
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) +
                    ((size_t)qrow[nb] * a.num_q_heads + qhead[nb]) * HD;
      for (int d = grp * 4; d < HD; d += 16) *reinterpret_cast<uint2*>(o + d) = make_uint2(0, 0);
    }
    return;
  }

  // ---- stage the needed slice of the block table; invalid ids become -1
  int* tbl = reinterpret_cast<int*>(smem + 2 * G::STAGE);
  const int ntbl = ((nkeys - 1) >> bshift) + 1;
  const int* trow = a.tables + (size_t)s * a.max_blocks;
  int bad = 0;
  for (int i = tid; i < ntbl; i += kThreads) {
    const int b = trow[i];
    const bool ok = (unsigned)b < (unsigned)a.num_blocks;
    tbl[i] = ok ? b : -1;
    bad |= !ok;
  }
  const bool any_bad = __syncthreads_or(bad);

  // ---- Q^T fragments (B operand of S^T = K Q^T): row l16, dims kk*32+grp*8..+7
  bf16x8_t qf[NBLK][G::KK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) +
                       ((size_t)(qrow[nb] < 0 ? 0 : qrow[nb]) * a.num_q_heads + qhead[nb]) * HD +
                       grp * 8;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qp + kk * 32);
      if (qrow[nb] < 0) v = bf16x8_t{};
      qf[nb][kk] = v;
    }
  }

  // ---- DMA geometry: wave w fills bytes [w*LOADS*1024, (w+1)*LOADS*1024) of
  // each tile; lane l of op i writes tile row dr[i], physical chunk pc[i].
  const int bmask = (1 << bshift) - 1;
  const size_t slot_bytes = (size_t)a.num_kv_heads * G::ROWB;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * G::ROWB;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * G::ROWB;
  int dr[G::LOADS], dc[G::LOADS];
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int o = (w * G::LOADS + i) * 1024 + 16 * l;
    dr[i] = o / G::ROWB;
    dc[i] = ((o % G::ROWB) >> 4) ^ swz<HD>(dr[i]);   // logical chunk to fetch
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int t) {
    const uint32_t kdst = lds0 + (t & 1) * G::STAGE + w * G::LOADS * 1024;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int key = t * KT + dr[i];
      const int b = key <= a_max ? tbl[key >> bshift] : -1;
      const char* kp;
      const char* vp;
      if (b >= 0) {
        const size_t off = ((size_t)(uint32_t)b << bshift | (uint32_t)(key & bmask)) * slot_bytes +
                           (dc[i] << 4);
        kp = kbase + off;
        vp = vbase + off;
      } else {
        kp = vp = reinterpret_cast<const char*>(g_zero_row) + (dc[i] << 4);
      }
      dma16(kp, kdst + i * 1024);
      dma16(vp, kdst + G::TILEB + i * 1024);
    }
  };

  f32x4_t o[G::DB][NBLK];
#pragma unroll
  for (int d = 0; d < G::DB; ++d)
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) o[d][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[NBLK], lsum[NBLK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    m[nb] = -INFINITY;
    lsum[nb] = 0.f;
  }

  const int ntiles = (nkeys + KT - 1) / KT;
  __builtin_amdgcn_s_waitcnt(0);   // q fragments and table reads are in
  issue(0);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();
    __syncthreads();   // tile t is in LDS; tile t-1's stage is free
    if (t + 1 < ntiles) issue(t + 1);

    const unsigned char* kt = smem + (t & 1) * G::STAGE;
    const unsigned char* vt = kt + G::TILEB;
    const int k0 = t * KT;

    // S^T blocks: keys kb*16 + grp*4 + i, row l16
    f32x4_t sc[4][NBLK];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) sc[kb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r = kb * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < G::KK; ++kk) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt + lds_off<HD>(r, kk * 4 + grp));
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb)
          sc[kb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nb][kk], sc[kb][nb], 0, 0, 0);
      }
    }

    // online softmax per row
    const bool masked = any_bad || k0 + KT - 1 > a_min;
    bf16x8_t pf[2][NBLK];
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sc[kb][nb][i] * a.scale_log2;
          if (masked) {
            const int key = k0 + kb * 16 + grp * 4 + i;
            const bool vis = key <= arow[nb] && (!any_bad || tbl[key >> bshift] >= 0);
            v = vis ? v : -INFINITY;
          }
          sc[kb][nb][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, swz_xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const float mn = fmaxf(m[nb], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[nb] - mu);
      m[nb] = mn;
      float sum = 0.f;
      f32x8_t p0v, p1v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = fast_exp2(sc[0][nb][i] - mu);
        const float e1 = fast_exp2(sc[1][nb][i] - mu);
        const float e2 = fast_exp2(sc[2][nb][i] - mu);
        const float e3 = fast_exp2(sc[3][nb][i] - mu);
        sum += (e0 + e1) + (e2 + e3);
        p0v[i] = e0;
        p0v[4 + i] = e1;
        p1v[i] = e2;
        p1v[4 + i] = e3;
      }
      lsum[nb] = lsum[nb] * alpha + sum;
      pf[0][nb] = __builtin_convertvector(p0v, bf16x8_t);
      pf[1][nb] = __builtin_convertvector(p1v, bf16x8_t);
#pragma unroll
      for (int d = 0; d < G::DB; ++d) o[d][nb] *= alpha;
    }

    // O^T += V^T P^T over the two 32-key halves of the tile
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int r0 = sb * 32 + grp * 4 + (l16 >> 2);
      const int r1 = r0 + 16;
      const int half = (l16 & 1) << 3;
      const int cq = (l16 & 3) >> 1;
#pragma unroll
      for (int d = 0; d < G::DB; ++d) {
        const int cc = d * 2 + cq;
        const i16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(vt + lds_off<HD>(r0, cc) + half));
        const i16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(vt + lds_off<HD>(r1, cc) + half));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb)
          o[d][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[sb][nb], o[d][nb], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store: lane holds dims d*16 + grp*4 .. +3 of row l16
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    float tot = lsum[nb];
    tot += swz_xor16(tot);
    tot += xor32(tot);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (qrow[nb] < 0) continue;
    __bf16* op = reinterpret_cast<__bf16*>(a.out) +
                 ((size_t)qrow[nb] * a.num_q_heads + qhead[nb]) * HD + grp * 4;
#pragma unroll
    for (int d = 0; d < G::DB; ++d) {
      const f32x4_t v = o[d][nb] * inv;
      *reinterpret_cast<bf16x4_t*>(op + d * 16) = __builtin_convertvector(v, bf16x4_t);
    }
  }
}

template <int HD, int REP>
pkv_status launch_mfma(const PrefillArgs& p, hipStream_t st) {
  using G = MG<HD>;
  constexpr int QTP = kRows / REP;
  const int tiles_per_seq = (p.max_q_len + QTP - 1) / QTP;
  const int64_t units = (int64_t)p.num_seqs * p.num_kv_heads * tiles_per_seq;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds;
  if (grid > INT32_MAX) {
    set_error("prefill: %lld query tiles exceed the grid limit", (long long)units);
    return PKV_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL((prefill_mfma_kernel<HD, REP>), dim3((unsigned)grid), dim3(kThreads), G::LDS,
                     st, p, tiles_per_seq, (int)units);
  return launch_status("prefill_mfma_kernel");
}

template <int HD>
pkv_status mfma_rep(const PrefillArgs& p, int rep, hipStream_t st) {
  switch (rep) {
    case 1: return launch_mfma<HD, 1>(p, st);
    case 2: return launch_mfma<HD, 2>(p, st);
    case 3: return launch_mfma<HD, 3>(p, st);
    case 4: return launch_mfma<HD, 4>(p, st);
    case 5: return launch_mfma<HD, 5>(p, st);
    case 6: return launch_mfma<HD, 6>(p, st);
    case 7: return launch_mfma<HD, 7>(p, st);
    case 8: return launch_mfma<HD, 8>(p, st);
    default: break;
  }
  set_error("prefill: group size %d is not compiled", rep);
  return PKV_ERR_UNSUPPORTED;
}

int table_reach(const PrefillArgs& p) {
  const int64_t reach = (int64_t)p.max_blocks << p.block_shift;
  return (int)(p.max_ctx < reach ? p.max_ctx : reach);
}

pkv_status launch_rows(const PrefillArgs& p, int dtype, int head_dim, int rep, hipStream_t st) {
  const int isz = dtype == PKV_F32 ? 4 : 2;
  const int tile = decode_tile_tokens(head_dim * isz);
  const int bs = 1 << p.block_shift;
  const int align = tile > bs ? tile : bs;
  const int lim = table_reach(p);
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
  a.k_new = nullptr;
  a.v_new = nullptr;
  return launch_decode_partials(a, dtype, head_dim, rep, st);
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int rep) {
  return decode_supported(dtype, head_dim, rep);
}

namespace {
bool uses_mfma(const PrefillArgs& p, int dtype, int head_dim, int rep) {
  if (dtype != PKV_BF16 || (head_dim != 64 && head_dim != 128) || rep < 1 || rep > 8) return false;
  const int lim = table_reach(p);
  return ((int64_t)lim + (1 << p.block_shift) - 1) >> p.block_shift <= kMaxTbl;
}
}  // namespace

pkv_status launch_prefill(const PrefillArgs& p, int dtype, int head_dim, int rep,
                          hipStream_t st) {
  if (!uses_mfma(p, dtype, head_dim, rep))
    return launch_rows(p, dtype, head_dim, rep, st);
  return head_dim == 64 ? mfma_rep<64>(p, rep, st) : mfma_rep<128>(p, rep, st);
}

}  // namespace pkv
