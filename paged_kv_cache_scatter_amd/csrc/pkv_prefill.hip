// Attention of many query rows over the same paged keys, on matrix cores:
//  * causal prefill ("Build a Mini vLLM" section 4: a query sees keys at its
//    own and earlier positions only; softmax of the scores, weighted V) for a
//    chunk of rows that ends at each sequence's last position;
//  * the shared pass of the shared-prefix decode ("nano-vLLM" "Where the time
//    went" and "Next steps": a prompt shared by many sequences is read once per
//    step instead of once per sequence): the rows are (member, head) pairs of a
//    group of sequences whose tables begin with the same blocks, the keys one
//    split of the shared tokens, and the result a split partial (m, l, o) that
//    the decode merge combines with the member's own tail.
//
// Matrix-core path (bf16 or fp32 pools, head_dim 64 or 128). One workgroup (4
// waves) per (KV head g, tile of 128 rows[, key split]). The rows are (query,
// head-of-group) pairs, so every K/V row staged in LDS serves the whole GQA
// group and, in the shared pass, every member. Each wave owns NBLK blocks of
// 16 rows. Per tile of KT keys:
//   S^T = K . Q^T   K rows from LDS as the A operand, the wave's Q rows resident
//                   in registers as the B operand (bf16: v_mfma_f32_16x16x32_bf16,
//                   one 16-byte chunk = 8 dims per lane; fp32:
//                   v_mfma_f32_16x16x4_f32, the chunk's 4 dims in 4 products;
//                   lane group grp takes chunks grp, grp + 4, ... of its K row,
//                   so every lane reads whole 16-byte chunks and the dims are
//                   summed in that order). The transposed product leaves
//                   lane l holding 16 scores of query row l%16, which is the
//                   B-operand layout the PV product needs, so probabilities
//                   never leave registers.
//   softmax         online max/sum in the log2 domain; the row max is joined
//                   across the four 16-lane groups; the row sum stays per lane
//                   and is joined once at the end.
//   O^T += V^T.P^T  bf16: V^T fragments from ds_read_b64_tr_b16 transposing
//                   reads, 32 keys per product; fp32: one V element per lane,
//                   4 keys per product. The keys of each product are taken in
//                   the order the score layout produced them (the same
//                   permutation on both operands leaves the sum unchanged).
// K/V tiles are filled by global_load_lds_dwordx4 (double-buffered, one
// barrier per tile), with a per-row XOR swizzle of 16-byte chunks (below).
// Measured LDS read rates on gfx950 (bytes per clock per CU, 8 or more waves):
// the bf16 swizzle gives the transposing V reads 225-239 (conflict-free) but
// the 16-row K reads only 128, a 2-way bank conflict; swizzling K by r & 15
// instead gives K 231 and V 128. A layout with separate K and V swizzles,
// conflict-free on both, ran the chunked prefill in the same time, so the
// conflicts are not what bounds this kernel and the single layout is kept.
// Keys past the last
// visible one, and keys of invalid table entries, are loaded from a zero row
// and masked, so masked V rows contribute exactly 0. Workgroups are numbered
// so that all tiles of one (sequence or group, KV head) run on one XCD and
// share its L2; the prefill deals the (sequence, KV head) pairs to the XCDs
// in turn, which balances them.
//
// Prefill row path (other head sizes, very long tables): each query row is run
// as its own decode problem whose context is the row's causal prefix
// (positions 0 .. ctx - n + i), on the decode kernel with one split. It
// re-reads each row's prefix.
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
constexpr int KT = kSharedAlign;            // keys per LDS tile
constexpr int NBLK = 2;                     // 16-row blocks per wave
constexpr int kRows = kWaves * NBLK * 16;   // query rows per workgroup
constexpr int kMaxTbl = kSharedMaxTbl;      // table entries staged in LDS
constexpr int kXcds = 8;
static_assert(kRows == kSharedRows, "rows per workgroup");

// 512 zero bytes: the source of masked K/V rows (head_dim up to 128 fp32).
__device__ __attribute__((aligned(16))) unsigned char g_zero_row[512];

// T = uint16_t (bf16 bits) or float.
template <typename T, int HD>
struct MG {
  static constexpr int ISZ = (int)sizeof(T);
  static constexpr int ROWB = HD * ISZ;            // bytes of one K or V row
  static constexpr int NC = ROWB / 16;             // 16-byte chunks per row
  static constexpr int RPB = ROWB >= 256 ? 1 : 256 / ROWB;   // rows per 256-byte bank line
  static constexpr int TILEB = KT * ROWB;          // bytes of a K (or V) tile
  static constexpr int LOADS = TILEB / 1024 / kWaves;   // DMA ops per wave per tile
  static constexpr int KK = NC / 4;                // 16-byte chunk steps of the QK product
  static constexpr int DB = HD / 16;               // 16-dim blocks of O
  static constexpr int STAGE = 2 * TILEB;          // K tile then V tile
  static constexpr int LDS = 2 * STAGE + kMaxTbl * 4;
  static constexpr int MINB = LDS <= 80 * 1024 ? 2 : 1;   // workgroups per CU the LDS allows
  static_assert(LOADS >= 1 && LOADS * kWaves * 1024 == TILEB, "tile split");
  static_assert(HD == 64 || HD == 128, "head_dim 64 or 128");
  static_assert(ROWB <= 512, "zero row");
};

// Physical 16-byte chunk of logical chunk c in tile row r is c ^ swz(r).
// bf16: the 16 rows a K read touches get distinct chunks, and so do the 8 rows
// of each half-wave of a transposing V read (two adjacent logical chunks).
// Distinct chunks are not enough for the K reads on gfx950: a 16-byte read is
// conflict-free only when each group of 8 lanes also spreads over distinct
// 16-byte slots of a 128-byte half line, which this mapping does not give (K
// reads run 2-way conflicted; the V reads are conflict-free). fp32: the 16
// rows of a K read get distinct chunks modulo 16 (one 256-byte bank line), and
// the four rows r, r+4, r+8, r+12 of a V read get disjoint 64-byte quarters of
// the line.
template <typename T, int HD>
__device__ __forceinline__ int swz(int r) {
  using G = MG<T, HD>;
  if constexpr (G::ISZ == 4) {
    return r & 15;
  } else {
    const int t = r / G::RPB;
    return ((t & (G::NC / 2 - 1)) << 1) | ((t / (G::NC / 2)) & 1);
  }
}

template <typename T, int HD>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * MG<T, HD>::ROWB + ((c ^ swz<T, HD>(r)) << 4);
}

// Q^T fragment of one 16-byte chunk (B operand): 8 bf16 or 4 fp32 dims.
template <typename T>
struct QFrag;
template <>
struct QFrag<uint16_t> {
  using type = bf16x8_t;
};
template <>
struct QFrag<float> {
  using type = f32x4_t;
};

// S^T block += K rows (one 16-byte chunk per lane) x Q^T chunk.
template <typename T>
__device__ __forceinline__ f32x4_t qk_chunk(const unsigned char* kp,
                                            const typename QFrag<T>::type& q, f32x4_t acc) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kp);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, q, acc, 0, 0, 0);
  } else {
    const f32x4_t kf = *reinterpret_cast<const f32x4_t*>(kp);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], q[e], acc, 0, 0, 0);
    return acc;
  }
}

// What one workgroup computes: KV head g, keys [key_lo, key_hi) of the table
// row trow, rows (w, nb, l16) -> q/out row qrow (-1 = none), query head qhead,
// and the row sees keys [key_lo, rhi).
struct Work {
  int g;
  const int* trow;
  int key_lo, key_hi;
};

template <typename T, int HD, int REP, bool SHARED>
__device__ __forceinline__ void attend_rows(const PrefillArgs& a, const Work& wk,
                                            const int (&qrow)[NBLK], const int (&qhead)[NBLK],
                                            const int (&rhi)[NBLK], int slot, bool (&emit)[NBLK],
                                            unsigned char* smem) {
  using G = MG<T, HD>;
  using QF = typename QFrag<T>::type;
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = l & 15;
  const int grp = l >> 4;
  const int bshift = a.block_shift;
  const int key_lo = wk.key_lo, key_hi = wk.key_hi;

  // ---- stage the needed slice of the block table; invalid ids become -1
  int* tbl = reinterpret_cast<int*>(smem + 2 * G::STAGE);
  const int tb0 = key_lo >> bshift;
  const int ntbl = ((key_hi - 1) >> bshift) - tb0 + 1;
  int bad = 0;
  for (int i = tid; i < ntbl; i += kThreads) {
    const int b = wk.trow[tb0 + i];
    const bool ok = (unsigned)b < (unsigned)a.num_blocks;
    tbl[i] = ok ? b : -1;
    bad |= !ok;
  }
  const bool any_bad = __syncthreads_or(bad);

  // ---- Q^T fragments (B operand of S^T = K Q^T): row l16, chunk kk*4 + grp
  QF qf[NBLK][G::KK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    const T* qp = reinterpret_cast<const T*>(a.q) +
                  ((size_t)(qrow[nb] < 0 ? 0 : qrow[nb]) * a.num_q_heads + qhead[nb]) * HD +
                  grp * (16 / G::ISZ);
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) {
      QF v = *reinterpret_cast<const QF*>(qp + kk * 4 * (16 / G::ISZ));
      if (qrow[nb] < 0) v = QF{};
      qf[nb][kk] = v;
    }
  }
  int rmin = rhi[0];
#pragma unroll
  for (int nb = 1; nb < NBLK; ++nb) rmin = min(rmin, rhi[nb]);

  // ---- DMA geometry: wave w fills bytes [w*LOADS*1024, (w+1)*LOADS*1024) of
  // each tile; lane l of op i writes tile row dr[i], physical chunk pc[i].
  const int bmask = (1 << bshift) - 1;
  const size_t slot_bytes = (size_t)a.num_kv_heads * G::ROWB;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)wk.g * G::ROWB;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)wk.g * G::ROWB;
  int dr[G::LOADS], dc[G::LOADS];
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int o = (w * G::LOADS + i) * 1024 + 16 * l;
    dr[i] = o / G::ROWB;
    dc[i] = ((o % G::ROWB) >> 4) ^ swz<T, HD>(dr[i]);   // logical chunk to fetch
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // block id of each of the lane's rows of tile t (-1 past the keys or for an
  // invalid entry), read from LDS a tile before its loads are issued
  auto ids = [&](int t, int (&b)[G::LOADS]) {
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int key = key_lo + t * KT + dr[i];
      b[i] = key < key_hi ? tbl[(key >> bshift) - tb0] : -1;
    }
  };
  auto issue = [&](int t, const int (&bid)[G::LOADS]) {
    const uint32_t kdst = lds0 + (t & 1) * G::STAGE + w * G::LOADS * 1024;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int key = key_lo + t * KT + dr[i];
      const int b = bid[i];
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

  const int ntiles = (key_hi - key_lo + KT - 1) / KT;
  __builtin_amdgcn_s_waitcnt(0);   // q fragments and table reads are in
  int bnext[G::LOADS];
  ids(0, bnext);
  issue(0, bnext);
  if (ntiles > 1) ids(1, bnext);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();
    __syncthreads();   // tile t is in LDS; tile t-1's stage is free
    if (t + 1 < ntiles) {
      issue(t + 1, bnext);
      if (t + 2 < ntiles) ids(t + 2, bnext);   // consumed at the next issue
    }

    const unsigned char* kt = smem + (t & 1) * G::STAGE;
    const unsigned char* vt = kt + G::TILEB;
    const int k0 = key_lo + t * KT;

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
        const unsigned char* kp = kt + lds_off<T, HD>(r, kk * 4 + grp);
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb) sc[kb][nb] = qk_chunk<T>(kp, qf[nb][kk], sc[kb][nb]);
      }
    }

    // online softmax per row; p overwrites the scores. The mask test is
    // uniform over the tile: only the tiles that reach past a row's last
    // visible key (or hold an invalid block) run the masking pass. (Tested
    // inside the per-score loop it became a branch per score: 3.03 against
    // 2.93 ms for the LLaMA-2-70B layer's chunked prefill.)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) sc[kb][nb] *= a.scale_log2;
    if (any_bad || __any(k0 + KT > rmin)) {
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + kb * 16 + grp * 4 + i;
            const bool vis = key < rhi[nb] && (!any_bad || tbl[(key >> bshift) - tb0] >= 0);
            sc[kb][nb][i] = vis ? sc[kb][nb][i] : -INFINITY;
          }
    }
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kb][nb][i]);
      // the row's 16 lanes of each of the four lane groups: join the groups
      // with VALU cross-lane swaps (lanes i ^ 16, then i ^ 32)
      mx = join16<true>(mx);
      mx = join32<true>(mx);
      const float mn = fmaxf(m[nb], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[nb] - mu);
      const bool moved = __any(mn > m[nb]);
      m[nb] = mn;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = fast_exp2(sc[0][nb][i] - mu);
        const float e1 = fast_exp2(sc[1][nb][i] - mu);
        const float e2 = fast_exp2(sc[2][nb][i] - mu);
        const float e3 = fast_exp2(sc[3][nb][i] - mu);
        sum += (e0 + e1) + (e2 + e3);
        sc[0][nb][i] = e0;
        sc[1][nb][i] = e1;
        sc[2][nb][i] = e2;
        sc[3][nb][i] = e3;
      }
      lsum[nb] = lsum[nb] * alpha + sum;
      // no row's max moved: alpha is 1 everywhere and o needs no rescale
      // (nor does the next product have to wait for o's previous value)
      if (moved) {
#pragma unroll
        for (int d = 0; d < G::DB; ++d) o[d][nb] *= alpha;
      }
    }

    if constexpr (G::ISZ == 2) {
      // O^T += V^T P^T over the two 32-key halves of the tile; probabilities
      // rounded to bf16, keys kb*16 + grp*4 + i of half sb = kb / 2
      bf16x8_t pf[2][NBLK];
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) {
        f32x8_t p0v, p1v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p0v[i] = sc[0][nb][i];
          p0v[4 + i] = sc[1][nb][i];
          p1v[i] = sc[2][nb][i];
          p1v[4 + i] = sc[3][nb][i];
        }
        pf[0][nb] = __builtin_convertvector(p0v, bf16x8_t);
        pf[1][nb] = __builtin_convertvector(p1v, bf16x8_t);
      }
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
              (lds_i16x4_t*)(vt + lds_off<T, HD>(r0, cc) + half));
          const i16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(vt + lds_off<T, HD>(r1, cc) + half));
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int nb = 0; nb < NBLK; ++nb)
            o[d][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[sb][nb], o[d][nb], 0, 0, 0);
        }
      }
    } else {
      // O^T += V^T P^T four keys at a time: product (kb, i) takes key
      // kb*16 + grp*4 + i from lane group grp (A: V element of dim
      // d*16 + l16, B: the lane's own probability)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = kb * 16 + grp * 4 + i;
#pragma unroll
          for (int d = 0; d < G::DB; ++d) {
            const float vv = *reinterpret_cast<const float*>(
                vt + lds_off<T, HD>(r, d * 4 + (l16 >> 2)) + (l16 & 3) * 4);
#pragma unroll
            for (int nb = 0; nb < NBLK; ++nb)
              o[d][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, sc[kb][nb][i], o[d][nb], 0, 0, 0);
          }
        }
    }
  }

  // ---- lane holds dims d*16 + grp*4 .. +3 of row l16
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    float tot = lsum[nb];
    tot = join16<false>(tot);
    tot = join32<false>(tot);
    if constexpr (SHARED) {
      // split partial: running max (log2 units), exp-sum, unnormalised o
      if (!emit[nb]) continue;
      const size_t row = ((size_t)qrow[nb] * a.num_q_heads + qhead[nb]) * a.num_slots + slot;
      float* op = a.ws_o + row * HD + grp * 4;
#pragma unroll
      for (int d = 0; d < G::DB; ++d) *reinterpret_cast<f32x4_t*>(op + d * 16) = o[d][nb];
      if (grp == 0) *reinterpret_cast<float2*>(a.ws_ml + row * 2) = make_float2(m[nb], tot);
    } else {
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
      if (qrow[nb] < 0) continue;
      T* op = reinterpret_cast<T*>(a.out) + ((size_t)qrow[nb] * a.num_q_heads + qhead[nb]) * HD +
              grp * 4;
#pragma unroll
      for (int d = 0; d < G::DB; ++d) {
        const f32x4_t v = o[d][nb] * inv;
        if constexpr (G::ISZ == 2)
          *reinterpret_cast<bf16x4_t*>(op + d * 16) = __builtin_convertvector(v, bf16x4_t);
        else
          *reinterpret_cast<f32x4_t*>(op + d * 16) = v;
      }
    }
  }
}

// Workgroup index -> unit, so that consecutive units run on one XCD.
__device__ __forceinline__ int xcd_unit() {
  const int bid = blockIdx.x;
  const int per_xcd = gridDim.x / kXcds;
  return (bid % kXcds) * per_xcd + bid / kXcds;
}

// Workgroup index -> unit for units grouped T to a (sequence, KV head) pair:
// the pairs are dealt to the XCDs in turn (pair p to XCD p mod 8) and each
// pair's T units run together on its XCD, sharing its L2. With 8 KV heads
// every XCD gets one head of every sequence, so the XCDs get equal work
// whatever the lengths; dealing blocks of consecutive pairs instead gave the
// LLaMA-2-70B layer's chunked prefill one XCD 1.34 times the mean work
// (4.13 ms per call against 2.98 ms dealt in turn).
__device__ __forceinline__ int pair_xcd_unit(int T) {
  const int bid = blockIdx.x;
  const int x = bid % kXcds, k = bid / kXcds;
  return ((k / T) * kXcds + x) * T + k % T;
}

// Causal prefill: unit = (sequence, KV head, tile of QTP query positions).
template <typename T, int HD, int REP>
__global__ __launch_bounds__(kThreads, (MG<T, HD>::MINB)) void prefill_mfma_kernel(
    PrefillArgs a, int tiles_per_seq, int num_units) {
  constexpr int QTP = kRows / REP;   // query positions per workgroup
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int unit = pair_xcd_unit(tiles_per_seq);
  if (unit >= num_units) return;
  const int qt = unit % tiles_per_seq;
  const int g = (unit / tiles_per_seq) % a.num_kv_heads;
  const int s = unit / tiles_per_seq / a.num_kv_heads;

  const int cu0 = a.cu_q[s];
  const int n = a.cu_q[s + 1] - cu0;
  const int p0 = qt * QTP;
  if (p0 >= n) return;
  const int lim = min(a.max_ctx, a.max_blocks << a.block_shift);
  int c = a.ctx_lens[s];
  c = c < 0 ? 0 : (c > lim ? lim : c);
  const int pend = min(n, p0 + QTP);
  const int a_max = c - n + pend - 1;    // position of the tile's last query; keys 0..a_max

  const int l = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int qrow[NBLK], qhead[NBLK], rhi[NBLK];
  bool emit[NBLK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    const int r = (w * NBLK + nb) * 16 + (l & 15);
    const int i = p0 + r / REP;
    const bool ok = r < QTP * REP && i < n;
    qrow[nb] = ok ? cu0 + i : -1;
    qhead[nb] = g * REP + r % REP;
    rhi[nb] = ok ? c - n + i + 1 : a_max + 1;   // keys 0 .. position
    emit[nb] = ok;
  }

  if (a_max < 0) {   // every row precedes position 0: zeros
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      if (qrow[nb] < 0) continue;
      T* o = reinterpret_cast<T*>(a.out) + ((size_t)qrow[nb] * a.num_q_heads + qhead[nb]) * HD;
      for (int d = (l >> 4) * 4; d < HD; d += 16)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[d + e] = T{};
    }
    return;
  }
  Work wk;
  wk.g = g;
  wk.trow = a.tables + (size_t)s * a.max_blocks;
  wk.key_lo = 0;
  wk.key_hi = a_max + 1;
  attend_rows<T, HD, REP, false>(a, wk, qrow, qhead, rhi, 0, emit, smem);
}

// Shared pass: unit = (group, KV head, key split, tile of 128 (member, head) rows).
template <typename T, int HD, int REP>
__global__ __launch_bounds__(kThreads, (MG<T, HD>::MINB)) void shared_prefix_mfma_kernel(
    PrefillArgs a, int row_tiles, int key_splits, int num_units) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int wave_max[kWaves];
  const int unit = xcd_unit();
  if (unit >= num_units) return;
  const int rt = unit % row_tiles;
  const int ks = (unit / row_tiles) % key_splits;
  const int g = (unit / row_tiles / key_splits) % a.num_kv_heads;
  const int gi = unit / row_tiles / key_splits / a.num_kv_heads;

  const int S = a.num_seqs;
  int gs0 = a.sh.group_start[gi];
  gs0 = gs0 < 0 ? 0 : (gs0 > S ? S : gs0);
  int gs1 = a.sh.group_start[gi + 1];
  gs1 = gs1 < gs0 ? gs0 : (gs1 > S ? S : gs1);
  const int nmem = gs1 - gs0;
  if (rt * kRows >= nmem * REP) return;
  const int lim = min(a.max_ctx, a.max_blocks << a.block_shift);
  const int pre = shared_len(a.sh, gi, lim, a.block_shift);
  const int key_lo = ks * a.sh.prefix_part;
  if (key_lo >= pre) return;

  // keys past every member's context are never loaded
  const int tid = threadIdx.x;
  int cmax = 0;
  for (int i = tid; i < nmem; i += kThreads) {
    int c = a.ctx_lens[gs0 + i];
    c = c < 0 ? 0 : (c > lim ? lim : c);
    cmax = max(cmax, c);
  }
#pragma unroll
  for (int off = 32; off; off >>= 1) cmax = max(cmax, __shfl_xor(cmax, off));
  if ((tid & 63) == 0) wave_max[tid >> 6] = cmax;
  __syncthreads();
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) cmax = max(cmax, wave_max[ww]);
  const int key_hi = min(min(key_lo + a.sh.prefix_part, pre), cmax);
  if (key_hi <= key_lo) return;

  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int qrow[NBLK], qhead[NBLK], rhi[NBLK];
  bool emit[NBLK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    const int r = rt * kRows + (w * NBLK + nb) * 16 + (l & 15);
    const int mem = r / REP;
    const bool ok = mem < nmem;
    qrow[nb] = ok ? gs0 + mem : -1;
    qhead[nb] = g * REP + r % REP;
    int c = ok ? a.ctx_lens[gs0 + mem] : 0;
    c = c < 0 ? 0 : (c > lim ? lim : c);
    const int rl = min(c, pre);               // the member's shared tokens
    rhi[nb] = ok ? min(rl, key_hi) : key_hi;
    emit[nb] = ok && rl > key_lo;             // the merge counts this split
  }
  Work wk;
  wk.g = g;
  wk.trow = a.tables + (size_t)gs0 * a.max_blocks;
  wk.key_lo = key_lo;
  wk.key_hi = key_hi;
  attend_rows<T, HD, REP, true>(a, wk, qrow, qhead, rhi, ks, emit, smem);
}

template <typename T, int HD, int REP>
pkv_status launch_mfma(const PrefillArgs& p, hipStream_t st) {
  using G = MG<T, HD>;
  constexpr int QTP = kRows / REP;
  const int tiles_per_seq = (p.max_q_len + QTP - 1) / QTP;
  const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
  const int64_t units = pairs * tiles_per_seq;
  const int64_t grid = (pairs + kXcds - 1) / kXcds * kXcds * tiles_per_seq;   // see pair_xcd_unit
  if (grid > INT32_MAX) {
    set_error("prefill: %lld query tiles exceed the grid limit", (long long)units);
    return PKV_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL((prefill_mfma_kernel<T, HD, REP>), dim3((unsigned)grid), dim3(kThreads),
                     G::LDS, st, p, tiles_per_seq, (int)units);
  return launch_status("prefill_mfma_kernel");
}

template <typename T, int HD, int REP>
pkv_status launch_shared(const PrefillArgs& p, hipStream_t st) {
  using G = MG<T, HD>;
  const int64_t row_tiles = ((int64_t)p.max_group * REP + kRows - 1) / kRows;
  const int64_t key_splits = p.sh.prefix_slots;
  const int64_t units = (int64_t)p.sh.num_groups * p.num_kv_heads * key_splits * row_tiles;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds;
  if (grid > INT32_MAX || row_tiles > INT32_MAX) {
    set_error("shared pass: %lld work units exceed the grid limit", (long long)units);
    return PKV_ERR_UNSUPPORTED;
  }
  if (units == 0) return PKV_OK;
  hipLaunchKernelGGL((shared_prefix_mfma_kernel<T, HD, REP>), dim3((unsigned)grid),
                     dim3(kThreads), G::LDS, st, p, (int)row_tiles, (int)key_splits, (int)units);
  return launch_status("shared_prefix_mfma_kernel");
}

template <bool SHARED, typename T, int HD>
pkv_status mfma_rep(const PrefillArgs& p, int rep, hipStream_t st) {
  switch (rep) {
#define PKV_REP_CASE(R) \
    case R: return SHARED ? launch_shared<T, HD, R>(p, st) : launch_mfma<T, HD, R>(p, st);
    PKV_REP_CASE(1)
    PKV_REP_CASE(2)
    PKV_REP_CASE(3)
    PKV_REP_CASE(4)
    PKV_REP_CASE(5)
    PKV_REP_CASE(6)
    PKV_REP_CASE(7)
    PKV_REP_CASE(8)
#undef PKV_REP_CASE
    default: break;
  }
  set_error("matrix-core attention: group size %d is not compiled", rep);
  return PKV_ERR_UNSUPPORTED;
}

template <bool SHARED>
pkv_status mfma_dispatch(const PrefillArgs& p, int dtype, int head_dim, int rep,
                         hipStream_t st) {
  if (dtype == PKV_BF16)
    return head_dim == 64 ? mfma_rep<SHARED, uint16_t, 64>(p, rep, st)
                          : mfma_rep<SHARED, uint16_t, 128>(p, rep, st);
  return head_dim == 64 ? mfma_rep<SHARED, float, 64>(p, rep, st)
                        : mfma_rep<SHARED, float, 128>(p, rep, st);
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
  DecodeArgs a{};
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
  a.sh = SharedDesc{};
  return launch_decode_partials(a, dtype, head_dim, rep, st);
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int rep) {
  return decode_supported(dtype, head_dim, rep);
}

bool shared_pass_supported(int dtype, int head_dim, int rep) {
  return (dtype == PKV_BF16 || dtype == PKV_F32) && (head_dim == 64 || head_dim == 128) &&
         rep >= 1 && rep <= 8;
}

namespace {
bool uses_mfma(const PrefillArgs& p, int dtype, int head_dim, int rep) {
  if (!shared_pass_supported(dtype, head_dim, rep)) return false;
  const int lim = table_reach(p);
  return ((int64_t)lim + (1 << p.block_shift) - 1) >> p.block_shift <= kMaxTbl;
}
}  // namespace

pkv_status launch_prefill(const PrefillArgs& p, int dtype, int head_dim, int rep,
                          hipStream_t st) {
  if (!uses_mfma(p, dtype, head_dim, rep))
    return launch_rows(p, dtype, head_dim, rep, st);
  return mfma_dispatch<false>(p, dtype, head_dim, rep, st);
}

pkv_status launch_shared_pass(const PrefillArgs& p, int dtype, int head_dim, int rep,
                              hipStream_t st) {
  if (!shared_pass_supported(dtype, head_dim, rep)) {
    set_error("shared pass: dtype %d, head_dim %d, group %d not compiled", dtype, head_dim, rep);
    return PKV_ERR_UNSUPPORTED;
  }
  return mfma_dispatch<true>(p, dtype, head_dim, rep, st);
}

}  // namespace pkv
