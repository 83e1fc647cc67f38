// Paged decode attention for gfx950: reads each sequence's K/V blocks in place
// through its block table (no gathered copy), GQA group sharing, online softmax,
// split-K partials plus a merge kernel.
//
// What is computed follows "Build a Mini vLLM" section 3 "PagedAttention"
// (gather in table order, repeat KV heads onto query heads, softmax of
// scale * q.k, weighted sum of V) and "nano-vLLM" "How it works" (masked
// attention over padded tables, query heads grouped on their K/V head). The
// pages gather a contiguous copy first; here the blocks are read where they lie.
//
// Work decomposition: one workgroup (4 waves) per (KV head g, split j,
// sequence s). The split's slice of the block table is staged in LDS once.
// Each wave takes token tiles of TILE tokens in turn (tiles w, w+4, ...):
//   K stage   lanes own (token, two 16-byte chunks of its K row); the REP query
//             heads of the group sit in registers, so each K row is read once
//             for the whole group. The partial dot products of a token are
//             combined across its lanes by a DPP reduce-scatter that leaves each
//             lane holding the complete score of one head (or a few).
//   softmax   each lane runs the online max/sum for its own head(s) over its
//             tokens; a strided DPP max joins the lanes of one head. Every exp
//             is computed once. Probabilities go to a small LDS tile.
//   V stage   lanes own (token, one 16-byte chunk of its V row); probabilities
//             are broadcast reads from LDS; o[REP][chunk] accumulates in fp32.
//             The rescale of o is skipped when no head's running max moved.
// Loads are software-pipelined across tiles: the next tile's K rows are issued
// as soon as this tile's scores are formed, its V rows as soon as this tile's
// V has been consumed. Only the split's last partial tile (or a split with an
// invalid table entry) takes the masked, unpipelined path.
// At the end the four waves' (m, l, o) are merged in LDS and either the
// normalised output (single split) or the split partial is written.
#include "pkv_internal.h"

#include <math.h>

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

constexpr int pow2ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <typename T, int HD, int REP>
struct Geo {
  static constexpr int ISZ = (int)sizeof(T);
  static constexpr int ROWB = HD * ISZ;  // bytes of one K (or V) row of one KV head
  static constexpr int EPC = 16 / ISZ;   // elements per 16-byte chunk
  // tokens per tile: 8 KB of K plus V per wave and tile (at most 64 tokens)
  static constexpr int TILE = ROWB >= 1024 ? 4 : ROWB >= 512 ? 8 : ROWB >= 256 ? 16 : ROWB >= 128 ? 32 : 64;
  static constexpr int KCH = ROWB >= 32 ? 2 : 1;    // K chunks per lane per row
  static constexpr int LPT_K = ROWB / (16 * KCH);   // lanes per token (K stage)
  static constexpr int TPW_K = 64 / LPT_K;          // tokens per wave load (K)
  static constexpr int RK = TILE / TPW_K;           // K rows per lane per tile
  static constexpr int LPT_V = ROWB / 16;           // lanes per token (V stage)
  static constexpr int TPW_V = 64 / LPT_V;
  static constexpr int RV = TILE / TPW_V;           // V rows per lane per tile
  // heads after the reduce-scatter of the K stage
  static constexpr int REPP = pow2ceil(REP);        // heads padded to a power of two
  static constexpr int RS = REPP < LPT_K ? REPP : LPT_K;   // lanes one head set spreads over
  static constexpr int HPL = REPP / RS;             // heads per lane
  static constexpr int DUP = LPT_K / RS;            // lanes holding the same heads
  static_assert(RK >= 1 && RV >= 1 && LPT_K >= 1 && LPT_K <= 32 && LPT_V <= 64, "geometry");
};

__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <typename T>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc);

template <>
__device__ __forceinline__ float chunk_dot<float>(const uint4& q, const uint4& k, float acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<uint16_t>(const uint4& q, const uint4& k, float acc) {
  acc = dot2_bf16(q.x, k.x, acc);
  acc = dot2_bf16(q.y, k.y, acc);
  acc = dot2_bf16(q.z, k.z, acc);
  acc = dot2_bf16(q.w, k.w, acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ void chunk_to_f32(const uint4& c, float* v);

template <>
__device__ __forceinline__ void chunk_to_f32<float>(const uint4& c, float* v) {
  v[0] = __uint_as_float(c.x);
  v[1] = __uint_as_float(c.y);
  v[2] = __uint_as_float(c.z);
  v[3] = __uint_as_float(c.w);
}

template <>
__device__ __forceinline__ void chunk_to_f32<uint16_t>(const uint4& c, float* v) {
  v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x);
  v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
  v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z);
  v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16 and packed (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16_rne(x); }

// Partner lane of a W-lane token group for one reduction step: lane i of each
// aligned W-lane segment is paired with the lane W/2 away in the other half
// (i <-> W-1-i for W = 8, 16; i <-> i^(W/2) otherwise).
template <int W>
__device__ __forceinline__ float pair_lane(float x) {
  if constexpr (W == 2) return dpp<kQuadXor1>(x);
  else if constexpr (W == 4) return dpp<kQuadXor2>(x);
  else if constexpr (W == 8) return dpp<kRowHalfMirror>(x);
  else if constexpr (W == 16) return dpp<kRowMirror>(x);
  else return swz_xor16(x);  // W == 32
}

// Reduce-scatter of N per-head partial sums over a W-lane token group. While
// more than HPL values remain, lanes in the upper half of each segment keep the
// upper half of the values and the others the lower half, each adding the
// partner's copy of what it keeps; once HPL values remain the remaining steps
// are plain sums. Values are compacted into cur[0 .. HPL).
template <int W, int N, int HPL>
__device__ __forceinline__ void reduce_scatter(float* cur, int kc) {
  if constexpr (W >= 2) {
    if constexpr (N > HPL) {
      constexpr int H = N / 2;
      const bool side = (kc & (W >> 1)) != 0;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const float keep = side ? cur[j + H] : cur[j];
        const float send = side ? cur[j] : cur[j + H];
        cur[j] = keep + pair_lane<W>(send);
      }
      reduce_scatter<W / 2, H, HPL>(cur, kc);
    } else {
#pragma unroll
      for (int j = 0; j < HPL; ++j) cur[j] += pair_lane<W>(cur[j]);
      reduce_scatter<W / 2, N, HPL>(cur, kc);
    }
  }
}

// First head a lane holds after reduce_scatter<W, N, HPL>.
template <int W, int N, int HPL>
__device__ __forceinline__ int head_base(int kc) {
  if constexpr (W >= 2 && N > HPL) {
    return ((kc & (W >> 1)) ? N / 2 : 0) + head_base<W / 2, N / 2, HPL>(kc);
  } else {
    return 0;
  }
}

// Max / sum over lanes congruent modulo STRIDE (power of two), result in every lane.
template <int STRIDE, bool MAX>
__device__ __forceinline__ float strided_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (STRIDE <= 1) x = op(x, dpp<kRowRor + 1>(x));
  if constexpr (STRIDE <= 2) x = op(x, dpp<kRowRor + 2>(x));
  if constexpr (STRIDE <= 4) x = op(x, dpp<kRowRor + 4>(x));
  if constexpr (STRIDE <= 8) x = op(x, dpp<kRowRor + 8>(x));
  if constexpr (STRIDE <= 16) x = op(x, swz_xor16(x));
  if constexpr (STRIDE <= 32) x = op(x, xor32(x));
  return x;
}

template <typename T, int HD, int REP>
struct WaveState {
  using G = Geo<T, HD, REP>;
  float m[G::HPL];          // running max (log2 units) of the lane's heads
  float lsum[G::HPL];       // this lane's share of the exp-sum of its heads
  float o[REP][G::EPC];     // unnormalised output chunk (V-stage layout)
};

struct SplitCtx {
  const char* kb;     // lane base into k_pool: + g*HD*isz + kc*16
  const char* vb;     // lane base into v_pool: + g*HD*isz + vc*16
  const char* kh;     // head base into k_pool: + g*HD*isz (uniform)
  const char* vh;     // head base into v_pool: + g*HD*isz (uniform)
  uint32_t koff;      // lane offset of its K chunk within a row group: kg*rsb + kc*16
  uint32_t voff;      // lane offset of its V chunk within a row group: vg*rsb + vc*16
  const int* tbl;     // LDS block ids of this split (-1 = invalid)
  int tbl_base;       // logical block index of tbl[0]
  int bshift;
  uint32_t blk_bytes; // bytes of one block of one pool (all heads)
  uint32_t rsb;       // bytes of one token row (all heads)
  int t1;             // end of the split (exclusive)
  float scale_log2;
};

template <typename T, int HD, int REP, bool MASKED>
__device__ __forceinline__ void load_k(const SplitCtx& c, int tb, int kg,
                                       uint4 (&kr)[Geo<T, HD, REP>::RK][Geo<T, HD, REP>::KCH],
                                       bool (&kval)[Geo<T, HD, REP>::RK]) {
  using G = Geo<T, HD, REP>;
  const int bmask = (1 << c.bshift) - 1;
#pragma unroll
  for (int r = 0; r < G::RK; ++r) {
    const int t = tb + r * G::TPW_K + kg;
    bool ok = true;
    int blk;
    if (MASKED) {
      blk = t < c.t1 ? c.tbl[(t >> c.bshift) - c.tbl_base] : -1;
      ok = blk >= 0;
      blk = ok ? blk : 0;
    } else {
      blk = c.tbl[(t >> c.bshift) - c.tbl_base];
    }
    kval[r] = ok;
    const char* p = c.kb + (uint64_t)(uint32_t)blk * c.blk_bytes +
                    (uint32_t)(t & bmask) * c.rsb;
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      if (MASKED) {
        kr[r][i] = make_uint4(0, 0, 0, 0);
        if (ok) kr[r][i] = ld16(p + i * G::LPT_K * 16);
      } else {
        kr[r][i] = ld16(p + i * G::LPT_K * 16);
      }
    }
  }
}

template <typename T, int HD, int REP, bool MASKED>
__device__ __forceinline__ void load_v(const SplitCtx& c, int tb, int vg,
                                       uint4 (&vr)[Geo<T, HD, REP>::RV]) {
  using G = Geo<T, HD, REP>;
  const int bmask = (1 << c.bshift) - 1;
#pragma unroll
  for (int r = 0; r < G::RV; ++r) {
    const int t = tb + r * G::TPW_V + vg;
    bool ok = true;
    int blk;
    if (MASKED) {
      blk = t < c.t1 ? c.tbl[(t >> c.bshift) - c.tbl_base] : -1;
      ok = blk >= 0;
      blk = ok ? blk : 0;
    } else {
      blk = c.tbl[(t >> c.bshift) - c.tbl_base];
    }
    const char* p = c.vb + (uint64_t)(uint32_t)blk * c.blk_bytes +
                    (uint32_t)(t & bmask) * c.rsb;
    if (MASKED) {
      vr[r] = make_uint4(0, 0, 0, 0);
      if (ok) vr[r] = ld16(p);
    } else {
      vr[r] = ld16(p);
    }
  }
}

// Full tiles when a wave's load row never straddles a block (tokens per wave
// load <= block size): the row's block id is one wave-uniform value, read once
// from LDS into a scalar register, and each lane only adds its fixed offset.
__device__ __forceinline__ const char* row_base(const SplitCtx& c, const char* head, int t) {
  const int blk = __builtin_amdgcn_readfirstlane(c.tbl[(t >> c.bshift) - c.tbl_base]);
  const uint32_t in_blk = (uint32_t)(t & ((1 << c.bshift) - 1));
  return head + (uint64_t)(uint32_t)blk * c.blk_bytes + in_blk * c.rsb;
}

template <typename T, int HD, int REP>
__device__ __forceinline__ void load_k_uni(const SplitCtx& c, int tb,
                                           uint4 (&kr)[Geo<T, HD, REP>::RK][Geo<T, HD, REP>::KCH]) {
  using G = Geo<T, HD, REP>;
#pragma unroll
  for (int r = 0; r < G::RK; ++r) {
    const char* base = row_base(c, c.kh, tb + r * G::TPW_K);
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) kr[r][i] = ld16(base + c.koff + i * G::LPT_K * 16);
  }
}

template <typename T, int HD, int REP>
__device__ __forceinline__ void load_v_uni(const SplitCtx& c, int tb,
                                           uint4 (&vr)[Geo<T, HD, REP>::RV]) {
  using G = Geo<T, HD, REP>;
#pragma unroll
  for (int r = 0; r < G::RV; ++r) vr[r] = ld16(row_base(c, c.vh, tb + r * G::TPW_V) + c.voff);
}

// Scores of the tile's K rows (log2 units), reduce-scattered to the lane's heads.
template <typename T, int HD, int REP, bool MASKED>
__device__ __forceinline__ void tile_scores(
    const SplitCtx& c, int kc, const uint4 (&qr)[REP][Geo<T, HD, REP>::KCH],
    const uint4 (&kr)[Geo<T, HD, REP>::RK][Geo<T, HD, REP>::KCH],
    const bool (&kval)[Geo<T, HD, REP>::RK],
    float (&sc)[Geo<T, HD, REP>::RK][Geo<T, HD, REP>::HPL]) {
  using G = Geo<T, HD, REP>;
#pragma unroll
  for (int r = 0; r < G::RK; ++r) {
    float acc[G::REPP];
#pragma unroll
    for (int h = 0; h < G::REPP; ++h) {
      acc[h] = 0.f;
      if (h < REP) {
#pragma unroll
        for (int i = 0; i < G::KCH; ++i) acc[h] = chunk_dot<T>(qr[h][i], kr[r][i], acc[h]);
      }
    }
    reduce_scatter<G::LPT_K, G::REPP, G::HPL>(acc, kc);
#pragma unroll
    for (int j = 0; j < G::HPL; ++j) {
      float s = acc[j] * c.scale_log2;
      if (MASKED) s = kval[r] ? s : -INFINITY;
      sc[r][j] = s;
    }
  }
}

// Online softmax of the lane's heads over the tile; writes probabilities (and,
// when some running max moved, the rescale factors) to the wave's LDS tile.
// Returns whether any head's running max moved in this wave.
template <typename T, int HD, int REP>
__device__ __forceinline__ bool tile_softmax(
    WaveState<T, HD, REP>& st, const float (&sc)[Geo<T, HD, REP>::RK][Geo<T, HD, REP>::HPL],
    int kg, int hb, bool dup0, float* pbuf, float* cbuf) {
  using G = Geo<T, HD, REP>;
  bool moved = false;
  float corr[G::HPL];
#pragma unroll
  for (int j = 0; j < G::HPL; ++j) {
    float tm = sc[0][j];
#pragma unroll
    for (int r = 1; r < G::RK; ++r) tm = fmaxf(tm, sc[r][j]);
    tm = strided_reduce<G::LPT_K, true>(tm);
    const float mold = st.m[j];
    const float mnew = fmaxf(mold, tm);
    moved |= mnew > mold;
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    corr[j] = fast_exp2(mold - mref);
    st.m[j] = mnew;
    float ps = 0.f;
    const int h = hb + j;
#pragma unroll
    for (int r = 0; r < G::RK; ++r) {
      const float p = fast_exp2(sc[r][j] - mref);
      ps += p;
      if (dup0 && h < REP) pbuf[(r * G::TPW_K + kg) * G::REPP + h] = p;
    }
    st.lsum[j] = fmaf(st.lsum[j], corr[j], dup0 ? ps : 0.f);
  }
  const bool any_moved = __any(moved);
  if (any_moved) {
#pragma unroll
    for (int j = 0; j < G::HPL; ++j) {
      const int h = hb + j;
      if (kg == 0 && dup0 && h < REP) cbuf[h] = corr[j];
    }
  }
  return any_moved;
}

template <typename T, int HD, int REP>
__device__ __forceinline__ void tile_pv(WaveState<T, HD, REP>& st,
                                        const uint4 (&vr)[Geo<T, HD, REP>::RV], int vg,
                                        bool rescale, const float* pbuf, const float* cbuf) {
  using G = Geo<T, HD, REP>;
  if (rescale) {
    float cr[G::REPP];
#pragma unroll
    for (int h = 0; h < REP; ++h) cr[h] = cbuf[h];
#pragma unroll
    for (int h = 0; h < REP; ++h)
#pragma unroll
      for (int e = 0; e < G::EPC; ++e) st.o[h][e] *= cr[h];
  }
  if constexpr (sizeof(T) == 2) {
    // bf16: two tokens at a time. Their probabilities are rounded to a bf16
    // pair and their V values for one dimension are packed side by side, so
    // one fp32-accumulating bf16 dot2 adds both tokens' terms.
    static_assert(G::RV % 2 == 0, "bf16 V rows come in pairs");
#pragma unroll
    for (int r = 0; r < G::RV; r += 2) {
      const float* pa = pbuf + (r * G::TPW_V + vg) * G::REPP;
      const float* pb = pbuf + ((r + 1) * G::TPW_V + vg) * G::REPP;
      uint32_t pp[G::REPP];
#pragma unroll
      for (int h = 0; h < REP; ++h) pp[h] = pack_bf16x2(pa[h], pb[h]);
      const uint32_t va[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
      const uint32_t vb[4] = {vr[r + 1].x, vr[r + 1].y, vr[r + 1].z, vr[r + 1].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = __builtin_amdgcn_perm(vb[q], va[q], 0x05040100u);  // dim 2q of a, b
        const uint32_t hi = __builtin_amdgcn_perm(vb[q], va[q], 0x07060302u);  // dim 2q+1
#pragma unroll
        for (int h = 0; h < REP; ++h) {
          st.o[h][2 * q] = dot2_bf16(pp[h], lo, st.o[h][2 * q]);
          st.o[h][2 * q + 1] = dot2_bf16(pp[h], hi, st.o[h][2 * q + 1]);
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < G::RV; ++r) {
      const float* pp = pbuf + (r * G::TPW_V + vg) * G::REPP;
      float pr[G::REPP];
#pragma unroll
      for (int h = 0; h < REP; ++h) pr[h] = pp[h];
      float v[G::EPC];
      chunk_to_f32<T>(vr[r], v);
#pragma unroll
      for (int h = 0; h < REP; ++h)
#pragma unroll
        for (int e = 0; e < G::EPC; ++e) st.o[h][e] = fmaf(pr[h], v[e], st.o[h][e]);
    }
  }
}

constexpr int kStages = 2;   // tiles in a wave's LDS ring

template <typename T, int HD, int REP>
struct Ring {
  using G = Geo<T, HD, REP>;
  static constexpr int LOADS = G::RK * G::KCH + G::RV;   // 16-byte loads per lane per tile
  static constexpr int STAGE = LOADS * 1024;              // bytes of one tile of one wave
};

// The wave's full tiles from tb (step kStep) up to t_end. Tiles stream into the
// wave's LDS ring kStages - 1 tiles ahead of the one being computed; each lane
// reads back exactly the 16-byte pieces it loaded (conflict-free).
template <typename T, int HD, int REP, bool UNI, int kStep>
__device__ __forceinline__ void full_tiles(const SplitCtx& c, WaveState<T, HD, REP>& st,
                                           const uint4 (&qr)[REP][Geo<T, HD, REP>::KCH], int tb,
                                           int t_end, int lane, int kg, int kc, int vg, int hb,
                                           bool dup0, float* pbuf, float* cbuf,
                                           const unsigned char* ring) {
  using G = Geo<T, HD, REP>;
  using R = Ring<T, HD, REP>;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const int bmask = (1 << c.bshift) - 1;
  auto issue = [&](int t, int stg) {
    const uint32_t base = ring_lds + stg * R::STAGE;
#pragma unroll
    for (int r = 0; r < G::RK; ++r) {
      const int tr = t + r * G::TPW_K;
      if (UNI) {
        const char* rb = row_base(c, c.kh, tr);
#pragma unroll
        for (int i = 0; i < G::KCH; ++i)
          dma16s(rb + i * G::LPT_K * 16, c.koff, base + (r * G::KCH + i) * 1024);
      } else {
        const int tt = tr + kg;
        const int blk = c.tbl[(tt >> c.bshift) - c.tbl_base];
        const char* p = c.kb + (uint64_t)(uint32_t)blk * c.blk_bytes + (uint32_t)(tt & bmask) * c.rsb;
#pragma unroll
        for (int i = 0; i < G::KCH; ++i)
          dma16(p + i * G::LPT_K * 16, base + (r * G::KCH + i) * 1024);
      }
    }
#pragma unroll
    for (int r = 0; r < G::RV; ++r) {
      const int tr = t + r * G::TPW_V;
      const uint32_t dst = base + (G::RK * G::KCH + r) * 1024;
      if (UNI) {
        dma16s(row_base(c, c.vh, tr), c.voff, dst);
      } else {
        const int tt = tr + vg;
        const int blk = c.tbl[(tt >> c.bshift) - c.tbl_base];
        dma16(c.vb + (uint64_t)(uint32_t)blk * c.blk_bytes + (uint32_t)(tt & bmask) * c.rsb, dst);
      }
    }
  };
  const int n = (t_end - 1 - tb) / kStep + 1;   // tiles of this wave
  // The prologue's own loads (q) are back before the ring starts. Issued as the
  // builtin so the compiler's wait bookkeeping sees it (and inserts no waits for
  // q inside the loop, where they would also stall on the ring's loads).
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int q = 0; q < kStages - 1; ++q)
    if (q < n) issue(tb + q * kStep, q);
  for (int k = 0; k < n; ++k) {
    if (k + kStages - 1 < n) {
      wait_lgkmcnt0();   // the stage about to be refilled has been read
      issue(tb + (k + kStages - 1) * kStep, (k + kStages - 1) % kStages);
      wait_vmcnt<(kStages - 1) * R::LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    const uint4* sp = reinterpret_cast<const uint4*>(ring + (k % kStages) * R::STAGE) + lane;
    uint4 kr[G::RK][G::KCH];
    uint4 vr[G::RV];
    bool kval[G::RK];
#pragma unroll
    for (int r = 0; r < G::RK; ++r)
#pragma unroll
      for (int i = 0; i < G::KCH; ++i) kr[r][i] = sp[(r * G::KCH + i) * 64];
#pragma unroll
    for (int r = 0; r < G::RV; ++r) vr[r] = sp[(G::RK * G::KCH + r) * 64];
    float sc[G::RK][G::HPL];
    tile_scores<T, HD, REP, false>(c, kc, qr, kr, kval, sc);
    const bool moved = tile_softmax<T, HD, REP>(st, sc, kg, hb, dup0, pbuf, cbuf);
    tile_pv<T, HD, REP>(st, vr, vg, moved, pbuf, cbuf);
  }
}

__host__ __device__ constexpr int round16(int b) { return (b + 15) & ~15; }

// Query heads of a group are split over HS waves when the group is large:
// each wave then holds q and o for REP/HS heads only (fewer registers, more
// resident waves); the HS waves of a pair read the same K/V rows.
template <int REP>
struct HeadSplit {
  static constexpr int HS = 1;
  static constexpr int REPW = REP / HS;              // query heads per wave
  static constexpr int NSTREAM = kWaves / HS;       // token streams per workgroup
};

template <typename T, int HD, int REP>
struct Lds {
  using H = HeadSplit<REP>;
  using G = Geo<T, HD, H::REPW>;
  static constexpr int kWaveFloats = G::TILE * G::REPP + G::REPP;   // probabilities + rescale
  static constexpr int kMergeFloats = H::REPW * (HD + 2);           // m, l, o per wave
  static constexpr int kRingBytes = kStages * Ring<T, HD, H::REPW>::STAGE;  // per wave
  __host__ __device__ static int ring_offset(int tbl_entries) {
    return round16(tbl_entries * 4) + kWaves * kWaveFloats * 4;
  }
  // The merge area reuses the front of LDS once every wave has left the tile loop.
  static int bytes(int tbl_entries) {
    const int loop = ring_offset(tbl_entries) + kWaves * kRingBytes;
    const int merge = kWaves * kMergeFloats * 4;
    return loop > merge ? loop : merge;
  }
};

template <typename T, int HD, int REP>
__global__ void __launch_bounds__(kThreads)
decode_partials_kernel(DecodeArgs a) {
  using H = HeadSplit<REP>;
  constexpr int REPW = H::REPW;
  using G = Geo<T, HD, REPW>;
  using L = Lds<T, HD, REP>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int g = blockIdx.x;
  int j = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int hh = w % H::HS, stream = w / H::HS;             // head half, token stream
  const int bshift = a.block_shift;
  const int lim = min(a.max_ctx, a.max_blocks << bshift);
  int qrow = s;   // row of q and out
  int ctx;
  if (a.cu_q) {
    // prefill row: its own causal context, one split
    qrow = blockIdx.y * gridDim.z + blockIdx.z;
    j = 0;
    if (qrow >= a.total_q) return;
    int lo = 0, hi = a.num_seqs;   // last sequence with cu_q[s] <= qrow
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_q[mid] <= qrow) lo = mid;
      else hi = mid;
    }
    s = lo;
    int c = a.ctx_lens[s];
    c = c < 0 ? 0 : (c > lim ? lim : c);
    const int n = a.cu_q[s + 1] - a.cu_q[s];
    ctx = c - n + (qrow - a.cu_q[s]) + 1;
    ctx = ctx < 0 ? 0 : (ctx > lim ? lim : ctx);
  } else {
    ctx = a.ctx_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > lim ? lim : ctx);
  }
  const int P = a.partition;
  const int nsplit = (ctx + P - 1) / P;
  const int hq0 = g * REP;
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)qrow * a.num_q_heads + hq0) * HD;

  if (j >= nsplit) {
    if (j == 0) {  // empty sequence: zeros
      for (int i = tid; i < REP * HD; i += kThreads) out[i] = from_f32<T>(0.f);
    }
    return;
  }
  const int t0 = j * P;
  const int t1 = min(ctx, t0 + P);

  const int tbl_entries = (P >> bshift) + 1;
  int* tbl = reinterpret_cast<int*>(smem);
  float* pbuf = reinterpret_cast<float*>(smem + round16(tbl_entries * 4)) + w * L::kWaveFloats;
  float* cbuf = pbuf + G::TILE * G::REPP;
  float* merge = reinterpret_cast<float*>(smem);
  const unsigned char* ring = smem + L::ring_offset(tbl_entries) + w * L::kRingBytes;

  // ---- stage this split's block ids in LDS (invalid ids become -1)
  const int tbl_base = t0 >> bshift;
  const int nb = ((t1 - 1) >> bshift) - tbl_base + 1;
  const int* trow = a.tables + (size_t)s * a.max_blocks + tbl_base;
  int bad = 0;
  for (int i = tid; i < nb; i += kThreads) {
    const int id = trow[i];
    const bool ok = (unsigned)id < (unsigned)a.num_blocks;
    tbl[i] = ok ? id : -1;
    bad |= !ok;
  }
  const int any_bad = __syncthreads_or(bad);

  // ---- this wave's query heads, in the K-stage lane layout
  const int kg = lane / G::LPT_K, kc = lane % G::LPT_K;
  const int vg = lane / G::LPT_V, vc = lane % G::LPT_V;
  const T* qp = reinterpret_cast<const T*>(a.q) +
                ((size_t)qrow * a.num_q_heads + hq0 + hh * REPW) * HD;
  uint4 qr[REPW][G::KCH];
#pragma unroll
  for (int h = 0; h < REPW; ++h)
#pragma unroll
    for (int i = 0; i < G::KCH; ++i)
      qr[h][i] = *reinterpret_cast<const uint4*>(qp + h * HD + (kc + i * G::LPT_K) * G::EPC);

  SplitCtx c;
  {
    const size_t head_off = (size_t)g * HD * G::ISZ;
    c.kh = reinterpret_cast<const char*>(a.k_pool) + head_off;
    c.vh = reinterpret_cast<const char*>(a.v_pool) + head_off;
    c.kb = c.kh + kc * 16;
    c.vb = c.vh + vc * 16;
    c.tbl = tbl;
    c.tbl_base = tbl_base;
    c.bshift = bshift;
    c.rsb = (uint32_t)a.num_kv_heads * HD * G::ISZ;
    c.blk_bytes = c.rsb << bshift;
    c.koff = (uint32_t)kg * c.rsb + kc * 16;
    c.voff = (uint32_t)vg * c.rsb + vc * 16;
    c.t1 = t1;
    c.scale_log2 = a.scale_log2;
  }
  const int hb = head_base<G::LPT_K, G::REPP, G::HPL>(kc);
  const bool dup0 = (kc & (G::DUP - 1)) == 0;

  WaveState<T, HD, REPW> st;
#pragma unroll
  for (int jj = 0; jj < G::HPL; ++jj) {
    st.m[jj] = -INFINITY;
    st.lsum[jj] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < REPW; ++h)
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) st.o[h][e] = 0.f;

  // ---- full tiles: pipelined; the partial last tile (or all, with a bad id): masked
  const int n_full = any_bad ? 0 : (t1 - t0) / G::TILE;
  const int n_tiles = (t1 - t0 + G::TILE - 1) / G::TILE;
  constexpr int kStep = H::NSTREAM * G::TILE;
  const int t_full_end = t0 + n_full * G::TILE;
  int tb = t0 + stream * G::TILE;
  if (tb < t_full_end) {
    const bool uni = G::TPW_K <= (1 << bshift) && G::TPW_V <= (1 << bshift);
    if (uni)
      full_tiles<T, HD, REPW, true, kStep>(c, st, qr, tb, t_full_end, lane, kg, kc, vg, hb,
                                          dup0, pbuf, cbuf, ring);
    else
      full_tiles<T, HD, REPW, false, kStep>(c, st, qr, tb, t_full_end, lane, kg, kc, vg, hb,
                                           dup0, pbuf, cbuf, ring);
    tb += ((t_full_end - 1 - tb) / kStep + 1) * kStep;
  }
  for (int k = (tb - t0) / G::TILE; k < n_tiles; k += H::NSTREAM) {
    const int tm = t0 + k * G::TILE;
    uint4 kr[G::RK][G::KCH];
    uint4 vr[G::RV];
    bool kval[G::RK];
    load_k<T, HD, REPW, true>(c, tm, kg, kr, kval);
    load_v<T, HD, REPW, true>(c, tm, vg, vr);
    float sc[G::RK][G::HPL];
    tile_scores<T, HD, REPW, true>(c, kc, qr, kr, kval, sc);
    const bool moved = tile_softmax<T, HD, REPW>(st, sc, kg, hb, dup0, pbuf, cbuf);
    tile_pv<T, HD, REPW>(st, vr, vg, moved, pbuf, cbuf);
  }

  // ---- per-wave totals, then merge the waves in LDS
  float* mw = merge + w * L::kMergeFloats;
#pragma unroll
  for (int jj = 0; jj < G::HPL; ++jj) st.lsum[jj] = strided_reduce<G::LPT_K, false>(st.lsum[jj]);
#pragma unroll
  for (int h = 0; h < REPW; ++h)
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) st.o[h][e] = strided_sum<G::LPT_V>(st.o[h][e]);
  __syncthreads();  // every wave is done with the table and tile buffers
  if (kg == 0 && dup0) {
#pragma unroll
    for (int jj = 0; jj < G::HPL; ++jj) {
      const int h = hb + jj;
      if (h < REPW) {
        mw[h] = st.m[jj];
        mw[REPW + h] = st.lsum[jj];
      }
    }
  }
  if (vg == 0) {
#pragma unroll
    for (int h = 0; h < REPW; ++h)
#pragma unroll
      for (int e = 0; e < G::EPC; ++e) mw[2 * REPW + h * HD + vc * G::EPC + e] = st.o[h][e];
  }
  __syncthreads();

  const int J = a.num_splits;
  for (int idx = tid; idx < REP * HD; idx += kThreads) {
    const int h = idx / HD, d = idx % HD;
    const int hw = h / REPW, hl = h % REPW;   // head half and head within it
    float M = -INFINITY;
#pragma unroll
    for (int ss = 0; ss < H::NSTREAM; ++ss)
      M = fmaxf(M, merge[(ss * H::HS + hw) * L::kMergeFloats + hl]);
    float Ls = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ss = 0; ss < H::NSTREAM; ++ss) {
        const float* mv = merge + (ss * H::HS + hw) * L::kMergeFloats;
        const float f = fast_exp2(mv[hl] - M);
        Ls = fmaf(mv[REPW + hl], f, Ls);
        O = fmaf(mv[2 * REPW + hl * HD + d], f, O);
      }
    }
    if (nsplit == 1) {
      out[h * HD + d] = from_f32<T>(Ls > 0.f ? O / Ls : 0.f);
    } else {
      const size_t row = ((size_t)s * a.num_q_heads + hq0 + h) * J + j;
      a.ws_o[row * HD + d] = O;
      if (d == 0) {
        a.ws_ml[row * 2] = M;
        a.ws_ml[row * 2 + 1] = Ls;
      }
    }
  }
}

// Merge split partials of sequences with more than one split: one wave per
// (query head, sequence).
template <typename T>
__global__ void __launch_bounds__(64) decode_reduce_kernel(DecodeArgs a, int head_dim) {
  extern __shared__ __align__(16) float wts[];
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int lim = min(a.max_ctx, a.max_blocks << a.block_shift);
  int ctx = a.ctx_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > lim ? lim : ctx);
  const int P = a.partition;
  const int nsplit = (ctx + P - 1) / P;
  if (nsplit <= 1) return;
  const int J = a.num_splits;
  const size_t row0 = ((size_t)s * a.num_q_heads + h) * J;
  const float* ml = a.ws_ml + row0 * 2;
  float M = -INFINITY;
  for (int j = lane; j < nsplit; j += 64) M = fmaxf(M, ml[2 * j]);
  M = group_max<64>(M);
  float Ls = 0.f;
  for (int j = lane; j < nsplit; j += 64) {
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(ml[2 * j] - M);
    wts[j] = f;
    Ls = fmaf(ml[2 * j + 1], f, Ls);
  }
  Ls = group_sum<64>(Ls);
  __syncthreads();
  const float* po = a.ws_o + row0 * head_dim;
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * head_dim;
  for (int d = lane; d < head_dim; d += 64) {
    float O = 0.f;
    for (int j = 0; j < nsplit; ++j) O = fmaf(wts[j], po[(size_t)j * head_dim + d], O);
    out[d] = from_f32<T>(Ls > 0.f ? O / Ls : 0.f);
  }
}

template <typename T, int HD, int REP>
pkv_status launch_split(const DecodeArgs& a, hipStream_t st) {
  const int tbl_entries = (a.partition >> a.block_shift) + 1;
  const int lds = Lds<T, HD, REP>::bytes(tbl_entries);
  dim3 grid(a.num_kv_heads, a.num_splits, a.num_seqs);
  if (a.cu_q) {
    const int z = a.total_q < kRowGridZ ? a.total_q : kRowGridZ;
    grid = dim3(a.num_kv_heads, (a.total_q + z - 1) / z, z);
  }
  hipLaunchKernelGGL((decode_partials_kernel<T, HD, REP>), grid, dim3(kThreads), lds, st, a);
  return launch_status("decode_partials_kernel");
}

template <typename T, int HD>
pkv_status dispatch_rep(const DecodeArgs& a, int rep, hipStream_t st) {
  switch (rep) {
    case 1: return launch_split<T, HD, 1>(a, st);
    case 2: return launch_split<T, HD, 2>(a, st);
    case 3: return launch_split<T, HD, 3>(a, st);
    case 4: return launch_split<T, HD, 4>(a, st);
    case 5: return launch_split<T, HD, 5>(a, st);
    case 6: return launch_split<T, HD, 6>(a, st);
    case 7: return launch_split<T, HD, 7>(a, st);
    case 8: return launch_split<T, HD, 8>(a, st);
    default: break;
  }
  set_error("group size %d (num_q_heads / num_kv_heads) is not compiled (1..8)", rep);
  return PKV_ERR_UNSUPPORTED;
}

template <typename T>
pkv_status dispatch_hd(const DecodeArgs& a, int hd, int rep, hipStream_t st) {
  switch (hd) {
    case 16: return dispatch_rep<T, 16>(a, rep, st);
    case 32: return dispatch_rep<T, 32>(a, rep, st);
    case 64: return dispatch_rep<T, 64>(a, rep, st);
    case 128: return dispatch_rep<T, 128>(a, rep, st);
    case 256: return dispatch_rep<T, 256>(a, rep, st);
    default: break;
  }
  set_error("head_dim %d is not compiled (16, 32, 64, 128, 256)", hd);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace

int decode_tile_tokens(int row_bytes) {
  return row_bytes >= 1024 ? 4 : row_bytes >= 512 ? 8 : row_bytes >= 256 ? 16 : row_bytes >= 128 ? 32 : 64;
}

bool decode_supported(int dtype, int head_dim, int rep) {
  (void)dtype;
  const bool hd_ok = head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 ||
                     head_dim == 256;
  return hd_ok && rep >= 1 && rep <= 8;
}

pkv_status launch_decode_partials(const DecodeArgs& a, int dtype, int head_dim, int rep,
                                  hipStream_t st) {
  if (dtype == PKV_F32) return dispatch_hd<float>(a, head_dim, rep, st);
  return dispatch_hd<uint16_t>(a, head_dim, rep, st);
}

pkv_status launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st) {
  if (a.num_splits <= 1) return PKV_OK;
  dim3 grid(a.num_q_heads, a.num_seqs);
  const int lds = a.num_splits * (int)sizeof(float);
  if (dtype == PKV_F32)
    hipLaunchKernelGGL((decode_reduce_kernel<float>), grid, dim3(64), lds, st, a, head_dim);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<uint16_t>), grid, dim3(64), lds, st, a, head_dim);
  return launch_status("decode_reduce_kernel");
}

}  // namespace pkv
