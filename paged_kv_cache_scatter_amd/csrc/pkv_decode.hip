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
// sequence s). Each wave takes token tiles of TILE tokens in turn (tiles w,
// w+4, ...) and streams them into its own two-stage LDS ring with 16-byte
// direct-to-LDS loads, one tile ahead of the one it computes. When a load
// instruction's 64 lanes stay inside one block (tokens per instruction <=
// block size), the tile's block ids are scalar loads issued a tile ahead and
// every row address is one scalar base plus a fixed lane offset; otherwise the
// split's ids are staged in LDS first. Tokens past the split or in an invalid
// block are read from a zero row and get a -inf score, so every tile, the
// partial last one included, goes through the same pipelined ring.
//   K stage   lanes own (token, KCH 16-byte chunks of its K row); the REP query
//             heads of the group sit in registers, so each K row is read once
//             for the whole group. The partial dot products of a token are
//             combined across its lanes by a DPP reduce-scatter that leaves each
//             lane holding the complete score of one head (or a few).
//   softmax   each lane runs the online max/sum for its own head(s) over its
//             tokens; a strided DPP max joins the lanes of one head. Every exp
//             is computed once. Probabilities go to a small LDS tile (bf16: a
//             rounded pair of tokens per word).
//   V stage   each lane owns DPL output dims of HPV heads for the whole tile and
//             reads the V rows from the ring (all lanes of a head set read one
//             row contiguously); o accumulates in fp32 and needs no cross-lane
//             reduction. The rescale of o is skipped when no running max moved.
// At the end the four waves' (m, l, o) are merged in LDS and either the
// normalised output (single split) or the split partial is written.
#include "pkv_internal.h"

#include <math.h>

namespace pkv {
namespace {

using namespace dev;

// Phase timestamps of the benchmark's traced build (PKV_PHASE, PKV_PHASE_VALUE;
// nothing in the normal build).
#include "pkv_phase_trace.h"

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

constexpr int pow2ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Largest power of two p with p * p <= x (1 for x < 4).
constexpr int isqrt_p2(int x) {
  int p = 1;
  while (4 * p * p <= x) p <<= 1;
  return p;
}

template <typename T, int HD, int REP>
struct Geo {
  static constexpr int ISZ = (int)sizeof(T);
  static constexpr int ROWB = HD * ISZ;  // bytes of one K (or V) row of one KV head
  static constexpr int EPC = 16 / ISZ;   // elements per 16-byte chunk
  // tokens per tile: 4 KB of K plus V per wave and tile for rows of 256 bytes
  // or more, 8 KB for shorter rows (at most 64 tokens)
  static constexpr int TILE = ROWB >= 1024 ? 2 : ROWB >= 512 ? 4 : ROWB >= 256 ? 8 : ROWB >= 128 ? 32 : 64;
  static constexpr int KCH = ROWB >= 32 ? 2 : 1;    // K chunks per lane per row
  static constexpr int LPT_K = ROWB / (16 * KCH);   // lanes per token (K stage)
  static constexpr int TPW_K = 64 / LPT_K;          // tokens per wave load (K)
  static constexpr int RK = TILE / TPW_K;           // K rows per lane per tile
  static constexpr int LPT_V = ROWB / 16;           // lanes per token (V loads)
  static constexpr int TPW_V = 64 / LPT_V;
  static constexpr int RV = TILE / TPW_V;           // V rows per lane per tile
  // heads after the reduce-scatter of the K stage
  static constexpr int REPP = pow2ceil(REP);        // heads padded to a power of two
  static constexpr int RS = REPP < LPT_K ? REPP : LPT_K;   // lanes one head set spreads over
  static constexpr int HPL = REPP / RS;             // heads per lane
  static constexpr int DUP = LPT_K / RS;            // lanes holding the same heads
  // V stage: lane owns DPL dims of HPV heads. DPL near sqrt(REP * HD / 64)
  // balances the probability words and the V bytes each lane reads per tile.
  static constexpr int DPL_MIN = HD / 64 > 2 ? HD / 64 : 2;
  static constexpr int DPL = isqrt_p2(REP * HD / 64) > DPL_MIN ? isqrt_p2(REP * HD / 64) : DPL_MIN;
  static constexpr int LPH = HD / DPL;              // lanes per head set
  static constexpr int HG = 64 / LPH;               // head sets across the wave
  static constexpr int HPV = (REP + HG - 1) / HG;   // heads per lane
  static constexpr int PSTR = REPP > HG * HPV ? REPP : HG * HPV;   // probability row stride
  static constexpr int PROWS = ISZ == 2 ? TILE / 2 : TILE;          // probability rows
  // ring stage: RK*KCH K loads then RV V loads, 1 KB per wave each
  static constexpr int LOADS = RK * KCH + RV;
  static constexpr int STAGE = LOADS * 1024;
  static constexpr int VOFF = RK * KCH * 1024;      // V rows (token-major) in a stage
  static constexpr int NID = TILE / (TPW_K > TPW_V ? TPW_K : TPW_V);   // block ids per tile
  static constexpr int STAGES = 2;                  // tiles in a wave's LDS ring
  // K/V loads carry the non-temporal hint for rows of 256 bytes or more
  // (measured: 4% faster at head_dim 128 bf16, 3% slower at 128-byte rows)
  static constexpr bool NT = ROWB >= 256;
  static_assert(RK >= 1 && RV >= 1 && LPT_K >= 1 && LPT_K <= 32 && LPT_V <= 64, "geometry");
  static_assert(LPH >= 1 && LPH <= 64 && DPL * ISZ <= 16 && (ISZ == 4 || TILE % 2 == 0), "PV");
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

// The value of lane + W (W <= 8: a DPP row shift, lane i reads lane i + W of
// its 16-lane row, which holds the next token for lanes of even tokens).
template <int W>
__device__ __forceinline__ float next_token(float x) {
  if constexpr (W <= 8) return dpp<0x100 + W>(x);   // row_shl:W
  else return __shfl_xor(x, W);
}

// Max / sum over lanes congruent modulo STRIDE (power of two), result in every lane.
template <int STRIDE, bool MAX>
__device__ __forceinline__ float strided_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (STRIDE <= 1) x = op(x, dpp<kRowRor + 1>(x));
  if constexpr (STRIDE <= 2) x = op(x, dpp<kRowRor + 2>(x));
  if constexpr (STRIDE <= 4) x = op(x, dpp<kRowRor + 4>(x));
  if constexpr (STRIDE <= 8) x = op(x, dpp<kRowRor + 8>(x));
  if constexpr (STRIDE <= 16) x = join16<MAX>(x);
  if constexpr (STRIDE <= 32) x = join32<MAX>(x);
  return x;
}

// PV-stage lane layout: HG head sets of HPV heads, LPH lanes per set, each
// lane DPL dims starting at dim0(hg, dl). Paired heads (PR > 0): twice the
// sets, each holding heads of one real head only and only that head's half
// of the (virtual) dims, so no lane accumulates dims it will not store.
template <typename T, int HD, int REP, int PR>
struct PvGeo {
  using G = Geo<T, HD, REP>;
  static constexpr int HG = PR ? 2 * G::HG : G::HG;
  static constexpr int LPH = PR ? G::LPH / 2 : G::LPH;
  static constexpr int HPV = PR ? REP / HG : G::HPV;
  static constexpr int DPL = G::DPL;
  static_assert(PR == 0 || (HG * HPV == REP && LPH * DPL == HD / 2 && HPV <= PR),
                "paired PV layout: every head set within one half");
  __device__ static int dim0(int hg, int dl) {
    return (PR ? (hg * HPV / (PR > 0 ? PR : 1)) * (HD / 2) : 0) + dl * DPL;
  }
};

template <typename T, int HD, int REP>
struct WaveState {
  using G = Geo<T, HD, REP>;
  float m[G::HPL];          // running max (log2 units) of the lane's K-stage heads
  float lsum[G::HPL];       // this lane's share of the exp-sum of those heads
  float o[G::HPV][G::DPL];  // unnormalised output: DPL dims of HPV heads (PV layout)
};

// 16-byte pieces of dead tokens are read from here (longest row: fp32 x 256).
__device__ __attribute__((aligned(16))) unsigned char g_zero_row[1024];

// Wave-uniform description of one split (scalar registers).
struct SplitCtx {
  const char* kh;     // head base into k_pool: + g*HD*isz
  const char* vh;     // head base into v_pool: + g*HD*isz
  const int* trow;    // this sequence's block table row (global)
  const int* tbl;     // LDS block ids of this split (-1 = invalid); per-lane path only
  int tbl_base;       // logical block index of tbl[0]
  int bshift;
  int num_blocks;
  uint32_t blk_bytes; // bytes of one block of one pool (all heads)
  uint32_t rsb;       // bytes of one token row (all heads)
  int t1;             // end of the split (exclusive)
  float scale_log2;
  int tnew;           // position read from k_new/v_new (fused step), else -1
  const char* knew;   // k_new row of this sequence and head (fused step)
  const char* vnew;
};

// Block ids of one tile on the uniform path (every 16-byte load instruction of
// the wave stays inside one block): one id per block the tile touches. ok bit
// i: id[i] is a valid block.
template <int NID>
struct TileIds {
  int id[NID];
  uint32_t ok;
  bool masked;        // partial tile or an invalid id: zero rows and -inf scores
};

template <int NID>
__device__ __forceinline__ int pick(const TileIds<NID>& ti, int i) {
  int v = ti.id[0];
#pragma unroll
  for (int k = 1; k < NID; ++k) v = i == k ? ti.id[k] : v;
  return v;
}

// Block ids on the uniform path are copied from the table into LDS in batches
// of 64 entries (TPB tiles of NID entries), one direct-to-LDS word per lane,
// into one of two batch slots. A batch is requested when the first tile of the
// previous one is issued, so it retires long before it is read, in order with
// the tile loads.
template <typename T, int HD, int REP>
__device__ __forceinline__ void ids_batch_dma(const SplitCtx& c, int tb0, int step, int n,
                                              int b, int lane, uint32_t slots) {
  using G = Geo<T, HD, REP>;
  constexpr int TPB = 64 / G::NID;
  const int m = min(b * TPB + lane / G::NID, n - 1);   // this lane's tile
  const int tb = tb0 + m * step;
  const int fb = tb >> c.bshift;
  const int lb = (min(tb + G::TILE, c.t1) - 1) >> c.bshift;   // last block with a live token
  dma4(c.trow + min(fb + lane % G::NID, lb), slots + (b & 1) * 256);
}

template <typename T, int HD, int REP>
__device__ __forceinline__ TileIds<Geo<T, HD, REP>::NID> read_ids(const SplitCtx& c, int tb, int m,
                                                                 const int* slots) {
  using G = Geo<T, HD, REP>;
  constexpr int TPB = 64 / G::NID;
  const int* e = slots + ((m / TPB) & 1) * 64 + (m % TPB) * G::NID;
  TileIds<G::NID> ti;
  const int fb = tb >> c.bshift;
  const int lb = (min(tb + G::TILE, c.t1) - 1) >> c.bshift;
  ti.ok = 0;
#pragma unroll
  for (int i = 0; i < G::NID; ++i) {
    const int id = __builtin_amdgcn_readfirstlane(e[i]);
    const bool ok = fb + i <= lb && (unsigned)id < (unsigned)c.num_blocks;
    ti.id[i] = ok ? id : 0;
    ti.ok |= (uint32_t)ok << i;
  }
  ti.masked = tb + G::TILE > c.t1 || ti.ok != (2u << (lb - fb)) - 1u ||
              (c.tnew >= tb && c.tnew < tb + G::TILE);
  return ti;
}

// Token tt of a tile starting at tb is live: inside the split and in a valid block.
template <typename T, int HD, int REP, bool UNI>
__device__ __forceinline__ bool live(const SplitCtx& c, const TileIds<Geo<T, HD, REP>::NID>& ti,
                                     int tb, int tt) {
  if (tt >= c.t1) return false;
  if (UNI) return (ti.ok >> ((tt - tb) >> c.bshift)) & 1u;
  return c.tbl[(tt >> c.bshift) - c.tbl_base] >= 0;
}

// Scores of the tile's K rows (log2 units), reduce-scattered to the lane's heads.
template <typename T, int HD, int REP, bool MASKED, int PR>
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
        for (int i = 0; i < G::KCH; ++i) {
          // paired heads: chunk i lies in real head i's half of the row
          if (PR == 0 || i == h / (PR > 0 ? PR : 1))
            acc[h] = chunk_dot<T>(qr[h][i], kr[r][i], acc[h]);
        }
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

// Online softmax of the lane's heads over the tile. Probabilities go to the
// wave's LDS tile: bf16 as a pair (token 2i, token 2i+1) rounded and packed
// in one word per head, fp32 one float per (token, head); the rescale factors
// go to cbuf when some running max moved. Returns whether one moved.
template <typename T, int HD, int REP>
__device__ __forceinline__ bool tile_softmax(
    WaveState<T, HD, REP>& st, const float (&sc)[Geo<T, HD, REP>::RK][Geo<T, HD, REP>::HPL],
    int kg, int hb, bool dup0, uint32_t* pbuf, float* cbuf) {
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
      const int tt = r * G::TPW_K + kg;
      if constexpr (G::ISZ == 2) {
        const float pn = next_token<G::LPT_K>(p);   // same head, token tt + 1
        if (dup0 && h < REP && !(kg & 1)) pbuf[(tt >> 1) * G::PSTR + h] = pack_bf16x2(p, pn);
      } else {
        if (dup0 && h < REP) reinterpret_cast<float*>(pbuf)[tt * G::PSTR + h] = p;
      }
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

// N consecutive 32-bit words from LDS, in the widest aligned pieces.
template <int N, int STR>
__device__ __forceinline__ void lds_words(const uint32_t* p, uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0 && STR % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + i);
      w[i] = x.x; w[i + 1] = x.y; w[i + 2] = x.z; w[i + 3] = x.w;
    }
  } else if constexpr (N % 2 == 0 && STR % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(p + i);
      w[i] = x.x; w[i + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = p[i];
  }
}

// o[h][d] += sum_t p[t][h] * V[t][d] for the lane's DPL dims of HPV heads,
// reading the tile's V rows (token-major, ROWB bytes each) from LDS.
template <typename T, int HD, int REP, int PR>
__device__ __forceinline__ void tile_pv(WaveState<T, HD, REP>& st, const unsigned char* vt,
                                        int hg, int d0, bool rescale, const uint32_t* pbuf,
                                        const float* cbuf) {
  using G = Geo<T, HD, REP>;
  using PV = PvGeo<T, HD, REP, PR>;
  if (rescale) {
#pragma unroll
    for (int i = 0; i < PV::HPV; ++i) {
      const float cr = cbuf[hg * PV::HPV + i];
#pragma unroll
      for (int e = 0; e < G::DPL; ++e) st.o[i][e] *= cr;
    }
  }
  const unsigned char* vl = vt + d0 * G::ISZ;
  if constexpr (G::ISZ == 2) {
    // bf16: two tokens at a time. Their probabilities are a packed bf16 pair
    // and their V values of one dimension are packed side by side, so one
    // fp32-accumulating bf16 dot2 adds both tokens' terms.
    constexpr int W = G::DPL / 2;   // words of V per token and lane
#pragma unroll
    for (int pp = 0; pp < G::TILE / 2; ++pp) {
      uint32_t a[W], b[W], pr[PV::HPV];
      lds_words<W, G::ROWB / 4>(reinterpret_cast<const uint32_t*>(vl + 2 * pp * G::ROWB), a);
      lds_words<W, G::ROWB / 4>(reinterpret_cast<const uint32_t*>(vl + (2 * pp + 1) * G::ROWB), b);
      lds_words<PV::HPV, G::PSTR>(pbuf + pp * G::PSTR + hg * PV::HPV, pr);
#pragma unroll
      for (int q = 0; q < W; ++q) {
        const uint32_t lo = __builtin_amdgcn_perm(b[q], a[q], 0x05040100u);  // dim 2q
        const uint32_t hi = __builtin_amdgcn_perm(b[q], a[q], 0x07060302u);  // dim 2q+1
#pragma unroll
        for (int i = 0; i < PV::HPV; ++i) {
          st.o[i][2 * q] = dot2_bf16(pr[i], lo, st.o[i][2 * q]);
          st.o[i][2 * q + 1] = dot2_bf16(pr[i], hi, st.o[i][2 * q + 1]);
        }
      }
    }
  } else {
    const float* pf = reinterpret_cast<const float*>(pbuf);
#pragma unroll
    for (int t = 0; t < G::TILE; ++t) {
      uint32_t v[G::DPL], pr[PV::HPV];
      lds_words<G::DPL, G::ROWB / 4>(reinterpret_cast<const uint32_t*>(vl + t * G::ROWB), v);
      lds_words<PV::HPV, G::PSTR>(
          reinterpret_cast<const uint32_t*>(pf) + t * G::PSTR + hg * PV::HPV, pr);
#pragma unroll
      for (int i = 0; i < PV::HPV; ++i)
#pragma unroll
        for (int e = 0; e < G::DPL; ++e)
          st.o[i][e] = fmaf(__uint_as_float(pr[i]), __uint_as_float(v[e]), st.o[i][e]);
    }
  }
}

// Lane layout and per-lane address offsets (the same for every split).
struct Lanes {
  int lane, kg, kc, vg, hb, hg, vd0;   // vd0: first dim of the lane's PV share
  bool dup0;
  uint32_t kc16, vc16;   // lane's 16-byte chunk within a K / V row
  uint32_t koff, voff;   // lane's chunk within a row group: kg*rsb + kc*16, vg*rsb + vc*16
};

// Issue the 16-byte direct-to-LDS loads of one tile (K rows, then V rows) into
// LDS stage `base`. Unmasked uniform tiles address each row group from one
// scalar block id; other tiles compute a per-lane address and read dead
// tokens (past the split, or in an invalid block) from the zero row.
template <typename T, int HD, int REP, bool UNI>
__device__ __forceinline__ void issue_tile(const SplitCtx& c, const Lanes& ln, int tb,
                                           const TileIds<Geo<T, HD, REP>::NID>& ti,
                                           uint32_t base) {
  using G = Geo<T, HD, REP>;
  const int bmask = (1 << c.bshift) - 1;
  if (UNI && !ti.masked) {
#pragma unroll
    for (int r = 0; r < G::RK; ++r) {
      const int tr = tb + r * G::TPW_K;
      const int blk = __builtin_amdgcn_readfirstlane(pick(ti, (r * G::TPW_K) >> c.bshift));
      const char* rb = c.kh + (uint64_t)(uint32_t)blk * c.blk_bytes + (uint32_t)(tr & bmask) * c.rsb;
#pragma unroll
      for (int i = 0; i < G::KCH; ++i)
        dma16s<G::NT>(rb + i * G::LPT_K * 16, ln.koff, base + (r * G::KCH + i) * 1024);
    }
#pragma unroll
    for (int r = 0; r < G::RV; ++r) {
      const int tr = tb + r * G::TPW_V;
      const int blk = __builtin_amdgcn_readfirstlane(pick(ti, (r * G::TPW_V) >> c.bshift));
      const char* rb = c.vh + (uint64_t)(uint32_t)blk * c.blk_bytes + (uint32_t)(tr & bmask) * c.rsb;
      dma16s<G::NT>(rb, ln.voff, base + (G::RK * G::KCH + r) * 1024);
    }
    return;
  }
  auto row = [&](int tt, const char* lb, const char* zb, const char* nb) -> const char* {
    int blk;
    bool ok = tt < c.t1;
    if (UNI) {
      const int i = (tt - tb) >> c.bshift;
      blk = pick(ti, i);
      ok = ok && ((ti.ok >> i) & 1u);
    } else {
      blk = ok ? c.tbl[(tt >> c.bshift) - c.tbl_base] : -1;
      ok = blk >= 0;
    }
    if (ok && tt == c.tnew) return nb;
    return ok ? lb + (uint64_t)(uint32_t)blk * c.blk_bytes + (uint32_t)(tt & bmask) * c.rsb : zb;
  };
#pragma unroll
  for (int r = 0; r < G::RK; ++r) {
    const char* p = row(tb + r * G::TPW_K + ln.kg, c.kh + ln.kc16,
                        reinterpret_cast<const char*>(g_zero_row) + ln.kc16, c.knew + ln.kc16);
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) dma16<G::NT>(p + i * G::LPT_K * 16, base + (r * G::KCH + i) * 1024);
  }
#pragma unroll
  for (int r = 0; r < G::RV; ++r)
    dma16<G::NT>(row(tb + r * G::TPW_V + ln.vg, c.vh + ln.vc16,
              reinterpret_cast<const char*>(g_zero_row) + ln.vc16, c.vnew + ln.vc16),
          base + (G::RK * G::KCH + r) * 1024);
}

template <typename T, int HD, int REP, bool UNI, int PR>
__device__ __forceinline__ void compute_tile(const SplitCtx& c, const Lanes& ln,
                                             WaveState<T, HD, REP>& st,
                                             const uint4 (&qr)[REP][Geo<T, HD, REP>::KCH], int tb,
                                             const TileIds<Geo<T, HD, REP>::NID>& ti,
                                             const unsigned char* stage, uint32_t* pbuf,
                                             float* cbuf) {
  using G = Geo<T, HD, REP>;
  const uint4* sp = reinterpret_cast<const uint4*>(stage) + ln.lane;
  uint4 kr[G::RK][G::KCH];
#pragma unroll
  for (int r = 0; r < G::RK; ++r)
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) kr[r][i] = sp[(r * G::KCH + i) * 64];
  float sc[G::RK][G::HPL];
  bool kval[G::RK];
#pragma unroll
  for (int r = 0; r < G::RK; ++r) kval[r] = true;
  if (ti.masked) {
#pragma unroll
    for (int r = 0; r < G::RK; ++r) kval[r] = live<T, HD, REP, UNI>(c, ti, tb, tb + r * G::TPW_K + ln.kg);
    tile_scores<T, HD, REP, true, PR>(c, ln.kc, qr, kr, kval, sc);
  } else {
    tile_scores<T, HD, REP, false, PR>(c, ln.kc, qr, kr, kval, sc);
  }
  const bool moved = tile_softmax<T, HD, REP>(st, sc, ln.kg, ln.hb, ln.dup0, pbuf, cbuf);
  tile_pv<T, HD, REP, PR>(st, stage + G::VOFF, ln.hg, ln.vd0, moved, pbuf, cbuf);
}

template <int LOADS, int S>
__device__ __forceinline__ void wait_tiles_after(int behind) {
  // loads of `behind` newer tiles may stay in flight (behind < S)
  if constexpr (S > 3) {
    if (behind >= 3) { wait_vmcnt<3 * LOADS>(); return; }
  }
  if constexpr (S > 2) {
    if (behind == 2) { wait_vmcnt<2 * LOADS>(); return; }
  }
  if (behind == 1) { wait_vmcnt<LOADS>(); return; }
  wait_vmcnt<0>();
}

// The wave's tiles tb0, tb0 + kStep, ... below t1. Tiles stream into the wave's
// STAGES-deep LDS ring, STAGES - 1 tiles ahead of the one being computed.
template <typename T, int HD, int REP, bool UNI, int kStep, int PR>
__device__ __forceinline__ void wave_tiles(const SplitCtx& c, const Lanes& ln,
                                           WaveState<T, HD, REP>& st,
                                           const uint4 (&qr)[REP][Geo<T, HD, REP>::KCH], int tb0,
                                           bool any_bad, uint32_t* pbuf, float* cbuf,
                                           int* idslots, const unsigned char* ring) {
  using G = Geo<T, HD, REP>;
  using TI = TileIds<G::NID>;
  constexpr int S = G::STAGES;
  constexpr int TPB = 64 / G::NID;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const uint32_t slots_lds = (uint32_t)(uintptr_t)idslots;
  const int n = (c.t1 - 1 - tb0) / kStep + 1;   // tiles of this wave (tb0 < t1)
  auto ids = [&](int m) -> TI {
    const int tb = tb0 + m * kStep;
    if (UNI) return read_ids<T, HD, REP>(c, tb, m, idslots);
    TI ti;
#pragma unroll
    for (int i = 0; i < G::NID; ++i) ti.id[i] = 0;
    ti.ok = 0;
    ti.masked = any_bad || tb + G::TILE > c.t1 || (c.tnew >= tb && c.tnew < tb + G::TILE);
    return ti;
  };
  if (UNI) {
    ids_batch_dma<T, HD, REP>(c, tb0, kStep, n, 0, ln.lane, slots_lds);
    if (n > TPB) ids_batch_dma<T, HD, REP>(c, tb0, kStep, n, 1, ln.lane, slots_lds);
  }
  // The prologue's own loads (q, table) are back before the ring starts, so the
  // compiler puts no waits for them inside the loop (where they would also
  // stall on the ring's loads).
  __builtin_amdgcn_s_waitcnt(0);
  PKV_PHASE(2);
  TI ti[S];
#pragma unroll
  for (int q = 0; q < S - 1; ++q) {
    ti[q] = ti[0];
    if (q < n) {
      ti[q] = ids(q);
      issue_tile<T, HD, REP, UNI>(c, ln, tb0 + q * kStep, ti[q], ring_lds + q * G::STAGE);
    }
  }
  for (int k = 0; k < n; ++k) {
    const int m = k + S - 1;   // tile issued in this iteration
    if (m < n) {
      wait_lgkmcnt0();   // the stage about to be refilled has been read
      ti[S - 1] = ids(m);
      if (UNI && m % TPB == 0 && m > 0 && (m / TPB + 1) * TPB < n)
        ids_batch_dma<T, HD, REP>(c, tb0, kStep, n, m / TPB + 1, ln.lane, slots_lds);
      issue_tile<T, HD, REP, UNI>(c, ln, tb0 + m * kStep, ti[S - 1],
                                  ring_lds + (m % S) * G::STAGE);
      wait_vmcnt<(S - 1) * G::LOADS>();
    } else {
      wait_tiles_after<G::LOADS, S>(n - 1 - k);
    }
    if (k == 0) PKV_PHASE(3);
    compute_tile<T, HD, REP, UNI, PR>(c, ln, st, qr, tb0 + k * kStep, ti[0],
                                      ring + (k % S) * G::STAGE, pbuf, cbuf);
#pragma unroll
    for (int q = 0; q < S - 1; ++q) ti[q] = ti[q + 1];
  }
}

__host__ __device__ constexpr int round16(int b) { return (b + 15) & ~15; }

template <typename T, int HD, int REP>
struct Lds {
  using G = Geo<T, HD, REP>;
  // per wave: two 64-entry block id slots, probabilities, rescale factors
  static constexpr int kWaveWords = 128 + round16((G::PROWS * G::PSTR + G::PSTR) * 4) / 4;
  static constexpr int kMergeFloats = REP * (HD + 2);                                 // m, l, o per wave
  static constexpr int kRingBytes = G::STAGES * G::STAGE;                             // per wave
  __host__ __device__ static int ring_offset(int tbl_entries) {
    return round16(tbl_entries * 4) + kWaves * kWaveWords * 4;
  }
  // The merge area reuses the front of LDS once every wave has left the tile loop.
  __host__ __device__ static int bytes(int tbl_entries) {
    const int loop = ring_offset(tbl_entries) + kWaves * kRingBytes;
    const int merge = kWaves * kMergeFloats * 4;
    return loop > merge ? loop : merge;
  }
  // Table entries staged in LDS: only the per-lane path uses them.
  __host__ __device__ static int table_entries(int partition, int bshift) {
    return uniform(bshift) ? 0 : (partition >> bshift) + 1;
  }
  __host__ __device__ static bool uniform(int bshift) {
    return G::TPW_K <= (1 << bshift) && G::TPW_V <= (1 << bshift);
  }
};


// Merge of one (sequence, KV head)'s split partials into the output rows of
// its REP query heads: M = max m_i, L = sum l_i 2^(m_i - M), out = sum
// 2^(m_i - M) o_i / L. Slots 0 .. nps-1 hold the shared pass's partials, the
// decode splits follow from slot0. Head h is merged by wave h % kWaves; lane
// l owns dims l, l + 64, ... Lane i reads slot i's (m, l) with one 8-byte
// load; the o rows of kMergeBatch slots are loaded together before they are
// summed, in slot order (the same order, hence the same bits, as the merge
// kernel). wl is the wave's 64-float LDS scratch (more than 64 partials).
constexpr int kMergeBatch = 8;


template <typename T, int HD, int REP, int PR>
__device__ __forceinline__ void merge_partials(const DecodeArgs& a, int s, int hq0, int nps,
                                               int slot0, int nsplit, T* out, float* wl, int w,
                                               int lane) {
  constexpr int QHD = PR ? HD / 2 : HD;          // dims of one query head's output
  constexpr int DPT = QHD >= 64 ? QHD / 64 : 1;  // dims per lane
  const int n = nps + nsplit;
  const int J = a.num_splits;
  auto slot = [&](int i) { return i < nps ? i : slot0 + i - nps; };
  for (int h = w; h < REP; h += kWaves) {
    const size_t row0 = ((size_t)s * a.num_q_heads + hq0 + h) * J;
    const float* ml = a.ws_ml + row0 * 2;
    const float* po = a.ws_o + row0 * HD + (PR ? h / (PR > 0 ? PR : 1) : 0) * QHD;
    float M = -INFINITY, Ls = 0.f, f = 0.f;
    if (n <= 64) {
      const float2 v = lane < n ? ld_agent2(ml + 2 * slot(lane)) : make_float2(-INFINITY, 0.f);
      M = group_max<64>(v.x);
      if (lane < n && M != -INFINITY) {
        f = fast_exp2(v.x - M);
        Ls = fmaf(v.y, f, 0.f);
      }
    } else {
      for (int i = lane; i < n; i += 64) M = fmaxf(M, ld_agent(ml + 2 * slot(i)));
      M = group_max<64>(M);
    }
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
    for (int c = 0; c < n; c += 64) {
      if (n > 64) {
        const int i = c + lane;
        f = 0.f;
        if (i < n && M != -INFINITY) {
          f = fast_exp2(ld_agent(ml + 2 * slot(i)) - M);
          Ls = fmaf(ld_agent(ml + 2 * slot(i) + 1), f, Ls);
        }
      }
      wl[lane] = f;   // read back by the same wave: LDS keeps a wave's order
      const int m = min(64, n - c);
      for (int k0 = 0; k0 < m; k0 += kMergeBatch) {
        float ov[kMergeBatch][DPT];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          const float* pk = po + (size_t)slot(c + min(k0 + k, m - 1)) * HD;
#pragma unroll
          for (int e = 0; e < DPT; ++e) {
            const int d = lane + 64 * e;
            ov[k][e] = d < QHD ? ld_agent(pk + d) : 0.f;
          }
        }
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          if (k0 + k < m) {
            const float fk = wl[k0 + k];
#pragma unroll
            for (int e = 0; e < DPT; ++e) acc[e] = fmaf(fk, ov[k][e], acc[e]);
          }
        }
      }
    }
    Ls = group_sum<64>(Ls);
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const int d = lane + 64 * e;
      if (d < QHD) out[h * QHD + d] = from_f32<T>(Ls > 0.f ? acc[e] / Ls : 0.f);
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then
// the row broadcasts of lanes 15 and 31).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u<0x111>(x);         // row_shr:1
  x += dpp_u<0x112>(x);         // row_shr:2
  x += dpp_u<0x114>(x);         // row_shr:4
  x += dpp_u<0x118>(x);         // row_shr:8
  x += dpp_u<0x142, 0xA>(x);    // row_bcast:15 into rows 1 and 3
  x += dpp_u<0x143, 0xC>(x);    // row_bcast:31 into rows 2 and 3
  return x;
}

// A workgroup's piece under the piece schedule.
struct Piece {
  int s, t0, t1, slot, n, ctx;
  int start;   // first token of a shared-prefix tail (0 without sharing)
};

// Piece number `pid` of the schedule (see DecodeArgs::sched_q): every thread
// counts the pieces of four consecutive sequences, a workgroup scan gives
// each thread its offsets among the large pieces, the long tail pieces and
// the short tail pieces (the order they run in), and the thread holding the
// piece publishes it. Returns false (uniformly) when pid is past the last
// piece. `lds` holds at least 32 ints; the caller synchronises before
// reusing it.
__device__ __forceinline__ bool find_piece(const DecodeArgs& a, int pid, int lim, Piece& pc,
                                           int* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int P = a.partition;
  const int lp = __builtin_ctz((unsigned)P), lq = __builtin_ctz((unsigned)a.sched_q),
            la = __builtin_ctz((unsigned)a.sched_align);
  int L[4];
  PieceCounts pcs[4];
  uint32_t nbig = 0, ntail = 0;   // ntail: (long << 16) | short
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // all four loads in flight together
    const int sq = tid * 4 + i;
    L[i] = sq < a.num_seqs ? a.ctx_lens[sq] : 0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sq = tid * 4 + i;
    L[i] = L[i] < 0 ? 0 : (L[i] > lim ? lim : L[i]);
    pcs[i] = sq < a.num_seqs ? piece_counts(L[i], lp, lq, la) : PieceCounts{0, 0, 0, 0};
    nbig += pcs[i].big;
    ntail += ((uint32_t)pcs[i].nlong << 16) | (uint32_t)(pcs[i].tail - pcs[i].nlong);
  }
  const uint32_t ib = wave_incl_scan(nbig), it = wave_incl_scan(ntail);
  if (lane == 63) {
    lds[w] = (int)ib;
    lds[4 + w] = (int)it;
  }
  lds[16] = -1;
  __syncthreads();
  uint32_t pb = 0, pt = 0, tb = 0, tt = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const uint32_t vb = (uint32_t)lds[k], vt = (uint32_t)lds[4 + k];
    if (k < w) {
      pb += vb;
      pt += vt;
    }
    tb += vb;
    tt += vt;
  }
  const uint32_t tlong = tt >> 16, tshort = tt & 0xFFFF;
  const uint32_t et = pt + it - ntail;   // this thread's packed tail offsets
  const uint32_t u = (uint32_t)pid;
  if (u >= tb + tlong + tshort) return false;
  // segment (0 large, 1 long tail, 2 short tail) and index among this
  // thread's pieces of it (unsigned: an index below the thread's wraps)
  const int seg = u < tb ? 0 : u < tb + tlong ? 1 : 2;
  uint32_t k = seg == 0 ? u - (pb + ib - nbig)
             : seg == 1 ? u - tb - (et >> 16)
                        : u - tb - tlong - (et & 0xFFFF);
  const uint32_t mine = seg == 0 ? nbig : seg == 1 ? (ntail >> 16) : (ntail & 0xFFFF);
  if (k < mine) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const PieceCounts& c = pcs[i];
      const uint32_t ni = seg == 0 ? c.big : seg == 1 ? c.nlong : c.tail - c.nlong;
      if (k < ni) {
        int t0 = 0, t1 = 0, slot = 0;
        if (seg == 0) {
          t0 = (int)k * P;
          t1 = ((int)k == c.big - 1 && c.tail == 0) ? L[i] : t0 + P;
          slot = (int)k;
        } else {
          // the k-th tail piece of this class, in piece order
          int left = (int)k;
          for (int j = 0; j < c.tail; ++j) {
            const int a0 = c.big * P + j * c.base;
            const int a1 = j == c.tail - 1 ? L[i] : a0 + c.base;
            if (long_tail(a1 - a0, lq) == (seg == 1)) {
              if (left == 0) {
                t0 = a0;
                t1 = a1;
                slot = c.big + j;
                break;
              }
              --left;
            }
          }
        }
        lds[16] = tid * 4 + i;
        lds[17] = t0;
        lds[18] = t1;
        lds[19] = slot;
        lds[20] = c.big + c.tail;
        lds[21] = L[i];
        break;
      }
      k -= ni;
    }
  }
  __syncthreads();
  pc.s = lds[16];
  pc.t0 = lds[17];
  pc.t1 = lds[18];
  pc.slot = lds[19];
  pc.n = lds[20];
  pc.ctx = lds[21];
  return pc.s >= 0;
}

// Rank (longest first) of the sequence that grid index `pid` runs, when the
// CUs take the grid in passes of n sequences, position k of every pass on
// the same CUs. The aim is an equal sum of lengths per position. Pairs of
// full passes run the second reversed (rank k with rank n - 1 - k). An odd
// count of full passes ends with three passes dealt as k, (k + n/2) mod n and
// n - 1 - (2 (k mod n/2) + [k >= n/2]) (n even), whose position sums differ
// by at most one rank step; a partial last pass keeps its order.
__device__ __forceinline__ int lpt_rank(int pid, int n, int num_seqs) {
  const int full = num_seqs / n;
  const int ps = pid / n, k = pid - ps * n;
  if (ps >= full) return pid;
  int off;
  if ((full & 1) && full >= 3 && ps >= full - 3 && (n & 1) == 0) {
    const int q = ps - (full - 3), h = n >> 1;
    off = q == 0 ? k : q == 1 ? (k + h) % n : n - 1 - (2 * (k % h) + (k >= h));
  } else {
    off = (ps & 1) ? n - 1 - k : k;
  }
  return ps * n + off;
}

// Sequence number `pid` in longest-first order (see DecodeArgs::sched_lpt):
// every thread classifies four consecutive sequences by length (class
// floor(kLenClasses * L / (lim + 1)), longest class first) and counts them
// into an LDS histogram; the rank's class and its place within the class
// follow from the counts, and a workgroup scan of the thread's own members of
// that class finds the sequence (index order within a class), which the
// thread holding it publishes as a one-piece Piece. With lpt_pass > 0 the
// ranks are dealt in passes of lpt_pass, every second pass reversed, so that
// the CUs that take the longest of one pass take the shortest of the next.
// Returns false (uniformly) when pid is past the last sequence.
__device__ __forceinline__ bool find_sequence_lpt(const DecodeArgs& a, int pid, int lim,
                                                  Piece& pc, int* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int* hist = lds + 32;   // kLenClasses counts
  const float cls_scale = (float)kLenClasses / (float)(lim + 1);
  int L[4], cls[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // all four loads in flight together
    const int sq = tid * 4 + i;
    L[i] = sq < a.num_seqs ? a.ctx_lens[sq] : 0;
  }
  for (int c = tid; c < kLenClasses; c += kThreads) hist[c] = 0;
  if (tid == 0) lds[16] = -1;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sq = tid * 4 + i;
    L[i] = L[i] < 0 ? 0 : (L[i] > lim ? lim : L[i]);
    int c = (int)((float)L[i] * cls_scale);
    c = c > kLenClasses - 1 ? kLenClasses - 1 : c;
    cls[i] = sq < a.num_seqs ? kLenClasses - 1 - c : -1;   // longest class first
    if (cls[i] >= 0) atomicAdd(&hist[cls[i]], 1);
  }
  __syncthreads();
  if (pid >= a.num_seqs) return false;
  int r = pid;
  if (a.lpt_pass > 0) r = lpt_rank(pid, a.lpt_pass, a.num_seqs);
  int seg = 0, base = 0;   // the class holding rank r, and its first rank
  for (; seg < kLenClasses - 1; ++seg) {
    const int h = hist[seg];
    if (r < base + h) break;
    base += h;
  }
  const uint32_t k = (uint32_t)(r - base);   // place within the class
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) mine += cls[i] == seg;
  const uint32_t incl = wave_incl_scan(mine);
  if (lane == 63) lds[w] = (int)incl;
  __syncthreads();
  uint32_t pre = 0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q)
    if (q < w) pre += (uint32_t)lds[q];
  const uint32_t exc = pre + incl - mine;
  if (k >= exc && k < exc + mine) {
    uint32_t kk = k - exc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (cls[i] == seg) {
        if (kk == 0) {
          lds[16] = tid * 4 + i;
          lds[17] = L[i];
          break;
        }
        --kk;
      }
    }
  }
  __syncthreads();
  pc.s = lds[16];
  pc.t0 = 0;
  pc.t1 = pc.ctx = lds[17];
  pc.slot = 0;
  pc.n = 1;
  return pc.s >= 0;
}

// Stream-K layout of one KV head's stream (see DecodeArgs::sched_sk): every
// thread takes four consecutive sequences, a workgroup scan of their unit
// counts (a non-empty sequence costs sk_alpha + ceil(L / A) units) gives
// st[s], the unit where sequence s's tokens start, and len[s], its clamped
// length. With shared-prefix groups (a.sh.group_start) L is the tail past
// the group's shared tokens, which start in `first` gets (the same group
// and shared length as group_of and shared_len give, from the group table
// staged in `gtab`, 2 * num_seqs ints). Returns the stream's total units.
// `tmp` holds kWaves ints; the caller's later reads of st, len and first
// follow the barrier at the end.
template <bool TAILS>
__device__ __forceinline__ int sk_layout(const DecodeArgs& a, int lim, int* st, int* len,
                                         int* tmp, int* first, int* gtab) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int la = __builtin_ctz((unsigned)a.sched_align);
  constexpr bool shared = TAILS;
  int L[4], F[4] = {0, 0, 0, 0};
  uint32_t u[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // all four loads in flight together
    const int sq = tid * 4 + i;
    L[i] = sq < a.num_seqs ? a.ctx_lens[sq] : 0;
  }
  if constexpr (shared) {
    const int G = a.sh.num_groups;   // at most num_seqs (checked by the planner)
    for (int k = tid; k < G; k += kThreads) {
      gtab[k] = a.sh.group_start[k];
      gtab[a.num_seqs + k] = shared_len(a.sh, k, lim, a.block_shift);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sq = tid * 4 + i;
      int lo = 0, hi = G;   // the last group starting at or before sq (0 if none)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (gtab[mid] <= sq) lo = mid;
        else hi = mid;
      }
      const int c = L[i] < 0 ? 0 : (L[i] > lim ? lim : L[i]);
      F[i] = G > 0 ? min(c, gtab[a.num_seqs + lo]) : 0;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    L[i] = L[i] < 0 ? 0 : (L[i] > lim ? lim : L[i]);
    L[i] -= F[i];
    u[i] = ((uint32_t)L[i] + (uint32_t)a.sched_align - 1u) >> la;
    sum += u[i] ? u[i] + (uint32_t)a.sk_alpha : 0u;
  }
  const uint32_t incl = wave_incl_scan(sum);
  if (lane == 63) tmp[w] = (int)incl;
  __syncthreads();
  uint32_t base = 0, total = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const uint32_t v = (uint32_t)tmp[k];
    if (k < w) base += v;
    total += v;
  }
  uint32_t at = base + incl - sum;   // this thread's first sequence's cost starts here
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sq = tid * 4 + i;
    const uint32_t pad = u[i] ? (uint32_t)a.sk_alpha : 0u;
    if (sq < a.num_seqs) {
      st[sq] = (int)(at + pad);
      len[sq] = L[i];
      if constexpr (shared) first[sq] = F[i];
    }
    at += u[i] + pad;
  }
  __syncthreads();
  return (int)total;
}

// SK: the stream-K variant (DecodeArgs::sched_sk), compiled for rows of 256
// bytes or more only; the other variant runs one piece per workgroup. TAILS:
// stream-K over shared-prefix tails (a.sh.group_start set), an instance of its
// own so that the plain stream-K kernel carries none of its code (the TP=8
// shard of the LLaMA-2-70B layer ran 29.8 us with one kernel for both, 28.7 us
// apart).
template <typename T, int HD, int REP, int PR, bool SK, bool TAILS>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
  using G = Geo<T, HD, REP>;
  using L = Lds<T, HD, REP>;
  // PR > 0: paired KV heads (see DecodeArgs::pair_rep); chunk i of a lane's
  // K row then lies in real head i's half, and q / out rows have QHD dims
  static_assert(PR == 0 || (REP == 2 * PR && G::KCH == 2 && G::LPT_K * 16 * 2 == G::ROWB),
                "paired heads need two K chunks per lane, one in each half");
  constexpr int QHD = PR ? HD / 2 : HD;
  extern __shared__ __align__(16) unsigned char smem[];

  // Splits are dispatched last-index first: the later splits exist only for
  // the longer sequences, so their work starts early and the tail of the
  // launch is made of the short first splits.
  PKV_PHASE(0);
  const int g = blockIdx.x;
  int s = blockIdx.y, j = gridDim.z - 1 - blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int bshift = a.block_shift;
  const int lim = min(a.max_ctx, a.max_blocks << bshift);
  int qrow = s;   // row of q and out
  int ctx;
  // piece schedule: this workgroup's sequence, token range and partial slot
  Piece pc{};
  const bool sched = a.sched_q > 0 || a.sched_lpt || SK;
  if (SK) {
    // the pieces come from the loop over this workgroup's range at the end
  } else if (sched) {
    const int pid = blockIdx.y + gridDim.y * blockIdx.z;
    int* scan_lds = reinterpret_cast<int*>(smem);
    if (a.sched_lpt ? !find_sequence_lpt(a, pid, lim, pc, scan_lds)
                    : !find_piece(a, pid, lim, pc, scan_lds))
      return;
    // memory safety whatever the scan gave: an inconsistent piece does no work
    if ((unsigned)pc.s >= (unsigned)a.num_seqs || pc.t0 < 0 || pc.t0 > pc.t1 ||
        pc.t1 > pc.ctx || pc.ctx > lim || (unsigned)pc.slot >= (unsigned)a.num_splits ||
        pc.n > a.num_splits)
      return;
    __syncthreads();   // the scan's LDS words are reused below
    s = qrow = pc.s;
    j = pc.slot;
    ctx = pc.ctx;
  } else if (a.cu_q) {
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
  // One piece (s, j, ctx, pc): everything from here to the end of the lambda
  // runs once per piece; its returns end the piece.
  auto piece = [&]() __attribute__((always_inline)) {
  // Shared-prefix decode: the group's shared pass covers positions < start
  // (nps partials in the leading slots); this kernel covers the tail.
  int start = 0, nps = 0, slot0 = 0;
  const int P = a.partition;
  int nsplit;
  if (sched) {
    nsplit = pc.n;
    if constexpr (TAILS) {
      // a shared-prefix tail: the shared pass's partials lead
      start = pc.start;
      nps = (start + a.sh.prefix_part - 1) / a.sh.prefix_part;
      slot0 = a.sh.prefix_slots;
    }
  } else if (a.sh.group_start) {
    start = min(ctx, shared_len(a.sh, group_of(a.sh, s), lim, bshift));
    nps = (start + a.sh.prefix_part - 1) / a.sh.prefix_part;
    slot0 = a.sh.prefix_slots;
    nsplit = min((ctx - start + P - 1) / P, a.num_splits - slot0);
  } else {
    nsplit = (ctx + P - 1) / P;
  }
  const int hq0 = g * REP;
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)qrow * a.num_q_heads + hq0) * QHD;

  PKV_PHASE(1);
  if (sched ? ctx == start : j >= nsplit) {
    if (j == 0 && nps == 0) {  // empty sequence: zeros
      for (int i = tid; i < REP * QHD; i += kThreads) out[i] = from_f32<T>(0.f);
    } else if (j == 0 && a.counters) {
      // context inside the shared prompt: only the shared pass's partials,
      // written by the previous launch
      merge_partials<T, HD, REP, PR>(a, s, hq0, nps, slot0, 0, out,
                                 reinterpret_cast<float*>(smem) + w * 64, w, lane);
    }
    return;
  }
  const int t0 = sched ? pc.t0 : start + j * P;
  const int t1 = sched ? pc.t1 : min(ctx, t0 + P);
  const bool uni = L::uniform(bshift);

  const int tbl_entries = L::table_entries(a.sched_q > 0 ? max_piece(P, a.sched_q) : P, bshift);
  int* tbl = reinterpret_cast<int*>(smem);
  int* idslot = reinterpret_cast<int*>(smem + round16(tbl_entries * 4)) + w * L::kWaveWords;
  uint32_t* pbuf = reinterpret_cast<uint32_t*>(idslot + 128);
  float* cbuf = reinterpret_cast<float*>(pbuf + G::PROWS * G::PSTR);
  float* merge = reinterpret_cast<float*>(smem);
  const unsigned char* ring = smem + L::ring_offset(tbl_entries) + w * L::kRingBytes;

  SplitCtx c;
  c.trow = a.tables + (size_t)s * a.max_blocks;
  c.tbl = tbl;
  c.tbl_base = t0 >> bshift;
  c.bshift = bshift;
  c.num_blocks = a.num_blocks;
  c.t1 = t1;
  c.scale_log2 = a.scale_log2;
  c.tnew = -1;
  c.knew = c.vnew = nullptr;
  if (a.k_new && t1 == ctx) {
    // fused step: this workgroup owns the new token of KV head g
    const int tn = ctx - 1;
    const size_t row_off = ((size_t)s * a.num_kv_heads + g) * HD * G::ISZ;
    c.tnew = tn;
    c.knew = reinterpret_cast<const char*>(a.k_new) + row_off;
    c.vnew = reinterpret_cast<const char*>(a.v_new) + row_off;
    const int id = c.trow[tn >> bshift];
    if ((unsigned)id < (unsigned)a.num_blocks) {
      constexpr int CH = G::ROWB / 16;   // 16-byte chunks of one head's row
      const size_t dst = ((size_t)(uint32_t)id << bshift | (uint32_t)(tn & ((1 << bshift) - 1))) *
                             ((size_t)a.num_kv_heads * G::ROWB) +
                         (size_t)g * G::ROWB;
      if (tid < 2 * CH) {
        const bool isv = tid >= CH;
        const int ch = isv ? tid - CH : tid;
        const uint4 v = *reinterpret_cast<const uint4*>((isv ? c.vnew : c.knew) + ch * 16);
        char* pool = reinterpret_cast<char*>(const_cast<void*>(isv ? a.v_pool : a.k_pool));
        *reinterpret_cast<uint4*>(pool + dst + ch * 16) = v;
      }
    }
  }

  // ---- per-lane path: stage this split's block ids in LDS (invalid -> -1)
  int any_bad = 0;
  if (!uni) {
    const int nb = ((t1 - 1) >> bshift) - c.tbl_base + 1;
    int bad = 0;
    for (int i = tid; i < nb; i += kThreads) {
      const int id = c.trow[c.tbl_base + i];
      const bool ok = (unsigned)id < (unsigned)a.num_blocks;
      tbl[i] = ok ? id : -1;
      bad |= !ok;
    }
    any_bad = __syncthreads_or(bad);
  }

  // ---- this wave's query heads, in the K-stage lane layout
  Lanes ln;
  ln.lane = lane;
  ln.kg = lane / G::LPT_K;
  ln.kc = lane % G::LPT_K;
  ln.vg = lane / G::LPT_V;
  const int vc = lane % G::LPT_V;
  using PV = PvGeo<T, HD, REP, PR>;
  ln.hg = lane / PV::LPH;
  ln.vd0 = PV::dim0(ln.hg, lane % PV::LPH);
  ln.hb = head_base<G::LPT_K, G::REPP, G::HPL>(ln.kc);
  ln.dup0 = (ln.kc & (G::DUP - 1)) == 0;
  const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)qrow * a.num_q_heads + hq0) * QHD;
  uint4 qr[REP][G::KCH];
#pragma unroll
  for (int h = 0; h < REP; ++h)
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      if (PR == 0)
        qr[h][i] = *reinterpret_cast<const uint4*>(qp + h * HD + (ln.kc + i * G::LPT_K) * G::EPC);
      else   // only the chunk in the head's own half is used
        qr[h][i] = i == h / (PR > 0 ? PR : 1)
                       ? *reinterpret_cast<const uint4*>(qp + h * QHD + ln.kc * G::EPC)
                       : make_uint4(0u, 0u, 0u, 0u);
    }

  {
    const size_t head_off = (size_t)g * HD * G::ISZ;
    c.kh = reinterpret_cast<const char*>(a.k_pool) + head_off;
    c.vh = reinterpret_cast<const char*>(a.v_pool) + head_off;
    c.rsb = (uint32_t)a.num_kv_heads * HD * G::ISZ;
    c.blk_bytes = c.rsb << bshift;
    ln.kc16 = (uint32_t)ln.kc * 16;
    ln.vc16 = (uint32_t)vc * 16;
    ln.koff = (uint32_t)ln.kg * c.rsb + ln.kc16;
    ln.voff = (uint32_t)ln.vg * c.rsb + ln.vc16;
  }

  WaveState<T, HD, REP> st;
#pragma unroll
  for (int jj = 0; jj < G::HPL; ++jj) {
    st.m[jj] = -INFINITY;
    st.lsum[jj] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < G::HPV; ++i)
#pragma unroll
    for (int e = 0; e < G::DPL; ++e) st.o[i][e] = 0.f;

  // ---- tiles w, w + 4, ... of the split, every one through the LDS ring
  constexpr int kStep = kWaves * G::TILE;
  const int tb0 = t0 + w * G::TILE;
  if (tb0 < t1) {
    if (uni)
      wave_tiles<T, HD, REP, true, kStep, PR>(c, ln, st, qr, tb0, false, pbuf, cbuf, idslot,
                                              ring);
    else
      wave_tiles<T, HD, REP, false, kStep, PR>(c, ln, st, qr, tb0, any_bad, pbuf, cbuf, idslot,
                                               ring);
  }

  PKV_PHASE(4);
  // ---- per-wave totals, then merge the waves in LDS
  float* mw = merge + w * L::kMergeFloats;
#pragma unroll
  for (int jj = 0; jj < G::HPL; ++jj) st.lsum[jj] = strided_reduce<G::LPT_K, false>(st.lsum[jj]);
  __syncthreads();  // every wave is done with the table and tile buffers
  if (ln.kg == 0 && ln.dup0) {
#pragma unroll
    for (int jj = 0; jj < G::HPL; ++jj) {
      const int h = ln.hb + jj;
      if (h < REP) {
        mw[h] = st.m[jj];
        mw[REP + h] = st.lsum[jj];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PV::HPV; ++i) {
    const int h = ln.hg * PV::HPV + i;
    if (h < REP) {
#pragma unroll
      for (int e = 0; e < G::DPL; ++e) mw[2 * REP + h * HD + ln.vd0 + e] = st.o[i][e];
    }
  }
  __syncthreads();

  const int J = a.num_splits;
  for (int idx = tid; idx < REP * QHD; idx += kThreads) {
    // d: dim of the (virtual) row; a paired head's own half only
    const int h = idx / QHD, dq = idx % QHD;
    const int d = PR ? dq + (h / (PR > 0 ? PR : 1)) * QHD : dq;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, merge[ww * L::kMergeFloats + h]);
    float Ls = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float* mv = merge + ww * L::kMergeFloats;
        const float f = fast_exp2(mv[h] - M);
        Ls = fmaf(mv[REP + h], f, Ls);
        O = fmaf(mv[2 * REP + h * HD + d], f, O);
      }
    }
    if (nsplit == 1 && nps == 0) {
      out[h * QHD + dq] = from_f32<T>(Ls > 0.f ? O / Ls : 0.f);
    } else {
      const size_t row = ((size_t)s * a.num_q_heads + hq0 + h) * J + slot0 + j;
      if (a.counters) {
        // read back in this launch by another workgroup, possibly on another
        // XCD: device-coherent stores, written through the XCD's L2
        st_agent(a.ws_o + row * HD + d, O);
        if (dq == 0) {
          st_agent(a.ws_ml + row * 2, M);
          st_agent(a.ws_ml + row * 2 + 1, Ls);
        }
      } else {
        a.ws_o[row * HD + d] = O;
        if (dq == 0) {
          a.ws_ml[row * 2] = M;
          a.ws_ml[row * 2 + 1] = Ls;
        }
      }
    }
  }
  PKV_PHASE(5);
  if (!a.counters || (nsplit == 1 && nps == 0)) {
#ifdef PKV_PHASE_TRACE
    wait_vmcnt<0>();
    PKV_PHASE(8);
#endif
    return;
  }

  // ---- in-launch merge: the last workgroup of (s, g) to count itself merges.
  // Each wave waits until its device-coherent partial stores are complete
  // before the barrier; only then is the workgroup counted, so a workgroup
  // that sees the full count reads every partial back with device-coherent
  // loads. The atomics are relaxed, so the ordering comes from how gfx950
  // executes them, which the merge relies on (the GFX942 memory model that
  // LLVM's AMDGPU backend documents and applies to gfx950; a CPU test compiles
  // these helpers and checks the first three):
  //  1. an agent-scope atomic store is a global store with sc1 set: it is
  //     written through the XCD's own L2 (L2s of different XCDs are not
  //     coherent with each other), so no partial sits dirty in one L2;
  //  2. an agent-scope atomic load is a global load with sc1 set: it is not
  //     served from a line the reading XCD's L2 may hold stale;
  //  3. the counter is a returning global atomic add at agent scope, which
  //     the memory system performs at the device's coherence point;
  //  4. on this GFX9-family target vmcnt counts stores too, and a store's
  //     count is released only when the memory system has acknowledged it,
  //     so s_waitcnt vmcnt(0) followed by the barrier puts every wave's
  //     partial stores before the counting add.
  // With these, no cache-wide write-back or invalidate is needed (an
  // agent-scope release/acquire pair would emit buffer_wbl2 / buffer_inv of
  // the whole L2 per workgroup: measured 660 us per launch instead of 173).
  wait_vmcnt<0>();
  int* last = reinterpret_cast<int*>(smem) + kWaves * 64;
  __syncthreads();
  PKV_PHASE(6);
  if (nsplit > 1) {
    if (tid == 0) {
      int* cnt = a.counters + (size_t)s * a.num_kv_heads + g;
      const int before = count_agent(cnt);
      *last = before == nsplit - 1;
      // every split has counted: reset for the next launch
      if (before == nsplit - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    PKV_PHASE(7);
    PKV_PHASE_VALUE(9, *last);
    if (!*last) {
      PKV_PHASE(8);
      return;
    }
  }
  merge_partials<T, HD, REP, PR>(a, s, hq0, nps, slot0, nsplit, out,
                             reinterpret_cast<float*>(smem) + w * 64, w, lane);
#ifdef PKV_PHASE_TRACE
  wait_vmcnt<0>();
  __syncthreads();
  PKV_PHASE(8);
#endif
  };

  if constexpr (!SK) {
    piece();
  } else {
  // ---- stream-K: the pieces of workgroup i's range [start(i), start(i + 1))
  // of the head's stream of U units, in sequence order. The first H =
  // sched_sk / 2 ranges are E1 = ceil(U (64 + sk_first_extra) / (64 sched_sk))
  // units long, the others E2 = ceil((U - H E1) / (sched_sk - H)), both at
  // least sk_min_units: the first half of a head's workgroups reaches each
  // CU first, and the older workgroup of a CU streams faster (with equal
  // ranges it ended ~15 us before the other, leaving its CU half occupied).
  // The range of the last workgroup with tokens runs to the end, so that
  // empty sequences after the last token belong to it. A sequence's tokens
  // occupy units [a0, a1); its piece in range i is partial slot i - idx(a0)
  // of idx(a1 - 1) - idx(a0) + 1, idx(u) being the range holding unit u. An
  // empty sequence (a0 == a1) is one piece, of the range holding a0.
  if (!Lds<T, HD, REP>::uniform(bshift)) return;   // the planner never asks for it
  int* st_lds = reinterpret_cast<int*>(smem + round16(Lds<T, HD, REP>::bytes(0)));
  int* len_lds = st_lds + a.num_seqs;
  int* first_lds = len_lds + a.num_seqs + kWaves;   // shared-prefix tails only
  constexpr bool tails = TAILS;
  const int U = sk_layout<TAILS>(a, lim, st_lds, len_lds, len_lds + a.num_seqs, first_lds,
                                 first_lds + a.num_seqs);
  const int la = __builtin_ctz((unsigned)a.sched_align);
  const int i = blockIdx.y;
  const int Nh = a.sched_sk, H = Nh / 2, mu = a.sk_min_units;
  const int64_t e1 = ((int64_t)U * (64 + a.sk_first_extra) + 64ll * Nh - 1) / (64ll * Nh);
  const int E1 = (int)(e1 < mu ? mu : e1);
  const int64_t HE = (int64_t)H * E1, rest = (int64_t)U - HE;
  const int64_t e2 = Nh == H ? E1 : rest > 0 ? (rest + (Nh - H) - 1) / (Nh - H) : mu;
  const int E2 = (int)(e2 < mu ? mu : e2);
  auto start = [&](int k) -> int64_t {
    return k <= H ? (int64_t)k * E1 : HE + (int64_t)(k - H) * E2;
  };
  auto idx = [&](int u) -> int { return u < HE ? u / E1 : H + (int)((u - HE) / E2); };
  const int last_active = U > 0 ? idx(U - 1) : 0;
  if (i > last_active) return;
  const int lo = (int)start(i);
  const int64_t hi = i == last_active ? INT64_MAX : start(i + 1);
  auto units = [&](int sq) { return (len_lds[sq] + a.sched_align - 1) >> la; };
  // first sequence with tokens past lo, or empty at or after it
  int l = 0, r = a.num_seqs;
  while (l < r) {
    const int m = (l + r) >> 1;
    if (st_lds[m] + units(m) > lo || st_lds[m] >= lo) r = m;
    else l = m + 1;
  }
  for (int sq = l; sq < a.num_seqs; ++sq) {
    // c: the tokens of the stream (a tail with sharing), from token f on
    const int a0 = st_lds[sq], a1 = a0 + units(sq), c = len_lds[sq];
    if ((int64_t)a0 >= hi) break;
    const int f = tails ? first_lds[sq] : 0;
    Piece p;
    p.s = sq;
    p.start = f;
    p.ctx = f + c;
    if (a1 == a0) {
      p.t0 = p.t1 = f;
      p.slot = 0;
      p.n = 1;
    } else {
      const int b0 = a0 > lo ? a0 : lo;
      const int b1 = (int64_t)a1 < hi ? a1 : (int)hi;
      const int e1 = (b1 - a0) << la;
      p.t0 = f + ((b0 - a0) << la);
      p.t1 = f + (e1 < c ? e1 : c);
      p.slot = i - idx(a0);
      p.n = idx(a1 - 1) - idx(a0) + 1;
    }
    // memory safety whatever the layout gave: an inconsistent piece does no work
    if (p.start < 0 || p.t0 < p.start || p.t0 > p.t1 || p.t1 > p.ctx || p.ctx > lim ||
        p.slot < 0 || p.slot >= p.n ||
        p.n > a.num_splits - (tails ? a.sh.prefix_slots : 0))
      continue;
    __syncthreads();   // the previous piece is done with LDS
    s = qrow = p.s;
    j = p.slot;
    ctx = p.ctx;
    pc = p;
    piece();
  }
  }
}

template <typename T, int HD, int REP, int PR, bool SK>
__global__ void __launch_bounds__(kThreads) decode_partials_kernel(DecodeArgs a) {
  decode_body<T, HD, REP, PR, SK, false>(a);
}

template <typename T, int HD, int REP>
__global__ void __launch_bounds__(kThreads) decode_tails_kernel(DecodeArgs a) {
  decode_body<T, HD, REP, 0, true, true>(a);
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
  const int J = a.num_splits;
  // partials: slots 0 .. nps-1 (shared pass), then slot0 .. slot0+nsplit-1
  int nps = 0, slot0 = 0, nsplit;
  if (a.sched_q > 0) {
    const PieceCounts c = piece_counts(ctx, __builtin_ctz((unsigned)P),
                                       __builtin_ctz((unsigned)a.sched_q),
                                       __builtin_ctz((unsigned)a.sched_align));
    nsplit = ctx > 0 ? c.big + c.tail : 0;
  } else if (a.sh.group_start) {
    const int start = min(ctx, shared_len(a.sh, group_of(a.sh, s), lim, a.block_shift));
    nps = (start + a.sh.prefix_part - 1) / a.sh.prefix_part;
    slot0 = a.sh.prefix_slots;
    nsplit = min((ctx - start + P - 1) / P, J - slot0);
  } else {
    nsplit = (ctx + P - 1) / P;
  }
  if (nps == 0 && nsplit <= 1) return;   // written by the partials kernel
  const int n = nps + nsplit;
  auto slot = [&](int i) { return i < nps ? i : slot0 + i - nps; };
  const size_t row0 = ((size_t)s * a.num_q_heads + h) * J;
  const float* ml = a.ws_ml + row0 * 2;
  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, ml[2 * slot(i)]);
  M = group_max<64>(M);
  float Ls = 0.f;
  for (int i = lane; i < n; i += 64) {
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(ml[2 * slot(i)] - M);
    wts[i] = f;
    Ls = fmaf(ml[2 * slot(i) + 1], f, Ls);
  }
  Ls = group_sum<64>(Ls);
  __syncthreads();
  // paired heads: virtual rows of head_dim, this head's half of them
  const int qhd = a.pair_rep > 0 ? head_dim / 2 : head_dim;
  const int half = a.pair_rep > 0 ? (h % (2 * a.pair_rep)) / a.pair_rep : 0;
  const float* po = a.ws_o + row0 * head_dim + half * qhd;
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * qhd;
  for (int d = lane; d < qhd; d += 64) {
    float O = 0.f;
    for (int i = 0; i < n; ++i) O = fmaf(wts[i], po[(size_t)slot(i) * head_dim + d], O);
    out[d] = from_f32<T>(Ls > 0.f ? O / Ls : 0.f);
  }
}


template <typename T, int HD, int REP, int PR = 0>
pkv_status launch_split(const DecodeArgs& a, hipStream_t st) {
  using L = Lds<T, HD, REP>;
  const int piece = a.sched_q > 0 ? max_piece(a.partition, a.sched_q) : a.partition;
  int lds = L::bytes(L::table_entries(piece, a.block_shift));
  // shared-prefix decode: the leading slots belong to the shared pass
  dim3 grid(a.num_kv_heads, a.num_seqs, a.num_splits - a.sh.prefix_slots);
  if (a.sched_sk > 0) {
    // stream-K: sched_sk ranges per KV head; the layout (start, length per
    // sequence, the scan's words) after the piece's LDS
    // (and, for shared-prefix tails, the tails' first tokens and the group table)
    lds = round16(L::bytes(0)) +
          ((a.sh.group_start ? 5 : 2) * a.num_seqs + kWaves) * (int)sizeof(int);
    grid = dim3(a.num_kv_heads, a.sched_sk, 1);
  } else if (a.sched_q > 0 || a.sched_lpt) {
    // pieces: at most num_splits per sequence (one in longest-first order)
    const int planes = a.num_seqs * a.num_splits;
    const int y = planes < kRowGridZ ? planes : kRowGridZ;
    grid = dim3(a.num_kv_heads, y, (planes + y - 1) / y);
  } else if (a.cu_q) {
    const int z = a.total_q < kRowGridZ ? a.total_q : kRowGridZ;
    grid = dim3(a.num_kv_heads, (a.total_q + z - 1) / z, z);
  }
  if (a.sched_sk > 0) {
    if constexpr (PR == 0 && HD * sizeof(T) >= 256) {
      if (a.sh.group_start) {
        hipLaunchKernelGGL((decode_tails_kernel<T, HD, REP>), grid, dim3(kThreads), lds, st, a);
        return launch_status("decode_tails_kernel");
      }
      hipLaunchKernelGGL((decode_partials_kernel<T, HD, REP, PR, true>), grid, dim3(kThreads),
                         lds, st, a);
      return launch_status("decode_partials_kernel");
    }
    set_error("stream-K ranges are compiled for unpaired rows of 256 bytes or more only");
    return PKV_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL((decode_partials_kernel<T, HD, REP, PR, false>), grid, dim3(kThreads), lds,
                     st, a);
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
  return row_bytes >= 1024 ? 2 : row_bytes >= 512 ? 4 : row_bytes >= 256 ? 8 : row_bytes >= 128 ? 32 : 64;
}

bool decode_supported(int dtype, int head_dim, int rep) {
  (void)dtype;
  const bool hd_ok = head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 ||
                     head_dim == 256;
  return hd_ok && rep >= 1 && rep <= 8;
}

pkv_status launch_decode_partials(const DecodeArgs& a, int dtype, int head_dim, int rep,
                                  hipStream_t st) {
  if (a.pair_rep > 0) {
    // paired bf16 heads of 64 dims: virtual heads of 128, groups of 2 * pair_rep
    if (dtype == PKV_BF16 && head_dim == 128 && rep == 2 * a.pair_rep) {
      switch (a.pair_rep) {
        case 1: return launch_split<uint16_t, 128, 2, 1>(a, st);
        case 2: return launch_split<uint16_t, 128, 4, 2>(a, st);
        case 3: return launch_split<uint16_t, 128, 6, 3>(a, st);
        case 4: return launch_split<uint16_t, 128, 8, 4>(a, st);
        default: break;
      }
    }
    set_error("paired heads: no kernel for dtype %d, virtual head_dim %d, group %d", dtype,
              head_dim, rep);
    return PKV_ERR_UNSUPPORTED;
  }
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

#ifdef PKV_PHASE_TRACE
// The traced build's access to the timestamps (host memory, kTraceRows x
// kTraceCols uint64): clear before a call, copy after it has completed.
extern "C" int pkv_phase_trace_clear(const void* zeros, size_t bytes) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(pkv::g_phase_trace), zeros, bytes, 0,
                                hipMemcpyHostToDevice);
}
extern "C" int pkv_phase_trace_copy(void* host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(pkv::g_phase_trace), bytes, 0,
                                  hipMemcpyDeviceToHost);
}
#endif
