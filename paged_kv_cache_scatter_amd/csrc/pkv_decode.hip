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
// Each wave takes token tiles of TILE tokens in turn:
//   K stage   lanes own (token, two 16-byte chunks of its K row); the REP query
//             heads of the group are held in registers, so each K row is read
//             once for the whole group; partial dots are summed across the
//             lanes of a token with DPP.
//   softmax   scores go through LDS to a lane-per-token layout; per-head tile
//             max by DPP; running max/sum per head (online softmax, log2 units).
//   V stage   lanes own (token, one 16-byte chunk of its V row); p from LDS;
//             o[REP][chunk] accumulates in fp32.
// At the end the four waves' (m, l, o) are merged in LDS and either the
// normalised output (single split) or the split partial is written.
#include "pkv_internal.h"

#include <math.h>

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

template <typename T, int HD>
struct Geo {
  static constexpr int ISZ = (int)sizeof(T);
  static constexpr int ROWB = HD * ISZ;  // bytes of one K (or V) row of one KV head
  static constexpr int EPC = 16 / ISZ;   // elements per 16-byte chunk
  static constexpr int TILE = ROWB >= 1024 ? 8 : ROWB >= 512 ? 16 : ROWB >= 256 ? 32 : 64;
  static constexpr int KCH = ROWB >= 32 ? 2 : 1;    // K chunks per lane per row
  static constexpr int LPT_K = ROWB / (16 * KCH);   // lanes per token (K stage)
  static constexpr int TPW_K = 64 / LPT_K;          // tokens per wave load (K)
  static constexpr int RK = TILE / TPW_K;           // K rows per lane per tile
  static constexpr int LPT_V = ROWB / 16;           // lanes per token (V stage)
  static constexpr int TPW_V = 64 / LPT_V;
  static constexpr int RV = TILE / TPW_V;           // V rows per lane per tile
  static_assert(RK >= 1 && RV >= 1 && LPT_K >= 1 && LPT_V >= 1 && LPT_V <= 64, "geometry");
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

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

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16_rne(x); }

// One tile of TILE tokens starting at tb (absolute position) for one wave.
// MASKED handles the split's last tile and tables holding invalid block ids.
template <typename T, int HD, int REP, bool MASKED>
__device__ __forceinline__ void decode_tile(
    const T* __restrict__ kbase, const T* __restrict__ vbase, size_t row_stride,
    const int* tbl, int tbl_base, int bshift, int tb, int t1,
    const uint4 (&qr)[REP][Geo<T, HD>::KCH], float scale_log2,
    float* sbuf, float* pbuf, int lane,
    float (&m)[REP], float (&lsum)[REP], float (&o)[REP][Geo<T, HD>::EPC]) {
  using G = Geo<T, HD>;
  const int kg = lane / G::LPT_K, kc = lane % G::LPT_K;
  const int vg = lane / G::LPT_V, vc = lane % G::LPT_V;
  const int bmask = (1 << bshift) - 1;

  // ---- issue K and V loads for the whole tile
  uint4 kr[G::RK][G::KCH];
  bool kval[G::RK];
#pragma unroll
  for (int r = 0; r < G::RK; ++r) {
    const int t = tb + r * G::TPW_K + kg;
    int blk = 0;
    bool ok = true;
    if (MASKED) {
      blk = (t < t1) ? tbl[(t >> bshift) - tbl_base] : -1;
      ok = blk >= 0;
    } else {
      blk = tbl[(t >> bshift) - tbl_base];
    }
    kval[r] = ok;
    const int bsafe = ok ? blk : 0;
    const T* p = kbase + ((size_t)bsafe * (size_t)(bmask + 1) + (size_t)(t & bmask)) * row_stride;
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      if (MASKED) {
        kr[r][i] = make_uint4(0, 0, 0, 0);
        if (ok) kr[r][i] = ld16(p + (kc + i * G::LPT_K) * G::EPC);
      } else {
        kr[r][i] = ld16(p + (kc + i * G::LPT_K) * G::EPC);
      }
    }
  }
  uint4 vr[G::RV];
#pragma unroll
  for (int r = 0; r < G::RV; ++r) {
    const int t = tb + r * G::TPW_V + vg;
    int blk = 0;
    bool ok = true;
    if (MASKED) {
      blk = (t < t1) ? tbl[(t >> bshift) - tbl_base] : -1;
      ok = blk >= 0;
    } else {
      blk = tbl[(t >> bshift) - tbl_base];
    }
    const int bsafe = ok ? blk : 0;
    const T* p = vbase + ((size_t)bsafe * (size_t)(bmask + 1) + (size_t)(t & bmask)) * row_stride;
    if (MASKED) {
      vr[r] = make_uint4(0, 0, 0, 0);
      if (ok) vr[r] = ld16(p + vc * G::EPC);
    } else {
      vr[r] = ld16(p + vc * G::EPC);
    }
  }

  // ---- scores: one K row shared by the REP query heads of the group
#pragma unroll
  for (int r = 0; r < G::RK; ++r) {
    float sc[REP];
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < G::KCH; ++i) acc = chunk_dot<T>(qr[h][i], kr[r][i], acc);
      acc = group_sum<G::LPT_K>(acc);
      sc[h] = acc * scale_log2;
      if (MASKED) sc[h] = kval[r] ? sc[h] : -INFINITY;
    }
    if (kc == 0) {
      float* dst = sbuf + (r * G::TPW_K + kg) * REP;
#pragma unroll
      for (int h = 0; h < REP; ++h) dst[h] = sc[h];
    }
  }

  // ---- online softmax over the tile, lane tl <-> token tl
  const int tl = lane % G::TILE;
  float corr[REP];
  {
    float pv[REP];
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      const float sv = sbuf[tl * REP + h];
      const float tmax = group_max<G::TILE>(sv);
      const float mnew = fmaxf(m[h], tmax);
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      corr[h] = fast_exp2(m[h] - mref);
      pv[h] = fast_exp2(sv - mref);
      lsum[h] = lsum[h] * corr[h] + ((G::TILE >= 64 || lane < G::TILE) ? pv[h] : 0.f);
      m[h] = mnew;
    }
    if (G::TILE >= 64 || lane < G::TILE) {
      float* dst = pbuf + tl * REP;
#pragma unroll
      for (int h = 0; h < REP; ++h) dst[h] = pv[h];
    }
  }

  // ---- o = o * corr + sum_t p_t v_t
#pragma unroll
  for (int h = 0; h < REP; ++h)
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) o[h][e] *= corr[h];
#pragma unroll
  for (int r = 0; r < G::RV; ++r) {
    const float* pp = pbuf + (r * G::TPW_V + vg) * REP;
    float pr[REP];
#pragma unroll
    for (int h = 0; h < REP; ++h) pr[h] = pp[h];
    float v[G::EPC];
    chunk_to_f32<T>(vr[r], v);
#pragma unroll
    for (int h = 0; h < REP; ++h)
#pragma unroll
      for (int e = 0; e < G::EPC; ++e) o[h][e] = fmaf(pr[h], v[e], o[h][e]);
  }
}

__host__ __device__ constexpr int round16(int b) { return (b + 15) & ~15; }

template <typename T, int HD, int REP>
struct Lds {
  using G = Geo<T, HD>;
  static constexpr int kTileFloats = 2 * G::TILE * REP;          // scores + probabilities
  static constexpr int kMergeFloats = REP * (HD + 2);            // m, l, o per wave
  // The merge area reuses the table/tile area once every wave has left the tile loop.
  static int bytes(int tbl_entries) {
    const int loop = round16(tbl_entries * 4) + kWaves * kTileFloats * 4;
    const int merge = kWaves * kMergeFloats * 4;
    return loop > merge ? loop : merge;
  }
};

template <typename T, int HD, int REP>
__global__ void __launch_bounds__(kThreads)
decode_partials_kernel(DecodeArgs a) {
  using G = Geo<T, HD>;
  using L = Lds<T, HD, REP>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int g = blockIdx.x, j = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bshift = a.block_shift;
  const int lim = min(a.max_ctx, a.max_blocks << bshift);
  int ctx = a.ctx_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > lim ? lim : ctx);
  const int P = a.partition;
  const int nsplit = (ctx + P - 1) / P;
  const int hq0 = g * REP;
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + hq0) * HD;

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
  float* tiles = reinterpret_cast<float*>(smem + round16(tbl_entries * 4));
  float* sbuf = tiles + w * L::kTileFloats;
  float* pbuf = sbuf + G::TILE * REP;
  float* merge = reinterpret_cast<float*>(smem);

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

  // ---- query heads of this group, in the K-stage lane layout
  const int kc = lane % G::LPT_K;
  const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)s * a.num_q_heads + hq0) * HD;
  uint4 qr[REP][G::KCH];
#pragma unroll
  for (int h = 0; h < REP; ++h)
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) qr[h][i] = ld16(qp + h * HD + (kc + i * G::LPT_K) * G::EPC);

  const size_t row_stride = (size_t)a.num_kv_heads * HD;
  const T* kbase = reinterpret_cast<const T*>(a.k_pool) + (size_t)g * HD;
  const T* vbase = reinterpret_cast<const T*>(a.v_pool) + (size_t)g * HD;

  float m[REP], lsum[REP], o[REP][G::EPC];
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) o[h][e] = 0.f;
  }

  for (int tb = t0 + w * G::TILE; tb < t1; tb += kWaves * G::TILE) {
    if (!any_bad && tb + G::TILE <= t1)
      decode_tile<T, HD, REP, false>(kbase, vbase, row_stride, tbl, tbl_base, bshift, tb, t1, qr,
                                     a.scale_log2, sbuf, pbuf, lane, m, lsum, o);
    else
      decode_tile<T, HD, REP, true>(kbase, vbase, row_stride, tbl, tbl_base, bshift, tb, t1, qr,
                                    a.scale_log2, sbuf, pbuf, lane, m, lsum, o);
  }

  // ---- per-wave totals, then merge the waves in LDS
  const int vg = lane / G::LPT_V, vc = lane % G::LPT_V;
  float* mw = merge + w * L::kMergeFloats;
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    lsum[h] = group_sum<64>(lsum[h]);
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) o[h][e] = strided_sum<G::LPT_V>(o[h][e]);
  }
  __syncthreads();  // every wave is done with the table and tile buffers
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      mw[h] = m[h];
      mw[REP + h] = lsum[h];
    }
  }
  if (vg == 0) {
#pragma unroll
    for (int h = 0; h < REP; ++h)
#pragma unroll
      for (int e = 0; e < G::EPC; ++e) mw[2 * REP + h * HD + vc * G::EPC + e] = o[h][e];
  }
  __syncthreads();

  const int J = a.num_splits;
  for (int idx = tid; idx < REP * HD; idx += kThreads) {
    const int h = idx / HD, d = idx % HD;
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
  return row_bytes >= 1024 ? 8 : row_bytes >= 512 ? 16 : row_bytes >= 256 ? 32 : 64;
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
