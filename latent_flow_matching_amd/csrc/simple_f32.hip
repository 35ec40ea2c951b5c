// The fp32 path's GEMMs and attention, and the small projections with 128-wide latents:
//   * gemm_simple: fp32 activations times fp32, bf16 or fp16 weights, fp32 accumulation.
//     fp32 weights (every GEMM of the fp32 compute path) run on the fp32 MFMA
//     (k_gemm_f32m, one wave per 64 x 64 tile, operands straight into registers); 16-bit
//     weights (img_in and final.out on the 16-bit paths, whose inputs are the caller's
//     unpadded fp32 latents) on an LDS-tiled FMA kernel.  Launches with few tiles cut k into
//     slices, and a second kernel adds them in a fixed order, so that few tokens still stream
//     the weights through the whole device.
//   * attention_f32: the fp32 path's softmax attention, one wave per (query, head), online
//     softmax over 64-key chunks.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int TN = 64, TM = 64, TK = 16;

// First token tile of each row group (entries past the last group hold the total).
struct TileStarts {
  int t[kMaxGroups + 1];
};

// The epilogue of one 64 x 64 tile (or of its first 16 NJ rows): thread (tx, ty) holds
// features n0 + tx + 16 i of tokens m0 + ty + 16 j (rows inside the group).
template <int EPI, int NJ = 4>
__device__ __forceinline__ void simple_epilogue(const GemmArgs &a, const GemmGroup &grp, int n0,
                                                int m0, int tx, int ty, const float (&acc)[4][4]) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int m = m0 + ty + 16 * j;
    if (m >= grp.rows) continue;
    const int tok = grp.out_row0 + m;
    if constexpr (EPI == EPI_STORE_F32) {
      float *o = a.out + (size_t)tok * a.ldo + n0 + tx;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[16 * i] = a.accumulate == 1   ? o[16 * i] + a.alpha * acc[i][j]
                    : a.accumulate == 2 ? a.alpha * acc[i][j]
                                        : acc[i][j];
    } else if constexpr (EPI == EPI_RESID) {
      const float *gate = a.gate[segment_of(tok, a.b1, a.b2, a.per)] + n0 + tx;
      float *xr = a.x + (size_t)tok * a.ldres + n0 + tx;
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[16 * i] += gate[16 * i] * acc[i][j];
    } else {
      if (n0 < a.split) {
        float *q = reinterpret_cast<float *>(a.qkv) + (size_t)tok * a.ldq + n0 + tx;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[16 * i] = acc[i][j];
      } else {
        // 64-row tile = gate rows of features [32c, 32c+32) then their up rows
        float *c = reinterpret_cast<float *>(a.cat) + (size_t)tok * a.ldc + a.cat_off +
                   (n0 - a.split) / 2 + tx;
#pragma unroll
        for (int i = 0; i < 2; ++i) c[16 * i] = silu(acc[i][j]) * acc[i + 2][j];
      }
    }
  }
}

// Tile coordinates of workgroup tile `lt` (feature tile major, then the groups' token tiles of
// tm rows).
struct SimpleTile {
  int gi, n0, m0;
};
__device__ __forceinline__ SimpleTile simple_tile(const TileStarts &tb, int m_tiles_total, int lt,
                                                  int tm = TM) {
  const int tile_n = lt / m_tiles_total;
  const int mt = lt - tile_n * m_tiles_total;
  int gi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) gi += mt >= tb.t[i];
  return SimpleTile{gi, tile_n * TN, (mt - tb.t[gi]) * tm};
}

// k-slices: workgroup (tile, slice) takes the slice's TK-steps [kt0, kt1) of the tile's k;
// with splits > 1 it stores its 64 x 64 partial sums to a.part ([slice][tile][m][n]), and
// k_gemm_simple_reduce adds the slices in slice order and applies the epilogue.
template <typename TW, int EPI>
__global__ __launch_bounds__(256) void k_gemm_simple(GemmArgs a, TileStarts tb, int m_tiles_total,
                                                     int splits) {
  __shared__ float ws[TK][TN + 4];
  __shared__ float xs[TK][TM + 4];
  const int lt = blockIdx.x / splits, slice = blockIdx.x - lt * splits;
  const SimpleTile st = simple_tile(tb, m_tiles_total, lt);
  const GemmGroup grp = a.g[st.gi];
  const int n0 = st.n0, m0 = st.m0;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const TW *W = reinterpret_cast<const TW *>(grp.w);
  const float *X = reinterpret_cast<const float *>(grp.x);
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int kt_all = a.k / TK;
  const int kt0 = (int)((long long)kt_all * slice / splits);
  const int kt1 = (int)((long long)kt_all * (slice + 1) / splits);
  // the next k-step's operands load into registers while the current one multiplies
  const TW *wrow = W + (size_t)(n0 + lr) * (a.ldw > 0 ? a.ldw : a.k) + lk;
  const int xrow = m0 + lr;
  const float *xp = X + (size_t)xrow * a.ldx + lk;
  float wn[4], xn[4];
  auto fetch = [&](int kt) {
    const int k0 = kt * TK;
#pragma unroll
    for (int e = 0; e < 4; ++e) wn[e] = to_f32(wrow[k0 + e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) xn[e] = xrow < grp.rows ? xp[k0 + e] : 0.f;
  };
  float acc[4][4] = {};
  if (kt0 < kt1) fetch(kt0);
  for (int kt = kt0; kt < kt1; ++kt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ws[lk + e][lr] = wn[e];
      xs[lk + e][lr] = xn[e];
    }
    __syncthreads();
    if (kt + 1 < kt1) fetch(kt + 1);
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float wv[4], xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = ws[kk][tx + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = xs[kk][ty + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += wv[i] * xv[j];
    }
    __syncthreads();
  }
  if (splits > 1) {
    const int tiles = gridDim.x / splits;
    float *pp = a.part + ((size_t)slice * tiles + lt) * (TM * TN);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[(ty + 16 * j) * TN + tx + 16 * i] = acc[i][j];
    return;
  }
  simple_epilogue<EPI>(a, grp, n0, m0, tx, ty, acc);
}

// Sum of the k-slices of a tile's partials in slice order, and the epilogue: workgroup
// (tile, r) takes the tile's rows 16 r .. 16 r + 15 (tiles of tm rows, partials laid out as
// 64 x 64).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_simple_reduce(GemmArgs a, TileStarts tb,
                                                            int m_tiles_total, int splits, int tm) {
  const int lt = blockIdx.x, tiles = gridDim.x, r = blockIdx.y;
  const SimpleTile st = simple_tile(tb, m_tiles_total, lt, tm);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int s = 0; s < splits; ++s) {
    const float *pp = a.part + ((size_t)s * tiles + lt) * (TM * TN) + (16 * r + ty) * TN + tx;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] += pp[16 * i];
  }
  simple_epilogue<EPI, 1>(a, a.g[st.gi], st.n0, st.m0 + 16 * r, tx, ty, acc);
}

// fp32 weights: v_mfma_f32_16x16x4_f32, one wave per 64 x 64 tile, operands straight from
// global memory into registers (no LDS).  For each 16-wide chunk of k, lane (c, q) (c = lane %
// 16, q = lane / 16) loads k0 + 4q .. k0 + 4q + 3 of weight row 16 fb + c and of token row
// 16 tb + c; MFMA step s takes component s, so lane group q stands for k = k0 + 4q + s in both
// operands and the four steps cover the chunk once.  Lane (c, q) then holds features
// n0 + 16 fb + 4q + {0..3} of token m0 + 16 tb + c.  Two chunks are in flight while the
// previous one multiplies.  A tile has TB blocks of 16 token rows (up to 64): groups of at
// most 48 rows, such as 32 + 16 tokens, do not multiply padding.
template <int EPI, int TB>
__device__ __forceinline__ void mfma32_epilogue(const GemmArgs &a, const GemmGroup &grp, int n0,
                                                int m0, int lane, const f32x4 (&acc)[4][TB]) {
  const int c = lane & 15, q = lane >> 4;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int m = m0 + 16 * tb + c;
    if (m >= grp.rows) continue;
    const int tok = grp.out_row0 + m;
    if constexpr (EPI == EPI_STORE_F32) {
      float *o = a.out + (size_t)tok * a.ldo + n0 + 4 * q;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        f32x4 *op = reinterpret_cast<f32x4 *>(o + 16 * fb);
        f32x4 v = acc[fb][tb];
        if (a.accumulate == 1) v = *op + a.alpha * v;
        else if (a.accumulate == 2) v = a.alpha * v;
        *op = v;
      }
    } else if constexpr (EPI == EPI_RESID) {
      const float *gate = a.gate[segment_of(tok, a.b1, a.b2, a.per)] + n0 + 4 * q;
      float *xr = a.x + (size_t)tok * a.ldres + n0 + 4 * q;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        f32x4 *xp = reinterpret_cast<f32x4 *>(xr + 16 * fb);
        *xp = *xp + *reinterpret_cast<const f32x4 *>(gate + 16 * fb) * acc[fb][tb];
      }
    } else {
      if (n0 < a.split) {
        float *o = reinterpret_cast<float *>(a.qkv) + (size_t)tok * a.ldq + n0 + 4 * q;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) *reinterpret_cast<f32x4 *>(o + 16 * fb) = acc[fb][tb];
      } else {
        // 64-row tile = gate rows of features [32c, 32c+32) then their up rows
        float *o = reinterpret_cast<float *>(a.cat) + (size_t)tok * a.ldc + a.cat_off +
                   (n0 - a.split) / 2 + 4 * q;
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = silu(acc[fb][tb][e]) * acc[fb + 2][tb][e];
          *reinterpret_cast<f32x4 *>(o + 16 * fb) = v;
        }
      }
    }
  }
}

template <int EPI, int TB>
__global__ __launch_bounds__(64) void k_gemm_f32m(GemmArgs a, TileStarts tb, int m_tiles_total,
                                                  int splits) {
  const int lt = blockIdx.x / splits, slice = blockIdx.x - lt * splits;
  const SimpleTile st = simple_tile(tb, m_tiles_total, lt, 16 * TB);
  const GemmGroup grp = a.g[st.gi];
  const int lane = threadIdx.x, c = lane & 15, q = lane >> 4;
  const int LW = a.ldw > 0 ? a.ldw : a.k;
  const float *W = reinterpret_cast<const float *>(grp.w) + (size_t)st.n0 * LW;
  const float *X = reinterpret_cast<const float *>(grp.x) + (size_t)st.m0 * a.ldx;
  // descriptors over the tile's 64 weight rows and its token rows up to the group's end: rows
  // past it read as zero (the range check includes the scalar offset)
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void *)W, (short)0, (int)min((long long)TN * LW * 4, 0x7FFFFFFFll), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
      (void *)X, (short)0, (int)min((long long)(grp.rows - st.m0) * a.ldx * 4, 0x7FFFFFFFll),
      0x00020000);
  const int vo_w = (c * LW + 4 * q) * 4, vo_x = (c * a.ldx + 4 * q) * 4;
  const int kc_all = a.k / TK;
  const int kc0 = (int)((long long)kc_all * slice / splits);
  const int kc1 = (int)((long long)kc_all * (slice + 1) / splits);
  f32x4 w0[4], x0[TB], w1[4], x1[TB];
  auto load = [&](int kc, f32x4 (&w)[4], f32x4 (&x)[TB]) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      w[b] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs_w, vo_w, (16 * b * LW + kc * TK) * 4, 0));
#pragma unroll
    for (int b = 0; b < TB; ++b)
      x[b] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs_x, vo_x, (16 * b * a.ldx + kc * TK) * 4, 0));
  };
  f32x4 acc[4][TB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const f32x4 (&w)[4], const f32x4 (&x)[TB]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb2 = 0; tb2 < TB; ++tb2)
          acc[fb][tb2] = __builtin_amdgcn_mfma_f32_16x16x4f32(w[fb][s], x[tb2][s], acc[fb][tb2], 0, 0, 0);
  };
  // chunks past the slice's end are clamped to its last one (repeated loads, never used)
  int kc = kc0;
  load(kc, w0, x0);
  load(min(kc + 1, kc1 - 1), w1, x1);
  for (; kc + 2 <= kc1; kc += 2) {
    mma(w0, x0);
    load(min(kc + 2, kc1 - 1), w0, x0);
    mma(w1, x1);
    load(min(kc + 3, kc1 - 1), w1, x1);
  }
  if (kc < kc1) mma(w0, x0);
  if (splits > 1) {  // partial tile [slice][tile][m][n], as k_gemm_simple_reduce reads it
    float *pp = a.part + ((size_t)slice * (gridDim.x / splits) + lt) * (TM * TN);
#pragma unroll
    for (int tb2 = 0; tb2 < TB; ++tb2)
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
        *reinterpret_cast<f32x4 *>(pp + (16 * tb2 + c) * TN + 16 * fb + 4 * q) = acc[fb][tb2];
    return;
  }
  mfma32_epilogue<EPI, TB>(a, grp, st.n0, st.m0, lane, acc);
}

template <typename TW, int EPI>
hipError_t launch_simple(const GemmArgs &a, hipStream_t s) {
  TileStarts tb = {};
  for (int i = 0; i < kMaxGroups; ++i)
    tb.t[i + 1] = tb.t[i] + (i < a.ng ? (a.g[i].rows + TM - 1) / TM : 0);
  const int m_tiles = tb.t[kMaxGroups];
  if (m_tiles == 0) return hipSuccess;
  const int tiles = m_tiles * (a.n / TN);
  // k-slices when the tiles give under eight workgroups per compute unit (few tokens: the
  // weights then stream through many more workgroups at once), at least 8 k-steps each
  int splits = 1;
  if (a.part != nullptr && a.cus > 0 && tiles < 8 * a.cus) {
    splits = min(16, min((8 * a.cus + tiles - 1) / tiles, (a.k / TK) / 8));
    const long long room = (long long)a.part_tiles * gemm_part_floats / (TM * TN);
    while (splits > 1 && (long long)splits * tiles > room) --splits;
    if (splits < 2) splits = 1;
  }
  k_gemm_simple<TW, EPI><<<tiles * splits, 256, 0, s>>>(a, tb, m_tiles, splits);
  if (splits > 1)
    k_gemm_simple_reduce<EPI><<<dim3(tiles, TM / 16), 256, 0, s>>>(a, tb, m_tiles, splits, TM);
  return hipGetLastError();
}

// fp32 weights on the fp32 MFMA: one 64-thread wave per tile and k-slice.  k is cut into as
// many slices as keep every wave resident at once (the occupancy the runtime reports for the
// kernel, times the compute units): one more wave than fits would start a second round that
// takes as long as the first.  At most 32 slices (their partials cost HBM traffic), at least
// 8 chunks of 16 k each.
template <int EPI, int TB>
hipError_t run_f32m(const GemmArgs &a, hipStream_t s) {
  TileStarts tb = {};
  for (int i = 0; i < kMaxGroups; ++i)
    tb.t[i + 1] = tb.t[i] + (i < a.ng ? (a.g[i].rows + 16 * TB - 1) / (16 * TB) : 0);
  const int m_tiles = tb.t[kMaxGroups];
  if (m_tiles == 0) return hipSuccess;
  const int tiles = m_tiles * (a.n / TN);
  // resident waves per compute unit (initialised once, thread-safely)
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gemm_f32m<EPI, TB>, 64, 0) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  int splits = 1;
  const int slots = per_cu * a.cus;
  if (a.part != nullptr && a.cus > 0 && 2 * tiles <= slots) {
    splits = min(32, min(slots / tiles, (a.k / TK) / 8));
    const long long room = (long long)a.part_tiles * gemm_part_floats / (TM * TN);
    while (splits > 1 && (long long)splits * tiles > room) --splits;
    if (splits < 2) splits = 1;
  }
  k_gemm_f32m<EPI, TB><<<tiles * splits, 64, 0, s>>>(a, tb, m_tiles, splits);
  if (splits > 1)
    k_gemm_simple_reduce<EPI><<<dim3(tiles, TB), 256, 0, s>>>(a, tb, m_tiles, splits, 16 * TB);
  return hipGetLastError();
}

// Token rows per tile: the fewest 16-row blocks that keep the number of token tiles (each of
// which streams the weights once) what 64-row tiles give.
template <int EPI>
hipError_t launch_f32m(const GemmArgs &a, hipStream_t s) {
  auto tiles_of = [&](int rows_per_tile) {
    int t = 0;
    for (int i = 0; i < a.ng; ++i) t += (a.g[i].rows + rows_per_tile - 1) / rows_per_tile;
    return t;
  };
  const int t64 = tiles_of(64);
  if (tiles_of(16) == t64) return run_f32m<EPI, 1>(a, s);
  if (tiles_of(32) == t64) return run_f32m<EPI, 2>(a, s);
  if (tiles_of(48) == t64) return run_f32m<EPI, 3>(a, s);
  return run_f32m<EPI, 4>(a, s);
}

template <typename TW>
hipError_t dispatch_simple(const GemmArgs &a, int epi, hipStream_t s) {
  if constexpr (std::is_same<TW, float>::value) {
    switch (epi) {
      case EPI_STORE_F32: return launch_f32m<EPI_STORE_F32>(a, s);
      case EPI_QKV_SWIGLU: return launch_f32m<EPI_QKV_SWIGLU>(a, s);
      case EPI_RESID: return launch_f32m<EPI_RESID>(a, s);
    }
  } else {
    switch (epi) {
      case EPI_STORE_F32: return launch_simple<TW, EPI_STORE_F32>(a, s);
      case EPI_QKV_SWIGLU: return launch_simple<TW, EPI_QKV_SWIGLU>(a, s);
      case EPI_RESID: return launch_simple<TW, EPI_RESID>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a, int total_q) {
  __shared__ float qs[4][128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qi = blockIdx.x * 4 + wave;
  const int head = blockIdx.y;
  // locate the group of the qi-th query (waves past the end idle but reach the barrier)
  const bool active = qi < total_q;
  int gi = 0, off = active ? qi : 0;
  while (gi < a.ng - 1 && off >= a.g[gi].q1 - a.g[gi].q0) {
    off -= a.g[gi].q1 - a.g[gi].q0;
    ++gi;
  }
  const AttnGroup grp = a.g[gi];
  const int q = grp.q0 + off;
  const float *base = reinterpret_cast<const float *>(a.qkv);
  const float *qp = base + (size_t)q * a.ldqkv + head * 128;
  qs[wave][2 * lane] = qp[2 * lane];
  qs[wave][2 * lane + 1] = qp[2 * lane + 1];
  __syncthreads();
  if (!active) return;
  float m_run = -INFINITY, l_run = 0.f, o0 = 0.f, o1 = 0.f;
  for (int c = grp.k0; c < grp.k1; c += 64) {
    const int key = c + lane;
    float sc = -INFINITY;
    if (key < grp.k1) {
      const float *kp = base + (size_t)key * a.ldqkv + a.d_model + head * 128;
      float dot = 0.f;
      for (int d = 0; d < 128; ++d) dot += qs[wave][d] * kp[d];
      sc = dot * a.scale;
    }
    const float m_new = fmaxf(m_run, wave_max(sc));
    const float alpha = expf(m_run - m_new);
    const float p = key < grp.k1 ? expf(sc - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    const int nk = min(64, grp.k1 - c);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(p, j, 64);
      const float *vp = base + (size_t)(c + j) * a.ldqkv + 2 * a.d_model + head * 128;
      o0 += pj * vp[2 * lane];
      o1 += pj * vp[2 * lane + 1];
    }
    m_run = m_new;
  }
  float *op = reinterpret_cast<float *>(a.out) + (size_t)q * a.ldo + head * 128;
  op[2 * lane] = o0 / l_run;
  op[2 * lane + 1] = o1 / l_run;
}

}  // namespace

hipError_t gemm_simple(const GemmArgs &a, int epi, int w_type, hipStream_t s) {
  if (a.n % TN || a.k % TK || a.ng < 1 || a.ng > kMaxGroups) return hipErrorInvalidValue;
  switch (w_type) {
    case OP_F32: return dispatch_simple<float>(a, epi, s);
    case OP_BF16: return dispatch_simple<bf16>(a, epi, s);
    case OP_F16: return dispatch_simple<f16>(a, epi, s);
  }
  return hipErrorInvalidValue;
}

hipError_t attention_f32(const AttnArgs &a, hipStream_t s) {
  int total_q = 0;
  for (int i = 0; i < a.ng; ++i) total_q += a.g[i].q1 - a.g[i].q0;
  if (total_q <= 0) return hipSuccess;
  dim3 grid((total_q + 3) / 4, a.heads);
  k_attn_f32<<<grid, 256, 0, s>>>(a, total_q);
  return hipGetLastError();
}

}  // namespace dit
