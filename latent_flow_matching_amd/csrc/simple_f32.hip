// fp32-accumulating kernels without MFMA:
//   * gemm_simple: LDS-tiled FMA GEMM with fp32 activations and fp32 or bf16 weights.  It
//     runs every GEMM of the fp32 compute path and, in both paths, the two small
//     projections with 128-wide latents (img_in, final.out), whose inputs are the caller's
//     unpadded fp32 latents.  Launches with few tiles cut k into slices (a second kernel
//     adds them in a fixed order), so that few tokens still stream the weights through
//     the whole device.
//   * attention_f32: the fp32 path's softmax attention, one wave per (query, head), online
//     softmax over 64-key chunks.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int TN = 64, TM = 64, TK = 16;

// First token tile of each row group (entries past the last group hold the total).
struct TileStarts {
  int t[kMaxGroups + 1];
};

// The epilogue of one 64 x 64 tile: thread (tx, ty) holds features n0 + tx + 16 i of tokens
// m0 + ty + 16 j (rows inside the group).
template <int EPI>
__device__ __forceinline__ void simple_epilogue(const GemmArgs &a, const GemmGroup &grp, int n0,
                                                int m0, int tx, int ty, const float (&acc)[4][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
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

// Tile coordinates of workgroup tile `lt` (feature tile major, then the groups' token tiles).
struct SimpleTile {
  int gi, n0, m0;
};
__device__ __forceinline__ SimpleTile simple_tile(const TileStarts &tb, int m_tiles_total, int lt) {
  const int tile_n = lt / m_tiles_total;
  const int mt = lt - tile_n * m_tiles_total;
  int gi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) gi += mt >= tb.t[i];
  return SimpleTile{gi, tile_n * TN, (mt - tb.t[gi]) * TM};
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

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_simple_reduce(GemmArgs a, TileStarts tb,
                                                            int m_tiles_total, int splits) {
  const int lt = blockIdx.x, tiles = gridDim.x;
  const SimpleTile st = simple_tile(tb, m_tiles_total, lt);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int s = 0; s < splits; ++s) {
    const float *pp = a.part + ((size_t)s * tiles + lt) * (TM * TN);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] += pp[(ty + 16 * j) * TN + tx + 16 * i];
  }
  simple_epilogue<EPI>(a, a.g[st.gi], st.n0, st.m0, tx, ty, acc);
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
  if (splits > 1) k_gemm_simple_reduce<EPI><<<tiles, 256, 0, s>>>(a, tb, m_tiles, splits);
  return hipGetLastError();
}

template <typename TW>
hipError_t dispatch_simple(const GemmArgs &a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE_F32: return launch_simple<TW, EPI_STORE_F32>(a, s);
    case EPI_QKV_SWIGLU: return launch_simple<TW, EPI_QKV_SWIGLU>(a, s);
    case EPI_RESID: return launch_simple<TW, EPI_RESID>(a, s);
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
