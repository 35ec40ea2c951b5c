// Row-wise FP8 GEMM on gfx950: OCP E4M3 operands, one fp32 scale per weight row and per
// token, fp32 accumulation ("FLUX.3 Image Klein: offene Gewichte ...", "Was sich geändert
// hat": the transformer ships in row-wise FP8; we0.ai "FLUX 3 Image Klein" article,
// "Hardwareanforderungen, Quantisierung und Inferenzlatenz": GPUs with FP8 kernels compute
// with it directly).
//
//   out[token][n] = xs[token] * ws[n] * sum_k X[token][k] * W[n][k]     (X, W: E4M3 codes)
//
// v_mfma_f32_16x16x128_f8f6f4 (both operands E4M3, no block scales) takes 32 bytes of k per
// lane: row (A) or column (B) lane % 16, k-quarter lane / 16.  Any assignment of bytes to k
// works as long as both operands use the same one; here lane l takes 16-byte chunks q and
// 4 + q (q = l / 16) of the 128-byte row, which are the chunks the 16-bit kernel reads for its
// two k-steps, so the LDS layout, the swizzle and the global loads are those of the 16-bit
// GEMM with one byte per value.  The MFMA adds the products of a group with limited
// alignment: a product more than about 12 bits below the group's largest is truncated.
//
// Workgroup tile 256 features x 256 tokens, 4 waves each 128 x 128 (8 x 8 accumulators of
// 16 x 16), k advances 128 per LDS stage (two stages, 128 KB).  Per k-tile each wave reads its
// 16 fragments once (32 bytes per lane each) and issues 64 MFMAs of 32 cycles, in row order
// (weight sub-tile outer); weight fragment i + 1 is read during row i.  The LDS writes of the
// next tile and the global loads two tiles ahead sit between the MFMAs of rows 1..4; a second
// barrier after them publishes the next tile, whose weight fragment 0 is read then and whose
// token fragment j is read right after the last MFMA that uses token fragment j of this
// tile, so the next tile starts without waiting on LDS.  Scales are applied to the accumulators before the
// shared epilogues (gemm_common.h).
#include "gemm_common.h"

namespace dit {

namespace {

constexpr int BK8 = 128;  // k (bytes) per LDS stage
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma8(const i32x8 &a, const i32x8 &b, f32x4 c) {
  // format 0 (E4M3) for both operands, scales off
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int EPI, int BM>
__global__ __launch_bounds__(256) void k_gemm8(GemmArgs a, TileBounds tb, int m_tiles_total,
                                               int total_tiles, int splits) {
  constexpr int WN = 2, WM = 2, NT = 256;
  constexpr int WTN = BN / WN, WTM = BM / WM;  // 128 x 128 (or 128 x 112)
  constexpr int FS = WTN / 16, TS = WTM / 16;  // 8 x 8 (or 8 x 7) sub-tiles of 16 x 16
  constexpr int LA = BN * 8 / NT, LB = BM * 8 / NT;  // 8 + 8 (or 8 + 7) 16-byte loads per thread
  constexpr int STAGE = (BN + BM) * BK8;       // 64 KB (or 60 KB)
  constexpr int MEND = 8 + 2 * (LA + LB);     // the LDS writes and global loads sit at m in [8, MEND)
  static_assert(BM % 32 == 0 && MEND < (FS - 1) * TS, "tile shape");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int per = gridDim.x >> 3;
  const int uid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (uid >= total_tiles * splits) return;
  const int lid = uid / splits, slice = uid - lid * splits;  // tile, k-slice
  const int n_tiles = a.n / BN;
  const int in_group = kGroupN * m_tiles_total;
  const int group = lid / in_group;
  const int first_n = group * kGroupN;
  const int gsize = min(n_tiles - first_n, kGroupN);
  const int rem = lid - group * in_group;
  const int tile_n = EPI == EPI_QKV_SWIGLU ? qkv_feature_tile(first_n + rem % gsize, n_tiles, a.split)
                                          : first_n + rem % gsize;
  const int mt = rem / gsize;
  int gi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) gi += mt >= tb.t[i];
  const int lmt = mt - tb.t[gi];
  const GemmGroup grp = a.g[gi];
  const int n0 = tile_n * BN;
  const int m0 = lmt * BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int K = a.k, LW = a.ldw > 0 ? a.ldw : a.k;  // bytes: reduction length, weight row stride
  const uint8_t *W = reinterpret_cast<const uint8_t *>(grp.w) + (size_t)n0 * LW;
  const uint8_t *X = reinterpret_cast<const uint8_t *>(grp.x) + (size_t)m0 * a.ldx;
  const int lchunk = tid & 7, lrow = tid >> 3;

  const int kt_all = K / BK8;
  const int kt0 = (int)((long long)kt_all * slice / splits);
  const int KT = (int)((long long)kt_all * (slice + 1) / splits) - kt0;
  W += (size_t)kt0 * BK8;
  X += (size_t)kt0 * BK8;
  // buffer descriptors: the weight tile's 256 rows; token rows from m0 to the group's end
  // (rows past it read as zero)
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void *)W, (short)0, (int)min((long long)BN * LW, 0x7FFFFFFFll), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
      (void *)X, (short)0, (int)min((long long)(grp.rows - m0) * a.ldx, 0x7FFFFFFFll), 0x00020000);
  const int vo_w = lrow * LW + lchunk * 16, vo_x = lrow * a.ldx + lchunk * 16;
  auto load_w = [&](int kt, int i) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rs_w, vo_w, i * (NT / 8) * LW + kt * BK8, 0);
  };
  auto load_x = [&](int kt, int i) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rs_x, vo_x, i * (NT / 8) * a.ldx + kt * BK8, 0);
  };
  // staging registers: tile kt+2 loads while tile kt+1 is written to LDS
  u32x4 ra[LA], rb[LB];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = load_w(kt, i);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = load_x(kt, i);
  };
  auto sstore = [&](int stage) {
    char *As = smem + stage * STAGE;
    char *Bs = As + BN * BK8;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *reinterpret_cast<u32x4 *>(As + swz(lrow + i * (NT / 8), lchunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<u32x4 *>(Bs + swz(lrow + i * (NT / 8), lchunk)) = rb[i];
  };
  const int r16 = lane & 15, q4 = lane >> 4;
  i32x8 fr[FS + TS];  // [weight sub-tiles | token sub-tiles]: chunks q4 and 4 + q4
  auto read_frag = [&](int stage, int f) {
    const char *As = smem + stage * STAGE;
    const char *Bs = As + BN * BK8;
    const char *base = f < FS ? As : Bs;
    const int row = f < FS ? wn * WTN + f * 16 + r16 : wm * WTM + (f - FS) * 16 + r16;
    fr[f].lo = *reinterpret_cast<const i32x4 *>(base + swz(row, q4));
    fr[f].hi = *reinterpret_cast<const i32x4 *>(base + swz(row, 4 + q4));
  };
  auto write_one = [&](int stage, int i) {  // i < 8: weights
    char *As = smem + stage * STAGE;
    char *Bs = As + BN * BK8;
    if (i < LA)
      *reinterpret_cast<u32x4 *>(As + swz(lrow + i * (NT / 8), lchunk)) = ra[i];
    else
      *reinterpret_cast<u32x4 *>(Bs + swz(lrow + (i - LA) * (NT / 8), lchunk)) = rb[i - LA];
  };
  auto gload_one = [&](int kt, int i) {
    if (i < LA) ra[i] = load_w(kt, i);
    else rb[i - LA] = load_x(kt, i - LA);
  };
  f32x4 acc[FS][TS];
#pragma unroll
  for (int i = 0; i < FS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  gload(0);
  sstore(0);
  gload(min(1, KT - 1));
  lds_sync();
  read_frag(0, 0);
#pragma unroll
  for (int j = 0; j < TS; ++j) read_frag(0, FS + j);

  // one k-tile from stage kt & 1; the staging registers hold tile kt+1 and receive tile kt+2
  // (indices past the slice are clamped: the repeats are harmless)
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const int nk = min(kt + 2, KT - 1);
    lds_sync();  // every wave is done reading the other stage (tile kt-1)
#pragma unroll
    for (int m = 0; m < FS * TS; ++m) {
      const int i = m / TS, j = m % TS;
      acc[i][j] = mma8(fr[i], fr[FS + j], acc[i][j]);
      if (j == 0 && i < FS - 1) read_frag(cur, i + 1);
      if (m >= 8 && m < MEND) {
        const int r = (m - 8) >> 1;
        if ((m & 1) == 0) write_one(cur ^ 1, r);
        else gload_one(nk, r);
      }
      if (m == MEND - 1) lds_sync();  // tile kt+1 written by every wave
      if (m == MEND) read_frag(cur ^ 1, 0);            // its weight fragment 0 (free since row 0)
      if (i == FS - 1) read_frag(cur ^ 1, FS + j);   // its token fragment j, just freed
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // row-wise scales: token scale per lane row, weight scales of the lane's four features
  {
    const float *xs = a.xs + grp.out_row0;
    const float *ws = grp.ws;
#pragma unroll
    for (int j = 0; j < TS; ++j) {
      const int m = m0 + wm * WTM + j * 16 + r16;
      const float sx = m < grp.rows ? xs[m] : 0.f;
#pragma unroll
      for (int i = 0; i < FS; ++i) {
        const f32x4 sw = *reinterpret_cast<const f32x4 *>(ws + n0 + wn * WTN + i * 16 + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] *= sx * sw[e];
      }
    }
  }
  if (splits > 1) {  // partial tile: [wave][sub-tile][lane] float4, in slice-major order
    f32x4 *pp = reinterpret_cast<f32x4 *>(a.part) +
                ((size_t)(slice * total_tiles + lid) * 4 + wave) * (FS * TS * 64) + lane;
#pragma unroll
    for (int i = 0; i < FS; ++i)
#pragma unroll
      for (int j = 0; j < TS; ++j) pp[(i * TS + j) * 64] = acc[i][j];
    return;
  }
  static_assert(2 * STAGE >= 4 * kVtLds, "LDS for the fused V transpose");
  static_assert(2 * STAGE >= 4 * WTM * 256, "LDS for the fused Q / K normalisation");
  epilogue<f16, BM, WN, WM, EPI, false>(a, grp, n0, m0, wn, wm, lane, acc, smem);
}

// A launch plan for tile height bm: token tiles, tiles, k-slices.
struct Plan8 {
  TileBounds tb;
  int m_tiles, total, splits;
};
template <int EPI>
Plan8 make_plan8(const GemmArgs &a, int bm) {
  Plan8 p;
  p.tb = TileBounds{};
  for (int i = 0; i < kMaxGroups; ++i)
    p.tb.t[i + 1] = p.tb.t[i] + (i < a.ng ? (a.g[i].rows + bm - 1) / bm : 0);
  p.m_tiles = p.tb.t[kMaxGroups];
  p.total = p.m_tiles * (a.n / BN);
  // k-slices: only for tiles that fill under half of the compute units, with at least 8
  // k-tiles per slice
  p.splits = 1;
  if (EPI != EPI_QKV_SWIGLU && a.part != nullptr && a.split_grid > 0 && 2 * p.total <= a.split_grid) {
    p.splits = min(8, min(a.split_grid / p.total, (a.k / BK8) / 8));
    p.splits = min(p.splits, a.part_tiles / p.total);  // as many partial tiles as the workspace holds
    if (p.splits < 2) p.splits = 1;
  }
  return p;
}

template <int EPI, int BM>
hipError_t run_plan8(const GemmArgs &a, const Plan8 &p, hipStream_t s) {
  const int grid = (p.total * p.splits + 7) / 8 * 8;
  k_gemm8<EPI, BM><<<grid, 256, 0, s>>>(a, p.tb, p.m_tiles, p.total, p.splits);
  if constexpr (EPI != EPI_QKV_SWIGLU)
    if (p.splits > 1)
      k_gemm_reduce<EPI, BM><<<dim3(p.total, BM / 4), 256, 0, s>>>(a, p.tb, p.m_tiles, p.total, p.splits);
  return hipGetLastError();
}

// linear2: 224-row tiles when the rounds of workgroups over the compute units, times the rows
// and k each workgroup takes, come out at least 5% lower (the 16-bit GEMM's rule)
template <int EPI>
hipError_t launch8(const GemmArgs &a, hipStream_t s) {
  const Plan8 p256 = make_plan8<EPI>(a, 256);
  if (p256.m_tiles == 0) return hipSuccess;
  if constexpr (EPI == EPI_RESID) {
    if (a.cus > 0) {
      const Plan8 p224 = make_plan8<EPI>(a, 224);
      auto cost = [&](const Plan8 &p, int bm) {
        return (double)((p.total * p.splits + a.cus - 1) / a.cus) * bm / p.splits;
      };
      if (20 * cost(p224, 224) < 19 * cost(p256, 256)) return run_plan8<EPI, 224>(a, p224, s);
    }
  }
  return run_plan8<EPI, 256>(a, p256, s);
}

}  // namespace

hipError_t gemm_fp8(const GemmArgs &a, int epi, hipStream_t s) {
  if (a.n % BN || a.k % BK8 || a.ng < 1 || a.ng > kMaxGroups || !a.xs) return hipErrorInvalidValue;
  if (!fused_heads_ok(a, epi)) return hipErrorInvalidValue;
  if (a.ldx % 16 || (a.ldw > 0 ? a.ldw : a.k) % 16) return hipErrorInvalidValue;
  for (int i = 0; i < a.ng; ++i)
    if (!a.g[i].ws) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_QKV_SWIGLU: return launch8<EPI_QKV_SWIGLU>(a, s);
    case EPI_RESID: return launch8<EPI_RESID>(a, s);
    case EPI_STORE_F32: return launch8<EPI_STORE_F32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
