// MFMA GEMM (16-bit operands: bf16 or fp16, fp32 accumulation) for the block's two fused
// projections on gfx950.
//
//   out[token][n] = sum_k X[token][k] * W[n][k]       (X = activations, W = [N, K] weights)
//
// Both operands are K-contiguous, which is the per-lane layout of v_mfma_f32_16x16x32_{bf16,f16}
// (lane l holds 8 consecutive k of row l%16, k-quarter l/16).  The weight tile is the MFMA A
// operand and the token tile the B operand, so each lane's accumulator holds one token and
// four consecutive output features: stores are 8-byte (bf16) or 16-byte (fp32) vectors.
// The 16x16x32 form moves a quarter of the accumulator registers per flop of the 32x32x16
// one; under the chip's power limit it holds a clock about 15% higher on the same work.
//
// Workgroup tile 256 features x 256 tokens, 4 waves (2 x 2) each owning 128 x 128 (64
// accumulators of 16x16 in AGPRs, one wave per SIMD).  k advances in tiles of 64 through two
// LDS stages (128 KB) with one barrier per k-tile; global loads are staged through registers
// one k-tile ahead.  LDS rows are 128 B (64 values), swizzled as described in gemm_common.h.
#include "gemm_common.h"

namespace dit {

namespace {

constexpr int BK = 64;   // k per LDS stage

// Main loop.  Entering k-tile kt a wave holds the fragments of its k-steps 0 and 1.  Before
// the barrier it runs the MFMAs of k-steps 0..2 while it reads k-steps 2 and 3 of tile kt,
// writes tile kt+1 into the other stage and issues the global loads of tile kt+2; after the
// barrier the MFMAs of k-step 3 overlap the reads of k-steps 0 and 1 of tile kt+1.  A stage is
// rewritten only after the barrier that follows the last reads of its previous tile.  The
// order of every MFMA and memory operation is pinned (sched_barrier), one memory operation
// after each MFMA, so the LDS and global latencies sit under MFMAs.  Token rows, which miss L2
// more often than weight rows under the grouped tile order, get two staging sets and so two
// k-tiles of latency cover.
//
// BM (token rows per tile) is 256 or 224: 224-row tiles (7 token sub-tiles per wave) let a
// launch whose 256-row tiles would leave many compute units idle in its last round fill them
// (linear2 at 4608 tokens: 12 x 18 = 216 tiles of 256 rows for 256 compute units, 12 x 21 =
// 252 of 224 rows).  The schedule below is written for any TS; with TS = 8 it is the
// 256-row kernel's.
template <typename T, int EPI, int BM>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a, TileBounds tb, int m_tiles_total,
                                                  int total_tiles, int splits) {
  constexpr int WN = 2, WM = 2, NT = 256;
  constexpr int WTN = BN / WN, WTM = BM / WM;  // 128 x 128 (or 128 x 112)
  constexpr int FS = WTN / 16, TS = WTM / 16;  // 8 x 8 (or 8 x 7) sub-tiles of 16 x 16
  constexpr int LA = BN * 8 / NT, LB = BM * 8 / NT;  // 8 + 8 (or 8 + 7) 16-byte loads per thread
  constexpr int KS = BK / 32;                  // 2 k-steps of 32 per k-tile
  constexpr int STAGE = (BN + BM) * BK * 2;    // 64 KB (or 60 KB)
  constexpr int NK = FS * TS;                  // MFMAs per k-step
  constexpr int NMEM = 3 * (FS + TS);          // memory operations placed before the barrier
  static_assert(BM % 32 == 0 && LA == FS && LB == TS, "tile shape");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  typedef typename Mfma<T>::v8 V8;

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
  const int K = a.k, LW = a.ldw > 0 ? a.ldw : a.k;  // reduction length, weight row stride
  const T *W = reinterpret_cast<const T *>(grp.w) + (size_t)n0 * LW;
  const T *X = reinterpret_cast<const T *>(grp.x) + (size_t)m0 * a.ldx;
  const int lchunk = tid & 7, lrow = tid >> 3;

  // k-tiles [kt0, kt0 + KT) of the tile's K / BK are this unit's slice
  const int kt_all = K / BK;
  const int kt0 = (int)((long long)kt_all * slice / splits);
  const int KT = (int)((long long)kt_all * (slice + 1) / splits) - kt0;
  W += (size_t)kt0 * BK;
  X += (size_t)kt0 * BK;
  // Global loads are buffer loads: one descriptor per operand (the weight tile's 256 rows; the
  // token rows from m0 to the group's end, so rows past it read as zero), one per-lane byte
  // offset, and the row / k-tile offsets in scalar registers.
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void *)W, (short)0, (int)min((long long)BN * LW * 2, 0x7FFFFFFFll), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
      (void *)X, (short)0, (int)min((long long)(grp.rows - m0) * a.ldx * 2, 0x7FFFFFFFll),
      0x00020000);
  const int vo_w = (lrow * LW + lchunk * 8) * 2, vo_x = (lrow * a.ldx + lchunk * 8) * 2;
  auto load_w = [&](int kt, int i) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rs_w, vo_w, (i * (NT / 8) * LW + kt * BK) * 2, 0);
  };
  auto load_x = [&](int kt, int i) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rs_x, vo_x, (i * (NT / 8) * a.ldx + kt * BK) * 2, 0);
  };
  // staging registers: weight rows one set (tile kt+2 loads while tile kt+1 is written to
  // LDS), token rows two sets (tile j in set j % 2, loaded three k-tiles ahead)
  u32x4 ra[LA], rb0[LB], rb1[LB];
  auto gload_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = load_w(kt, i);
  };
  auto gload_b = [&](int kt, u32x4 (&rb)[LB]) {
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = load_x(kt, i);
  };
  auto sstore = [&](int stage, const u32x4 (&rb)[LB]) {
    char *As = smem + stage * STAGE;
    char *Bs = As + BN * 128;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *reinterpret_cast<u32x4 *>(As + swz(lrow + i * (NT / 8), lchunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<u32x4 *>(Bs + swz(lrow + i * (NT / 8), lchunk)) = rb[i];
  };
  const int r16 = lane & 15, q4 = lane >> 4;
  V8 fr[KS][FS + TS];  // fragments of a whole k-tile: [k-step][weight sub-tiles | token sub-tiles]
  auto lread = [&](int stage, int ks) {
    const char *As = smem + stage * STAGE;
    const char *Bs = As + BN * 128;
    const int ch = ks * 4 + q4;
#pragma unroll
    for (int i = 0; i < FS; ++i)
      fr[ks][i] = *reinterpret_cast<const V8 *>(As + swz(wn * WTN + i * 16 + r16, ch));
#pragma unroll
    for (int j = 0; j < TS; ++j)
      fr[ks][FS + j] = *reinterpret_cast<const V8 *>(Bs + swz(wm * WTM + j * 16 + r16, ch));
  };
  f32x4 acc[FS][TS];
#pragma unroll
  for (int i = 0; i < FS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;
  auto mma_step = [&](int ks) {
#pragma unroll
    for (int i = 0; i < FS; ++i)
#pragma unroll
      for (int j = 0; j < TS; ++j)
        acc[i][j] = Mfma<T>::mma16(fr[ks][i], fr[ks][FS + j], acc[i][j]);
  };

  // single operations, so the loop below can fix their order exactly
  auto mma_one = [&](int ks, int idx) {  // idx = TS i + j
    acc[idx / TS][idx % TS] =
        Mfma<T>::mma16(fr[ks][idx / TS], fr[ks][FS + idx % TS], acc[idx / TS][idx % TS]);
  };
  auto read_one = [&](int stage, int ks, int f) {  // f < FS: weight rows, else token rows
    const char *As = smem + stage * STAGE;
    const char *Bs = As + BN * 128;
    const int ch = ks * 4 + q4;
    if (f < FS)
      fr[ks][f] = *reinterpret_cast<const V8 *>(As + swz(wn * WTN + f * 16 + r16, ch));
    else
      fr[ks][f] = *reinterpret_cast<const V8 *>(Bs + swz(wm * WTM + (f - FS) * 16 + r16, ch));
  };
  auto write_one = [&](int stage, int i, const u32x4 (&rb)[LB]) {  // i < LA: weights
    char *As = smem + stage * STAGE;
    char *Bs = As + BN * 128;
    if (i < LA)
      *reinterpret_cast<u32x4 *>(As + swz(lrow + i * (NT / 8), lchunk)) = ra[i];
    else
      *reinterpret_cast<u32x4 *>(Bs + swz(lrow + (i - LA) * (NT / 8), lchunk)) = rb[i - LA];
  };
  auto gload_one = [&](int kta, int ktb, int i, u32x4 (&rb)[LB]) {  // weights kta, tokens ktb
    if (i < LA) ra[i] = load_w(kta, i);
    else rb[i - LA] = load_x(ktb, i - LA);
  };

  gload_a(0);
  gload_b(0, rb0);
  sstore(0, rb0);
  gload_a(min(1, KT - 1));
  gload_b(min(1, KT - 1), rb1);
  gload_b(min(2, KT - 1), rb0);
  lds_sync();
  lread(0, 0);
  // Order of the fragment reads: k-step 1 of the tile reads its token sub-tiles first (every
  // MFMA row needs all of them), the next tile's k-step 0 reads weight sub-tile 0, the token
  // sub-tiles, then the other weight sub-tiles (the order its first MFMAs use them).
  auto frag_k1 = [](int r) { return r < TS ? FS + r : r - TS; };
  auto frag_k0 = [](int r) { return r == 0 ? 0 : (r <= TS ? FS - 1 + r : r - TS); };
  // one k-tile; rb holds the token rows of tile kt+1 and receives those of tile kt+3
  auto ktile = [&](int kt, u32x4 (&rb)[LB]) {
    const int cur = kt & 1;
    const int na = min(kt + 2, KT - 1), nb = min(kt + 3, KT - 1);  // clamped: repeats harmless
    // before the barrier: 2 NMEM MFMAs (k-step 0 and part of k-step 1; 96 of 128 for 256-row
    // tiles); after every second one comes in turn a fragment read of k-step 1, an LDS write
    // of tile kt+1 or a global load
#pragma unroll
    for (int m = 0; m < 2 * NMEM; ++m) {
      mma_one(m / NK, m % NK);
      if ((m & 1) == 0) {
        const int q = m >> 1, r = q / 3;
        if (q % 3 == 0) read_one(cur, 1, frag_k1(r));
        else if (q % 3 == 1) write_one(cur ^ 1, r, rb);
        else gload_one(na, nb, r, rb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();  // tile kt+1 written by every wave; tile kt's reads done
    // after the barrier: the other MFMAs of k-step 1 (32 for 256-row tiles), the reads of
    // tile kt+1's k-step 0 spread evenly before them (every second one for 256-row tiles)
    constexpr int NPOST = 2 * NK - 2 * NMEM, NR = FS + TS;
#pragma unroll
    for (int m = 0; m < NPOST; ++m) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (r * NPOST / NR == m) read_one(cur ^ 1, 0, frag_k0(r));
      mma_one(1, NK - NPOST + m);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int kt = 0;
  for (; kt + 2 < KT; kt += 2) {
    ktile(kt, rb1);
    ktile(kt + 1, rb0);
  }
  if (kt + 1 < KT) ktile(kt, rb1);
  {
    const int cur = (KT - 1) & 1;
    mma_step(0);
    lread(cur, 1);
    mma_step(1);
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
  epilogue<T, BM, WN, WM, EPI>(a, grp, n0, m0, wn, wm, lane, acc, smem);
}

// Token-tile bounds of the row groups for tile height bm; returns the number of token tiles.
int tile_bounds(const GemmArgs &a, int bm, TileBounds *tb) {
  *tb = TileBounds{};
  for (int i = 0; i < kMaxGroups; ++i)
    tb->t[i + 1] = tb->t[i] + (i < a.ng ? (a.g[i].rows + bm - 1) / bm : 0);
  return tb->t[kMaxGroups];
}

// A launch plan for tile height bm: token tiles, tiles, k-slices.
struct Plan {
  TileBounds tb;
  int m_tiles, total, splits;
};
template <int EPI>
Plan make_plan(const GemmArgs &a, int bm) {
  Plan p;
  p.m_tiles = tile_bounds(a, bm, &p.tb);
  p.total = p.m_tiles * (a.n / BN);
  // k-slices: only for tiles that fill under half of the compute units, with at least 8
  // k-tiles per slice
  p.splits = 1;
  if (EPI != EPI_QKV_SWIGLU && a.part != nullptr && a.split_grid > 0 && 2 * p.total <= a.split_grid) {
    p.splits = min(16, min(a.split_grid / p.total, (a.k / BK) / 8));
    if (p.splits < 2 || (long long)p.splits * p.total > a.part_tiles) p.splits = 1;
  }
  return p;
}

template <typename T, int EPI, int BM>
hipError_t run_plan(const GemmArgs &a, const Plan &p, hipStream_t s) {
  const int grid = (p.total * p.splits + 7) / 8 * 8;
  k_gemm<T, EPI, BM><<<grid, 256, 0, s>>>(a, p.tb, p.m_tiles, p.total, p.splits);
  if constexpr (EPI != EPI_QKV_SWIGLU)
    if (p.splits > 1)
      k_gemm_reduce<EPI, BM><<<dim3(p.total, BM / 4), 256, 0, s>>>(a, p.tb, p.m_tiles, p.total, p.splits);
  return hipGetLastError();
}

template <typename T, int EPI>
hipError_t launch(const GemmArgs &a, hipStream_t s) {
  const Plan p256 = make_plan<EPI>(a, 256);
  if (p256.m_tiles == 0) return hipSuccess;
  // linear2: 224-row tiles when the rounds of workgroups over the compute units, times the
  // rows and k each workgroup takes, come out at least 5% lower (at 4608 tokens: 216 tiles of
  // 256 rows against 252 of 224 on 256 compute units).  Not linear1: at 1536 tokens its 648
  // tiles of 256 rows (3 rounds, the last half full) beat 756 of 224 (3 full rounds), 239
  // against 253 us: a half-empty round runs at a higher clock under the power limit.
  if constexpr (EPI == EPI_RESID) {
    if (a.cus > 0) {
      const Plan p224 = make_plan<EPI>(a, 224);
      auto cost = [&](const Plan &p, int bm) {
        return (double)((p.total * p.splits + a.cus - 1) / a.cus) * bm / p.splits;
      };
      if (20 * cost(p224, 224) < 19 * cost(p256, 256)) return run_plan<T, EPI, 224>(a, p224, s);
    }
  }
  return run_plan<T, EPI, 256>(a, p256, s);
}

}  // namespace

template <typename T>
hipError_t dispatch(const GemmArgs &a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_QKV_SWIGLU: return launch<T, EPI_QKV_SWIGLU>(a, s);
    case EPI_RESID: return launch<T, EPI_RESID>(a, s);
    case EPI_STORE_F32: return launch<T, EPI_STORE_F32>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t gemm_mfma(const GemmArgs &a, int epi, int op, hipStream_t s) {
  if (a.n % BN || a.k % BK || a.ng < 1 || a.ng > kMaxGroups) return hipErrorInvalidValue;
  if (!fused_heads_ok(a, epi)) return hipErrorInvalidValue;
  if (op == OP_BF16) return dispatch<bf16>(a, epi, s);
  if (op == OP_F16) return dispatch<f16>(a, epi, s);
  return hipErrorInvalidValue;
}

}  // namespace dit
