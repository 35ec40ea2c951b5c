// MFMA GEMM (16-bit operands: bf16 or fp16, fp32 accumulation) for the block's two fused
// projections on gfx950.
//
//   out[token][n] = sum_k X[token][k] * W[n][k]       (X = activations, W = [N, K] weights)
//
// Both operands are K-contiguous, which is the per-lane layout of v_mfma_f32_32x32x16_{bf16,f16}
// (lane l holds 8 consecutive k of row l%32, k-half l/32).  The weight tile is the MFMA A
// operand and the token tile the B operand, so each lane's accumulator holds one token and
// four consecutive output features: stores are 8-byte (bf16) or 16-byte (fp32) vectors.
//
// Workgroup tile 256 features x 256 tokens, 4 waves (2 x 2) each owning 128 x 128 (16
// accumulators of 32x32 in AGPRs, one wave per SIMD).  k advances in tiles of 64 through two
// LDS stages (128 KB) with one barrier per k-tile; global loads are staged through registers
// one k-tile ahead.  LDS rows are 128 B (64 values) with the 16-byte chunk index XOR-swizzled
// by ((row >> 1) & 7): gfx950's LDS serves 256 B (64 banks) per cycle, i.e. two consecutive
// rows, so the 16 rows of one quarter-wave ds_read_b128 land on 16 distinct 16-byte slots.
//
// Epilogues (the fusions of the block):
//   EPI_QKV_SWIGLU  linear1: columns [0, split) are Q|K|V and go to the qkv buffer; the
//                   rest holds gate and up rows interleaved in 32-row chunks, so one lane
//                   owns gate and up of the same feature and writes SiLU(gate) * up
//                   ("FLUX.3 Image Klein in Diffusers", "Entkoppelte Vorverarbeitung ...":
//                   the MLP is a SwiGLU MLP run in parallel with attention).
//   EPI_RESID       linear2: x[token] += gate_seg(token) * acc (gated residual, fp32).
//   EPI_STORE_F32   plain fp32 store or out += alpha * acc.
//
// Workgroups are remapped so that each of the 8 XCDs receives a contiguous range of tile ids,
// and ids are ordered in groups of 4 feature tiles (feature fastest, then tokens): the 32
// workgroups one XCD runs at a time then share 4 weight tiles and 8 token tiles in its L2.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BN = 256;  // output features per workgroup
constexpr int BK = 64;   // k per LDS stage

__device__ __forceinline__ int swz(int row, int chunk) {  // byte offset inside a tile
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

constexpr int kGroupN = 4;  // feature tiles per ordering group (4 x 8 tiles per XCD round)

// Epilogue: lane owns token (lane & 31) and features
// 8 g + 4 (lane >> 5) + {0..3} of every 32x32 sub-tile.
template <typename T, int BM, int WN, int WM, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const GemmGroup &grp, int n0, int m0,
                                         int wn, int wm, int lane,
                                         f32x16 (&acc)[BN / WN / 32][BM / WM / 32]) {
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int FS = WTN / 32, TS = WTM / 32;
  const int r32 = lane & 31, hk = lane >> 5;
  const int fbase = n0 + wn * WTN + 4 * hk;
#pragma unroll
  for (int j = 0; j < TS; ++j) {
    const int m = m0 + wm * WTM + j * 32 + r32;  // row inside the group
    if (m >= grp.rows) continue;
    const int tok = grp.out_row0 + m;
    if constexpr (EPI == EPI_RESID) {
      const int seg = segment_of(tok, a.b1, a.b2, a.per);
      const float *gate = a.gate[seg];
      float *xr = a.x + (size_t)tok * a.ldres;
#pragma unroll
      for (int i = 0; i < FS; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = fbase + i * 32 + 8 * g;
          f32x4 gv = *reinterpret_cast<const f32x4 *>(gate + n);
          f32x4 xv = *reinterpret_cast<const f32x4 *>(xr + n);
          xv.x += gv.x * acc[i][j][4 * g + 0];
          xv.y += gv.y * acc[i][j][4 * g + 1];
          xv.z += gv.z * acc[i][j][4 * g + 2];
          xv.w += gv.w * acc[i][j][4 * g + 3];
          *reinterpret_cast<f32x4 *>(xr + n) = xv;
        }
    } else if constexpr (EPI == EPI_QKV_SWIGLU) {
      if (n0 < a.split) {
        T *qr = reinterpret_cast<T *>(a.qkv) + (size_t)tok * a.ldq;
#pragma unroll
        for (int i = 0; i < FS; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store4(qr + fbase + i * 32 + 8 * g, acc[i][j][4 * g], acc[i][j][4 * g + 1],
                   acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      } else {
        // sub-tiles (2p, 2p+1) = gate / up rows of SwiGLU features [32c, 32c + 32)
        T *cr = reinterpret_cast<T *>(a.cat) + (size_t)tok * a.ldc + a.cat_off;
        const int jb = (n0 - a.split + wn * WTN) / 2;  // first SwiGLU feature of the wave
#pragma unroll
        for (int p = 0; p < FS / 2; ++p)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              o[r] = silu(acc[2 * p][j][4 * g + r]) * acc[2 * p + 1][j][4 * g + r];
            store4(cr + jb + p * 32 + 8 * g + 4 * hk, o[0], o[1], o[2], o[3]);
          }
      }
    } else {
      float *orow = a.out + (size_t)tok * a.ldo;
#pragma unroll
      for (int i = 0; i < FS; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = fbase + i * 32 + 8 * g;
          if (a.n_store > 0 && n >= a.n_store) continue;
          f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                     acc[i][j][4 * g + 3]};
          if (a.accumulate == 1) {
            f32x4 o = *reinterpret_cast<const f32x4 *>(orow + n);
            v = o + a.alpha * v;
          } else if (a.accumulate == 2) {
            v = a.alpha * v;
          }
          *reinterpret_cast<f32x4 *>(orow + n) = v;
        }
    }
  }
}

// Barrier for LDS hand-over only: global loads stay in flight across it (a workgroup fence
// would also drain them).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS traffic is done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Main loop.  Entering k-tile kt a wave holds the fragments of its k-steps 0 and 1.  Before
// the barrier it runs the MFMAs of k-steps 0..2 while it reads k-steps 2 and 3 of tile kt,
// writes tile kt+1 into the other stage and issues the global loads of tile kt+2; after the
// barrier the MFMAs of k-step 3 overlap the reads of k-steps 0 and 1 of tile kt+1.  A stage is
// rewritten only after the barrier that follows the last reads of its previous tile.  The
// order of every MFMA and memory operation is pinned (sched_barrier), one memory operation
// after each MFMA, so the LDS and global latencies sit under MFMAs.  Token rows, which miss L2
// more often than weight rows under the grouped tile order, get two staging sets and so two
// k-tiles of latency cover.
// First token tile of each row group (entries past the last group hold the total).
struct TileBounds {
  int t[kMaxGroups + 1];
};

template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a, TileBounds tb, int m_tiles_total,
                                                  int total_tiles) {
  constexpr int BM = 256, WN = 2, WM = 2, NT = 256;
  constexpr int WTN = BN / WN, WTM = BM / WM;  // 128 x 128
  constexpr int FS = WTN / 32, TS = WTM / 32;  // 4 x 4
  constexpr int LA = BN * 8 / NT, LB = BM * 8 / NT;  // 8 + 8 16-byte loads per thread
  constexpr int KS = BK / 16;                  // 4 k-steps per k-tile
  constexpr int STAGE = (BN + BM) * BK * 2;    // 64 KB
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  typedef typename Mfma<T>::v8 V8;

  const int per = gridDim.x >> 3;
  const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lid >= total_tiles) return;
  const int n_tiles = a.n / BN;
  const int in_group = kGroupN * m_tiles_total;
  const int group = lid / in_group;
  const int first_n = group * kGroupN;
  const int gsize = min(n_tiles - first_n, kGroupN);
  const int rem = lid - group * in_group;
  const int tile_n = first_n + rem % gsize;
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
  const int K = a.k;
  const T *W = reinterpret_cast<const T *>(grp.w) + (size_t)n0 * K;
  const T *X = reinterpret_cast<const T *>(grp.x) + (size_t)m0 * a.ldx;
  const int lchunk = tid & 7, lrow = tid >> 3;

  // Global loads are buffer loads: one descriptor per operand (the weight tile's 256 rows; the
  // token rows from m0 to the group's end, so rows past it read as zero), one per-lane byte
  // offset, and the row / k-tile offsets in scalar registers.
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void *)W, (short)0, (int)min((long long)BN * K * 2, 0x7FFFFFFFll), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
      (void *)X, (short)0, (int)min((long long)(grp.rows - m0) * a.ldx * 2, 0x7FFFFFFFll),
      0x00020000);
  const int vo_w = (lrow * K + lchunk * 8) * 2, vo_x = (lrow * a.ldx + lchunk * 8) * 2;
  auto load_w = [&](int kt, int i) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rs_w, vo_w, (i * (NT / 8) * K + kt * BK) * 2, 0);
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
  const int r32 = lane & 31, hk = lane >> 5;
  V8 fr[KS][FS + TS];
  auto lread = [&](int stage, int ks) {
    const char *As = smem + stage * STAGE;
    const char *Bs = As + BN * 128;
    const int ch = ks * 2 + hk;
#pragma unroll
    for (int i = 0; i < FS; ++i)
      fr[ks][i] = *reinterpret_cast<const V8 *>(As + swz(wn * WTN + i * 32 + r32, ch));
#pragma unroll
    for (int j = 0; j < TS; ++j)
      fr[ks][FS + j] = *reinterpret_cast<const V8 *>(Bs + swz(wm * WTM + j * 32 + r32, ch));
  };
  f32x16 acc[FS][TS];
#pragma unroll
  for (int i = 0; i < FS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto mma_step = [&](int ks) {
#pragma unroll
    for (int i = 0; i < FS; ++i)
#pragma unroll
      for (int j = 0; j < TS; ++j)
        acc[i][j] = Mfma<T>::mma(fr[ks][i], fr[ks][FS + j], acc[i][j]);
  };

  // single operations, so the loop below can fix their order exactly
  auto mma_one = [&](int ks, int idx) {  // idx = 4 i + j
    acc[idx >> 2][idx & 3] =
        Mfma<T>::mma(fr[ks][idx >> 2], fr[ks][FS + (idx & 3)], acc[idx >> 2][idx & 3]);
  };
  auto read_one = [&](int stage, int ks, int f) {  // f < 4: weight rows, else token rows
    const char *As = smem + stage * STAGE;
    const char *Bs = As + BN * 128;
    const int ch = ks * 2 + hk;
    if (f < FS)
      fr[ks][f] = *reinterpret_cast<const V8 *>(As + swz(wn * WTN + f * 32 + r32, ch));
    else
      fr[ks][f] = *reinterpret_cast<const V8 *>(Bs + swz(wm * WTM + (f - FS) * 32 + r32, ch));
  };
  auto write_one = [&](int stage, int i, const u32x4 (&rb)[LB]) {  // i < 8: weights
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

  const int KT = K / BK;
  gload_a(0);
  gload_b(0, rb0);
  sstore(0, rb0);
  gload_a(min(1, KT - 1));
  gload_b(min(1, KT - 1), rb1);
  gload_b(min(2, KT - 1), rb0);
  lds_sync();
  lread(0, 0);
  lread(0, 1);
  // one k-tile; rb holds the token rows of tile kt+1 and receives those of tile kt+3
  auto ktile = [&](int kt, u32x4 (&rb)[LB]) {
    const int cur = kt & 1;
    const int na = min(kt + 2, KT - 1), nb = min(kt + 3, KT - 1);  // clamped: repeats harmless
    // before the barrier: MFMAs of k-steps 0..2; after MFMA m comes fragment read m/3 (k-steps
    // 2 then 3 of tile kt), LDS write m/3 (tile kt+1) or global load m/3
#pragma unroll
    for (int m = 0; m < 48; ++m) {
      mma_one(m >> 4, m & 15);
      const int q = m / 3;
      if (m % 3 == 0) read_one(cur, 2 + (q >> 3), q & 7);
      else if (m % 3 == 1) write_one(cur ^ 1, q, rb);
      else gload_one(na, nb, q, rb);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();  // tile kt+1 written by every wave; tile kt's reads done
    // after the barrier: MFMAs of k-step 3, each after one read of tile kt+1 (k-steps 0, 1)
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      read_one(cur ^ 1, m >> 3, m & 7);
      mma_one(3, m);
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
    lread(cur, 2);
    mma_step(1);
    lread(cur, 3);
    mma_step(2);
    mma_step(3);
  }
  epilogue<T, BM, WN, WM, EPI>(a, grp, n0, m0, wn, wm, lane, acc);
}

template <typename T, int EPI>
hipError_t launch(const GemmArgs &a, hipStream_t s) {
  constexpr int BM = 256;
  TileBounds tb = {};
  for (int i = 0; i < kMaxGroups; ++i)
    tb.t[i + 1] = tb.t[i] + (i < a.ng ? (a.g[i].rows + BM - 1) / BM : 0);
  const int m_tiles = tb.t[kMaxGroups];
  if (m_tiles == 0) return hipSuccess;
  const int total = m_tiles * (a.n / BN);
  const int grid = (total + 7) / 8 * 8;
  k_gemm<T, EPI><<<grid, 256, 0, s>>>(a, tb, m_tiles, total);
  return hipGetLastError();
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
  if (op == OP_BF16) return dispatch<bf16>(a, epi, s);
  if (op == OP_F16) return dispatch<f16>(a, epi, s);
  return hipErrorInvalidValue;
}

}  // namespace dit
