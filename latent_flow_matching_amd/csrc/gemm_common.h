// Pieces shared by the MFMA GEMMs (16-bit and FP8 operands): the LDS swizzle, the XCD-aware
// tile order, the fused epilogues and the k-slice reduction.
//
// Workgroup tile 256 features x 256 tokens, 4 waves (2 x 2) each owning 128 x 128 as 8 x 8
// accumulators of 16 x 16: lane l holds token l % 16 and features 4 (l / 16) + {0..3} of
// every sub-tile.  LDS rows are 128 B with the 16-byte chunk index XOR-swizzled by
// ((row >> 1) & 7): gfx950's LDS serves 256 B (64 banks) per cycle, i.e. two consecutive
// rows, so the 16 rows of one quarter-wave 16-byte read land on 16 distinct slots.
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
#pragma once
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BN = 256;  // output features per workgroup
__device__ __forceinline__ int swz(int row, int chunk) {  // byte offset inside a tile
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

constexpr int kGroupN = 4;  // feature tiles per ordering group (4 x 8 tiles per XCD round)

// Epilogue: lane owns token (lane & 15) and features 4 (lane >> 4) + {0..3} of every 16x16
// sub-tile.
template <typename T, int BM, int WN, int WM, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const GemmGroup &grp, int n0, int m0,
                                         int wn, int wm, int lane,
                                         f32x4 (&acc)[BN / WN / 16][BM / WM / 16]) {
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int FS = WTN / 16, TS = WTM / 16;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int fbase = n0 + wn * WTN + 4 * q4;
#pragma unroll
  for (int j = 0; j < TS; ++j) {
    const int m = m0 + wm * WTM + j * 16 + r16;  // row inside the group
    if (m >= grp.rows) continue;
    const int tok = grp.out_row0 + m;
    if constexpr (EPI == EPI_RESID) {
      const int seg = segment_of(tok, a.b1, a.b2, a.per);
      const float *gate = a.gate[seg];
      float *xr = a.x + (size_t)tok * a.ldres;
#pragma unroll
      for (int i = 0; i < FS; ++i) {
        const int n = fbase + i * 16;
        f32x4 gv = *reinterpret_cast<const f32x4 *>(gate + n);
        f32x4 xv = *reinterpret_cast<const f32x4 *>(xr + n);
        xv.x += gv.x * acc[i][j][0];
        xv.y += gv.y * acc[i][j][1];
        xv.z += gv.z * acc[i][j][2];
        xv.w += gv.w * acc[i][j][3];
        *reinterpret_cast<f32x4 *>(xr + n) = xv;
      }
    } else if constexpr (EPI == EPI_QKV_SWIGLU) {
      if (n0 < a.split) {
        T *qr = reinterpret_cast<T *>(a.qkv) + (size_t)tok * a.ldq;
#pragma unroll
        for (int i = 0; i < FS; ++i)
          store4(qr + fbase + i * 16, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
        // rows of a 64-row chunk: gate of SwiGLU features [32c, 32c + 32), then their up rows;
        // sub-tiles 4p + h (gate) and 4p + 2 + h (up) hold features 32p + 16h + [0, 16)
        T *cr = reinterpret_cast<T *>(a.cat) + (size_t)tok * a.ldc + a.cat_off;
        const int jb = (n0 - a.split + wn * WTN) / 2;  // first SwiGLU feature of the wave
#pragma unroll
        for (int p = 0; p < FS / 4; ++p)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              o[r] = silu(acc[4 * p + h][j][r]) * acc[4 * p + 2 + h][j][r];
            store4(cr + jb + p * 32 + h * 16 + 4 * q4, o[0], o[1], o[2], o[3]);
          }
      }
    } else {
      float *orow = a.out + (size_t)tok * a.ldo;
#pragma unroll
      for (int i = 0; i < FS; ++i) {
          const int n = fbase + i * 16;
          if (a.n_store > 0 && n >= a.n_store) continue;
          f32x4 v = acc[i][j];
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

// First token tile of each row group (entries past the last group hold the total).
struct TileBounds {
  int t[kMaxGroups + 1];
};

// Sum of the k-slices of one partial tile (slice order fixed) and the tile's epilogue.  Grid:
// (tiles, 64 sub-tiles); 256 threads = the GEMM's 4 waves x 64 lanes, same accumulator layout.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmArgs a, TileBounds tb, int m_tiles_total,
                                                     int total_tiles, int splits) {
  constexpr int BM = 256, WTN = 128, WTM = 128, TS = 8;
  const int lid = blockIdx.x, sub = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  // tile coordinates, as in k_gemm
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
  const GemmGroup grp = a.g[gi];
  const int n0 = tile_n * BN, m0 = (mt - tb.t[gi]) * BM;
  const int i = sub / TS, j = sub - i * TS;
  const int m = m0 + wm * WTM + j * 16 + (lane & 15);
  if (m >= grp.rows) return;
  const f32x4 *pp = reinterpret_cast<const f32x4 *>(a.part) +
                    ((size_t)lid * 4 + wave) * (64 * 64) + sub * 64 + lane;
  const size_t slice_stride = (size_t)total_tiles * 4 * 64 * 64;
  f32x4 v = pp[0];
  for (int s = 1; s < splits; ++s) v += pp[s * slice_stride];
  const int tok = grp.out_row0 + m;
  const int n = n0 + wn * WTN + i * 16 + 4 * (lane >> 4);
  if constexpr (EPI == EPI_RESID) {
    const float *gate = a.gate[segment_of(tok, a.b1, a.b2, a.per)];
    float *xr = a.x + (size_t)tok * a.ldres + n;
    const f32x4 gv = *reinterpret_cast<const f32x4 *>(gate + n);
    f32x4 xv = *reinterpret_cast<const f32x4 *>(xr);
    xv.x += gv.x * v.x;
    xv.y += gv.y * v.y;
    xv.z += gv.z * v.z;
    xv.w += gv.w * v.w;
    *reinterpret_cast<f32x4 *>(xr) = xv;
  } else {
    if (a.n_store > 0 && n >= a.n_store) return;
    float *orow = a.out + (size_t)tok * a.ldo + n;
    if (a.accumulate == 1) {
      v = *reinterpret_cast<const f32x4 *>(orow) + a.alpha * v;
    } else if (a.accumulate == 2) {
      v = a.alpha * v;
    }
    *reinterpret_cast<f32x4 *>(orow) = v;
  }
}

}  // namespace

}  // namespace dit
