// Flash-style softmax attention, head_dim 128, 16-bit (bf16 or fp16) MFMA operands with fp32
// online softmax (gfx950).
//
// o_h = softmax(q_h k_h^T / sqrt(128)) v_h over the keys a query may see: all N tokens
// (joint / double / single blocks) or only its own stream (per-mode blocks, block-diagonal)
// ("FLUX.3 Image Klein in Diffusers", section "Entkoppelte Vorverarbeitung und gemeinsame
// Attention-Blöcke").  Padded prompt tokens are attended like any other token ("...",
// section "Verarbeitung einzelner Prompts und Batching-Architektur in der Praxis").
//
// Work split: a workgroup takes 128 queries of one head, 4 waves x 32 queries, and two
// workgroups share a CU (one wave of each per SIMD).  The two workgroups synchronise
// independently, so their phases drift apart and one wave's softmax (VALU) overlaps the
// other's MFMAs.  A workgroup walks the allowed keys in tiles of 64 staged through LDS (K and
// V^T tiles, double-buffered, one barrier per tile; the global loads of tile t+1 are in
// flight while tile t is computed).
//   S^T = K Q^T   (A = K tile from LDS, B = the wave's queries held in registers): each lane
//                 owns one query and 32 of the tile's keys, so the row max needs one exchange
//                 with the partner lane l^32.
//   O^T += V^T P^T (A = V^T tile from LDS, B = P straight from the S registers).
// The running max is raised lazily: P is formed against the stored max unless some row's
// max grew by more than 2^8, so O is rescaled only when that happens (P <= 256 fits fp16).
// V is read in the transposed layout written by the QK-norm kernel, vt[h][d][token'] with the
// middle two quads of every 16 tokens swapped, so that the eight keys a lane multiplies in
// one P.V MFMA form a single 16-byte chunk.  Scores
// are kept in the log2 domain (scale * log2(e) folded into one FMA before exp2).
// Groups: each (q0, q1, k0, k1) range gets its own query tiles; key tiles start at k0
// rounded down to 64 and keys outside [k0, k1) are masked to -inf.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BQ = 128, BKV = 64, HD = 128;
constexpr int KT_BYTES = BKV * HD * 2;   // K tile [64 keys][128 d]   (row 256 B)
constexpr int VT_BYTES = HD * BKV * 2;   // V^T tile [128 d][64 keys] (row 128 B)
constexpr float kLazy = 8.0f;            // log2 headroom before O is rescaled

// LDS swizzles for gfx950's 64 banks (256 B per cycle):
// K tile: 16 chunks of 16 B per 256-B row, chunk index XOR (row & 15), so the 16 rows of a
// quarter-wave ds_read_b128 hit 16 distinct slots.
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}
// V^T tile: 8 chunks of 16 B per 128-B row, chunk index XOR ((row >> 1) & 7), so the 16 rows
// of a quarter-wave ds_read_b128 (two rows per 256 B) hit 16 distinct slots.
__device__ __forceinline__ int v_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <typename T>
__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a, int qt_before1, int qt_before2,
                                                       int q_tiles, int total) {
  typedef typename Mfma<T>::v8 V8;
  __shared__ __attribute__((aligned(16))) char smem[2 * (KT_BYTES + VT_BYTES)];

  const int per = gridDim.x >> 3;
  const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lid >= total) return;
  const int head = lid / q_tiles;
  const int qt = lid - head * q_tiles;
  const int gi = (qt >= qt_before1) + (qt >= qt_before2);
  const AttnGroup grp = a.g[gi];
  const int q_tile0 = grp.q0 + (qt - (gi == 0 ? 0 : (gi == 1 ? qt_before1 : qt_before2))) * BQ;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, hk = lane >> 5;
  const T *qkv = reinterpret_cast<const T *>(a.qkv);
  const T *vt = reinterpret_cast<const T *>(a.vt) + (size_t)head * HD * a.ldv;

  // this lane's query row (rows past the group end are computed but never stored)
  const int q = q_tile0 + wave * 32 + r32;
  V8 qf[8];
  {
    const T *qp = qkv + (size_t)q * a.ldqkv + head * HD + hk * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const V8 *>(qp + kk * 16);
  }

  const int kv_begin = (grp.k0 / BKV) * BKV;
  const int n_tiles = (grp.k1 - kv_begin + BKV - 1) / BKV;

  // global -> register staging: 4 K chunks and 4 V^T chunks of 16 B per thread
  u32x4 rk[4], rv[4];
  const int k_row = tid >> 4, k_ch = tid & 15;   // K: rows k_row + 16 i
  const int v_row = tid >> 3, v_ch = tid & 7;    // V^T: rows v_row + 32 i
  auto gload = [&](int t) {
    const int kv0 = kv_begin + t * BKV;
    const T *kp = qkv + (size_t)(kv0 + k_row) * a.ldqkv + a.d_model + head * HD + k_ch * 8;
    const T *vp = vt + (size_t)v_row * a.ldv + kv0 + v_ch * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk[i] = *reinterpret_cast<const u32x4 *>(kp + (size_t)(16 * i) * a.ldqkv);
      rv[i] = *reinterpret_cast<const u32x4 *>(vp + (size_t)(32 * i) * a.ldv);
    }
  };
  auto sstore = [&](int buf) {
    char *ks = smem + buf * (KT_BYTES + VT_BYTES);
    char *vs = ks + KT_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4 *>(ks + k_off(k_row + 16 * i, k_ch)) = rk[i];
      *reinterpret_cast<u32x4 *>(vs + v_off(v_row + 32 * i, v_ch)) = rv[i];
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);
    const char *ks = smem + buf * (KT_BYTES + VT_BYTES);
    const char *vs = ks + KT_BYTES;
    const int kv0 = kv_begin + t * BKV;

    // ---- S^T for 64 keys: two 32-key sub-tiles
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[st][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        V8 kf = *reinterpret_cast<const V8 *>(ks + k_off(st * 32 + r32, 2 * kk + hk));
        s[st] = Mfma<T>::mma(kf, qf[kk], s[st]);
      }
    // ---- online softmax (lane: one query, keys 32 st + 8 g + 4 hk + r)
    if ((kv0 < grp.k0) || (kv0 + BKV > grp.k1)) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + st * 32 + 8 * (e >> 2) + 4 * hk + (e & 3);
          if (key < grp.k0 || key >= grp.k1) s[st][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[st][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
    if (__ballot(mx > m_run + kLazy)) {  // wave-uniform: raise the stored max, rescale O
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
    }
    const float nm = -m_run;
    float psum = 0.f;
    V8 pf[4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[st][e], sl2, nm));
        psum += p;
        // key chunk kc = 2 st + (e >> 3): k-index (e & 7) of the MFMA B operand
        pf[2 * st + (e >> 3)][e & 7] = from_f32_inrange<T>(p);  // p <= 256
      }
    l_run += psum;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const int row = ds * 32 + r32;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        // keys 16 kc + {4 hk .. 4 hk + 3, 8 + 4 hk .. 8 + 4 hk + 3}: one chunk of the
        // quad-permuted V^T row
        V8 vf = *reinterpret_cast<const V8 *>(vs + v_off(row, 2 * kc + hk));
        o[ds] = Mfma<T>::mma(vf, pf[kc], o[ds]);
      }
    }
    if (t + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }

  const float inv = 1.0f / (l_run + __shfl_xor(l_run, 32, 64));
  if (q < grp.q1) {
    T *op = reinterpret_cast<T *>(a.out) + (size_t)q * a.ldo + head * HD + 4 * hk;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(op + ds * 32 + 8 * g, o[ds][4 * g] * inv, o[ds][4 * g + 1] * inv,
               o[ds][4 * g + 2] * inv, o[ds][4 * g + 3] * inv);
  }
}

}  // namespace

hipError_t attention_mfma(const AttnArgs &a, int op, hipStream_t s) {
  if (a.ng < 1 || a.ng > 3) return hipErrorInvalidValue;
  int tb[4] = {0, 0, 0, 0};
  for (int i = 0; i < 3; ++i)
    tb[i + 1] = tb[i] + (i < a.ng ? (a.g[i].q1 - a.g[i].q0 + BQ - 1) / BQ : 0);
  const int q_tiles = tb[3];
  if (q_tiles == 0) return hipSuccess;
  const int total = q_tiles * a.heads;
  const int grid = (total + 7) / 8 * 8;
  if (op == OP_BF16)
    k_attn_mfma<bf16><<<grid, 256, 0, s>>>(a, tb[1], tb[2], q_tiles, total);
  else if (op == OP_F16)
    k_attn_mfma<f16><<<grid, 256, 0, s>>>(a, tb[1], tb[2], q_tiles, total);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dit
