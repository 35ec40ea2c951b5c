// Flash-style softmax attention, head_dim 128, 16-bit (bf16 or fp16) MFMA operands with fp32
// online softmax (gfx950).
//
// o_h = softmax(q_h k_h^T / sqrt(128)) v_h over the keys a query may see: all N tokens
// (joint / double / single blocks) or only its own stream (per-mode blocks, block-diagonal)
// ("FLUX.3 Image Klein in Diffusers", section "Entkoppelte Vorverarbeitung und gemeinsame
// Attention-Blöcke").  Padded prompt tokens are attended like any other token ("...",
// section "Verarbeitung einzelner Prompts und Batching-Architektur in der Praxis").
//
// Work split: a workgroup of 8 waves takes 256 queries of one head (32 per wave) and walks
// the allowed keys in tiles of 64, staged through LDS.  Per wave and key tile:
//   S^T = K Q^T   (A = K fragments from LDS, B = the wave's queries held in registers): each
//                 lane owns one query and 32 of the tile's keys, so the row max needs one
//                 exchange with the partner lane l^32.
//   O^T += V^T P^T (A = V^T fragments from LDS, B = P straight from the S registers).
// The running max is raised lazily: P is formed against the stored max unless some row's
// max grew by more than 2^8, so O is rescaled only when that happens (P <= 256 fits fp16).
// V is read in the transposed layout written by the QK-norm kernel, vt[h][d][token'] with the
// middle two quads of every 16 tokens swapped, so that the eight keys a lane multiplies in
// one P.V MFMA form a single 16-byte chunk.  Scores are kept in the log2 domain
// (scale * log2(e) folded into one FMA before exp2).
// Groups: each (q0, q1, k0, k1) range gets its own query tiles; key tiles start at k0
// rounded down to 64 and keys outside [k0, k1) are masked to -inf.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BKV = 64, HD = 128;
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

// A workgroup of 8 waves takes 256 queries (32 per wave) and the two waves
// that share a SIMD work in opposite phases, kept in step by workgroup barriers:
//   M phase of tile t:  S_t = K_t Q^T and O += V_{t-1} P_{t-1}   (32 MFMAs, raised priority)
//   V phase of tile t:  mask, row max, lazy rescale, exponentials -> P_t   (VALU)
// Half A runs M_0 V_0 M_1 V_1 ..., half B runs one phase later, so while one wave of a SIMD
// issues MFMAs the other issues its softmax.  Global phase 2t+1 also moves K_{t+1} and V_t
// from registers into LDS (two slots each) and starts the global loads of K_{t+2}, V_{t+1}:
// K_t is read in phases 2t and 2t+1 and V_t in phases 2t+2 and 2t+3, so no slot is written
// while a wave may still read it.
constexpr int BQ = 256;

template <typename T>
__global__ __launch_bounds__(512, 1) void k_attn_pp(AttnArgs a, int qt_before1, int qt_before2,
                                                     int q_tiles, int total) {
  typedef typename Mfma<T>::v8 V8;
  __shared__ __attribute__((aligned(16))) char smem[2 * KT_BYTES + 2 * VT_BYTES];

  const int per = gridDim.x >> 3;
  const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lid >= total) return;
  const int head = lid / q_tiles;
  const int qt = lid - head * q_tiles;
  const int gi = (qt >= qt_before1) + (qt >= qt_before2);
  const AttnGroup grp = a.g[gi];
  const int q_tile0 =
      grp.q0 + (qt - (gi == 0 ? 0 : (gi == 1 ? qt_before1 : qt_before2))) * BQ;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, hk = lane >> 5;
  const int half = wave >> 2;  // waves w and w+4 of a workgroup share a SIMD
  const T *qkv = reinterpret_cast<const T *>(a.qkv);
  const T *vt = reinterpret_cast<const T *>(a.vt) + (size_t)head * HD * a.ldv;

  const int q = q_tile0 + wave * 32 + r32;
  V8 qf[8];
  {
    const T *qp = qkv + (size_t)q * a.ldqkv + head * HD + hk * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const V8 *>(qp + kk * 16);
  }

  const int kv_begin = (grp.k0 / BKV) * BKV;
  const int n = (grp.k1 - kv_begin + BKV - 1) / BKV;

  u32x4 rk[2], rv[2];
  const int k_row = tid >> 4, k_ch = tid & 15;   // K: rows k_row + 32 i
  const int v_row = tid >> 3, v_ch = tid & 7;    // V^T: rows v_row + 64 i
  auto gload_k = [&](int t) {
    const T *kp = qkv + (size_t)(kv_begin + t * BKV + k_row) * a.ldqkv + a.d_model +
                  head * HD + k_ch * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rk[i] = *reinterpret_cast<const u32x4 *>(kp + (size_t)(32 * i) * a.ldqkv);
  };
  auto gload_v = [&](int t) {
    const T *vp = vt + (size_t)v_row * a.ldv + kv_begin + t * BKV + v_ch * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rv[i] = *reinterpret_cast<const u32x4 *>(vp + (size_t)(64 * i) * a.ldv);
  };
  auto store_k = [&](int t) {
    char *ks = smem + (t & 1) * KT_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4 *>(ks + k_off(k_row + 32 * i, k_ch)) = rk[i];
  };
  auto store_v = [&](int t) {
    char *vs = smem + 2 * KT_BYTES + (t & 1) * VT_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4 *>(vs + v_off(v_row + 64 * i, v_ch)) = rv[i];
  };
  auto sync = [&]() {  // LDS-only barrier: global loads stay in flight across it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 o[4], s[2];
  V8 pf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;

  // M phase: the 16 S MFMAs (K fragments) then the 16 P.V MFMAs (V^T fragments); fragment
  // j + kPre is read from LDS while MFMA j runs, so the LDS latency stays off the MFMA chain.
  constexpr int kPre = 4;
  auto frag = [&](int t, int j) __attribute__((always_inline)) -> V8 {
    if (j < 16) {  // K tile t: kk = j >> 1, st = j & 1
      const char *ks = smem + (t & 1) * KT_BYTES;
      return *reinterpret_cast<const V8 *>(ks + k_off((j & 1) * 32 + r32, 2 * (j >> 1) + hk));
    }
    const int i = j - 16;  // V tile t-1: kc = i >> 2, ds = i & 3 (accumulators alternate)
    const char *vs = smem + 2 * KT_BYTES + ((t - 1) & 1) * VT_BYTES;
    return *reinterpret_cast<const V8 *>(vs + v_off((i & 3) * 32 + r32, 2 * (i >> 2) + hk));
  };
  auto mphase = [&](auto j0c, auto j1c, int t) __attribute__((always_inline)) {
    constexpr int J0 = decltype(j0c)::value, J1 = decltype(j1c)::value;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (J0 == 0) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[st][e] = 0.f;
    }
    V8 fr[kPre];
#pragma unroll
    for (int j = J0; j < J0 + kPre; ++j) fr[j % kPre] = frag(t, j);
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const V8 f = fr[j % kPre];
      if (j + kPre < J1) fr[j % kPre] = frag(t, j + kPre);
      if (j < 16) s[j & 1] = Mfma<T>::mma(f, qf[j >> 1], s[j & 1]);
      else o[(j - 16) & 3] = Mfma<T>::mma(f, pf[(j - 16) >> 2], o[(j - 16) & 3]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int j = J0; j < J1 - kPre; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  auto vphase = [&](int t) __attribute__((always_inline)) {
    const int kv0 = kv_begin + t * BKV;
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
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[st][e], sl2, nm));
        psum += p;
        pf[2 * st + (e >> 3)][e & 7] = from_f32_inrange<T>(p);  // p <= 256
      }
    l_run += psum;
  };
  auto io = [&](int t) __attribute__((always_inline)) {  // global phase 2t+1
    if (t + 1 < n) store_k(t + 1);
    store_v(t);
    if (t + 2 < n) gload_k(t + 2);
    if (t + 1 < n) gload_v(t + 1);
  };

  using I0 = std::integral_constant<int, 0>;
  using I16 = std::integral_constant<int, 16>;
  using I32 = std::integral_constant<int, 32>;
  // Local phase 2t is M(t), 2t+1 is V(t); half B runs one global phase behind half A (one
  // extra barrier up front, one fewer at the end).  io(t) belongs to global phase 2t+1: the
  // V phase of half A, the M phase of half B.
  gload_k(0);
  store_k(0);
  if (n > 1) gload_k(1);
  gload_v(0);
  sync();
  if (half) sync();
  if (half) io(0);
  mphase(I0{}, I16{}, 0);
  sync();
  if (!half) io(0);
  vphase(0);
  sync();
  for (int t = 1; t < n; ++t) {
    if (half) io(t);
    mphase(I0{}, I32{}, t);
    sync();
    if (!half) io(t);
    vphase(t);
    sync();
  }
  mphase(I16{}, I32{}, n);
  if (!half) sync();

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
  if (op != OP_BF16 && op != OP_F16) return hipErrorInvalidValue;
  int tb[4] = {0, 0, 0, 0};
  for (int i = 0; i < 3; ++i)
    tb[i + 1] = tb[i] + (i < a.ng ? (a.g[i].q1 - a.g[i].q0 + BQ - 1) / BQ : 0);
  const int q_tiles = tb[3];
  if (q_tiles == 0) return hipSuccess;
  const int total = q_tiles * a.heads;
  const int grid = (total + 7) / 8 * 8;
  if (op == OP_BF16)
    k_attn_pp<bf16><<<grid, 512, 0, s>>>(a, tb[1], tb[2], q_tiles, total);
  else
    k_attn_pp<f16><<<grid, 512, 0, s>>>(a, tb[1], tb[2], q_tiles, total);
  return hipGetLastError();
}

}  // namespace dit
