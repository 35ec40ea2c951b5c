// Flash-style softmax attention, head_dim 128, 16-bit (bf16 or fp16) MFMA operands with fp32
// online softmax (gfx950).
//
// o_h = softmax(q_h k_h^T / sqrt(128)) v_h over the keys a query may see: all N tokens
// (joint / double / single blocks) or only its own stream (per-mode blocks, block-diagonal)
// ("FLUX.3 Image Klein in Diffusers", section "Entkoppelte Vorverarbeitung und gemeinsame
// Attention-Blöcke").  Padded prompt tokens are attended like any other token ("...",
// section "Verarbeitung einzelner Prompts und Batching-Architektur in der Praxis").
//
// Work split: a workgroup of 8 waves takes 256 queries of one head (32 per wave, two blocks of
// 16) and walks the allowed keys in tiles of 64, staged through LDS.  Per wave and key tile, with
// v_mfma_f32_16x16x32 (which holds a higher clock than the 32x32x16 form under the power limit):
//   S^T = K Q^T   (A = K fragments from LDS, B = the wave's queries held in registers): a lane
//                 owns one query of each block and 16 of the tile's keys, so a row max takes
//                 two exchanges (lanes l^16, l^32).
//   O^T += V^T P^T (A = V^T fragments from LDS, B = P straight from the S registers: a lane's S
//                 values of a 32-key chunk are keys 4q..4q+3 and 16+4q..16+4q+3, q = lane/16,
//                 the B operand's k positions 8q..8q+7 in that order).
// The running max is raised lazily: P is formed against the stored max unless some row's
// max grew by more than 2^8, so O is rescaled only when that happens (P <= 256 fits fp16).
// V is read in the transposed layout written by linear1's epilogue, vt[h][d][token'] with the
// tokens of every 32 reordered so that 16-byte chunk q holds tokens 4q..4q+3, 16+4q..16+4q+3:
// the eight keys a lane multiplies in one P.V MFMA form a single chunk.  Scores are kept in the log2 domain
// (scale * log2(e) folded into one FMA before exp2).
// Groups: each (q0, q1, k0, k1) range gets its own query tiles; key tiles start at k0
// rounded down to 64 and keys outside [k0, k1) are masked to -inf.
//
// Load balance: a unit is (head, 256-query tile) and needs one pass over its key tiles.  When
// there are more units than compute units, the grid is one workgroup per compute unit and
// each takes an equal share of all (unit, key tile) iterations, so the last round does not
// leave part of the chip idle.  A unit cut by a share boundary is computed in pieces; each
// piece stores its unnormalised O with its row max and row sum, and the piece that finishes
// last (a per-unit counter) merges the pieces in piece order, so the result does not depend
// on which workgroup finished first.  Nothing ever waits on another workgroup.
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

// Work plan: units are numbered head-major, query tiles within a head in group order; the
// iterations of a unit are its key tiles.
struct AttnPlan {
  int tb[kMaxGroups + 1];   // first query tile of each group (the rest: query tiles per head)
  int cum[kMaxGroups + 1];  // iterations of a head before each group (the rest: all of them)
  int nk[kMaxGroups];       // key tiles per unit of each group
  int q_tiles;              // query tiles per head
  int iters_head, iters;    // iterations per head, in total
  int total;              // units
  int lean;               // 1: equal iteration shares over the grid; 0: one unit per workgroup
  // lean: units [0, full) run whole, workgroup w taking units w, w + grid, ... (full is a
  // multiple of the grid); the iterations from it_full (unit full's first) to the end are
  // split into equal shares
  int full, it_full;
};

struct Unit {
  int head, qt, g, t;  // head, query tile, group, key tile within the unit
};
__device__ __forceinline__ Unit decode(const AttnPlan &p, int it) {
  Unit u;
  u.head = it / p.iters_head;
  const int r = it - u.head * p.iters_head;
  u.g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) u.g += r >= p.cum[i];
  const int rr = r - p.cum[u.g];
  const int ql = rr / p.nk[u.g];
  u.t = rr - ql * p.nk[u.g];
  u.qt = p.tb[u.g] + ql;
  return u;
}
// first iteration of the share of workgroup w, and the workgroup whose share holds iteration
// it (it >= it_full)
__device__ __forceinline__ int share_begin(const AttnPlan &p, int w, int grid) {
  return p.it_full + (int)((long long)(p.iters - p.it_full) * w / grid);
}
__device__ __forceinline__ int share_owner(const AttnPlan &p, int it, int grid) {
  const long long span = p.iters - p.it_full;
  return (int)(((long long)(it - p.it_full + 1) * grid + span - 1) / span) - 1;
}
// first iteration of unit u (head-major, query tiles in group order)
__device__ __forceinline__ int unit_begin(const AttnPlan &p, int u) {
  const int hd = u / p.q_tiles, qt = u - hd * p.q_tiles;
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) g += qt >= p.tb[i];
  return hd * p.iters_head + p.cum[g] + (qt - p.tb[g]) * p.nk[g];
}

// Partial results of a piece: O as 16 float4 per lane and wave, then (max, max, sum, sum) of the
// lane's two queries.
constexpr int kPartO = 8 * 16 * 64 * 4;
constexpr int kPartFloats = kPartO + 8 * 64 * 4;
static_assert(kPartFloats == attn_part_floats, "partial slot size");
constexpr int kSc1 = 16;  // buffer access cache policy: device-coherent (sc1)

template <typename T>
__global__ __launch_bounds__(512, 1) void k_attn_pp(AttnArgs a, AttnPlan p) {
  typedef typename Mfma<T>::v8 V8;
  __shared__ __attribute__((aligned(16))) char smem[2 * KT_BYTES + 2 * VT_BYTES];
  __shared__ int merge_flag;

  const int G = gridDim.x;
  const int per = G >> 3;
  const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  int it0, it1, n_whole = 0;  // the share (or the one unit), then whole units lid + G r, r < n_whole
  if (p.lean) {
    it0 = share_begin(p, lid, G);
    it1 = share_begin(p, lid + 1, G);
    n_whole = p.full / G;
  } else {
    if (lid >= p.total) return;
    it0 = unit_begin(p, lid);
    it1 = it0 + p.nk[decode(p, it0).g];
  }
  if (it0 >= it1 && n_whole == 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int half = wave >> 2;  // waves w and w+4 of a workgroup share a SIMD
  const T *qkv = reinterpret_cast<const T *>(a.qkv);

  // state of the piece being computed (set at the top of the piece loop)
  int head = 0, q = 0, kv_begin = 0, n = 0;
  AttnGroup grp = a.g[0];
  const T *vt = nullptr;
  V8 qf[2][4];  // [query block][32-d step]

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

  f32x4 o[2][8], s[2][4];  // O^T [query block][16-d block], S^T [query block][16-key block]
  V8 pf[2][2];              // P^T [query block][32-key chunk]
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const float sl2 = a.scale * 1.4426950408889634f;

  // M phase: 16 K fragments, each for the S MFMAs of both query blocks, then 16 V^T fragments,
  // each for the P.V MFMAs of both blocks; fragment j + kPre is read from LDS while fragment j's
  // MFMAs run, so the LDS latency stays off the MFMA chain.
  constexpr int kPre = 4;
  auto frag = [&](int t, int j) __attribute__((always_inline)) -> V8 {
    if (j < 16) {  // K tile t: key block kb = j & 3, 32-d step ds = j >> 2
      const char *ks = smem + (t & 1) * KT_BYTES;
      return *reinterpret_cast<const V8 *>(ks + k_off((j & 3) * 16 + r16, 4 * (j >> 2) + q4));
    }
    const int i = j - 16;  // V tile t-1: 16-d block db = i & 7, 32-key chunk kc = i >> 3
    const char *vs = smem + 2 * KT_BYTES + ((t - 1) & 1) * VT_BYTES;
    return *reinterpret_cast<const V8 *>(vs + v_off((i & 7) * 16 + r16, 4 * (i >> 3) + q4));
  };
  auto mphase = [&](auto j0c, auto j1c, int t) __attribute__((always_inline)) {
    constexpr int J0 = decltype(j0c)::value, J1 = decltype(j1c)::value;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (J0 == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[b][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    V8 fr[kPre];
#pragma unroll
    for (int j = J0; j < J0 + kPre; ++j) fr[j % kPre] = frag(t, j);
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const V8 f = fr[j % kPre];
      if (j + kPre < J1) fr[j % kPre] = frag(t, j + kPre);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (j < 16) s[b][j & 3] = Mfma<T>::mma16(f, qf[b][j >> 2], s[b][j & 3]);
        else o[b][(j - 16) & 7] = Mfma<T>::mma16(f, pf[b][(j - 16) >> 3], o[b][(j - 16) & 7]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int j = J0; j < J1 - kPre; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kPre, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  auto vphase = [&](int t) __attribute__((always_inline)) {
    const int kv0 = kv_begin + t * BKV;
    if ((kv0 < grp.k0) || (kv0 + BKV > grp.k1)) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = kv0 + kb * 16 + 4 * q4 + e;
            if (key < grp.k0 || key >= grp.k1) s[b][kb][e] = -INFINITY;
          }
    }
    float mx[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, s[b][kb][e]);
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      mx[b] = fmaxf(m, __shfl_xor(m, 32, 64)) * sl2;
    }
    // wave-uniform: raise the stored maxima, rescale O
    if (__ballot(mx[0] > m_run[0] + kLazy || mx[1] > m_run[1] + kLazy)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float m_new = fmaxf(m_run[b], mx[b]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_new);
        m_run[b] = m_new;
        l_run[b] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[b][i] *= alpha;
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float nm = -m_run[b];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[b][kb][e], sl2, nm));
          psum += p;
          pf[b][kb >> 1][4 * (kb & 1) + e] = from_f32_inrange<T>(p);  // p <= 256
        }
      l_run[b] += psum;
    }
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

  // Pieces of this workgroup's share: a partial piece at the end of the share first (the
  // head of a unit the next workgroup finishes), then the first piece, then the whole units
  // inside the share; then the whole units of the full rounds.
  int len_first = 0, len_last = 0, step = 3;
  if (it0 < it1) {
    const Unit uf = decode(p, it0);
    len_first = min(it1 - it0, p.nk[uf.g] - uf.t);
    const Unit ul = decode(p, it1 - 1);
    const bool last_partial = (it0 + len_first < it1) && (ul.t + 1 < p.nk[ul.g]);
    len_last = last_partial ? ul.t + 1 : 0;
    step = last_partial ? 0 : 1;
  }
  const int mid_end = it1 - len_last;
  int mid = it0 + len_first, r_whole = 0;
  for (;;) {
    int pit, plen, slot;
    if (step == 0) {
      pit = it1 - len_last;
      plen = len_last;
      slot = 2 * lid + 1;
      step = 1;
    } else if (step == 1) {
      pit = it0;
      plen = len_first;
      slot = 2 * lid;
      step = 2;
    } else if (step == 2 && mid < mid_end) {
      pit = mid;
      plen = p.nk[decode(p, mid).g];
      slot = -1;
      mid += plen;
    } else {
      if (r_whole >= n_whole) break;
      pit = unit_begin(p, lid + r_whole * G);
      plen = p.nk[decode(p, pit).g];
      slot = -1;
      ++r_whole;
    }
    const Unit u = decode(p, pit);
    const int nku = p.nk[u.g];
    head = u.head;
    grp = a.g[u.g];
    q = grp.q0 + (u.qt - p.tb[u.g]) * BQ + wave * 32 + r16;  // query of block 0; block 1: q + 16
    kv_begin = (grp.k0 / BKV) * BKV + u.t * BKV;
    n = plen;
    vt = reinterpret_cast<const T *>(a.vt) + (size_t)head * HD * a.ldv;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const T *qp = qkv + (size_t)(q + 16 * b) * a.ldqkv + head * HD + q4 * 8;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[b][ds] = *reinterpret_cast<const V8 *>(qp + ds * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[b] = -INFINITY;
      l_run[b] = 0.f;
    }

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

    // lane: query q (block 0) and q + 16 (block 1), dims 16 i + 4 q4 + {0..3} of each block
    auto store_rows = [&](const float inv[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (q + 16 * b >= grp.q1) continue;
        T *op = reinterpret_cast<T *>(a.out) + (size_t)(q + 16 * b) * a.ldo + head * HD + 4 * q4;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          store4(op + i * 16, o[b][i][0] * inv[b], o[b][i][1] * inv[b], o[b][i][2] * inv[b],
                 o[b][i][3] * inv[b]);
      }
    };
    // row sum: the four lanes l, l^16, l^32, l^48 hold a query's 64 keys between them
    auto full_sum = [](float l) __attribute__((always_inline)) {
      l += __shfl_xor(l, 16, 64);
      return l + __shfl_xor(l, 32, 64);
    };
    if (u.t == 0 && plen == nku) {  // the whole unit: normalise and store
      const float inv[2] = {1.0f / full_sum(l_run[0]), 1.0f / full_sum(l_run[1])};
      store_rows(inv);
      continue;
    }

    // A piece: publish (O, max, sum); the last piece of the unit to finish merges them.
    // Ordering, in the HIP memory model at agent scope: every wave's partial stores have
    // completed before the workgroup barrier, the counter increment is a release (it
    // happens after them), and the piece that sees the last count performs an acquire fence
    // before the barrier that lets its waves read the other pieces' partials.  The partials
    // are also written and read with device-coherent (sc1) buffer accesses, so the stores
    // leave no dirty lines for the release's writeback.
    const __amdgpu_buffer_rsrc_t rs_part = __builtin_amdgcn_make_buffer_rsrc(
        a.part, (short)0, (int)((size_t)2 * G * kPartFloats * 4), 0x00020000);
    const int o_off = (wave * 16 * 64 + lane) * 16, ml_off = kPartO * 4 + (wave * 64 + lane) * 16;
#pragma unroll
    for (int c = 0; c < 16; ++c)
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{__float_as_uint(o[c >> 3][c & 7][0]), __float_as_uint(o[c >> 3][c & 7][1]),
                __float_as_uint(o[c >> 3][c & 7][2]), __float_as_uint(o[c >> 3][c & 7][3])},
          rs_part, o_off + c * 64 * 16, slot * kPartFloats * 4, kSc1);
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(m_run[0]), __float_as_uint(m_run[1]), __float_as_uint(l_run[0]),
              __float_as_uint(l_run[1])},
        rs_part, ml_off, slot * kPartFloats * 4, kSc1);
    const int unit = u.head * p.q_tiles + u.qt;
    const int u0 = pit - u.t;  // first iteration of the unit
    const int w0 = share_owner(p, u0, G), w1 = share_owner(p, u0 + nku - 1, G);
    __builtin_amdgcn_s_waitcnt(0);  // the partial stores have completed
    __syncthreads();
    if (tid == 0) {
      const bool last = __hip_atomic_fetch_add(a.cnt + unit, 1, __ATOMIC_RELEASE,
                                               __HIP_MEMORY_SCOPE_AGENT) == w1 - w0;
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      merge_flag = last;
    }
    __syncthreads();
    if (merge_flag) {
      // two passes over the pieces (at most 8, checked by the launcher): the maxima, then the
      // weighted sums; each pass recomputes the piece's slot rather than holding a table
      const int np = w1 - w0 + 1;
      auto slot_of = [&](int i) __attribute__((always_inline)) {
        const int w = w0 + i;
        return share_begin(p, w, G) >= u0 ? 2 * w : 2 * w + 1;
      };
      float mx[2] = {-INFINITY, -INFINITY};
      for (int i = 0; i < np; ++i) {
        const u32x4 ml = __builtin_amdgcn_raw_buffer_load_b128(rs_part, ml_off,
                                                               slot_of(i) * kPartFloats * 4, kSc1);
        mx[0] = fmaxf(mx[0], __uint_as_float(ml.x));
        mx[1] = fmaxf(mx[1], __uint_as_float(ml.y));
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      float l[2] = {0.f, 0.f};
      for (int i = 0; i < np; ++i) {
        const int so = slot_of(i) * kPartFloats * 4;
        const u32x4 ml = __builtin_amdgcn_raw_buffer_load_b128(rs_part, ml_off, so, kSc1);
        const float wgt[2] = {__builtin_amdgcn_exp2f(__uint_as_float(ml.x) - mx[0]),
                              __builtin_amdgcn_exp2f(__uint_as_float(ml.y) - mx[1])};
        l[0] += wgt[0] * __uint_as_float(ml.z);
        l[1] += wgt[1] * __uint_as_float(ml.w);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs_part, o_off + c * 64 * 16, so, kSc1);
          const float w = wgt[c >> 3];
          o[c >> 3][c & 7][0] += w * __uint_as_float(v.x);
          o[c >> 3][c & 7][1] += w * __uint_as_float(v.y);
          o[c >> 3][c & 7][2] += w * __uint_as_float(v.z);
          o[c >> 3][c & 7][3] += w * __uint_as_float(v.w);
        }
      }
      const float inv[2] = {1.0f / full_sum(l[0]), 1.0f / full_sum(l[1])};
      store_rows(inv);
      if (tid == 0)  // ready for the next launch
        __hip_atomic_store(a.cnt + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t attention_mfma(const AttnArgs &a, int op, hipStream_t s) {
  if (a.ng < 1 || a.ng > kMaxGroups) return hipErrorInvalidValue;
  if (op != OP_BF16 && op != OP_F16) return hipErrorInvalidValue;
  AttnPlan p = {};
  for (int i = 0; i < kMaxGroups; ++i) {
    const bool on = i < a.ng && a.g[i].q1 > a.g[i].q0;
    if (on && a.g[i].k1 <= a.g[i].k0) return hipErrorInvalidValue;  // a query needs a key
    const int qt = on ? (a.g[i].q1 - a.g[i].q0 + BQ - 1) / BQ : 0;
    p.nk[i] = on ? (a.g[i].k1 - a.g[i].k0 / BKV * BKV + BKV - 1) / BKV : 1;
    p.tb[i + 1] = p.tb[i] + qt;
    p.cum[i + 1] = p.cum[i] + qt * p.nk[i];
  }
  p.q_tiles = p.tb[kMaxGroups];
  p.iters_head = p.cum[kMaxGroups];
  if (p.q_tiles == 0) return hipSuccess;
  p.total = p.q_tiles * a.heads;
  if ((long long)p.iters_head * a.heads > 0x7fffffffLL) return hipErrorInvalidValue;
  p.iters = p.iters_head * a.heads;
  int grid = (p.total + 7) / 8 * 8;
  const int lg = a.lean_grid / 8 * 8;
  // One unit per workgroup leaves compute units idle in a last, partly filled round, but the
  // chip is power-limited: the busy ones then run faster, so splitting units into pieces (with
  // the cost of publishing and merging them) pays only when that round is mostly empty.
  // Measured, one unit per workgroup against split: 56 against 69 us for 144 units on 256
  // CUs (1536 tokens), 274 against 275 us for 432 (4608), 1010 against 896 us for 816 (8704),
  // 213 against 190 us for 336 (3584).  A share of s iterations cuts a unit into at most
  // ceil(nk / s) + 1 pieces, which the merge supports up to 8; shares under 8 key tiles are
  // not worth a merge.
  if (a.part != nullptr && a.cnt != nullptr && lg > 0) {
    // Units of the full rounds run whole; the last round's units are split when they would
    // fill under 40% of it.
    const int full = p.total / lg * lg, rest = p.total - full;
    if (rest > 0 && 5LL * rest < 2LL * lg) {
      p.full = full;
      p.it_full = 0;
      if (full > 0) {  // first iteration of unit `full`, as unit_begin computes it
        const int hd = full / p.q_tiles, qt = full - hd * p.q_tiles;
        int g = 0;
        for (int i = 1; i < kMaxGroups; ++i) g += qt >= p.tb[i];
        p.it_full = hd * p.iters_head + p.cum[g] + (qt - p.tb[g]) * p.nk[g];
      }
      int nk_max = 1;
      for (int i = 0; i < kMaxGroups; ++i) nk_max = nk_max > p.nk[i] ? nk_max : p.nk[i];
      const int share = (p.iters - p.it_full) / lg;
      if (share >= 8 && (nk_max + share - 1) / share + 1 <= 8) {
        p.lean = 1;
        grid = lg;
      }
    }
  }
  if (op == OP_BF16)
    k_attn_pp<bf16><<<grid, 512, 0, s>>>(a, p);
  else
    k_attn_pp<f16><<<grid, 512, 0, s>>>(a, p);
  return hipGetLastError();
}

}  // namespace dit
