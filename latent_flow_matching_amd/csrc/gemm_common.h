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

// linear1's feature tiles in an interleaved order: head tile b's Q, K and V tiles, then its
// share of the SwiGLU tiles, for b = 0, 1, ...  Workgroups reach the XCDs in contiguous ranges
// of tile ids, so in plain order the Q and K tiles (whose fused epilogue costs the most) would
// all land on the first XCDs; interleaved, every XCD gets the same mix.  Identity when there
// are no Q / K / V columns (split == 0).
__device__ __forceinline__ int qkv_feature_tile(int l, int n_tiles, int split) {
  const int tq = split / (3 * BN);  // tiles of each of Q, K and V
  if (tq == 0) return l;
  const int tm = n_tiles - 3 * tq;  // SwiGLU tiles
  int b = 0;
  while (b + 1 < tq && 3 * (b + 1) + (b + 1) * tm / tq <= l) ++b;
  const int o = l - (3 * b + b * tm / tq);
  return o < 3 ? o * tq + b : 3 * tq + b * tm / tq + (o - 3);
}

// Bytes per row of a wave's V-transpose tile in LDS: 96 columns (three 32-token groups) of
// 16-bit values plus 16 B, so that the four dim rows one ds_write_b16 touches (dims 4 apart)
// start 16 banks apart.
constexpr int kVtPitch = 208;
constexpr int kVtLds = 128 * kVtPitch;  // per wave

// Column of token t inside its aligned 32-token group of vt: 16-byte chunk q holds tokens
// 4q..4q+3 then 16+4q..16+4q+3.
__device__ __forceinline__ int vt_col(int u) {
  return ((u & 15) >> 2) * 8 + (u >> 4) * 4 + (u & 3);
}

// Keeps accumulator v in its AGPRs up to this point, so that it is moved to VGPRs where it is
// used: left alone, the compiler reads every accumulator out at the start of an epilogue and
// spills.  PIN false (accumulators already rescaled in VGPRs by the caller) does nothing.
template <bool PIN>
__device__ __forceinline__ void keep_in_agpr(f32x4 &v) {
  if constexpr (PIN) asm volatile("" : "+a"(v)::"memory");
}

// Fused part of linear1's epilogue for a wave whose 128 features are one Q, K or V head
// (a.vt != nullptr).  Lane (r16, q4) holds dims 16 i + 4 q4 + {0..3} of token 16 j + r16.
//   Q, K: RMSNorm over the head's 128 dims ("FLUX.3 Image Klein in Diffusers", "Entkoppelte
//   Vorverarbeitung ...": queries and keys are RMS-normalised) -- the lane's 32 squares plus
//   those of lanes r16 + 16, + 32, + 48 -- times the segment's weight, then the rotary
//   embedding of adjacent pairs (2p, 2p + 1) with the token's (cos, sin) of pair p (the
//   lane's four dims are two whole pairs), stored to qkv.
//   V: written transposed to vt.  The wave's tokens go in halves of 64 through its own LDS
//   tile [128 dims][96 columns] (a half touches at most three aligned 32-token groups),
//   then out as 16-byte chunks; chunks that hold tokens outside the half or the group are
//   written element by element, so tiles that share a chunk write disjoint bytes.  The
//   caller has passed a workgroup barrier after the main loop's last LDS reads.
template <typename T, int BM, int WN, int WM, bool PIN>
__device__ __forceinline__ void epilogue_qkv_heads(const GemmArgs &a, const GemmGroup &grp,
                                                   int n0, int m0, int wn, int wm, int lane,
                                                   f32x4 (&acc)[BN / WN / 16][BM / WM / 16],
                                                   char *smem) {
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int FS = WTN / 16, TS = WTM / 16;
  static_assert(WTN == 128 && WTM % 16 == 0 && WTM >= 64 && WTM <= 128,
                "one head per wave, at most two token halves of up to 64");
  const int r16 = lane & 15, q4 = lane >> 4;
  const int dm = a.split / 3;
  const int fw = n0 + wn * WTN;  // the wave's first feature
  const int part = fw / dm;      // 0 Q, 1 K, 2 V
  const int h = (fw - part * dm) >> 7;
  const int mw = m0 + wm * WTM;  // the wave's first row in the group
  if (mw >= grp.rows) return;
  const int wave = wm * WN + wn;
  if (part < 2) {
    // Pass 1, registers only: each token's 1 / RMS from the fp32 accumulators (its 128 dims
    // are this lane's 32 and those of lanes +16, +32, +48), and the scaled values as fp16
    // into the wave's LDS tile [128 tokens][128 dims], 16-byte chunk c of token t at slot
    // c ^ (t & 15) so that the 16 tokens of one write land on distinct banks.
    char *tq = smem + wave * (WTM * 256);
#pragma unroll
    for (int j = 0; j < TS; ++j) {
#pragma unroll
      for (int i = 0; i < FS; ++i) keep_in_agpr<PIN>(acc[i][j]);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < FS; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss += acc[i][j][r] * acc[i][j][r];
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      const float rs = 1.0f / sqrtf(ss * (1.0f / 128.f) + a.rms_eps);
      const int t = j * 16 + r16;
#pragma unroll
      for (int i = 0; i < FS; ++i) {
        const int c = 2 * i + (q4 >> 1);  // 16-byte chunk of dims 16 i + 4 q4 ..
        f16x4 v = {(f16)(acc[i][j][0] * rs), (f16)(acc[i][j][1] * rs), (f16)(acc[i][j][2] * rs),
                   (f16)(acc[i][j][3] * rs)};
        *reinterpret_cast<f16x4 *>(tq + t * 256 + ((c ^ (t & 15)) << 4) + (q4 & 1) * 8) = v;
      }
    }
    // Pass 2, after the accumulators' last use: lane (c = lane % 16) takes dims 8c .. 8c + 7
    // (pairs 4c .. 4c + 3: axis c / 4, frequencies j0 = 4 (c % 4) .. j0 + 3) of tokens
    // lane / 16 + 4k.  It multiplies by the segment's weights and rotates each pair by
    // angle = pos * freq_j, taken in revolutions: x = pos * hi_j is exact for integer positions,
    // so r = (x - rint(x)) + pos * lo_j keeps the angle's precision within half a turn, where
    // the hardware sine and cosine are accurate.  The positions of all 32 tokens are loaded
    // at once; 16 lanes store one token's 256-byte head row.
    const int c = lane & 15, tl = lane >> 4;
    const int mlast = min(mw + WTM, grp.rows) - 1;
    const int seg0 = segment_of(grp.out_row0 + mw, a.b1, a.b2, a.per);
    const bool one_seg = seg0 == segment_of(grp.out_row0 + mlast, a.b1, a.b2, a.per);
    const float *const *wsel = part == 0 ? a.qn : a.kn;
    const f32x4 w0 = *reinterpret_cast<const f32x4 *>(wsel[seg0] + 8 * c);
    const f32x4 w1 = *reinterpret_cast<const f32x4 *>(wsel[seg0] + 8 * c + 4);
    const f32x4 fh = *reinterpret_cast<const f32x4 *>(a.rope_fr + 4 * (c & 3));
    const f32x4 fl = *reinterpret_cast<const f32x4 *>(a.rope_fr + 16 + 4 * (c & 3));
    constexpr int NT4 = WTM / 4;  // tokens per lane
    float pv[NT4];
#pragma unroll
    for (int k = 0; k < NT4; ++k) {
      const int tok = grp.out_row0 + min(mw + tl + 4 * k, grp.rows - 1);
      pv[k] = a.rope_pos[(size_t)tok * 4 + (c >> 2)];
    }
    constexpr int KB = 8;
    // y = weight * (value / RMS), then the rotation of its four pairs by pos * freq
    auto rotate = [&](const f16x8 &h, const f32x4 &wa, const f32x4 &wb, float p) {
      const float y[8] = {(float)h[0] * wa.x, (float)h[1] * wa.y, (float)h[2] * wa.z,
                          (float)h[3] * wa.w, (float)h[4] * wb.x, (float)h[5] * wb.y,
                          (float)h[6] * wb.z, (float)h[7] * wb.w};
      typename Mfma<T>::v8 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = p * fh[q];
        const float r = (x - __builtin_rintf(x)) + p * fl[q];
        const float co = __builtin_amdgcn_cosf(r), sn = __builtin_amdgcn_sinf(r);
        o[2 * q] = from_f32<T>(y[2 * q] * co - y[2 * q + 1] * sn);
        o[2 * q + 1] = from_f32<T>(y[2 * q] * sn + y[2 * q + 1] * co);
      }
      return o;
    };
    typedef typename Mfma<T>::v8 V8o;
    if (one_seg && mw + WTM <= grp.rows) {
      // every token of the wave in the group and in one segment: no per-token branches, so
      // the compiler can interleave the eight tokens of a batch
      V8o *dst = reinterpret_cast<V8o *>(reinterpret_cast<T *>(a.qkv) +
                                         (size_t)(grp.out_row0 + mw + tl) * a.ldq + fw + 8 * c);
      const size_t step = (size_t)4 * a.ldq / 8;  // four tokens, in 16-byte units
#pragma unroll
      for (int k0 = 0; k0 < NT4; k0 += KB) {
        f16x8 hv[KB];
#pragma unroll
        for (int k = 0; k < KB && k0 + k < NT4; ++k) {
          const int t = tl + 4 * (k0 + k);
          hv[k] = *reinterpret_cast<const f16x8 *>(tq + t * 256 + ((c ^ (t & 15)) << 4));
        }
#pragma unroll
        for (int k = 0; k < KB && k0 + k < NT4; ++k)
          dst[(k0 + k) * step] = rotate(hv[k], w0, w1, pv[k0 + k]);
      }
    } else {
#pragma unroll 1
      for (int k = 0; k < NT4; ++k) {
        const int t = tl + 4 * k, m = mw + t;
        if (m >= grp.rows) continue;
        const int tok = grp.out_row0 + m;
        const float *wr = wsel[segment_of(tok, a.b1, a.b2, a.per)] + 8 * c;
        const f16x8 h = *reinterpret_cast<const f16x8 *>(tq + t * 256 + ((c ^ (t & 15)) << 4));
        *reinterpret_cast<V8o *>(reinterpret_cast<T *>(a.qkv) + (size_t)tok * a.ldq + fw + 8 * c) =
            rotate(h, *reinterpret_cast<const f32x4 *>(wr), *reinterpret_cast<const f32x4 *>(wr + 4),
                   a.rope_pos[(size_t)tok * 4 + (c >> 2)]);
      }
    }
    return;
  }
  char *tile = smem + wave * kVtLds;
  T *vb = reinterpret_cast<T *>(a.vt) + (size_t)h * 128 * a.ldv;
  const int tw0 = grp.out_row0 + mw;        // the wave's first token
  const int gend = grp.out_row0 + grp.rows;  // the group's end
#pragma unroll
  for (int hf = 0; hf < (WTM + 63) / 64; ++hf) {
    constexpr int HL0 = 64;
    const int hl = min(HL0, WTM - 64 * hf);  // tokens of this half (48 for the second of 112)
    const int t0 = tw0 + 64 * hf, g0 = t0 & ~31;
    if (t0 >= gend) break;
#pragma unroll
    for (int jj = 0; jj < 4 && 16 * jj < WTM - 64 * hf; ++jj) {
      const int c = t0 + 16 * jj + r16 - g0;
      const int col = (c & ~31) + vt_col(c & 31);
#pragma unroll
      for (int i = 0; i < FS; ++i) keep_in_agpr<PIN>(acc[i][4 * hf + jj]);
#pragma unroll
      for (int i = 0; i < FS; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<T *>(tile + (16 * i + 4 * q4 + r) * kVtPitch + col * 2) =
              from_f32<T>(acc[i][4 * hf + jj][r]);
    }
    // (a wave's LDS operations complete in order: its reads below see its writes above)
    // Lane (ch = lane % 16, of which 12 are used) copies chunk ch of dim rows lane / 16 + 4k:
    // whether that chunk lies wholly in this half is the same for every row.
    const int t1 = min(t0 + hl, gend);
    const int ch = lane & 15, dl = lane >> 4;
    const int ta = g0 + (ch >> 2) * 32 + (ch & 3) * 4;  // tokens ta.., ta + 16.. of the chunk
    const bool any = ch < 12 && ta + 19 >= t0 && ta < t1;
    const bool whole = any && ta >= t0 && ta + 19 < t1;
    const char *src = tile + dl * kVtPitch + ch * 16;
    T *dst = vb + (size_t)dl * a.ldv + g0 + ch * 8;
    if (whole) {
#pragma unroll
      for (int k0 = 0; k0 < 32; k0 += 8) {
        u32x4 cv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          cv[k] = *reinterpret_cast<const u32x4 *>(src + (k0 + k) * 4 * kVtPitch);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          *reinterpret_cast<u32x4 *>(dst + (size_t)(k0 + k) * 4 * a.ldv) = cv[k];
      }
    } else if (any) {  // shared with the neighbouring half, wave or group: element by element
#pragma unroll 1
      for (int k = 0; k < 32; ++k) {
        const uint16_t *sv = reinterpret_cast<const uint16_t *>(src + k * 4 * kVtPitch);
        uint16_t *dv = reinterpret_cast<uint16_t *>(dst + (size_t)k * 4 * a.ldv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = ta + (e < 4 ? e : e + 12);
          if (t >= t0 && t < t1) dv[e] = sv[e];
        }
      }
    }
  }
  // the tile holding the last token also writes the zeros past it (this head, wm == 0 wave)
  if (wm == 0 && gend == a.n_tok && m0 + BM >= grp.rows) {
    const int z0 = a.n_tok & ~31, z1 = (a.n_tok / 64 + 2) * 64;
    const int nch = (z1 - z0) / 8;
    for (int k = lane; k < 128 * nch; k += 64) {
      const int d = k / nch, ch = k - d * nch;
      const int ta = z0 + (ch >> 2) * 32 + (ch & 3) * 4;
      T *dst = vb + (size_t)d * a.ldv + z0 + ch * 8;
      if (ta >= a.n_tok) {
        *reinterpret_cast<u32x4 *>(dst) = u32x4{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (ta + (e < 4 ? e : e + 12) >= a.n_tok) reinterpret_cast<uint16_t *>(dst)[e] = 0;
      }
    }
  }
}

// Epilogue: lane owns token (lane & 15) and features 4 (lane >> 4) + {0..3} of every 16x16
// sub-tile.  smem: the workgroup's LDS (at least 4 x kVtLds bytes), used by the fused
// Q / K / V epilogue, which every wave of a workgroup takes or none does.
template <typename T, int BM, int WN, int WM, int EPI, bool PIN = true>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const GemmGroup &grp, int n0, int m0,
                                         int wn, int wm, int lane,
                                         f32x4 (&acc)[BN / WN / 16][BM / WM / 16], char *smem) {
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int FS = WTN / 16, TS = WTM / 16;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int fbase = n0 + wn * WTN + 4 * q4;
  if constexpr (EPI == EPI_QKV_SWIGLU) {
    if (a.vt != nullptr && n0 < a.split) {
      __syncthreads();  // every wave's last fragment reads are done before LDS is reused
      epilogue_qkv_heads<T, BM, WN, WM, PIN>(a, grp, n0, m0, wn, wm, lane, acc, smem);
      return;
    }
  }
  if constexpr (EPI == EPI_RESID) {
    // Gated residual.  One wave per SIMD leaves load latency exposed: the gate is loaded once
    // when the wave's rows share a segment, so each token sub-tile's eight x loads go out
    // together and cost one round trip.
    const int mw = m0 + wm * WTM;  // the wave's first row in the group
    if (mw >= grp.rows) return;
    const int mlast = min(mw + WTM, grp.rows) - 1;
    const int seg0 = segment_of(grp.out_row0 + mw, a.b1, a.b2, a.per);
    if (seg0 == segment_of(grp.out_row0 + mlast, a.b1, a.b2, a.per)) {
      f32x4 g[FS];
#pragma unroll
      for (int i = 0; i < FS; ++i)
        g[i] = *reinterpret_cast<const f32x4 *>(a.gate[seg0] + fbase + i * 16);
      // the x rows of RB token sub-tiles are loaded before any of them is stored, so their
      // loads share one round trip
      constexpr int RB = PIN ? 2 : 1;
#pragma unroll
      for (int j0 = 0; j0 < TS; j0 += RB) {
        f32x4 xv[RB][FS];
#pragma unroll
        for (int jj = 0; jj < RB && j0 + jj < TS; ++jj) {
          const int m = mw + (j0 + jj) * 16 + r16;
          const float *xr = a.x + (size_t)(grp.out_row0 + min(m, grp.rows - 1)) * a.ldres + fbase;
#pragma unroll
          for (int i = 0; i < FS; ++i) xv[jj][i] = *reinterpret_cast<const f32x4 *>(xr + i * 16);
        }
#pragma unroll
        for (int jj = 0; jj < RB && j0 + jj < TS; ++jj) {
          const int j = j0 + jj, m = mw + j * 16 + r16;
          if (m >= grp.rows) continue;
          float *xr = a.x + (size_t)(grp.out_row0 + m) * a.ldres + fbase;
          // the accumulators leave their AGPRs here, not all at once at the epilogue's start
#pragma unroll
          for (int i = 0; i < FS; ++i) keep_in_agpr<PIN>(acc[i][j]);
#pragma unroll
          for (int i = 0; i < FS; ++i) {
            f32x4 v = xv[jj][i];
            v.x += g[i].x * acc[i][j][0];
            v.y += g[i].y * acc[i][j][1];
            v.z += g[i].z * acc[i][j][2];
            v.w += g[i].w * acc[i][j][3];
            *reinterpret_cast<f32x4 *>(xr + i * 16) = v;
          }
        }
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < TS; ++j) {
    const int m = m0 + wm * WTM + j * 16 + r16;  // row inside the group
    if (m >= grp.rows) continue;
    const int tok = grp.out_row0 + m;
#pragma unroll
    for (int i = 0; i < FS; ++i) keep_in_agpr<PIN>(acc[i][j]);
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

// Host check of the fused Q / K / V epilogue's shape: whole 256-feature tiles per Q, K and V
// region, and the table, weights and output it reads and writes.
inline bool fused_heads_ok(const GemmArgs &a, int epi) {
  if (epi != EPI_QKV_SWIGLU || a.vt == nullptr) return true;
  if (a.split % 3 || (a.split / 3) % BN || a.split > a.n || !a.qkv) return false;
  if (!a.rope_pos || !a.rope_fr) return false;
  if (a.n_tok < 0 || a.ldv < (a.n_tok / 64 + 2) * 64) return false;
  for (int s = 0; s < 3; ++s)
    if (!a.qn[s] || !a.kn[s]) return false;
  return true;
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
// (tiles, sub-tiles per wave); 256 threads = the GEMM's 4 waves x 64 lanes, same accumulator
// layout (BM token rows per tile: 8 or 7 sub-tiles of 16 per wave).
template <int EPI, int BM>
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmArgs a, TileBounds tb, int m_tiles_total,
                                                     int total_tiles, int splits) {
  constexpr int WTN = 128, WTM = BM / 2, FS = WTN / 16, TS = WTM / 16;
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
                    ((size_t)lid * 4 + wave) * (FS * TS * 64) + sub * 64 + lane;
  const size_t slice_stride = (size_t)total_tiles * 4 * FS * TS * 64;
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
