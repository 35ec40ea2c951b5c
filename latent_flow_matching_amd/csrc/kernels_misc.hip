// Memory-bound kernels of the block and the conditioning path (gfx950):
//   positions + RoPE tables, LayerNorm + adaLN modulation, QK RMSNorm + RoPE (+ V transpose),
//   GEMV for timestep MLP and modulation, timestep embedding, Philox noise.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dit {

// ------------------------------------------------------------------------------------------
// 4D RoPE coordinates: text i -> (0,0,0,i), image (r,c) -> (0,r,c,0), token (r,c) of reference
// k -> (0,r,c,-(k+1)), tokens ordered text | image | references, row-major inside an image
// ("FLUX.3 Image Klein in Diffusers", section "Modulation pro Token-Typ, Flow-Map-Destillation
// und 4D-RoPE").  The page's row/2, col/2 counts VAE-latent cells, two per token side.
// ------------------------------------------------------------------------------------------
struct RefGrids {
  int start[kMaxRefs + 1];  // first token of each reference after the image (then the end)
  int cols[kMaxRefs];
  int n;
};

__global__ void k_positions(float *pos, int n_txt, int gw, int n_img, RefGrids rg) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  int n = n_txt + n_img + rg.start[rg.n];
  if (i >= n) return;
  float h = 0.f, w = 0.f, l = 0.f;
  if (i < n_txt) {
    l = (float)i;
  } else if (i < n_txt + n_img) {
    int j = i - n_txt;
    h = (float)(j / gw);
    w = (float)(j % gw);
  } else {
    int j = i - n_txt - n_img;
    int k = 0;
    while (k + 1 < rg.n && j >= rg.start[k + 1]) ++k;
    j -= rg.start[k];
    h = (float)(j / rg.cols[k]);
    w = (float)(j % rg.cols[k]);
    l = -(float)(k + 1);
  }
  f32x4 v = {0.f, h, w, l};
  *reinterpret_cast<f32x4 *>(pos + 4 * (size_t)i) = v;
}

hipError_t fill_positions(float *pos, int n_txt, int gh, int gw, const int *ref_grids,
                          int n_refs, hipStream_t s) {
  if (n_refs < 0 || n_refs > kMaxRefs) return hipErrorInvalidValue;
  RefGrids rg = {};
  rg.n = n_refs;
  for (int k = 0; k < n_refs; ++k) {
    if (ref_grids[2 * k] < 1 || ref_grids[2 * k + 1] < 1) return hipErrorInvalidValue;
    rg.start[k + 1] = rg.start[k] + ref_grids[2 * k] * ref_grids[2 * k + 1];
    rg.cols[k] = ref_grids[2 * k + 1];
  }
  int n = n_txt + gh * gw + rg.start[n_refs];
  if (n <= 0) return hipSuccess;
  k_positions<<<(n + 255) / 256, 256, 0, s>>>(pos, n_txt, gw > 0 ? gw : 1, gh * gw, rg);
  return hipGetLastError();
}

// cs[i][p] = (cos, sin) of pos[i][p/16] * theta^(-2 (p%16) / 32), p = 0..63: one rotation
// angle per adjacent pair of the four 32-dim axis slices (t, h, w, l).  Angles in fp64.
__global__ void k_rope_table(float *cs, const float *pos, int n, double log_theta) {
  int i = blockIdx.x;
  int p = threadIdx.x;  // 64 threads
  if (i >= n) return;
  int axis = p >> 4, j = p & 15;
  double freq = exp(-log_theta * (2.0 * j) / 32.0);
  double ang = (double)pos[4 * (size_t)i + axis] * freq;
  double sn, cn;
  sincos(ang, &sn, &cn);
  cs[(size_t)i * 128 + 2 * p] = (float)cn;
  cs[(size_t)i * 128 + 2 * p + 1] = (float)sn;
}

hipError_t rope_table(float *cs, const float *pos, int n, float theta, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_rope_table<<<n, 64, 0, s>>>(cs, pos, n, log((double)theta));
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// LayerNorm without affine parameters, then y * (1 + scale_s) + shift_s with the segment's
// modulation ("FLUX.3 Image Klein in Diffusers", "Modulation pro Token-Typ ...": each block
// starts with a parameter-free LayerNorm whose scale and shift come from the timestep
// embedding).  One 256-thread workgroup per row (D <= 4096, D % 256 == 0): thread t holds
// the float4 columns t, t + 256, ... and that row's shift/scale, all loaded up front, and the
// two-pass mean/variance reduce through LDS.  Many small workgroups with few registers keep
// HBM busier than one wave per row with the whole row in one wave's registers.
// ------------------------------------------------------------------------------------------
constexpr int kLnMaxVec = 4;  // float4 per thread -> D <= 256 * 4 * 4 = 4096

template <typename TO>
__global__ __launch_bounds__(256) void k_ln_modulate(TO *out, int ldo, const float *x, int ldx,
                                                      int row0, int d, float eps,
                                                      const float *m0, const float *m1,
                                                      const float *m2, int b1, int b2, int per,
                                                      float *out_scale) {
  __shared__ float red[3][4];
  const int t = threadIdx.x, w = t >> 6;
  const int r = blockIdx.x, tok = row0 + r;
  const int nv4 = d >> 2;  // float4 columns; a multiple of 64, so each wave is all in or all out
  const float *xr = x + (size_t)tok * ldx;
  const int seg = segment_of(tok, b1, b2, per);
  const float *shift = seg == 0 ? m0 : (seg == 1 ? m1 : m2), *scale = shift + d;
  f32x4 v[kLnMaxVec], sh[kLnMaxVec], sc[kLnMaxVec];
#pragma unroll
  for (int i = 0; i < kLnMaxVec; ++i)
    if (i * 256 + t < nv4) v[i] = *reinterpret_cast<const f32x4 *>(xr + (i * 256 + t) * 4);
#pragma unroll
  for (int i = 0; i < kLnMaxVec; ++i)
    if (i * 256 + t < nv4) {
      sh[i] = *reinterpret_cast<const f32x4 *>(shift + (i * 256 + t) * 4);
      sc[i] = *reinterpret_cast<const f32x4 *>(scale + (i * 256 + t) * 4);
    }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kLnMaxVec; ++i)
    if (i * 256 + t < nv4) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  sum = wave_sum(sum);
  if ((t & 63) == 0) red[0][w] = sum;
  __syncthreads();
  const float mean = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) / (float)d;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < kLnMaxVec; ++i)
    if (i * 256 + t < nv4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, e = v[i].w - mean;
      sq += (a * a + b * b) + (c * c + e * e);
    }
  sq = wave_sum(sq);
  if ((t & 63) == 0) red[1][w] = sq;
  __syncthreads();
  const float var = ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) / (float)d;
  const float rstd = 1.0f / sqrtf(var + eps);
  TO *orow = out + (size_t)r * ldo;
  if constexpr (sizeof(TO) == 1) {
    // E4M3 codes of the modulated row: y * (448 / max |y|), dequantization scale max |y| / 448
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kLnMaxVec; ++i)
      if (i * 256 + t < nv4) {
        v[i].x = (v[i].x - mean) * rstd * (1.f + sc[i].x) + sh[i].x;
        v[i].y = (v[i].y - mean) * rstd * (1.f + sc[i].y) + sh[i].y;
        v[i].z = (v[i].z - mean) * rstd * (1.f + sc[i].z) + sh[i].z;
        v[i].w = (v[i].w - mean) * rstd * (1.f + sc[i].w) + sh[i].w;
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
      }
    amax = wave_max(amax);
    if ((t & 63) == 0) red[2][w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[2][0], red[2][1]), fmaxf(red[2][2], red[2][3]));
    if (t == 0) out_scale[r] = amax / 448.0f;
    const float rcp = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
    for (int i = 0; i < kLnMaxVec; ++i)
      if (i * 256 + t < nv4)
        *reinterpret_cast<uint32_t *>(orow + (i * 256 + t) * 4) =
            e4m3_pack4(v[i].x * rcp, v[i].y * rcp, v[i].z * rcp, v[i].w * rcp);
  } else {
#pragma unroll
    for (int i = 0; i < kLnMaxVec; ++i)
      if (i * 256 + t < nv4) {
        const int c = (i * 256 + t) * 4;
        const float y0 = (v[i].x - mean) * rstd * (1.f + sc[i].x) + sh[i].x;
        const float y1 = (v[i].y - mean) * rstd * (1.f + sc[i].y) + sh[i].y;
        const float y2 = (v[i].z - mean) * rstd * (1.f + sc[i].z) + sh[i].z;
        const float y3 = (v[i].w - mean) * rstd * (1.f + sc[i].w) + sh[i].w;
        store4(orow + c, y0, y1, y2, y3);
      }
  }
}

template <typename TO>
void launch_ln(void *out, int ldo, const float *x, int ldx, int rows, int row0, int d, float eps,
               const float *const m[3], Segs sg, hipStream_t s, float *out_scale) {
  k_ln_modulate<TO><<<rows, 256, 0, s>>>((TO *)out, ldo, x, ldx, row0, d, eps, m[0], m[1], m[2],
                                          sg.b1, sg.b2, sg.per, out_scale);
}

hipError_t ln_modulate(void *out, int out_type, int ldo, const float *x, int ldx, int rows,
                       int row0, int d, float eps, const float *const mod_seg[3], Segs segs,
                       hipStream_t s, float *out_scale) {
  if (rows <= 0) return hipSuccess;
  if (d % 256 || d > 256 * 4 * kLnMaxVec) return hipErrorInvalidValue;
  switch (out_type) {
    case OP_F32: launch_ln<float>(out, ldo, x, ldx, rows, row0, d, eps, mod_seg, segs, s, nullptr); break;
    case OP_BF16: launch_ln<bf16>(out, ldo, x, ldx, rows, row0, d, eps, mod_seg, segs, s, nullptr); break;
    case OP_F16: launch_ln<f16>(out, ldo, x, ldx, rows, row0, d, eps, mod_seg, segs, s, nullptr); break;
    case OP_FP8:
      if (!out_scale || ldo % 4) return hipErrorInvalidValue;
      launch_ln<uint8_t>(out, ldo, x, ldx, rows, row0, d, eps, mod_seg, segs, s, out_scale);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Queries and keys: RMSNorm over the 128 dims of each head with the weight set's learned
// scale ("FLUX.3 Image Klein in Diffusers", "Entkoppelte Vorverarbeitung ...": queries and
// keys are RMS-normalised before attention), then the 4D rotary embedding: lane p rotates
// the adjacent pair (2p, 2p+1) by the angle of axis p/16, frequency index p%16.
// The fp32 path runs this kernel; the 16-bit and FP8 paths do the same work in linear1's
// epilogue (gemm_common.h), which also writes V transposed for the attention kernel.
// Grid: (ceil(n/64) token tiles, heads); 4 waves, each 16 tokens of the tile.
// ------------------------------------------------------------------------------------------
template <typename T> struct Pair;
template <> struct Pair<float> {
  typedef float2 type;
  static __device__ float lo(float2 v) { return v.x; }
  static __device__ float hi(float2 v) { return v.y; }
  static __device__ float2 make(float a, float b) { return make_float2(a, b); }
};
template <typename T>
__global__ __launch_bounds__(256) void k_qk_norm_rope(T *qkv, int ldq, int d_model,
                                                       const float *cs, int n,
                                                       const float *qn0, const float *qn1,
                                                       const float *qn2, const float *kn0,
                                                       const float *kn1, const float *kn2,
                                                       int b1, int b2, int per, float eps) {
  typedef typename Pair<T>::type P2;
  int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int h = blockIdx.y;
  int t0 = blockIdx.x * 64;
  for (int i = 0; i < 16; ++i) {
    int tok = t0 + wave * 16 + i;
    if (tok >= n) break;
    int seg = segment_of(tok, b1, b2, per);
    const float *qn = seg == 0 ? qn0 : (seg == 1 ? qn1 : qn2);
    const float *kn = seg == 0 ? kn0 : (seg == 1 ? kn1 : kn2);
    T *qp = qkv + (size_t)tok * ldq + h * 128 + 2 * lane;
    T *kp = qp + d_model;
    P2 qv = *reinterpret_cast<const P2 *>(qp);
    P2 kv = *reinterpret_cast<const P2 *>(kp);
    float q0 = Pair<T>::lo(qv), q1 = Pair<T>::hi(qv);
    float k0 = Pair<T>::lo(kv), k1 = Pair<T>::hi(kv);
    float qs = wave_sum(q0 * q0 + q1 * q1);
    float ks = wave_sum(k0 * k0 + k1 * k1);
    float rq = 1.0f / sqrtf(qs * (1.0f / 128.f) + eps);
    float rk = 1.0f / sqrtf(ks * (1.0f / 128.f) + eps);
    float2 wq = *reinterpret_cast<const float2 *>(qn + 2 * lane);
    float2 wk = *reinterpret_cast<const float2 *>(kn + 2 * lane);
    q0 *= rq * wq.x;
    q1 *= rq * wq.y;
    k0 *= rk * wk.x;
    k1 *= rk * wk.y;
    float2 c = *reinterpret_cast<const float2 *>(cs + (size_t)tok * 128 + 2 * lane);
    *reinterpret_cast<P2 *>(qp) = Pair<T>::make(q0 * c.x - q1 * c.y, q0 * c.y + q1 * c.x);
    *reinterpret_cast<P2 *>(kp) = Pair<T>::make(k0 * c.x - k1 * c.y, k0 * c.y + k1 * c.x);
  }
}

hipError_t qk_norm_rope(void *qkv, int type, int ldq, int d_model, int heads,
                        const float *cs, int n, const float *const qn[3],
                        const float *const kn[3], Segs segs, float eps, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  switch (type) {
    case OP_F32:
      k_qk_norm_rope<float><<<dim3((n + 63) / 64, heads), 256, 0, s>>>(
          (float *)qkv, ldq, d_model, cs, n, qn[0], qn[1], qn[2], kn[0], kn[1], kn[2],
          segs.b1, segs.b2, segs.per, eps);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// GEMV for the conditioning path: y[v][i] = sum_k W[i][k] * act(x[v][k]), act = SiLU or
// identity.  Used for the timestep MLP and for mod = W_mod . SiLU(cond) ("FLUX.3 Image Klein
// in Diffusers", "Modulation pro Token-Typ ...": scale, shift and gate come from the
// timestep embedding).  8 rows per workgroup, k sliced over its 256 threads.
// ------------------------------------------------------------------------------------------
// Eight consecutive weights as raw registers (16-bit: one 16-byte load; fp32: two) and their
// conversion to floats.
template <typename TW> struct Load16;
template <> struct Load16<bf16> {
  typedef u32x4 raw;
  static __device__ __forceinline__ raw load(const bf16 *p) { return *reinterpret_cast<const u32x4 *>(p); }
  static __device__ __forceinline__ void unpack(float (&o)[8], const raw &v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = __uint_as_float(u[e] << 16);
      o[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  }
};
template <> struct Load16<f16> {
  typedef _Float16 raw __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ raw load(const f16 *p) { return *reinterpret_cast<const raw *>(p); }
  static __device__ __forceinline__ void unpack(float (&o)[8], const raw &v) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
  }
};
struct F32x8 {
  f32x4 a, b;
};
template <> struct Load16<float> {
  typedef F32x8 raw;
  static __device__ __forceinline__ raw load(const float *p) {
    return F32x8{*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 4)};
  }
  static __device__ __forceinline__ void unpack(float (&o)[8], const raw &v) {
    o[0] = v.a.x; o[1] = v.a.y; o[2] = v.a.z; o[3] = v.a.w;
    o[4] = v.b.x; o[5] = v.b.y; o[6] = v.b.z; o[7] = v.b.w;
  }
};

// GEMV over up to 3 vectors, bound by streaming the weights once.  k-sliced: thread t owns
// the 16-byte pieces t and t + 256 of every row (k <= 4096), so it loads the (activated)
// vector values of its pieces once, into registers, and reuses them for the workgroup's
// kGemvRows rows, whose weight loads it issues first.  Each (row, vector) sum is then reduced
// over the workgroup: three halving exchanges inside each wave (a lane keeps half of its sums
// and adds its partner's), a butterfly over the remaining 8 lanes, then the 4 waves' partial
// sums in a fixed order through LDS.
constexpr int kGemvRows = 8;              // rows per workgroup
constexpr int kGemvSums = 3 * kGemvRows;  // (row, vector) sums per thread
static_assert(kGemvSums % 8 == 0, "three halving exchanges");

template <int N>
__device__ __forceinline__ void halve(const float (&in)[2 * N], float (&out)[N], int lane, int offset) {
  const bool up = lane & offset;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float keep = up ? in[i + N] : in[i], send = up ? in[i] : in[i + N];
    out[i] = keep + __shfl_xor(send, offset, kWave);
  }
}

template <typename TW, bool SILU>
__global__ __launch_bounds__(256) void k_gemv(float *y, const TW *w, int rows, int k,
                                               const float *x, int nvec, int ldy) {
  constexpr int NS = kGemvSums;
  __shared__ float red[4][NS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row0 = blockIdx.x * kGemvRows;
  const int np = k >> 3;  // 16-byte pieces per row
  typedef typename Load16<TW>::raw Raw;
  Raw raw[kGemvRows][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = t + 256 * j;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
      if (p < np && row0 + r < rows) raw[r][j] = Load16<TW>::load(w + (size_t)(row0 + r) * k + 8 * p);
  }
  float xv[2][3][8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = t + 256 * j;
#pragma unroll
    for (int v = 0; v < 3; ++v) {
      f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
      if (p < np && v < nvec) {
        lo = *reinterpret_cast<const f32x4 *>(x + v * k + 8 * p);
        hi = *reinterpret_cast<const f32x4 *>(x + v * k + 8 * p + 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[j][v][e] = SILU ? silu(lo[e]) : lo[e];
        xv[j][v][4 + e] = SILU ? silu(hi[e]) : hi[e];
      }
    }
  }
  float acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (t + 256 * j >= np) continue;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      if (row0 + r >= rows) continue;
      float wv[8];
      Load16<TW>::unpack(wv, raw[r][j]);
#pragma unroll
      for (int v = 0; v < 3; ++v) {
        const float *xx = xv[j][v];
        acc[r * 3 + v] += ((wv[0] * xx[0] + wv[1] * xx[1]) + (wv[2] * xx[2] + wv[3] * xx[3])) +
                          ((wv[4] * xx[4] + wv[5] * xx[5]) + (wv[6] * xx[6] + wv[7] * xx[7]));
      }
    }
  }
  // after the halvings, lane group g = lane / 8 holds sums b5 * NS/2 + b4 * NS/4 + b3 * NS/8 + i
  // (b5 b4 b3 the bits of g); the butterfly completes them over the group's 8 lanes
  float h1[NS / 2], h2[NS / 4], h3[NS / 8];
  halve<NS / 2>(acc, h1, lane, 32);
  halve<NS / 4>(h1, h2, lane, 16);
  halve<NS / 8>(h2, h3, lane, 8);
#pragma unroll
  for (int i = 0; i < NS / 8; ++i)
#pragma unroll
    for (int o = 4; o >= 1; o >>= 1) h3[i] += __shfl_xor(h3[i], o, kWave);
  if ((lane & 7) == 0) {
    const int g = lane >> 3;
    const int base = ((g >> 2) & 1) * (NS / 2) + ((g >> 1) & 1) * (NS / 4) + (g & 1) * (NS / 8);
#pragma unroll
    for (int i = 0; i < NS / 8; ++i) red[wave][base + i] = h3[i];
  }
  __syncthreads();
  if (t < NS) {
    const int r = t / 3, v = t - 3 * r;
    if (v < nvec && row0 + r < rows)
      y[(size_t)v * ldy + row0 + r] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
  }
}

template <typename TW>
hipError_t launch_gemv(float *y, const TW *w, int rows, int k, const float *x, int nvec,
                       int silu_in, hipStream_t s, int ldy) {
  const dim3 grid((rows + kGemvRows - 1) / kGemvRows);
  if (silu_in)
    k_gemv<TW, true><<<grid, 256, 0, s>>>(y, w, rows, k, x, nvec, ldy);
  else
    k_gemv<TW, false><<<grid, 256, 0, s>>>(y, w, rows, k, x, nvec, ldy);
  return hipGetLastError();
}

hipError_t gemv(float *y, const void *w, int w_type, int rows, int k, const float *x, int nvec,
                int silu_in, hipStream_t s, int ldy) {
  if (nvec < 1 || nvec > 3 || k % 8 || k > 4096) return hipErrorInvalidValue;
  if (ldy == 0) ldy = rows;
  if (ldy < rows) return hipErrorInvalidValue;
  switch (w_type) {
    case OP_BF16: return launch_gemv(y, (const bf16 *)w, rows, k, x, nvec, silu_in, s, ldy);
    case OP_F16: return launch_gemv(y, (const f16 *)w, rows, k, x, nvec, silu_in, s, ldy);
    case OP_F32: return launch_gemv(y, (const float *)w, rows, k, x, nvec, silu_in, s, ldy);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------
// Row-wise E4M3 quantization: one 256-thread workgroup per row, which it reads once into
// registers (8 values per thread and step, up to kQuantSteps steps: 16384 columns); the codes
// are v * (448 / max |v|) rounded to E4M3, the row's dequantization scale max |v| / 448.  A
// row of zeros gets scale 0 and codes 0.
// ------------------------------------------------------------------------------------------
constexpr int kQuantSteps = 8;

template <typename TS>
__global__ __launch_bounds__(256) void k_quant_rows(uint8_t *q, int ldq, float *scale,
                                                    const TS *src, int lds, int cols) {
  __shared__ float red[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const TS *row = src + (size_t)r * lds;
  float v[kQuantSteps][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kQuantSteps; ++i) {
    const int c = (i * 256 + t) * 8;
    if (c < cols) {
      typename Load16<TS>::raw raw = Load16<TS>::load(row + c);
      Load16<TS>::unpack(v[i], raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (t == 0) scale[r] = amax / 448.0f;
  const float rcp = amax > 0.f ? 448.0f / amax : 0.f;
  uint8_t *qr = q + (size_t)r * ldq;
#pragma unroll
  for (int i = 0; i < kQuantSteps; ++i) {
    const int c = (i * 256 + t) * 8;
    if (c < cols)
      *reinterpret_cast<uint2 *>(qr + c) =
          make_uint2(e4m3_pack4(v[i][0] * rcp, v[i][1] * rcp, v[i][2] * rcp, v[i][3] * rcp),
                     e4m3_pack4(v[i][4] * rcp, v[i][5] * rcp, v[i][6] * rcp, v[i][7] * rcp));
  }
}

hipError_t quant_rows_fp8(uint8_t *q, int ldq, float *scale, const void *src, int src_type, int lds,
                          int rows, int cols, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cols % 8 || ldq % 8 || lds % 8 || cols > 256 * 8 * kQuantSteps) return hipErrorInvalidValue;
  switch (src_type) {
    case OP_F32: k_quant_rows<float><<<rows, 256, 0, s>>>(q, ldq, scale, (const float *)src, lds, cols); break;
    case OP_BF16: k_quant_rows<bf16><<<rows, 256, 0, s>>>(q, ldq, scale, (const bf16 *)src, lds, cols); break;
    case OP_F16: k_quant_rows<f16><<<rows, 256, 0, s>>>(q, ldq, scale, (const f16 *)src, lds, cols); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// fp32 -> 16-bit rounding of a contiguous array (four elements per thread).
template <typename T>
__global__ void k_to_half(T *dst, const float *src, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(src + i);
    store4(dst + i, v.x, v.y, v.z, v.w);
  } else {
    for (int64_t j = i; j < n; ++j) dst[j] = from_f32<T>(src[j]);
  }
}

hipError_t to_half(void *dst, int type, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (type == OP_BF16) k_to_half<bf16><<<blocks, 256, 0, s>>>((bf16 *)dst, src, n);
  else if (type == OP_F16) k_to_half<f16><<<blocks, 256, 0, s>>>((f16 *)dst, src, n);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Sinusoidal timestep embedding (reading: the Transformer / DiT sinusoid with time factor
// 1000 and max period 10000), in fp64: e = [cos(1000 t f_j) | sin(1000 t f_j)].
struct TVals {
  double t[4];
};
__global__ void k_timestep_embed(float *e, TVals tv, int nvec, int dim) {
  int j = blockIdx.x * blockDim.x + threadIdx.x;
  int half = dim / 2;
  if (j >= nvec * dim) return;
  int v = j / dim, c = j % dim;
  int idx = c < half ? c : c - half;
  double f = exp(-log(10000.0) * (double)idx / (double)half);
  double arg = 1000.0 * tv.t[v] * f;
  e[j] = (float)(c < half ? cos(arg) : sin(arg));
}

hipError_t timestep_embed(float *e, const double *t_host, int nvec, int dim, hipStream_t s) {
  if (nvec < 1 || nvec > 4) return hipErrorInvalidValue;
  TVals tv = {{0.0, 0.0, 0.0, 0.0}};
  for (int i = 0; i < nvec; ++i) tv.t[i] = t_host[i];
  int tot = nvec * dim;
  k_timestep_embed<<<(tot + 255) / 256, 256, 0, s>>>(e, tv, nvec, dim);
  return hipGetLastError();
}

__global__ void k_copy_rows(float *dst, int ldd, const float *src, int lds, int rows, int cols) {
  int r = blockIdx.y;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < cols; c += gridDim.x * blockDim.x)
    dst[(size_t)r * ldd + c] = src[(size_t)r * lds + c];
}

hipError_t copy_rows_f32(float *dst, int ldd, const float *src, int lds, int rows, int cols,
                         hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  k_copy_rows<<<dim3(4, rows), 256, 0, s>>>(dst, ldd, src, lds, rows, cols);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Seeded N(0,1) noise: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with counter
// (element / 4, 0, 0) and key (seed low, seed high) words, then Box-Muller on the pairs
// (x0, x1) and (x2, x3); uniforms u = (x + 0.5) / 2^32.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k[0];
  uint32_t n1 = (uint32_t)p1;
  uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k[1];
  uint32_t n3 = (uint32_t)p0;
  c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

__global__ void k_philox_normal(float *dst, int64_t n, uint64_t seed) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 4 elements
  if (g * 4 >= n) return;
  uint32_t c[4] = {(uint32_t)g, (uint32_t)((uint64_t)g >> 32), 0u, 0u};
  uint32_t k[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(c, k);
  }
  const double inv = 1.0 / 4294967296.0;
  double out[4];
  for (int p = 0; p < 2; ++p) {
    double u0 = ((double)c[2 * p] + 0.5) * inv;
    double u1 = ((double)c[2 * p + 1] + 0.5) * inv;
    double rad = sqrt(-2.0 * log(u0));
    double sn, cn;
    sincospi(2.0 * u1, &sn, &cn);
    out[2 * p] = rad * cn;
    out[2 * p + 1] = rad * sn;
  }
  for (int e = 0; e < 4; ++e)
    if (g * 4 + e < n) dst[g * 4 + e] = (float)out[e];
}

__global__ void k_noise_mix(float *x, const float *noise, int64_t n, float t) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = t * noise[i] + (1.0f - t) * x[i];
}

hipError_t noise_mix(float *x, const float *noise, int64_t n, float t, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_noise_mix<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, noise, n, t);
  return hipGetLastError();
}

__global__ void k_add_row(float *y, int nrows, int d, const float *v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d) return;
  const float a = v[i];
  for (int r = 0; r < nrows; ++r) y[(size_t)r * d + i] += a;
}

hipError_t add_row(float *y, int nrows, int d, const float *v, hipStream_t s) {
  if (nrows <= 0 || d <= 0) return hipSuccess;
  k_add_row<<<(d + 255) / 256, 256, 0, s>>>(y, nrows, d, v);
  return hipGetLastError();
}

// Debug guard: over rows x cols of a buffer (row stride ld), cnt[0] += fp16 values at the limit
// +-65504 (where the saturating conversion puts out-of-range values, and NaN), cnt[1] += NaN or
// infinite values.  A grid-stride loop; one atomic per wave.
template <typename T>
__global__ void k_count_nonfinite(const T *p, int rows, int cols, int ld, unsigned *cnt) {
  unsigned sat = 0, bad = 0;
  const int64_t total = (int64_t)rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i - r * cols;
    const float v = to_f32(p[r * ld + c]);
    if (!__builtin_isfinite(v)) ++bad;
    else if (std::is_same<T, f16>::value && fabsf(v) >= 65504.f) ++sat;
  }
  for (int o = 32; o > 0; o >>= 1) {
    sat += __shfl_xor(sat, o, kWave);
    bad += __shfl_xor(bad, o, kWave);
  }
  if ((threadIdx.x & 63) == 0 && (sat | bad)) {
    atomicAdd(cnt, sat);
    atomicAdd(cnt + 1, bad);
  }
}

hipError_t count_nonfinite(unsigned *cnt, const void *p, int type, int rows, int cols, int ld,
                           hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t total = (int64_t)rows * cols;
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
  switch (type) {
    case OP_F32: k_count_nonfinite<float><<<blocks, 256, 0, s>>>((const float *)p, rows, cols, ld, cnt); break;
    case OP_BF16: k_count_nonfinite<bf16><<<blocks, 256, 0, s>>>((const bf16 *)p, rows, cols, ld, cnt); break;
    case OP_F16: k_count_nonfinite<f16><<<blocks, 256, 0, s>>>((const f16 *)p, rows, cols, ld, cnt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t philox_normal(float *dst, int64_t n, uint64_t seed, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t groups = (n + 3) / 4;
  k_philox_normal<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(dst, n, seed);
  return hipGetLastError();
}

}  // namespace dit
