// Launchers of the gfx950 kernels (internal to the library; the C ABI is include/dit.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Element types of activations / weights (same codes as the C ABI's compute types).
enum ElemType { OP_F32 = 0, OP_BF16 = 1, OP_F16 = 2 };
// Row-wise OCP E4M3 codes (one byte per value) with one fp32 scale per row.
constexpr int OP_FP8 = 3;

// Token rows: one or two sequences of per rows each (the conditional and unconditional
// branches of classifier-free guidance), each ordered text [0, b1) | image [b1, b2) |
// reference [b2, per); n = rows in total.  A row's segment is that of its offset in its
// sequence.
struct Segs {
  int b1, b2, n, per;
};
// Most row groups of one GEMM or attention launch: three segments of two sequences.
constexpr int kMaxGroups = 6;

// --- GEMM row groups: up to three row ranges, each with its own input rows and weights.
struct GemmGroup {
  const void *x;   // first input row of the group (row stride ldx elements)
  const void *w;   // weights [N, K] row-major
  int rows;        // rows in the group
  int out_row0;    // token index of the first row (output row; segment lookup)
  const float *ws = nullptr;  // FP8 GEMM: scale of each weight row (output feature)
};

enum Epilogue {
  EPI_STORE_F32 = 0,   // out[r][n] = acc  or  out[r][n] += alpha * acc
  EPI_QKV_SWIGLU = 1,  // cols < split -> qkv; cols >= split (gate/up interleaved by 32) -> SiLU(g)*u
  EPI_RESID = 2,       // x[r][n] += gate_seg(r)[n] * acc
};

struct GemmArgs {
  GemmGroup g[kMaxGroups];
  int ng;
  int n, k;            // output columns, reduction length
  int ldx;             // input row stride (elements)
  int ldw;             // weight row stride (elements); 0: k
  // EPI_STORE_F32: accumulate 0: out = acc, 1: out += alpha * acc, 2: out = alpha * acc
  // (columns >= n_store are computed but not stored when n_store > 0)
  float *out; int ldo; int accumulate; float alpha; int n_store;
  // EPI_QKV_SWIGLU
  void *qkv; int ldq; int split; void *cat; int ldc; int cat_off;
  // EPI_QKV_SWIGLU, 16-bit and FP8 GEMMs, when vt != nullptr (split = 3 x 128-dim heads of
  // d_model = split / 3 each, and split % 256 == 0): each Q and K head is RMS-normalised with
  // the weights qn / kn of its token's segment (segments by b1, b2, per below) and rotated by
  // the 4D RoPE angles pos[token][axis] * freq_j, axis = pair / 16, j = pair % 16, then stored
  // to qkv; rope_fr holds freq_j / (2 pi) split as hi[16] (12 significant bits, so that an
  // integer position up to 4096 times hi is exact in fp32) then lo[16] = the remainder.
  // V is not stored to qkv but written transposed to vt [head][128][ldv] (the attention's
  // layout: in every 32 tokens, 16-byte chunk q holds tokens 4q..4q+3 and 16+4q..16+4q+3),
  // with zeros for the tokens in [n_tok, (n_tok / 64 + 2) * 64).
  void *vt; int ldv; int n_tok; const float *rope_pos; const float *rope_fr;
  const float *qn[3]; const float *kn[3]; float rms_eps;
  // EPI_RESID (b1, b2, per also give the segments of the fused Q / K norm)
  float *x; int ldres; const float *gate[3]; int b1, b2, per;
  // Split K (EPI_RESID and EPI_STORE_F32): when the tiles fill under half of split_grid
  // compute units and k is long, each tile's k-tiles are cut into S slices; every slice stores
  // its fp32 partial tile to part (room for part_tiles tiles of 256 x 256), and a second kernel
  // adds the slices in slice order and applies the epilogue.  split_grid = 0: never.
  float *part; int part_tiles; int split_grid;
  // Compute units of the device (EPI_RESID on the 16-bit GEMM: picks 224-row token tiles when
  // they fill the device in fewer tile-heights; 0: always 256-row tiles)
  int cus;
  // FP8 GEMM: scale of each input row, indexed by token (out_row0 + row)
  const float *xs;
};
// floats per 256 x 256 partial tile of the split-K GEMM
constexpr int gemm_part_floats = 256 * 256;

// MFMA GEMM: input and weights of 16-bit type op (OP_BF16 / OP_F16), fp32 accumulation.
// n % 256 == 0, k % 64 == 0, input rows readable up to 256 past each group's end.
hipError_t gemm_mfma(const GemmArgs &a, int epi, int op, hipStream_t s);
// Row-wise FP8 GEMM: E4M3 inputs and weights (ldx, ldw, k in bytes), out = xs[token] *
// ws[feature] * acc, then the epilogue (16-bit stores are fp16).  n % 256 == 0, k % 128 == 0,
// ldx and the weight row stride multiples of 16.
hipError_t gemm_fp8(const GemmArgs &a, int epi, hipStream_t s);
// q[r][c] = E4M3 code of src[r][c] * (448 / max_c |src[r][c]|), scale[r] = max_c |src[r][c]| / 448
// (fp32), for r < rows, c < cols; src of type src_type (OP_F32 / OP_BF16 / OP_F16);
// cols % 8 == 0, cols <= 16384.
hipError_t quant_rows_fp8(uint8_t *q, int ldq, float *scale, const void *src, int src_type, int lds,
                          int rows, int cols, hipStream_t s);
// fp32-accumulating general GEMM with fp32 inputs and weights of type w_type.
// n % 64 == 0, k % 16 == 0; any rows; input rows are not read past a group's end.
hipError_t gemm_simple(const GemmArgs &a, int epi, int w_type, hipStream_t s);

// --- attention
struct AttnGroup {
  int q0, q1, k0, k1;  // query rows [q0, q1) attend keys [k0, k1)
};
struct AttnArgs {
  const void *qkv; int ldqkv; int d_model;  // q at column h*128, k at d_model + h*128
  const void *vt; int ldv;                  // MFMA path: V transposed [heads][128][ldv]
  void *out; int ldo;                       // out[q][h*128 + d]
  AttnGroup g[kMaxGroups]; int ng;
  int heads;
  float scale;                              // 1/sqrt(head_dim)
  // MFMA path load balance: when one workgroup per (head, 256-query) unit would leave part
  // of the last round of lean_grid workgroups idle, lean_grid workgroups take equal shares of
  // the key-tile iterations, and units cut between shares merge through part (2 * lean_grid
  // slots of attn_part_floats) and cnt (one zeroed int per unit, left zeroed).  lean_grid = 0
  // or part = nullptr: one workgroup per unit.
  float *part; int *cnt; int lean_grid;
};
// floats per partial slot of the MFMA attention
constexpr int attn_part_floats = 8 * 16 * 64 * 4 + 8 * 64 * 4;
hipError_t attention_mfma(const AttnArgs &a, int op, hipStream_t s);
hipError_t attention_f32(const AttnArgs &a, hipStream_t s);  // V read from qkv at 2*d_model

// --- norms, RoPE, small ops
// Reference images per call: the model takes up to ten (we0.ai "FLUX 3 Image Klein" article,
// model summary).
constexpr int kMaxRefs = 10;
// pos [n_txt + gh*gw + sum of reference tokens][4]; ref_grids host [n_refs][2] (rows, cols)
hipError_t fill_positions(float *pos, int n_txt, int gh, int gw, const int *ref_grids,
                          int n_refs, hipStream_t s);
hipError_t rope_table(float *cs, const float *pos, int n, float theta, hipStream_t s);
// out[r] = LN(x[r]) * (1 + scale_seg) + shift_seg, mod_seg[s] = [shift | scale | ...]
// out_type OP_FP8: E4M3 codes with the row scales in out_scale[r] (row-wise quantization of
// the modulated row).
hipError_t ln_modulate(void *out, int out_type, int ldo, const float *x, int ldx, int rows,
                       int row0, int d, float eps, const float *const mod_seg[3], Segs segs,
                       hipStream_t s, float *out_scale = nullptr);
// q, k of every (token, head): RMSNorm with the segment's scale, then RoPE, in place (fp32
// path; the 16-bit and FP8 paths fuse this into linear1's epilogue).
hipError_t qk_norm_rope(void *qkv, int type, int ldq, int d_model, int heads,
                        const float *cs, int n, const float *const qn[3],
                        const float *const kn[3], Segs segs, float eps, hipStream_t s);
// dst[i] = src[i] rounded to the 16-bit type (OP_BF16 / OP_F16), i < n
hipError_t to_half(void *dst, int type, const float *src, int64_t n, hipStream_t s);
// y[v * ldy + i] = sum_k W[i][k] * act(x[v][k]) for v < nvec (x contiguous [nvec][k];
// ldy 0: rows).  silu_in: act = SiLU (applied as the vectors are loaded), else identity
hipError_t gemv(float *y, const void *w, int w_type, int rows, int k, const float *x, int nvec,
                int silu_in, hipStream_t s, int ldy = 0);
// e[v] = [cos(1000 t_v f_j), sin(1000 t_v f_j)], f_j = 10000^(-j/(dim/2)), 1 <= nvec <= 4
hipError_t timestep_embed(float *e, const double *t_host, int nvec, int dim, hipStream_t s);
hipError_t copy_rows_f32(float *dst, int ldd, const float *src, int lds, int rows, int cols,
                         hipStream_t s);
hipError_t philox_normal(float *dst, int64_t n, uint64_t seed, hipStream_t s);
// x = t * noise + (1 - t) * x  (the straight path from clean latents to noise)
hipError_t noise_mix(float *x, const float *noise, int64_t n, float t, hipStream_t s);
// y[r][:] += v for rows r < nrows of d floats
hipError_t add_row(float *y, int nrows, int d, const float *v, hipStream_t s);
// Sustained MFMA rate probe: blocks workgroups of 4 waves each run iters x 8 independent
// 16x16x32 MFMAs of type op (OP_F16 / OP_BF16) (sink [blocks] is written only in a case that
// never occurs).
hipError_t mfma_rate(int op, int blocks, int iters, float *sink, hipStream_t s);
double mfma_rate_flops(int blocks, int iters);
// Debug guard: cnt[0] += values of the rows x cols buffer p (row stride ld, element type
// OP_F32 / OP_BF16 / OP_F16) at the fp16 limit +-65504 (fp16 only), cnt[1] += NaN / Inf values.
hipError_t count_nonfinite(unsigned *cnt, const void *p, int type, int rows, int cols, int ld,
                           hipStream_t s);

}  // namespace dit
