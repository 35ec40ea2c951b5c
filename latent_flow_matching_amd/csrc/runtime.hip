// Runtime of the denoising-transformer library: context, weight upload and repack,
// workspace, the per-block launch sequence and the C ABI declared in include/dit.h.
//
// Launch sequence of one block (all on the caller's stream):
//   ln_modulate      x (fp32) -> xm                 LayerNorm + adaLN (shift, scale)
//   linear1          xm . W1^T -> qkv, V^T,         fused QKV (with QK RMSNorm + 4D RoPE and
//                    cat[:, D:]                     the V transpose) + SwiGLU epilogue
//   qk_norm_rope     qkv in place                   QK RMSNorm + 4D RoPE (fp32 path only)
//   attention        qkv, V^T -> cat[:, :D]         softmax attention (full or per stream)
//   linear2          cat . W2^T -> x += gate * .    gated residual
// Stream blocks (double / per-mode) run the two projections as row groups with one weight
// set per stream; shared blocks (single / joint) use one set for all rows.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "dit.h"
#include "kernels.h"

using namespace dit;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

}  // namespace

struct dit_ctx {
  dit_config cfg;
  int device = 0;
  int op = OP_BF16;          // element type of MFMA operands, activations and weights
  bool fp8 = false;          // DIT_FP8: block projections on E4M3 (op is OP_F16 for the rest)
  bool debug_sync = false;
  std::vector<void *> allocs;

  struct Set {
    void *w1 = nullptr, *w2 = nullptr;   // compute type, or E4M3 codes with DIT_FP8
    float *qn = nullptr, *kn = nullptr;
    float *s1 = nullptr, *s2 = nullptr;  // DIT_FP8: one scale per row of w1, w2
  };
  std::vector<std::vector<Set>> blk;
  // Modulation projections: the distinct device tensors (weight-table entries that name the
  // same host data share one), their row counts, and which one serves each (block, set).
  std::vector<void *> modw;
  std::vector<int> modw_rows;
  std::vector<std::vector<int>> mod_of;
  void *img_in = nullptr, *temb1 = nullptr, *temb2 = nullptr, *fmod = nullptr, *fout = nullptr;
  void *fout_pad = nullptr;  // 16-bit paths: final.out with zero rows up to a multiple of 256
  void *ttgt1 = nullptr, *ttgt2 = nullptr;  // flow-map target-time MLP
  void *txt_in = nullptr;                   // [D][txt_feat_dim] text-feature projection

  int rows_alloc = 0, ldv = 0;
  float *x = nullptr;        // [rows_alloc][D] residual of dit_forward / dit_denoise
  void *xm = nullptr;        // [rows_alloc][D]
  void *qkv = nullptr;       // [rows_alloc][3D]
  void *cat = nullptr;       // [rows_alloc][D+F]
  void *vt = nullptr;        // [H][128][ldv] (16-bit paths)
  float *pos = nullptr;      // [rows_alloc][4]
  const float *rope_pos = nullptr;  // positions of the call in flight (pos, or the caller's)
  float *rope_fr = nullptr;  // [32]: RoPE frequency / (2 pi), 12-bit high parts then remainders
  float *cs = nullptr;       // [rows_alloc][128]
  float *modbuf = nullptr;   // [modw.size()][3][mod_ld()]: one vector per cond row
  float *cond = nullptr;     // [3][D]
  float *temb_e = nullptr;   // [4][time_dim]: the three segment times, then the target time
  float *temb_h = nullptr;   // [4][D]
  float *tgt = nullptr;      // [D] target-time embedding (flow-map models)
  float *noise = nullptr;    // [max_tokens][C] image-to-image noise drawn from a seed
  float *fmodv = nullptr;    // [3][2D]
  float *xf = nullptr;       // fp32 path: [max_tokens][D] final-norm output
  int cus = 0;               // compute units, rounded down to a multiple of 8
  int lean_grid = 0;         // attention: one workgroup per compute unit (multiple of 8)
  float *attn_part = nullptr;  // [2 * lean_grid][attn_part_floats] partial pieces
  int *attn_cnt = nullptr;     // [heads * (max_tokens / 256 + 6)] per-unit piece counters
  float *gemm_part = nullptr;  // [cus][gemm_part_floats] split-K partial tiles
  unsigned *guard_cnt = nullptr;  // DIT_DEBUG_SYNC guard: (values at the fp16 limit, NaN/Inf)
  // DIT_FP8 workspace: E4M3 copy of cat, row scales of xm (codes in xm) and of cat's halves
  uint8_t *cat8 = nullptr;     // [rows_alloc][D+F]
  float *xs = nullptr, *cs_a = nullptr, *cs_b = nullptr;  // [rows_alloc] each

  // per-kernel timing: hipEvents recorded on the call's stream around each launch
  struct ProfRec {
    int cls;
    double flops, bytes;
    int e0, e1;
  };
  bool prof_on = false;
  unsigned prof_mask = ~0u;  // kernel classes that record events (bit per class)
  std::vector<hipEvent_t> prof_ev;
  std::vector<ProfRec> prof_rec;
  int prof_next = 0;

  int D() const { return cfg.hidden; }
  // lets a GEMM cut long k into slices when its tiles fill too few compute units
  void split_k(GemmArgs *a) const {
    a->part = gemm_part;
    a->part_tiles = gemm_part ? cus : 0;
    a->split_grid = gemm_part ? cus : 0;
    a->cus = cus;
  }
  int F() const { return cfg.mlp_hidden; }
  size_t esz() const { return op == OP_F32 ? 4 : 2; }
  int nblocks() const { return cfg.n_stream_blocks + cfg.n_shared_blocks; }
  int kind(int b) const { return b < cfg.n_stream_blocks ? 0 : 1; }
  void set_of_seg(int k, int out[3]) const {
    if (k == 1) {
      out[0] = out[1] = out[2] = 0;
    } else if (cfg.arch == DIT_FLUX2) {
      out[0] = 0; out[1] = 1; out[2] = 1;   // references travel with the image stream
    } else {
      out[0] = 0; out[1] = 1; out[2] = 2;
    }
  }
  // sequentially wired double blocks carry two (shift, scale, gate) triples per vector
  bool seq_block(int k) const { return k == 0 && cfg.double_wiring; }
  int mod_ld() const { return (cfg.double_wiring ? 6 : 3) * D(); }
  // (shift, scale, gate) of block b's weight set `set` for conditioning row `row`
  float *mod_vec(int b, int set, int row) const {
    return modbuf + ((size_t)mod_of[b][set] * 3 + row) * mod_ld();
  }
};

namespace {

int hip_fail(hipError_t e, const char *what) {
  return fail(DIT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define DIT_CHECK(call, what)                                   \
  do {                                                          \
    hipError_t e_ = (call);                                     \
    if (e_ != hipSuccess) return hip_fail(e_, what);            \
    if (ctx->debug_sync) {                                      \
      e_ = hipStreamSynchronize(stream);                        \
      if (e_ != hipSuccess) return hip_fail(e_, what);          \
    }                                                           \
  } while (0)

enum ProfClass { P_LN, P_LINEAR1, P_QKNORM, P_ATTN, P_LINEAR2, P_COND, P_EMBED, P_FINAL, P_QUANT,
                 P_NCLASS };
const char *const kProfNames[P_NCLASS] = {"ln_modulate", "linear1", "qk_norm_rope", "attention",
                                          "linear2", "conditioning", "embed", "final", "fp8_quant"};

// Start / end markers around one launch when timing is on (no-op otherwise).
int prof_begin(dit_ctx *ctx, int cls, hipStream_t stream) {
  if (!ctx->prof_on || !((ctx->prof_mask >> cls) & 1u) ||
      ctx->prof_next + 2 > (int)ctx->prof_ev.size())
    return -1;
  const int e = ctx->prof_next;
  ctx->prof_next += 2;
  (void)hipEventRecord(ctx->prof_ev[e], stream);
  return e;
}
void prof_end(dit_ctx *ctx, int e, int cls, double flops, double bytes, hipStream_t stream) {
  if (e < 0) return;
  (void)hipEventRecord(ctx->prof_ev[e + 1], stream);
  ctx->prof_rec.push_back(dit_ctx::ProfRec{cls, flops, bytes, e, e + 1});
}

#define DIT_TIMED(cls, flops, bytes, call, what)               \
  do {                                                          \
    const int pe_ = prof_begin(ctx, cls, stream);               \
    DIT_CHECK(call, what);                                      \
    prof_end(ctx, pe_, cls, flops, bytes, stream);              \
  } while (0)

// DIT_DEBUG_SYNC guard, after a launch that wrote rows x cols of p (row stride ld, element type
// type): counts the fp16 values at +-65504 (the saturating conversion puts out-of-range values,
// and NaN, there) and the NaN / Inf values, and fails the call with DIT_ENUMERIC if there are any.
int guard(dit_ctx *ctx, int block, const char *what, const void *p, int type, int rows, int cols,
          int ld, hipStream_t stream) {
  if (!ctx->debug_sync || rows <= 0 || cols <= 0) return 0;
  unsigned h[2] = {0, 0};
  hipError_t e = hipMemsetAsync(ctx->guard_cnt, 0, sizeof h, stream);
  if (e == hipSuccess) e = count_nonfinite(ctx->guard_cnt, p, type, rows, cols, ld, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(h, ctx->guard_cnt, sizeof h, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "debug guard");
  if (h[0] || h[1]) {
    char where[32] = "";
    if (block >= 0) snprintf(where, sizeof where, "block %d, ", block);
    return fail(DIT_ENUMERIC,
                "DIT_DEBUG_SYNC guard: %s%s: %u values at the fp16 limit +-65504 (saturated "
                "conversions, or NaN) and %u NaN/Inf values", where, what, h[0], h[1]);
  }
  return 0;
}

int dalloc(dit_ctx *ctx, void **p, size_t bytes) {
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return fail(DIT_ENOMEM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  }
  ctx->allocs.push_back(*p);
  e = hipMemset(*p, 0, bytes);
  if (e != hipSuccess) return hip_fail(e, "hipMemset");
  return 0;
}

int validate_config(const dit_config *c) {
  if (!c) return fail(DIT_EINVAL, "config is NULL");
  if (c->arch != DIT_FLUX2 && c->arch != DIT_FLUX3) return fail(DIT_EINVAL, "unknown arch %d", c->arch);
  if (c->head_dim != 128)
    return fail(DIT_EUNSUPPORTED, "head_dim must be 128 (four 32-dim RoPE axes), got %d", c->head_dim);
  if (c->heads < 1 || c->hidden != c->heads * c->head_dim)
    return fail(DIT_EINVAL, "hidden (%d) must equal heads (%d) * head_dim", c->hidden, c->heads);
  if (c->hidden % 256 || c->hidden > 4096)
    return fail(DIT_EUNSUPPORTED, "hidden must be a multiple of 256 and at most 4096, got %d", c->hidden);
  if (c->mlp_hidden < 128 || c->mlp_hidden % 128)
    return fail(DIT_EUNSUPPORTED, "mlp_hidden must be a positive multiple of 128, got %d", c->mlp_hidden);
  if (c->in_channels < 16 || c->in_channels % 64)
    return fail(DIT_EUNSUPPORTED, "in_channels must be a positive multiple of 64, got %d", c->in_channels);
  if (c->time_dim < 8 || c->time_dim % 16 || c->time_dim > 4096)
    return fail(DIT_EUNSUPPORTED, "time_dim must be a positive multiple of 16, at most 4096, got %d",
                c->time_dim);
  if (c->n_stream_blocks < 0 || c->n_shared_blocks < 0 || c->n_stream_blocks + c->n_shared_blocks < 1)
    return fail(DIT_EINVAL, "need at least one block");
  if (c->max_tokens < 1 || c->max_tokens > (1 << 20))
    return fail(DIT_EINVAL, "max_tokens out of range: %d", c->max_tokens);
  if (c->compute != DIT_F32 && c->compute != DIT_BF16 && c->compute != DIT_F16 && c->compute != DIT_FP8)
    return fail(DIT_EINVAL, "unknown compute type %d", c->compute);
  if (!(c->rope_theta > 0.f) || !(c->ln_eps > 0.f) || !(c->rms_eps > 0.f))
    return fail(DIT_EINVAL, "rope_theta, ln_eps and rms_eps must be positive");
  if (c->txt_feat_dim < 0 || c->txt_feat_dim % 64 || c->txt_feat_dim > 65536)
    return fail(DIT_EUNSUPPORTED, "txt_feat_dim must be 0 or a multiple of 64 up to 65536, got %d",
                c->txt_feat_dim);
  if (c->flow_map != 0 && c->flow_map != 1) return fail(DIT_EINVAL, "flow_map must be 0 or 1");
  if (c->double_wiring != 0 && c->double_wiring != 1) return fail(DIT_EINVAL, "double_wiring must be 0 or 1");
  if (c->double_wiring && c->arch != DIT_FLUX2)
    return fail(DIT_EUNSUPPORTED, "double_wiring applies to DIT_FLUX2 double blocks only");
  if (c->compute == DIT_FP8 && c->hidden + c->mlp_hidden > 16384)
    return fail(DIT_EUNSUPPORTED, "DIT_FP8 quantizes rows of at most 16384 values (hidden + mlp_hidden = %d)",
                c->hidden + c->mlp_hidden);
  return 0;
}

// Convert host data to the compute type (optionally as fp32 regardless) and upload.
// perm (optional): destination row r takes source row perm[r]; rows of `cols` elements.
// bf16 -> fp16 is exact for magnitudes >= 2^-14; smaller ones round to the fp16 subnormal grid.
int upload(dit_ctx *ctx, void **dst, const dit_tensor &t, bool as_f32,
           const std::vector<int> *perm = nullptr, int cols = 0) {
  const int64_t n = t.numel;
  const int out = as_f32 ? OP_F32 : ctx->op;
  const size_t es = out == OP_F32 ? 4 : 2;
  if (int rc = dalloc(ctx, dst, (size_t)n * es)) return rc;
  const bool same = (t.dtype == DIT_BF16 && out == OP_BF16) || (t.dtype == DIT_F32 && out == OP_F32);
  if (same && !perm) {  // no conversion, no reordering: copy straight from the caller
    hipError_t e = hipMemcpy(*dst, t.data, (size_t)n * es, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "upload");
    return 0;
  }
  std::vector<uint8_t> stage((size_t)n * es);
  if (same) {  // reorder rows only
    const int64_t rows = n / cols;
    for (int64_t r = 0; r < rows; ++r)
      memcpy(stage.data() + (size_t)r * cols * es,
             (const uint8_t *)t.data + (size_t)(*perm)[r] * cols * es, (size_t)cols * es);
  } else {
    auto src_at = [&](int64_t i) -> float {
      return t.dtype == DIT_BF16 ? bf16_to_f32(((const uint16_t *)t.data)[i]) : ((const float *)t.data)[i];
    };
    for (int64_t i = 0; i < n; ++i) {
      int64_t si = i;
      if (perm) si = (int64_t)(*perm)[i / cols] * cols + i % cols;
      const float v = src_at(si);
      if (out == OP_BF16)
        ((uint16_t *)stage.data())[i] = f32_to_bf16_rne(v);
      else if (out == OP_F16)
        ((_Float16 *)stage.data())[i] = (_Float16)v;
      else
        ((float *)stage.data())[i] = v;
    }
  }
  hipError_t e = hipMemcpy(*dst, stage.data(), stage.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "upload");
  return 0;
}

// Row-wise E4M3 copy of a weight [rows][cols] (rows optionally permuted: destination row r
// takes source row perm[r]): the fp32 values go to a temporary device buffer and the
// quantization kernel writes the codes and one scale per row.
int upload_fp8(dit_ctx *ctx, void **codes, float **scales, const dit_tensor &t, int cols,
               const std::vector<int> *perm = nullptr) {
  const int64_t n = t.numel, rows = n / cols;
  std::vector<float> stage((size_t)n);
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t sr = perm ? (*perm)[r] : r;
    for (int64_t c = 0; c < cols; ++c) {
      const int64_t si = sr * cols + c;
      stage[(size_t)(r * cols + c)] = t.dtype == DIT_BF16 ? bf16_to_f32(((const uint16_t *)t.data)[si])
                                                          : ((const float *)t.data)[si];
    }
  }
  if (int rc = dalloc(ctx, codes, (size_t)n)) return rc;
  if (int rc = dalloc(ctx, (void **)scales, (size_t)rows * 4)) return rc;
  float *tmp = nullptr;
  hipError_t e = hipMalloc(&tmp, (size_t)n * 4);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DIT_ENOMEM, "hipMalloc(%zu bytes) failed for weight quantization", (size_t)n * 4);
  }
  e = hipMemcpy(tmp, stage.data(), (size_t)n * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = quant_rows_fp8((uint8_t *)*codes, cols, *scales, tmp, OP_F32, cols, (int)rows, cols, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipFree(tmp);
  if (e != hipSuccess) return hip_fail(e, "weight quantization");
  return 0;
}

}  // namespace

// ------------------------------------------------------------------------------------------
extern "C" const char *dit_get_error(void) { return g_err.c_str(); }

extern "C" void dit_ctx_free(dit_ctx *ctx) {
  if (!ctx) return;
  (void)hipSetDevice(ctx->device);
  (void)hipDeviceSynchronize();
  for (void *p : ctx->allocs) (void)hipFree(p);
  for (hipEvent_t e : ctx->prof_ev) (void)hipEventDestroy(e);
  delete ctx;
}

extern "C" dit_ctx *dit_ctx_create(const dit_config *cfg, const dit_tensor *w, int n_w) {
  g_err.clear();
  if (validate_config(cfg)) return nullptr;
  if (n_w < 0 || (n_w > 0 && !w)) {
    fail(DIT_EINVAL, "weight table is NULL");
    return nullptr;
  }
  const dit_config &c = *cfg;
  const int D = c.hidden, F = c.mlp_hidden, C = c.in_channels, T = c.time_dim;
  // expected tensors
  std::unordered_map<std::string, int64_t> want;
  want["img_in"] = (int64_t)D * C;
  want["temb.l1"] = (int64_t)D * T;
  want["temb.l2"] = (int64_t)D * D;
  want["final.mod"] = (int64_t)2 * D * D;
  want["final.out"] = (int64_t)C * D;
  if (c.flow_map) {
    want["temb_tgt.l1"] = (int64_t)D * T;
    want["temb_tgt.l2"] = (int64_t)D * D;
  }
  if (c.txt_feat_dim > 0) want["txt_in"] = (int64_t)D * c.txt_feat_dim;
  const int nsets0 = c.arch == DIT_FLUX2 ? 2 : 3;
  const int nb = c.n_stream_blocks + c.n_shared_blocks;
  // Modulation: each (block, set) takes its own blk{b}.s{s}.mod, or else the projection its
  // block kind shares, mod.{kind}.s{s}; entries may name the same host data (aliases).
  std::unordered_map<std::string, int64_t> optional;
  auto mod_numel = [&](int kind) { return (int64_t)(kind == 0 && c.double_wiring ? 6 : 3) * D * D; };
  if (c.n_stream_blocks > 0)
    for (int s = 0; s < nsets0; ++s) optional["mod.0.s" + std::to_string(s)] = mod_numel(0);
  if (c.n_shared_blocks > 0) optional["mod.1.s0"] = mod_numel(1);
  for (int b = 0; b < nb; ++b)
    for (int s = 0; s < (b < c.n_stream_blocks ? nsets0 : 1); ++s)
      optional["blk" + std::to_string(b) + ".s" + std::to_string(s) + ".mod"] =
          mod_numel(b < c.n_stream_blocks ? 0 : 1);
  for (int b = 0; b < nb; ++b) {
    const int ns = b < c.n_stream_blocks ? nsets0 : 1;
    for (int s = 0; s < ns; ++s) {
      std::string p = "blk" + std::to_string(b) + ".s" + std::to_string(s);
      want[p + ".w1"] = (int64_t)(3 * D + 2 * F) * D;
      want[p + ".w2"] = (int64_t)D * (D + F);
      want[p + ".qn"] = 128;
      want[p + ".kn"] = 128;
    }
  }
  std::unordered_map<std::string, const dit_tensor *> have;
  for (int i = 0; i < n_w; ++i) {
    if (!w[i].name || !w[i].data) {
      fail(DIT_EINVAL, "weight %d has a NULL name or data pointer", i);
      return nullptr;
    }
    auto it = want.find(w[i].name);
    if (it == want.end()) {
      it = optional.find(w[i].name);
      if (it == optional.end()) {
        fail(DIT_EINVAL, "unknown weight '%s'", w[i].name);
        return nullptr;
      }
    }
    if (have.count(w[i].name)) {
      fail(DIT_EINVAL, "weight '%s' given twice", w[i].name);
      return nullptr;
    }
    if (w[i].numel != it->second) {
      fail(DIT_EINVAL, "weight '%s' has %lld elements, expected %lld", w[i].name,
           (long long)w[i].numel, (long long)it->second);
      return nullptr;
    }
    if (w[i].dtype != DIT_F32 && w[i].dtype != DIT_BF16) {
      fail(DIT_EINVAL, "weight '%s' has unknown dtype %d", w[i].name, w[i].dtype);
      return nullptr;
    }
    have[w[i].name] = &w[i];
  }
  for (auto &kv : want)
    if (!have.count(kv.first)) {
      fail(DIT_EINVAL, "missing weight '%s'", kv.first.c_str());
      return nullptr;
    }
  // the modulation source of every (block, set), and no shared entry left unused
  std::vector<std::vector<const dit_tensor *>> mod_src(nb);
  std::unordered_map<std::string, bool> shared_used;
  for (int b = 0; b < nb; ++b) {
    const int kind = b < c.n_stream_blocks ? 0 : 1;
    for (int s = 0; s < (kind == 0 ? nsets0 : 1); ++s) {
      const std::string own = "blk" + std::to_string(b) + ".s" + std::to_string(s) + ".mod";
      const std::string shared = "mod." + std::to_string(kind) + ".s" + std::to_string(s);
      if (have.count(own)) {
        mod_src[b].push_back(have[own]);
      } else if (have.count(shared)) {
        mod_src[b].push_back(have[shared]);
        shared_used[shared] = true;
      } else {
        fail(DIT_EINVAL, "missing weight '%s' (or the shared '%s')", own.c_str(), shared.c_str());
        return nullptr;
      }
    }
  }
  for (auto &kv : have)
    if (kv.first.rfind("mod.", 0) == 0 && !shared_used.count(kv.first)) {
      fail(DIT_EINVAL, "weight '%s' is used by no block (each has its own blk{b}.s{s}.mod)",
           kv.first.c_str());
      return nullptr;
    }

  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    fail(DIT_EHIP, "no HIP device available (%s)", e == hipSuccess ? "0 devices" : hipGetErrorString(e));
    return nullptr;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    fail(DIT_EHIP, "hipGetDevice failed");
    return nullptr;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    fail(DIT_EHIP, "hipGetDeviceProperties failed");
    return nullptr;
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    fail(DIT_EUNSUPPORTED, "this library is built for gfx950 (MI355X); device is %s", prop.gcnArchName);
    return nullptr;
  }

  dit_ctx *ctx = new dit_ctx();
  ctx->cfg = c;
  ctx->device = dev;
  ctx->fp8 = c.compute == DIT_FP8;
  ctx->op = ctx->fp8 ? OP_F16 : c.compute;  // DIT_F32 / DIT_BF16 / DIT_F16 share the OP_ codes
  ctx->cus = prop.multiProcessorCount / 8 * 8;
  ctx->lean_grid = ctx->cus;
  if (const char *ag = getenv("DIT_ATTN_GRID")) {  // attention share count (0: off)
    char *end = nullptr;
    const long v = strtol(ag, &end, 10);
    if (end == ag || *end != '\0' || v < 0 || v > 4096 || v % 8) {
      delete ctx;
      fail(DIT_EINVAL, "DIT_ATTN_GRID must be 0 or a multiple of 8 up to 4096, got '%s'", ag);
      return nullptr;
    }
    ctx->lean_grid = (int)v;
  }
  const char *ds = getenv("DIT_DEBUG_SYNC");
  ctx->debug_sync = ds && ds[0] == '1';

  // linear1 row order: Q | K | V unchanged, then gate / up rows interleaved in chunks of 32
  // (chunk c: gate rows of features [32c, 32c+32), then the up rows of the same features)
  std::vector<int> perm1(3 * D + 2 * F);
  for (int r = 0; r < 3 * D; ++r) perm1[r] = r;
  for (int j = 0; j < 2 * F; ++j) {
    const int chunk = j / 64, within = j % 64;
    const int feat = chunk * 32 + (within % 32);
    perm1[3 * D + j] = 3 * D + (within < 32 ? 0 : F) + feat;
  }

  auto up = [&](void **dst, const char *name, bool as_f32, const std::vector<int> *perm = nullptr,
                int cols = 0) { return upload(ctx, dst, *have[name], as_f32, perm, cols); };
  int rc = 0;
  // small projections run through the fp32 GEMM; keep their weights in the compute type
  rc = rc ? rc : up(&ctx->img_in, "img_in", false);
  rc = rc ? rc : up(&ctx->temb1, "temb.l1", false);
  rc = rc ? rc : up(&ctx->temb2, "temb.l2", false);
  if (c.flow_map) {
    rc = rc ? rc : up(&ctx->ttgt1, "temb_tgt.l1", false);
    rc = rc ? rc : up(&ctx->ttgt2, "temb_tgt.l2", false);
  }
  if (c.txt_feat_dim > 0) rc = rc ? rc : up(&ctx->txt_in, "txt_in", false);
  rc = rc ? rc : up(&ctx->fmod, "final.mod", false);
  rc = rc ? rc : up(&ctx->fout, "final.out", false);
  {
    // one device copy per distinct host tensor (same data pointer and element type)
    std::map<std::pair<const void *, int>, int> by_data;
    ctx->mod_of.resize(nb);
    for (int b = 0; b < nb && !rc; ++b)
      for (const dit_tensor *t : mod_src[b]) {
        const auto key = std::make_pair(t->data, t->dtype);
        auto f = by_data.find(key);
        if (f != by_data.end()) {
          ctx->mod_of[b].push_back(f->second);
          continue;
        }
        void *dst = nullptr;
        rc = upload(ctx, &dst, *t, false);
        if (rc) break;
        by_data[key] = (int)ctx->modw.size();
        ctx->mod_of[b].push_back((int)ctx->modw.size());
        ctx->modw.push_back(dst);
        ctx->modw_rows.push_back((int)(t->numel / D));
      }
  }
  ctx->blk.resize(nb);
  for (int b = 0; b < nb && !rc; ++b) {
    const int ns = b < c.n_stream_blocks ? nsets0 : 1;
    ctx->blk[b].resize(ns);
    for (int s = 0; s < ns && !rc; ++s) {
      std::string p = "blk" + std::to_string(b) + ".s" + std::to_string(s);
      dit_ctx::Set &st = ctx->blk[b][s];
      if (ctx->fp8) {
        rc = rc ? rc : upload_fp8(ctx, &st.w1, &st.s1, *have[p + ".w1"], D, &perm1);
        rc = rc ? rc : upload_fp8(ctx, &st.w2, &st.s2, *have[p + ".w2"], D + F);
      } else {
        rc = rc ? rc : up(&st.w1, (p + ".w1").c_str(), false, &perm1, D);
        rc = rc ? rc : up(&st.w2, (p + ".w2").c_str(), false);
      }
      rc = rc ? rc : up((void **)&st.qn, (p + ".qn").c_str(), true);
      rc = rc ? rc : up((void **)&st.kn, (p + ".kn").c_str(), true);
    }
  }
  // workspace
  const size_t es = ctx->esz();
  ctx->rows_alloc = c.max_tokens + 256;
  ctx->ldv = (c.max_tokens / 64 + 2) * 64;
  const size_t R = ctx->rows_alloc;
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->x, R * D * 4);
  rc = rc ? rc : dalloc(ctx, &ctx->xm, R * D * es);
  rc = rc ? rc : dalloc(ctx, &ctx->qkv, R * 3 * D * es);
  rc = rc ? rc : dalloc(ctx, &ctx->cat, R * (D + F) * es);
  if (ctx->op != OP_F32) rc = rc ? rc : dalloc(ctx, &ctx->vt, (size_t)c.heads * 128 * ctx->ldv * es);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->pos, R * 4 * 4);
  if (!rc) {
    // RoPE frequencies theta^(-2j / 32) in revolutions per unit position, each split into a
    // 12-significant-bit part (exact products with integer positions up to 4096) and the rest
    float fr[32];
    for (int j = 0; j < 16; ++j) {
      const double f = exp(-log((double)c.rope_theta) * (2.0 * j) / 32.0) / (2.0 * M_PI);
      int e = 0;
      const double m = frexp(f, &e);  // f = m 2^e, 0.5 <= m < 1
      const double hi = ldexp(nearbyint(m * 4096.0) / 4096.0, e);
      fr[j] = (float)hi;
      fr[16 + j] = (float)(f - hi);
    }
    rc = dalloc(ctx, (void **)&ctx->rope_fr, sizeof(fr));
    if (!rc) {
      hipError_t e = hipMemcpy(ctx->rope_fr, fr, sizeof(fr), hipMemcpyHostToDevice);
      if (e != hipSuccess) rc = hip_fail(e, "upload of the RoPE frequencies");
    }
  }
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->cs, R * 128 * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->modbuf, (ctx->modw.size() + 1) * 3 * ctx->mod_ld() * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->cond, (size_t)3 * D * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->temb_e, (size_t)4 * T * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->temb_h, (size_t)4 * D * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->tgt, (size_t)D * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->noise, (size_t)c.max_tokens * C * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->fmodv, (size_t)3 * 2 * D * 4);
  rc = rc ? rc : dalloc(ctx, (void **)&ctx->guard_cnt, 2 * sizeof(unsigned));
  if (ctx->op != OP_F32 && ctx->lean_grid > 0) {
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->attn_part,
                          (size_t)2 * ctx->lean_grid * attn_part_floats * 4);
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->attn_cnt,
                          (size_t)c.heads * (c.max_tokens / 256 + kMaxGroups) * 4);
  }
  if (ctx->cus > 0)
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->gemm_part, (size_t)ctx->cus * gemm_part_floats * 4);
  if (ctx->fp8) {
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->cat8, R * (D + F));
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->xs, R * 4);
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->cs_a, R * 4);
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->cs_b, R * 4);
  }
  if (ctx->op == OP_F32) {
    rc = rc ? rc : dalloc(ctx, (void **)&ctx->xf, (size_t)c.max_tokens * D * 4);
  } else if (!rc) {
    // the output head runs through the MFMA GEMM, whose feature tiles are 256 wide
    const size_t cpad = (size_t)(c.in_channels + 255) / 256 * 256;
    rc = dalloc(ctx, &ctx->fout_pad, cpad * D * es);
    if (!rc) {
      hipError_t e = hipMemcpy(ctx->fout_pad, ctx->fout, (size_t)c.in_channels * D * es,
                               hipMemcpyDeviceToDevice);
      if (e != hipSuccess) rc = hip_fail(e, "final.out padding");
    }
  }
  if (rc) {
    std::string msg = g_err;
    dit_ctx_free(ctx);
    g_err = msg;
    return nullptr;
  }
  return ctx;
}

// ------------------------------------------------------------------------------------------
namespace {

// nseq sequences (1, or 2 for the two branches of guidance) of [text | image | reference].
Segs make_segs(int n_txt, int n_img, int n_ref, int nseq = 1) {
  const int per = n_txt + n_img + n_ref;
  return Segs{n_txt, n_txt + n_img, per * nseq, per};
}

// Modulation vectors of the listed distinct projections i: slot (i, r) = W_mod[i] . SiLU(cond[r])
// for every conditioning row r < ncond.
int compute_mods(dit_ctx *ctx, const std::vector<int> &which, const float *cond, int ncond,
                 hipStream_t stream) {
  const int D = ctx->D();
  for (int i : which)
    DIT_CHECK(gemv(ctx->modbuf + (size_t)i * 3 * ctx->mod_ld(), ctx->modw[i], ctx->op, ctx->modw_rows[i], D,
                   cond, ncond, 1, stream, ctx->mod_ld()),
              "modulation gemv");
  return 0;
}

// One block on the residual x.  Parallel wiring: LayerNorm + modulation, linear1 (Q|K|V
// and the SwiGLU MLP), QK RMSNorm + RoPE, attention, linear2 over [attention || SwiGLU]
// with the gated residual.  Sequentially wired double blocks run the attention half
// (linear1 over the Q|K|V rows, linear2 over W2's first D columns, gate 1), then a second
// LayerNorm with the second (shift, scale) and the MLP half (linear1 over the gate/up
// rows, linear2 over W2's last F columns, gate 2).  With DIT_FP8 the LayerNorm writes E4M3
// codes with row scales, and linear2's input is quantized per token before its GEMM.
// mrow[s]: the conditioning row whose modulation vectors segment s uses.
int run_block(dit_ctx *ctx, int b, float *x, Segs sg, int mask, const int mrow[3], hipStream_t stream) {
  const dit_config &c = ctx->cfg;
  const int D = ctx->D(), F = ctx->F();
  const int kind = ctx->kind(b);
  const bool seq = ctx->seq_block(kind);
  const bool f8 = ctx->fp8;
  int sos[3];
  ctx->set_of_seg(kind, sos);
  const float *mseg[3], *gate[3], *qn[3], *kn[3], *mseg2[3], *gate2[3];
  for (int s = 0; s < 3; ++s) {
    mseg[s] = ctx->mod_vec(b, sos[s], mrow[s]);
    gate[s] = mseg[s] + 2 * D;
    mseg2[s] = mseg[s] + 3 * D;   // second triple: sequential blocks only
    gate2[s] = mseg2[s] + 2 * D;
    qn[s] = ctx->blk[b][sos[s]].qn;
    kn[s] = ctx->blk[b][sos[s]].kn;
  }
  if (mask == DIT_MASK_DEFAULT) mask = (kind == 0 && c.arch == DIT_FLUX3) ? DIT_MASK_SEGMENT : DIT_MASK_FULL;
  const int N = sg.n;
  const size_t es = ctx->esz();
  const size_t ex = f8 ? 1 : es;  // bytes per value of the projections' inputs and weights
  const bool mfma = ctx->op != OP_F32;
  const double es_d = (double)es;

  // debug guard on what a launch wrote (DIT_DEBUG_SYNC=1 only)
  auto chk = [&](const char *what, const void *p, int type, int rows, int cols, int ld) {
    return guard(ctx, b, what, p, type, rows, cols, ld, stream);
  };
  if (int rc = chk("input residual x", x, OP_F32, N, D, D)) return rc;
  auto ln = [&](const float *const ms[3]) -> int {
    DIT_TIMED(P_LN, 0.0, (double)N * D * (4.0 + (double)ex),
              ln_modulate(ctx->xm, f8 ? OP_FP8 : ctx->op, D, x, D, N, 0, D, c.ln_eps, ms, sg, stream,
                          ctx->xs),
              "ln_modulate");
    if (f8) return chk("ln_modulate -> E4M3 row scales", ctx->xs, OP_F32, N, 1, 1);
    return chk("ln_modulate -> xm", ctx->xm, ctx->op, N, D, D);
  };
  auto gemm = [&](const GemmArgs &ga, int epi) -> hipError_t {
    if (f8) return gemm_fp8(ga, epi, stream);
    if (mfma) return gemm_mfma(ga, epi, ctx->op, stream);
    return gemm_simple(ga, epi, OP_F32, stream);
  };
  if (int rc = ln(mseg)) return rc;

  // row groups: one per distinct weight set over contiguous rows, sequence by sequence
  const int nseq = sg.n / sg.per;
  const int lb[4] = {0, sg.b1, sg.b2, sg.per};
  const void *cat_in = f8 ? (const void *)ctx->cat8 : (const void *)ctx->cat;  // linear2 input
  GemmGroup g1[kMaxGroups], g2[kMaxGroups];
  int ng = 0;
  for (int qs = 0; qs < nseq; ++qs)
    for (int s = 0; s < 3; ++s) {
      const int r0 = qs * sg.per + lb[s], r1 = qs * sg.per + lb[s + 1];
      if (r1 == r0) continue;
      const dit_ctx::Set &ws = ctx->blk[b][sos[s]];
      if (ng > 0 && (const void *)g1[ng - 1].w == ws.w1 && g1[ng - 1].out_row0 + g1[ng - 1].rows == r0) {
        g1[ng - 1].rows += r1 - r0;  // extend
        g2[ng - 1].rows += r1 - r0;
        continue;
      }
      g1[ng] = GemmGroup{(const char *)ctx->xm + (size_t)r0 * D * ex, ws.w1, r1 - r0, r0, ws.s1};
      g2[ng] = GemmGroup{(const char *)cat_in + (size_t)r0 * (D + F) * ex, ws.w2, r1 - r0, r0, ws.s2};
      ++ng;
    }
  GemmArgs a1 = {};
  for (int i = 0; i < ng; ++i) a1.g[i] = g1[i];
  a1.ng = ng;
  a1.n = seq ? 3 * D : 3 * D + 2 * F;
  a1.k = D;
  a1.ldx = D;
  a1.qkv = ctx->qkv;
  a1.ldq = 3 * D;
  a1.split = 3 * D;
  a1.cat = ctx->cat;
  a1.ldc = D + F;
  a1.cat_off = D;
  a1.xs = ctx->xs;
  // MFMA paths: QK RMSNorm + RoPE and the V transpose run in linear1's epilogue
  if (mfma) {
    a1.vt = ctx->vt;
    a1.ldv = ctx->ldv;
    a1.n_tok = N;
    a1.rope_pos = ctx->rope_pos;
    a1.rope_fr = ctx->rope_fr;
    for (int s = 0; s < 3; ++s) {
      a1.qn[s] = qn[s];
      a1.kn[s] = kn[s];
    }
    a1.rms_eps = c.rms_eps;
    a1.b1 = sg.b1;
    a1.b2 = sg.b2;
    a1.per = sg.per;
  } else {
    ctx->split_k(&a1);  // the fp32 GEMM cuts k into slices when its tiles are few
  }
  DIT_TIMED(P_LINEAR1, 2.0 * N * D * (double)a1.n, 0.0, gemm(a1, EPI_QKV_SWIGLU), "linear1");
  if (mfma) {
    if (int rc = chk("linear1 -> q, k (normalised, rotated)", ctx->qkv, ctx->op, N, 2 * D, 3 * D)) return rc;
    if (int rc = chk("linear1 -> V^T", ctx->vt, ctx->op, D, N, ctx->ldv)) return rc;
  } else {
    if (int rc = chk("linear1 -> q, k, v", ctx->qkv, ctx->op, N, 3 * D, 3 * D)) return rc;
  }
  if (!seq)
    if (int rc = chk("linear1 -> SwiGLU output", (const char *)ctx->cat + (size_t)D * es, ctx->op, N, F, D + F))
      return rc;

  if (!mfma) {
    // bytes: q, k read + written, one cos/sin row per token
    DIT_TIMED(P_QKNORM, 0.0, (double)N * (4.0 * D * es_d + 512.0),
              qk_norm_rope(ctx->qkv, ctx->op, 3 * D, D, c.heads, ctx->cs, N, qn, kn, sg,
                           c.rms_eps, stream),
              "qk_norm_rope");
    if (int rc = chk("qk_norm_rope -> q, k", ctx->qkv, ctx->op, N, 2 * D, 3 * D)) return rc;
  }

  AttnArgs at = {};
  at.qkv = ctx->qkv;
  at.ldqkv = 3 * D;
  at.d_model = D;
  at.vt = ctx->vt;
  at.ldv = ctx->ldv;
  at.out = ctx->cat;
  at.ldo = D + F;
  at.heads = c.heads;
  at.scale = 1.0f / sqrtf(128.0f);
  at.part = ctx->attn_part;
  at.cnt = ctx->attn_cnt;
  at.lean_grid = ctx->lean_grid;
  // each sequence attends only to itself; per-mode blocks only within each segment
  for (int qs = 0; qs < nseq; ++qs) {
    if (mask == DIT_MASK_SEGMENT) {
      for (int s = 0; s < 3; ++s) {
        const int r0 = qs * sg.per + lb[s], r1 = qs * sg.per + lb[s + 1];
        if (r1 > r0) at.g[at.ng++] = AttnGroup{r0, r1, r0, r1};
      }
    } else {
      at.g[at.ng++] = AttnGroup{qs * sg.per, (qs + 1) * sg.per, qs * sg.per, (qs + 1) * sg.per};
    }
  }
  double pairs = 0.0;
  for (int i = 0; i < at.ng; ++i)
    pairs += (double)(at.g[i].q1 - at.g[i].q0) * (at.g[i].k1 - at.g[i].k0);
  const double fla = 4.0 * D * pairs;
  if (mfma)
    DIT_TIMED(P_ATTN, fla, 0.0, attention_mfma(at, ctx->op, stream), "attention");
  else
    DIT_TIMED(P_ATTN, fla, 0.0, attention_f32(at, stream), "attention");
  if (int rc = chk("attention -> output", ctx->cat, ctx->op, N, D, D + F)) return rc;

  // linear2 with the gated residual over k columns of cat starting at column k0 (W2 columns
  // k0 .. k0 + k of its D + F); with DIT_FP8 those columns are quantized first, scales in xsc
  auto linear2 = [&](int k0, int k, const float *const gt[3], float *xsc) -> int {
    if (f8) {
      DIT_TIMED(P_QUANT, 0.0, (double)N * k * 3.0,
                quant_rows_fp8(ctx->cat8 + k0, D + F, xsc, (const uint16_t *)ctx->cat + k0, OP_F16, D + F, N, k,
                               stream),
                "fp8 quantization");
      if (int rc = chk("E4M3 quantization -> row scales", xsc, OP_F32, N, 1, 1)) return rc;
    }
    GemmArgs a2 = {};
    for (int i = 0; i < ng; ++i) {
      a2.g[i] = g2[i];
      a2.g[i].x = (const char *)g2[i].x + (size_t)k0 * ex;
      a2.g[i].w = (const char *)g2[i].w + (size_t)k0 * ex;
    }
    a2.ng = ng;
    a2.n = D;
    a2.k = k;
    a2.ldx = D + F;
    a2.ldw = D + F;
    a2.x = x;
    a2.ldres = D;
    for (int s = 0; s < 3; ++s) a2.gate[s] = gt[s];
    a2.b1 = sg.b1;
    a2.b2 = sg.b2;
    a2.per = sg.per;
    a2.xs = xsc;
    ctx->split_k(&a2);
    DIT_TIMED(P_LINEAR2, 2.0 * N * (double)k * D, 0.0, gemm(a2, EPI_RESID), "linear2");
    return chk("linear2 -> residual x", x, OP_F32, N, D, D);
  };
  if (!seq) return linear2(0, D + F, gate, ctx->cs_a);

  // sequential double block: attention half, then the MLP half on the updated residual
  if (int rc = linear2(0, D, gate, ctx->cs_a)) return rc;
  if (int rc = ln(mseg2)) return rc;
  GemmArgs am = a1;
  for (int i = 0; i < ng; ++i) {  // gate/up rows of W1 (and their scales)
    am.g[i].w = (const char *)g1[i].w + (size_t)3 * D * D * ex;
    if (g1[i].ws) am.g[i].ws = g1[i].ws + 3 * D;
  }
  am.n = 2 * F;
  am.split = 0;
  DIT_TIMED(P_LINEAR1, 2.0 * N * D * (2.0 * F), 0.0, gemm(am, EPI_QKV_SWIGLU), "linear1");
  if (int rc = chk("linear1 -> SwiGLU output", (const char *)ctx->cat + (size_t)D * es, ctx->op, N, F, D + F))
    return rc;
  return linear2(D, F, gate2, ctx->cs_b);
}

int check_tokens(dit_ctx *ctx, int n_txt, int n_img, int n_ref, int nseq = 1) {
  if (n_txt < 0 || n_img < 0 || n_ref < 0) return fail(DIT_EINVAL, "negative token count");
  const long long n = (long long)n_txt + n_img + n_ref;
  if (n < 1) return fail(DIT_EINVAL, "empty sequence");
  if (n * nseq > ctx->cfg.max_tokens)
    return fail(DIT_EINVAL, "%lld tokens (%d sequence%s of %lld) exceed max_tokens %d", n * nseq, nseq,
                nseq > 1 ? "s" : "", n, ctx->cfg.max_tokens);
  return 0;
}

// Conditioning for one transformer call at time t: cond rows per segment, modulation of
// every block kind, output-head modulation.  FLUX.2: one timestep for all tokens; FLUX.3:
// image tokens at t, text and reference tokens at t = 0.  Flow-map models add the embedding
// of the target time t_target (its own MLP) to every cond row.
int prepare_conditioning(dit_ctx *ctx, double t, double t_target, hipStream_t stream) {
  const dit_config &c = ctx->cfg;
  const int D = c.hidden, T = c.time_dim;
  double tv[4] = {t, t, t, t_target};
  if (c.arch == DIT_FLUX3) tv[0] = tv[2] = 0.0;
  const int ne = c.flow_map ? 4 : 3;
  DIT_CHECK(timestep_embed(ctx->temb_e, tv, ne, T, stream), "timestep_embed");
  DIT_CHECK(gemv(ctx->temb_h, ctx->temb1, ctx->op, D, T, ctx->temb_e, 3, 0, stream), "temb l1");
  DIT_CHECK(gemv(ctx->cond, ctx->temb2, ctx->op, D, D, ctx->temb_h, 3, 1, stream), "temb l2");
  if (c.flow_map) {
    DIT_CHECK(gemv(ctx->temb_h + 3 * D, ctx->ttgt1, ctx->op, D, T, ctx->temb_e + 3 * T, 1, 0,
                   stream), "target temb l1");
    DIT_CHECK(gemv(ctx->tgt, ctx->ttgt2, ctx->op, D, D, ctx->temb_h + 3 * D, 1, 1, stream),
              "target temb l2");
    DIT_CHECK(add_row(ctx->cond, 3, D, ctx->tgt, stream), "target time");
  }
  std::vector<int> all(ctx->modw.size());
  for (size_t i = 0; i < all.size(); ++i) all[i] = (int)i;
  if (int rc = compute_mods(ctx, all, ctx->cond, 3, stream)) return rc;
  DIT_CHECK(gemv(ctx->fmodv, ctx->fmod, ctx->op, 2 * D, D, ctx->cond, 3, 1, stream), "final modulation");
  return 0;
}

// How the output head's velocity of one sequence lands in `out`: the GEMM's store modes
// (0: out = v, 1: out += alpha * v, 2: out = alpha * v).
struct HeadStore {
  int mode;
  float alpha;
};

// What one transformer call sees besides the latents: text (one sequence, or the two
// branches of guidance), the image grid and the reference images.
struct Req {
  const float *txt[2] = {nullptr, nullptr};
  int nseq = 1, n_txt = 0, gh = 0, gw = 0;
  float guidance = 1.f;
  const float *ref_lat = nullptr;
  int n_refs = 0;
  int grids[2 * kMaxRefs] = {0};
  int n_ref() const {
    int n = 0;
    for (int k = 0; k < n_refs; ++k) n += grids[2 * k] * grids[2 * k + 1];
    return n;
  }
};

// Embed, run every block, output head.  nseq = 1: the sequence of txt[0]; nseq = 2: the
// conditional (txt[0]) and unconditional (txt[1]) branches of guidance stacked as two
// sequences that share latents, references and time.  The head stores sequence 0 first,
// then sequence 1, each with its own HeadStore.
int run_forward(dit_ctx *ctx, const float *lat, const Req &rq, double t, double t_target,
                float *out, const HeadStore hs[2], hipStream_t stream) {
  const dit_config &c = ctx->cfg;
  const int D = c.hidden, C = c.in_channels;
  const int nseq = rq.nseq, n_txt = rq.n_txt, gh = rq.gh, gw = rq.gw;
  const float *const *txt = rq.txt;
  const float *ref_lat = rq.ref_lat;
  const int n_img = gh * gw, n_ref = rq.n_ref();
  const Segs sg = make_segs(n_txt, n_img, n_ref, nseq);
  const int per = sg.per;
  {
    const int pe = prof_begin(ctx, P_COND, stream);
    if (int rc = prepare_conditioning(ctx, t, t_target, stream)) return rc;
    prof_end(ctx, pe, P_COND, 0.0, 0.0, stream);
  }
  for (int qs = 0; qs < nseq; ++qs)
    DIT_CHECK(fill_positions(ctx->pos + (size_t)qs * per * 4, n_txt, gh, gw, rq.grids, rq.n_refs,
                             stream),
              "positions");
  if (ctx->op == OP_F32)  // the MFMA paths rotate in linear1's epilogue, from the positions
    DIT_CHECK(rope_table(ctx->cs, ctx->pos, sg.n, c.rope_theta, stream), "rope_table");
  ctx->rope_pos = ctx->pos;
  // sequence: text embeddings as they are, latents through the input projection
  for (int qs = 0; qs < nseq; ++qs)
    DIT_CHECK(copy_rows_f32(ctx->x + (size_t)qs * per * D, D, txt[qs], D, n_txt, D, stream),
              "copy text");
  GemmArgs ae = {};
  ae.n = D;
  ae.k = C;
  ae.ldx = C;
  ae.out = ctx->x;
  ae.ldo = D;
  const double fle = 2.0 * nseq * (n_img + n_ref) * (double)C * D;
  const void *lsrc = lat, *rsrc = ref_lat;
  if (ctx->op != OP_F32) {
    // latents rounded to the operand type (into the free xm buffer, [n_img + n_ref][C]), then
    // the MFMA GEMM
    char *lh = reinterpret_cast<char *>(ctx->xm);
    const size_t es = ctx->esz();
    DIT_TIMED(P_EMBED, 0.0, 0.0, to_half(lh, ctx->op, lat, (int64_t)n_img * C, stream), "img_in cast");
    lsrc = lh;
    if (n_ref > 0) {
      char *rh = lh + (size_t)n_img * C * es;
      DIT_TIMED(P_EMBED, 0.0, 0.0, to_half(rh, ctx->op, ref_lat, (int64_t)n_ref * C, stream), "img_in cast");
      rsrc = rh;
    }
  }
  for (int qs = 0; qs < nseq; ++qs) {
    ae.g[ae.ng++] = GemmGroup{lsrc, ctx->img_in, n_img, qs * per + n_txt};
    if (n_ref > 0) ae.g[ae.ng++] = GemmGroup{rsrc, ctx->img_in, n_ref, qs * per + n_txt + n_img};
  }
  if (ctx->op == OP_F32)
    DIT_TIMED(P_EMBED, fle, 0.0, gemm_simple(ae, EPI_STORE_F32, ctx->op, stream), "img_in");
  else
    DIT_TIMED(P_EMBED, fle, 0.0, gemm_mfma(ae, EPI_STORE_F32, ctx->op, stream), "img_in");
  if (int rc = guard(ctx, -1, "img_in -> residual x", ctx->x, OP_F32, sg.n, D, D, stream)) return rc;
  const int rows3[3] = {0, 1, 2};
  for (int b = 0; b < ctx->nblocks(); ++b)
    if (int rc = run_block(ctx, b, ctx->x, sg, DIT_MASK_DEFAULT, rows3, stream)) return rc;
  // output head on the image rows of each sequence
  const float *fm = ctx->fmodv + 2 * D;  // image segment's (shift, scale)
  const float *fms[3] = {fm, fm, fm};
  const double flf = 2.0 * n_img * (double)C * D;
  for (int qs = 0; qs < nseq; ++qs) {
    GemmArgs af = {};
    af.ng = 1;
    af.k = D;
    af.ldx = D;
    af.out = out;
    af.ldo = C;
    af.accumulate = hs[qs].mode;
    af.alpha = hs[qs].alpha;
    ctx->split_k(&af);
    const int row0 = qs * per + n_txt;
    if (ctx->op == OP_F32) {
      DIT_CHECK(ln_modulate(ctx->xf, OP_F32, D, ctx->x, D, n_img, row0, D, c.ln_eps, fms, sg, stream),
                "final norm");
      af.g[0] = GemmGroup{ctx->xf, ctx->fout, n_img, 0};
      af.n = C;
      DIT_TIMED(P_FINAL, flf, 0.0, gemm_simple(af, EPI_STORE_F32, ctx->op, stream), "final projection");
    } else {
      DIT_CHECK(ln_modulate(ctx->xm, ctx->op, D, ctx->x, D, n_img, row0, D, c.ln_eps, fms, sg, stream),
                "final norm");
      af.g[0] = GemmGroup{ctx->xm, ctx->fout_pad, n_img, 0};
      af.n = (C + 255) / 256 * 256;  // zero weight rows past C; only the first C columns are stored
      af.n_store = C;
      DIT_TIMED(P_FINAL, flf, 0.0, gemm_mfma(af, EPI_STORE_F32, ctx->op, stream), "final projection");
    }
    if (int rc = guard(ctx, -1, "output head -> velocity / latents", out, OP_F32, n_img, C, C, stream))
      return rc;
  }
  return 0;
}

int check_request(dit_ctx *ctx, const float *lat, const Req &rq) {
  if (rq.gh < 1 || rq.gw < 1) return fail(DIT_EINVAL, "image grid must be at least 1x1");
  if (!lat) return fail(DIT_EINVAL, "lat is NULL");
  if (rq.n_txt > 0 && !rq.txt[0]) return fail(DIT_EINVAL, "txt is NULL");
  if (rq.nseq == 2 && rq.n_txt > 0 && !rq.txt[1]) return fail(DIT_EINVAL, "txt_uncond is NULL");
  if (rq.nseq == 2 && !isfinite(rq.guidance)) return fail(DIT_EINVAL, "guidance must be finite");
  if (rq.n_refs < 0 || rq.n_refs > kMaxRefs)
    return fail(DIT_EINVAL, "n_refs %d out of range [0, %d]", rq.n_refs, kMaxRefs);
  for (int k = 0; k < rq.n_refs; ++k)
    if (rq.grids[2 * k] < 1 || rq.grids[2 * k + 1] < 1)
      return fail(DIT_EINVAL, "reference %d grid must be at least 1x1", k);
  if (rq.n_refs > 0 && !rq.ref_lat) return fail(DIT_EINVAL, "ref_lat is NULL");
  return check_tokens(ctx, rq.n_txt, rq.gh * rq.gw, rq.n_ref(), rq.nseq);
}

// The request of the single-reference entry points (rgh = rgw = 0: no reference).
int legacy_req(Req *rq, const float *txt, const float *txt_uncond, int nseq, int n_txt, int gh,
               int gw, const float *ref_lat, int rgh, int rgw, float guidance) {
  if (rgh < 0 || rgw < 0 || (rgh == 0) != (rgw == 0)) return fail(DIT_EINVAL, "bad reference grid");
  rq->txt[0] = txt;
  rq->txt[1] = txt_uncond;
  rq->nseq = nseq;
  rq->n_txt = n_txt;
  rq->gh = gh;
  rq->gw = gw;
  rq->guidance = guidance;
  rq->ref_lat = ref_lat;
  rq->n_refs = rgh > 0 ? 1 : 0;
  rq->grids[0] = rgh;
  rq->grids[1] = rgw;
  return 0;
}

// The request of dit_forward_ex / dit_denoise_ex.
int public_req(Req *rq, const dit_request *r) {
  if (!r) return fail(DIT_EINVAL, "request is NULL");
  if (r->n_refs < 0 || r->n_refs > kMaxRefs)
    return fail(DIT_EINVAL, "n_refs %d out of range [0, %d]", r->n_refs, kMaxRefs);
  if (r->n_refs > 0 && !r->ref_grids) return fail(DIT_EINVAL, "ref_grids is NULL");
  rq->txt[0] = r->txt;
  rq->txt[1] = r->txt_uncond;
  rq->nseq = r->txt_uncond ? 2 : 1;
  rq->n_txt = r->n_txt;
  rq->gh = r->gh;
  rq->gw = r->gw;
  rq->guidance = r->txt_uncond ? r->guidance : 1.f;
  rq->ref_lat = r->ref_lat;
  rq->n_refs = r->n_refs;
  for (int k = 0; k < 2 * r->n_refs; ++k) rq->grids[k] = r->ref_grids[k];
  return 0;
}

// Store modes of the output head for one call: plain velocity, or the guided combination.
void head_stores(const Req &rq, HeadStore hs[2]) {
  if (rq.nseq == 2) {  // v = g v_c + (1 - g) v_u  (= v_u + g (v_c - v_u))
    hs[0] = HeadStore{2, rq.guidance};
    hs[1] = HeadStore{1, 1.0f - rq.guidance};
  } else {
    hs[0] = HeadStore{0, 0.f};
    hs[1] = HeadStore{0, 0.f};
  }
}

int forward_call(dit_ctx *ctx, const float *lat, const Req &rq, double t, double t_target,
                 float *v, hipStream_t stream) {
  if (int rc = check_request(ctx, lat, rq)) return rc;
  if (!v) return fail(DIT_EINVAL, "v is NULL");
  if (!isfinite(t) || !isfinite(t_target)) return fail(DIT_EINVAL, "t and t_target must be finite");
  HeadStore hs[2];
  head_stores(rq, hs);
  return run_forward(ctx, lat, rq, t, t_target, v, hs, stream);
}

}  // namespace

extern "C" int dit_block_forward(dit_ctx *ctx, int block, float *x, int n_txt, int n_img, int n_ref,
                                 const float *pos, const float *cond, int mask, void *stream_) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  if (block < 0 || block >= ctx->nblocks())
    return fail(DIT_EINVAL, "block %d out of range [0, %d)", block, ctx->nblocks());
  if (!x || !pos || !cond) return fail(DIT_EINVAL, "x, pos and cond must be device pointers");
  if (mask != DIT_MASK_DEFAULT && mask != DIT_MASK_FULL && mask != DIT_MASK_SEGMENT)
    return fail(DIT_EINVAL, "unknown mask %d", mask);
  if (int rc = check_tokens(ctx, n_txt, n_img, n_ref)) return rc;
  hipStream_t stream = (hipStream_t)stream_;
  const Segs sg = make_segs(n_txt, n_img, n_ref);
  if (ctx->op == OP_F32)
    DIT_CHECK(rope_table(ctx->cs, pos, sg.n, ctx->cfg.rope_theta, stream), "rope_table");
  ctx->rope_pos = pos;
  // one conditioning row per non-empty segment, in the order text, image, reference
  const int count[3] = {n_txt, n_img, n_ref};
  int mrow[3], n_cond = 0;
  for (int s = 0; s < 3; ++s) mrow[s] = count[s] > 0 ? n_cond++ : 0;
  std::vector<int> which;
  for (int i : ctx->mod_of[block])
    if (std::find(which.begin(), which.end(), i) == which.end()) which.push_back(i);
  if (int rc = compute_mods(ctx, which, cond, n_cond, stream)) return rc;
  return run_block(ctx, block, x, sg, mask, mrow, stream);
}

extern "C" int dit_forward(dit_ctx *ctx, const float *lat, const float *ref_lat, const float *txt,
                           int n_txt, int gh, int gw, int rgh, int rgw, float t, float *v, void *stream) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  if (ctx->cfg.flow_map) return fail(DIT_EINVAL, "flow-map model: call dit_forward_flow with the target time");
  Req rq;
  if (int rc = legacy_req(&rq, txt, nullptr, 1, n_txt, gh, gw, ref_lat, rgh, rgw, 1.f)) return rc;
  return forward_call(ctx, lat, rq, t, t, v, (hipStream_t)stream);
}

extern "C" int dit_forward_flow(dit_ctx *ctx, const float *lat, const float *ref_lat,
                                const float *txt, int n_txt, int gh, int gw, int rgh, int rgw,
                                float t, float t_target, float *v, void *stream) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  if (!ctx->cfg.flow_map) return fail(DIT_EINVAL, "dit_forward_flow needs a flow-map model (flow_map = 1)");
  Req rq;
  if (int rc = legacy_req(&rq, txt, nullptr, 1, n_txt, gh, gw, ref_lat, rgh, rgw, 1.f)) return rc;
  return forward_call(ctx, lat, rq, t, t_target, v, (hipStream_t)stream);
}

extern "C" int dit_text_features(dit_ctx *ctx, const float *feat, int n_txt, float *txt,
                                 void *stream_) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  const int K = ctx->cfg.txt_feat_dim, D = ctx->cfg.hidden;
  if (K <= 0) return fail(DIT_EINVAL, "the model has no text-feature projection (txt_feat_dim = 0)");
  if (n_txt < 1 || n_txt > ctx->cfg.max_tokens)
    return fail(DIT_EINVAL, "n_txt %d out of range [1, max_tokens %d]", n_txt, ctx->cfg.max_tokens);
  if (!feat || !txt) return fail(DIT_EINVAL, "feat and txt must be device pointers");
  hipStream_t stream = (hipStream_t)stream_;
  GemmArgs a = {};
  a.ng = 1;
  a.n = D;
  a.k = K;
  a.ldx = K;
  a.ldo = D;
  ctx->split_k(&a);
  if (ctx->op == OP_F32) {
    a.g[0] = GemmGroup{feat, ctx->txt_in, n_txt, 0};
    a.out = txt;
    DIT_TIMED(P_EMBED, 2.0 * n_txt * (double)K * D, 0.0, gemm_simple(a, EPI_STORE_F32, ctx->op, stream),
              "text projection");
    return 0;
  }
  // 16-bit operands: features rounded in chunks of rows through the cat workspace
  const size_t cap = (size_t)ctx->rows_alloc * (D + ctx->F());  // 16-bit elements of cat
  size_t fit = cap / K;  // feature rows the workspace holds (whole 256-row tiles when it can)
  if (fit >= 256) fit = fit / 256 * 256;
  const int chunk = (int)std::min<size_t>((size_t)n_txt, fit);
  if (chunk < 1) return fail(DIT_EUNSUPPORTED, "txt_feat_dim %d too wide for the workspace", K);
  for (int r0 = 0; r0 < n_txt; r0 += chunk) {
    const int rows = std::min(chunk, n_txt - r0);
    DIT_TIMED(P_EMBED, 0.0, 0.0, to_half(ctx->cat, ctx->op, feat + (size_t)r0 * K, (int64_t)rows * K, stream),
              "feature cast");
    a.g[0] = GemmGroup{ctx->cat, ctx->txt_in, rows, 0};
    a.out = txt + (size_t)r0 * D;
    DIT_TIMED(P_EMBED, 2.0 * rows * (double)K * D, 0.0, gemm_mfma(a, EPI_STORE_F32, ctx->op, stream),
              "text projection");
  }
  return 0;
}

extern "C" int dit_forward_cfg(dit_ctx *ctx, const float *lat, const float *ref_lat,
                               const float *txt, const float *txt_uncond, int n_txt, int gh, int gw,
                               int rgh, int rgw, float t, float guidance, float *v, void *stream) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  if (ctx->cfg.flow_map)
    return fail(DIT_EINVAL, "flow-map model: dit_forward_cfg takes no target time; use dit_forward_ex");
  Req rq;
  if (int rc = legacy_req(&rq, txt, txt_uncond, 2, n_txt, gh, gw, ref_lat, rgh, rgw, guidance)) return rc;
  return forward_call(ctx, lat, rq, t, t, v, (hipStream_t)stream);
}

extern "C" int dit_forward_ex(dit_ctx *ctx, const dit_request *request, const float *lat,
                              float t, float t_target, float *v, void *stream) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  Req rq;
  if (int rc = public_req(&rq, request)) return rc;
  // only flow-map models read the target time
  return forward_call(ctx, lat, rq, t, ctx->cfg.flow_map ? t_target : t, v, (hipStream_t)stream);
}

namespace {

// The sampling loop.  strength 1: lat is the starting noise (drawn from seed when seed >= 0,
// copied from noise when given, else used as it is).  strength < 1 (image-to-image): lat holds
// clean latents; they are moved to t = floor(n s) / n on the straight path to the noise
// (noise, or drawn from seed) and the last floor(n s) Euler steps run.
int denoise(dit_ctx *ctx, const Req &rq, float *lat, int n_steps, float strength,
            const float *noise, int64_t seed, hipStream_t stream) {
  if (int rc = check_request(ctx, lat, rq)) return rc;
  if (n_steps < 1) return fail(DIT_EINVAL, "n_steps must be >= 1, got %d", n_steps);
  if (!(strength > 0.f && strength <= 1.f)) return fail(DIT_EINVAL, "strength must be in (0, 1], got %g", strength);
  const int steps_run = (int)floor((double)n_steps * strength);
  if (steps_run < 1)
    return fail(DIT_EINVAL, "strength %g runs no step of %d (needs n_steps * strength >= 1)", strength, n_steps);
  const int i0 = n_steps - steps_run;
  const int64_t nl = (int64_t)rq.gh * rq.gw * ctx->cfg.in_channels;
  if (i0 == 0) {
    if (noise) {
      DIT_CHECK(hipMemcpyAsync(lat, noise, (size_t)nl * 4, hipMemcpyDeviceToDevice, stream), "noise copy");
    } else if (seed >= 0) {
      DIT_CHECK(philox_normal(lat, nl, (uint64_t)seed, stream), "noise");
    }
  } else {
    const float *eps = noise;
    if (!eps) {
      if (seed < 0) return fail(DIT_EINVAL, "image-to-image needs noise or a seed >= 0");
      DIT_CHECK(philox_normal(ctx->noise, nl, (uint64_t)seed, stream), "noise");
      eps = ctx->noise;
    }
    DIT_CHECK(noise_mix(lat, eps, nl, (float)(1.0 - (double)i0 / n_steps), stream), "noise mix");
  }
  for (int i = i0; i < n_steps; ++i) {
    const double t_cur = 1.0 - (double)i / n_steps;
    const double t_next = 1.0 - (double)(i + 1) / n_steps;
    const float dt = (float)(t_cur - t_next);
    // Euler: lat += (t_i - t_{i+1}) * v, fused into the output projection's epilogue; with
    // guidance v = g v_c + (1 - g) v_u, added branch by branch
    HeadStore hs[2] = {{1, dt}, {1, 0.f}};
    if (rq.nseq == 2) {
      hs[0].alpha = dt * rq.guidance;
      hs[1].alpha = dt * (1.0f - rq.guidance);
    }
    // flow-map models also see the time the step jumps to
    if (int rc = run_forward(ctx, lat, rq, t_cur, t_next, lat, hs, stream)) return rc;
  }
  return 0;
}

}  // namespace

extern "C" int dit_denoise(dit_ctx *ctx, float *lat, const float *txt, int n_txt, int gh, int gw,
                           const float *ref_lat, int rgh, int rgw, int n_steps, int64_t seed, void *stream) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  Req rq;
  if (int rc = legacy_req(&rq, txt, nullptr, 1, n_txt, gh, gw, ref_lat, rgh, rgw, 1.f)) return rc;
  return denoise(ctx, rq, lat, n_steps, 1.f, nullptr, seed, (hipStream_t)stream);
}

extern "C" int dit_denoise_cfg(dit_ctx *ctx, float *lat, const float *txt, const float *txt_uncond,
                               int n_txt, int gh, int gw, const float *ref_lat, int rgh, int rgw,
                               int n_steps, float guidance, int64_t seed, void *stream) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  Req rq;
  if (int rc = legacy_req(&rq, txt, txt_uncond, 2, n_txt, gh, gw, ref_lat, rgh, rgw, guidance)) return rc;
  return denoise(ctx, rq, lat, n_steps, 1.f, nullptr, seed, (hipStream_t)stream);
}

extern "C" int dit_denoise_ex(dit_ctx *ctx, const dit_request *request, float *lat, int n_steps,
                              float strength, const float *noise, int64_t seed, void *stream) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  Req rq;
  if (int rc = public_req(&rq, request)) return rc;
  return denoise(ctx, rq, lat, n_steps, strength, noise, seed, (hipStream_t)stream);
}

extern "C" int dit_fill_noise(float *dst, int64_t n, int64_t seed, void *stream) {
  g_err.clear();
  if (!dst || n < 0 || seed < 0) return fail(DIT_EINVAL, "bad arguments");
  hipError_t e = philox_normal(dst, n, (uint64_t)seed, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "noise");
  return 0;
}

extern "C" int dit_quantize_rows_fp8(const float *x, int rows, int cols, int ldx, uint8_t *q, int ldq,
                                     float *scale, void *stream) {
  g_err.clear();
  if (!x || !q || !scale || rows < 0 || cols < 8 || cols % 8 || cols > 16384 || ldx < cols || ldx % 8 ||
      ldq < cols || ldq % 8)
    return fail(DIT_EINVAL, "bad arguments (8 <= cols <= 16384; cols, ldx, ldq multiples of 8, ldx, ldq >= cols)");
  hipError_t e = quant_rows_fp8(q, ldq, scale, x, OP_F32, ldx, rows, cols, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 quantization");
  return 0;
}

namespace {

// Arguments of the E4M3 GEMM entry points: checks, then the launch description.
int fp8_gemm_args(GemmArgs *a, const uint8_t *qx, const float *sx, int m, int ldx, const uint8_t *qw,
                  const float *sw, int n, int ldw, int k, float *y, int ldy) {
  if (!qx || !sx || !qw || !sw || !y || m < 0) return fail(DIT_EINVAL, "bad arguments");
  if (n < 256 || n % 256 || k < 128 || k % 128)
    return fail(DIT_EUNSUPPORTED, "dit_gemm_fp8 needs n %% 256 == 0 and k %% 128 == 0 (n %d, k %d)", n, k);
  if (ldx < k || ldx % 16 || ldw < k || ldw % 16 || ldy < n || ldy % 4)
    return fail(DIT_EINVAL, "bad strides (ldx, ldw >= k, multiples of 16; ldy >= n, multiple of 4)");
  *a = GemmArgs{};
  a->g[0] = GemmGroup{qx, qw, m, 0, sw};
  a->ng = 1;
  a->n = n;
  a->k = k;
  a->ldx = ldx;
  a->ldw = ldw;
  a->out = y;
  a->ldo = ldy;
  a->xs = sx;
  return 0;
}

// The allocation-free GEMM's k-slice partial tiles: a file-scope device array (each device
// holds its own copy until the process ends), 128 tiles of 256 x 256 fp32 = 32 MiB.  Host
// code never uses the array's name as an address: the device address is looked up once per
// device with hipGetSymbolAddress and kept in g_scratch.
constexpr int kStaticPartTiles = 128;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) float scratch[(size_t)kStaticPartTiles * gemm_part_floats];

struct ScratchOfDevice {
  float *ptr;
  int cus;
};
std::mutex g_scratch_mu;
ScratchOfDevice g_scratch[kMaxDevices] = {};

int scratch_of_current_device(ScratchOfDevice *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DIT_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchOfDevice &sd = g_scratch[dev];
  if (!sd.ptr) {
    float *p = nullptr;
    e = hipGetSymbolAddress((void **)&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    sd.cus = cus / 8 * 8;
    sd.ptr = p;
  }
  *out = sd;
  return 0;
}

}  // namespace

extern "C" int dit_gemm_fp8(const uint8_t *qx, const float *sx, int m, int ldx, const uint8_t *qw,
                            const float *sw, int n, int ldw, int k, float *y, int ldy, void *stream) {
  g_err.clear();
  GemmArgs a;
  if (int rc = fp8_gemm_args(&a, qx, sx, m, ldx, qw, sw, n, ldw, k, y, ldy)) return rc;
  if (m == 0) return 0;
  hipError_t e = gemm_fp8(a, EPI_STORE_F32, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 gemm");
  return 0;
}

extern "C" int dit_gemm_fp8_static(const uint8_t *qx, const float *sx, int m, int ldx,
                                   const uint8_t *qw, const float *sw, int n, int ldw, int k,
                                   float *y, int ldy, void *stream) {
  g_err.clear();
  GemmArgs a;
  if (int rc = fp8_gemm_args(&a, qx, sx, m, ldx, qw, sw, n, ldw, k, y, ldy)) return rc;
  if (m == 0) return 0;
  ScratchOfDevice sd;
  if (int rc = scratch_of_current_device(&sd)) return rc;
  // k-slices for launches whose tiles fill under half of the compute units, their partial
  // tiles in the static array (the launcher caps the slice count to what it holds)
  a.part = sd.ptr;
  a.part_tiles = kStaticPartTiles;
  a.split_grid = sd.cus;
  hipError_t e = gemm_fp8(a, EPI_STORE_F32, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 gemm");
  return 0;
}

extern "C" int dit_mfma_rate(int compute, int iters, double *tflops, double *ghz, void *stream_) {
  g_err.clear();
  if ((compute != DIT_F16 && compute != DIT_BF16) || iters < 1 || iters > (1 << 24) || !tflops || !ghz)
    return fail(DIT_EINVAL, "dit_mfma_rate: compute must be DIT_F16 or DIT_BF16, 1 <= iters <= 2^24");
  hipStream_t stream = (hipStream_t)stream_;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "dit_mfma_rate");
  const int blocks = 2 * cus;  // two waves on every SIMD
  float *sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  e = hipMalloc(&sink, (size_t)blocks * sizeof(float));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  float ms = 0.f;
  if (e == hipSuccess) e = mfma_rate(compute, blocks, 1000, sink, stream);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, stream);
  if (e == hipSuccess) e = mfma_rate(compute, blocks, iters, sink, stream);
  if (e == hipSuccess) e = hipEventRecord(e1, stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipFree(sink);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_fail(e, "dit_mfma_rate");
  *tflops = mfma_rate_flops(blocks, iters) / (ms * 1e-3) / 1e12;
  // one 16x16x32 MFMA (16384 flops) every 16 cycles on each of the 4 SIMDs of every CU
  *ghz = *tflops * 1e12 / (1024.0 * 4 * cus) / 1e9;
  return 0;
}

extern "C" const void *dit_debug_buffer(dit_ctx *ctx, const char *name, int *dtype, int64_t *row_stride) {
  if (!ctx || !name) return nullptr;
  const int D = ctx->D(), F = ctx->F();
  const int dt = ctx->op;
  auto ret = [&](const void *p, int t, int64_t rs) -> const void * {
    if (dtype) *dtype = t;
    if (row_stride) *row_stride = rs;
    return p;
  };
  if (!strcmp(name, "xm")) return ret(ctx->xm, ctx->fp8 ? DIT_FP8 : dt, D);
  if (!strcmp(name, "qkv")) return ret(ctx->qkv, dt, 3 * D);
  if (!strcmp(name, "vt")) return ctx->vt ? ret(ctx->vt, dt, ctx->ldv) : nullptr;
  if (!strcmp(name, "cat")) return ret(ctx->cat, dt, D + F);
  if (!strcmp(name, "mod")) return ret(ctx->modbuf, DIT_F32, ctx->mod_ld());  // [M][3][R]
  if (!strcmp(name, "x")) return ret(ctx->x, DIT_F32, D);
  return nullptr;
}

extern "C" int dit_profile_start(dit_ctx *ctx, int max_launches) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  if (max_launches < 1 || max_launches > (1 << 20)) return fail(DIT_EINVAL, "max_launches out of range");
  while ((int)ctx->prof_ev.size() < 2 * max_launches) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
    ctx->prof_ev.push_back(e);
  }
  ctx->prof_rec.clear();
  ctx->prof_next = 0;
  ctx->prof_on = true;
  return 0;
}

extern "C" int dit_profile_select(dit_ctx *ctx, const char *kernels) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  if (!kernels || !kernels[0]) {
    ctx->prof_mask = ~0u;
    return 0;
  }
  unsigned mask = 0;
  std::string list(kernels);
  size_t pos = 0;
  while (pos <= list.size()) {
    const size_t end = std::min(list.find(',', pos), list.size());
    const std::string name = list.substr(pos, end - pos);
    int cls = -1;
    for (int i = 0; i < P_NCLASS; ++i)
      if (name == kProfNames[i]) cls = i;
    if (cls < 0) return fail(DIT_EINVAL, "unknown kernel class '%s'", name.c_str());
    mask |= 1u << cls;
    pos = end + 1;
  }
  ctx->prof_mask = mask;
  return 0;
}

extern "C" int dit_profile_stop(dit_ctx *ctx) {
  g_err.clear();
  if (!ctx) return fail(DIT_EINVAL, "ctx is NULL");
  ctx->prof_on = false;
  if (!ctx->prof_rec.empty()) {
    hipError_t err = hipEventSynchronize(ctx->prof_ev[ctx->prof_rec.back().e1]);
    if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
  }
  return 0;
}

extern "C" int dit_profile_get(dit_ctx *ctx, const char *kernel, double *ms, int64_t *launches,
                               double *flops, double *bytes) {
  g_err.clear();
  if (!ctx || !kernel) return fail(DIT_EINVAL, "ctx or kernel is NULL");
  int cls = -1;
  for (int i = 0; i < P_NCLASS; ++i)
    if (!strcmp(kernel, kProfNames[i])) cls = i;
  if (cls < 0) return fail(DIT_EINVAL, "unknown kernel class '%s'", kernel);
  double t = 0.0, f = 0.0, b = 0.0;
  int64_t n = 0;
  for (const auto &r : ctx->prof_rec) {
    if (r.cls != cls) continue;
    float e = 0.f;
    hipError_t err = hipEventElapsedTime(&e, ctx->prof_ev[r.e0], ctx->prof_ev[r.e1]);
    if (err != hipSuccess) return hip_fail(err, "hipEventElapsedTime");
    t += e;
    f += r.flops;
    b += r.bytes;
    ++n;
  }
  if (ms) *ms = t;
  if (launches) *launches = n;
  if (flops) *flops = f;
  if (bytes) *bytes = b;
  return 0;
}
