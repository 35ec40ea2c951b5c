/*
 * dit.h - C ABI of the MI355X (gfx950) denoising-transformer library.
 *
 * The library computes the forward pass of the FLUX.2-klein / FLUX.3-Klein latent
 * flow-matching image transformer and its few-step Euler sampling loop on one GPU.
 * Its shape follows the small C library described for FLUX.2-klein: load a context,
 * generate, free it, read a thread-local error string, NULL / negative on failure
 * ("Flux 2 Klein: Reine C-basierte Inferenz", section "C-Bibliotheks-API"; hakusoku
 * FLUX.2-klein-4B article, sections "CライブラリAPI" and "エラーハンドリング").  It is narrowed
 * to the transformer: text embeddings come in precomputed (cf. the embeddings option,
 * hakusoku article, "コマンドラインオプション") and latents go out unpacked by any VAE.
 *
 * Conventions for every entry point:
 *   - Pointers marked "dev" are device memory owned by the caller (for example torch
 *     tensors).  They must stay valid until the work queued on `stream` has finished.
 *     Pointers marked "host" are read before the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is queued
 *     asynchronously on it; nothing synchronises unless DIT_DEBUG_SYNC=1 is set in the
 *     environment at dit_ctx_create, which synchronises and checks after every kernel, and
 *     checks what each launch of a block or forward wrote for saturated fp16 values and
 *     NaN / Inf (DIT_ENUMERIC).
 *   - One context serves one stream at a time: calls that overlap on one context race on
 *     its workspace.
 *   - DIT_ATTN_GRID=<n> in the environment at dit_ctx_create (0, or a multiple of 8 up to
 *     4096) sets the attention's grid when it splits work (default: the device's compute
 *     units; 0 = never split).  With n, (256-query tile, head) units of the full rounds of n
 *     run whole and the last round's units are split into n equal key-tile shares when they
 *     would fill under 40% of it.  Other values make dit_ctx_create fail with DIT_EINVAL.
 *   - Row-major everywhere.  "D" = hidden, "C" = in_channels, N = n_txt + n_img + n_ref.
 *   - Return values: 0 on success, or DIT_EINVAL / DIT_ENOMEM / DIT_EHIP / DIT_EUNSUPPORTED /
 *     DIT_ENUMERIC;
 *     dit_ctx_create returns NULL on failure.  dit_get_error() then describes the failure.
 *     Faults of queued kernels surface at a later call or synchronisation.
 */
#ifndef DIT_H
#define DIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dit_ctx dit_ctx;

/* element types.  Host weight data: DIT_F32 or DIT_BF16.  Compute types:
 *   DIT_F32   fp32 throughout (no MFMA)
 *   DIT_BF16  bf16 MFMA operands and activations, fp32 accumulation, fp32 residual
 *   DIT_F16   fp16 MFMA operands and activations (bf16 weights are held exactly, up to the
 *             fp16 subnormal grid below 2^-14), fp32 accumulation, fp32 residual; same MFMA
 *             rate as bf16 on gfx950 with 8x finer operand rounding; activations saturate at
 *             +-65504
 *   DIT_FP8   row-wise FP8 ("fp8r": "FLUX.3 Image Klein: offene Gewichte ...", "Was sich
 *             geändert hat"; we0.ai "FLUX 3 Image Klein" article, "Hardwareanforderungen,
 *             Quantisierung und Inferenzlatenz") for the two big projections of every block:
 *             W1 and W2 are held as OCP E4M3 codes with one fp32 scale per row (quantized at
 *             dit_ctx_create from the given values), their inputs (the modulated LayerNorm
 *             output, [attention || SwiGLU]) are quantized per token on the fly, and the
 *             products run on the E4M3 MFMA at twice the 16-bit rate.  Scale = max |row| / 448,
 *             code = value * (448 / max |row|) rounded to nearest even E4M3.  Everything else
 *             computes as DIT_F16.  Needs hidden + mlp_hidden <= 16384. */
enum { DIT_F32 = 0, DIT_BF16 = 1, DIT_F16 = 2, DIT_FP8 = 3 };

/* model families.
 * DIT_FLUX2: n_stream_blocks double-stream blocks (separate text / image weights, joint
 *   attention from the first block), then n_shared_blocks single-stream blocks
 *   ("Flux 2 Klein: Reine C-basierte Inferenz", "Modellarchitektur und Leistung": 5 double,
 *   20 single, hidden 3072, 24 heads).
 * DIT_FLUX3: n_stream_blocks per-mode blocks (text, image and reference streams each with
 *   their own weights, attending only within their stream), then n_shared_blocks joint
 *   blocks sharing one weight set, every token attending every token; image tokens are
 *   modulated with t, text and reference tokens with t = 0 ("FLUX.3 Image Klein in
 *   Diffusers", sections "Entkoppelte Vorverarbeitung und gemeinsame Attention-Blöcke" and
 *   "Modulation pro Token-Typ, Flow-Map-Destillation und 4D-RoPE"). */
enum { DIT_FLUX2 = 0, DIT_FLUX3 = 1 };

/* attention masks: DEFAULT = the block kind's own (per-mode: SEGMENT, others: FULL) */
enum { DIT_MASK_DEFAULT = -1, DIT_MASK_FULL = 0, DIT_MASK_SEGMENT = 1 };

/* error codes.  DIT_ENUMERIC comes only with DIT_DEBUG_SYNC=1: after every launch the library
 * counts, in what that launch wrote, the fp16 values at +-65504 (saturated conversions; the
 * saturating conversion also maps NaN there) and the NaN / Inf values, and fails the call at the
 * first launch that produced any, naming the block and the launch (the C library's error
 * reporting: NULL / negative return and a message, hakusoku FLUX.2-klein-4B article,
 * "エラーハンドリング"). */
enum { DIT_OK = 0, DIT_EINVAL = -1, DIT_ENOMEM = -2, DIT_EHIP = -3, DIT_EUNSUPPORTED = -4,
       DIT_ENUMERIC = -5 };

typedef struct {
  int arch;             /* DIT_FLUX2 or DIT_FLUX3 */
  int hidden;           /* D; multiple of 256, <= 4096, = heads * head_dim  (3072) */
  int heads;            /*                                                  (24)   */
  int head_dim;         /* must be 128: four 32-dim RoPE axes (t, h, w, l)  (128)  */
  int mlp_hidden;       /* F, SwiGLU width; multiple of 128                 (9216) */
  int in_channels;      /* C, latent channels per token; multiple of 64     (128)  */
  int time_dim;         /* sinusoidal timestep embedding width; mult. of 16, <= 4096 (256) */
  int n_stream_blocks;  /* double (FLUX2) or per-mode (FLUX3) blocks        (5)    */
  int n_shared_blocks;  /* single (FLUX2) or joint (FLUX3) blocks           (20/28) */
  int max_tokens;       /* largest N any call will use (sizes the workspace)       */
  int compute;          /* DIT_F16, DIT_BF16, DIT_F32 or DIT_FP8 (see above)        */
  float rope_theta;     /* RoPE base (10000)      */
  float ln_eps;         /* LayerNorm epsilon (1e-6) */
  float rms_eps;        /* QK RMSNorm epsilon (1e-6) */
  int txt_feat_dim;     /* 0, or the width of stacked text-encoder features that
                         * dit_text_features projects to D with txt_in (FLUX.3: 8 hidden
                         * states of 2560 = 20480); multiple of 64, <= 65536 */
  int flow_map;         /* 1: flow-map (timestep-distilled) model: every conditioning row
                         * also gets the embedding of the step's target time (temb_tgt) */
  int double_wiring;    /* DIT_FLUX2 double blocks: 0 parallel (attention and SwiGLU MLP on one
                         * normalised input, the form of the single blocks), 1 sequential
                         * (attention, then the MLP on the updated residual, each with its own
                         * LayerNorm, shift, scale and gate; mod.0.s{s} are then [6D, D]).
                         * "Flux 2 Klein: Reine C-basierte Inferenz" (GeekNews), model
                         * architecture: double-stream blocks with separate text
                         * and image weights; the pages leave their inner wiring open.  Must
                         * be 0 for DIT_FLUX3. */
} dit_config;

/* One named weight tensor in host memory, row-major [out, in].  dtype DIT_F32: float
 * values; DIT_BF16: uint16 bf16 bit patterns.  Values are converted to the compute type
 * (round-to-nearest-even) and copied during dit_ctx_create; the caller keeps ownership.
 * Names and shapes (b = block index, s = weight set):
 *   img_in      [D, C]       input projection of image and reference latents
 *   temb.l1     [D, time_dim], temb.l2 [D, D]   timestep MLP
 *   temb_tgt.l1 [D, time_dim], temb_tgt.l2 [D, D]   target-time MLP (flow_map = 1 only)
 *   txt_in      [D, txt_feat_dim]   text-feature projection (txt_feat_dim > 0 only)
 *   final.mod   [2D, D]      output-head modulation (shift || scale)
 *   final.out   [C, D]       output projection to the velocity
 *   mod.0.s{s}  [3D, D]      modulation (shift || scale || gate) shared by the stream blocks,
 *               per set; [6D, D] with double_wiring = 1: (shift || scale || gate) of the
 *               attention half, then of the MLP half
 *   mod.1.s0    [3D, D]      modulation shared by the shared (single / joint) blocks
 *   blk{b}.s{s}.mod  [3D, D] (or [6D, D] as above)  block b's own modulation of set s; when
 *               given it replaces the shared mod.{kind}.s{s} for that block.  The pages tie
 *               scale, shift and gate to the timestep embedding without saying whether each
 *               block has its own projection ("FLUX.3 Image Klein in Diffusers", section
 *               "Modulation pro Token-Typ, Flow-Map-Destillation und 4D-RoPE"); both forms are
 *               data.  Entries may alias: entries whose data pointer (and dtype) is the same
 *               are uploaded and computed once.  A shared entry that no block uses is an error.
 *   blk{b}.s{s}.w1 [3D+2F, D]  rows Q | K | V | gate | up (head-major Q, K, V)
 *   blk{b}.s{s}.w2 [D, D+F]    output projection of [attention || SwiGLU]
 *   blk{b}.s{s}.qn, .kn [128]  query / key RMSNorm scales
 * Sets: stream blocks have 2 (FLUX2: text, image; references use the image set) or 3
 * (FLUX3: text, image, reference); shared blocks have 1. */
typedef struct {
  const char *name;
  const void *data;     /* host */
  int64_t numel;
  int dtype;            /* DIT_F32 or DIT_BF16 */
} dit_tensor;

/* Validate cfg, upload and repack all weights, allocate the workspace for max_tokens.
 * Every tensor listed above must be present exactly once with the right numel; unknown
 * names are an error.  Returns NULL on failure (no device, bad config, missing or
 * misshaped tensor, out of device memory). */
dit_ctx *dit_ctx_create(const dit_config *cfg, const dit_tensor *weights, int n_weights);

/* Release all device memory of ctx (synchronises the device first).  NULL is a no-op. */
void dit_ctx_free(dit_ctx *ctx);

/* One transformer block in place on the residual stream.
 *   x     dev fp32 [N, D], in/out; rows ordered text || image || reference
 *   pos   dev fp32 [N, 4] RoPE coordinates (t, h, w, l) per token
 *   cond  dev fp32 [n_seg, D]: one conditioning vector per non-empty segment, in the order
 *         text, image, reference (n_seg = number of n_txt, n_img, n_ref that are > 0)
 *   mask  DIT_MASK_DEFAULT / FULL / SEGMENT
 * Computes x <- x + gate_s * ([attention || SwiGLU](LN(x) * (1 + scale_s) + shift_s) W2^T)
 * with (shift, scale, gate)_s = W_mod . SiLU(cond row of s), W_mod the block's modulation
 * projection of the segment's weight set
 * ("FLUX.3 Image Klein in Diffusers": parallel attention and SwiGLU MLP on one normalised
 * input, QK RMSNorm, adaLN from the timestep embedding, 4D RoPE).  Double blocks of a
 * double_wiring = 1 model run the two halves in sequence instead:
 *   x <- x + gate1_s * (attention(LN(x) * (1 + scale1_s) + shift1_s) W2[:, :D]^T)
 *   x <- x + gate2_s * (SwiGLU(LN(x) * (1 + scale2_s) + shift2_s) W2[:, D:]^T)
 * with the Q|K|V rows of W1 in the first and its gate/up rows in the second.
 * Requires 0 <= block < n_stream_blocks + n_shared_blocks, 1 <= N <= max_tokens. */
int dit_block_forward(dit_ctx *ctx, int block, float *x, int n_txt, int n_img, int n_ref,
                      const float *pos, const float *cond, int mask, void *stream);

/* One full transformer call at time t: v = velocity of the image tokens.
 *   lat      dev fp32 [gh*gw, C]      packed image latents (16x16 px per token)
 *   ref_lat  dev fp32 [rgh*rgw, C]    reference latents, or NULL with rgh = rgw = 0
 *   txt      dev fp32 [n_txt, D]      text embeddings (enter the residual as they are)
 *   v        dev fp32 [gh*gw, C]      output
 * Positions: text i -> (0,0,0,i), image (r,c) -> (0,r,c,0), reference (r,c) -> (0,r,c,-1)
 * ("FLUX.3 Image Klein in Diffusers", "Modulation pro Token-Typ, Flow-Map-Destillation und
 * 4D-RoPE"). */
int dit_forward(dit_ctx *ctx, const float *lat, const float *ref_lat, const float *txt,
                int n_txt, int gh, int gw, int rgh, int rgw, float t, float *v, void *stream);

/* Few-step Euler sampling from t = 1 (noise) to t = 0 (clean) on the uniform schedule
 * t_i = 1 - i/n_steps: lat <- lat + (t_i - t_{i+1}) * v(lat, t_i).
 *   lat   dev fp32 [gh*gw, C], in/out.  seed >= 0: first filled with N(0,1) noise from
 *         Philox4x32-10 (counter = element index / 4, key = seed) and Box-Muller;
 *         seed < 0: lat is used as given.
 * Other arguments as in dit_forward.  n_steps >= 1. */
int dit_denoise(dit_ctx *ctx, float *lat, const float *txt, int n_txt, int gh, int gw,
                const float *ref_lat, int rgh, int rgw, int n_steps, int64_t seed,
                void *stream);

/* FLUX.3 text features to transformer width: txt = feat . txt_in^T.
 *   feat  dev fp32 [n_txt, txt_feat_dim]: per text token the hidden states of text-encoder
 *         layers 4, 8, ..., 32 (of 36) stacked in that order, 8 x 2560 values
 *   txt   dev fp32 [n_txt, D] output, the txt argument of the calls below
 * ("FLUX.3 Image Klein in Diffusers", "Zweistufiger Transformer und Tokenisierung im
 * Detail": eight hidden states of Qwen3-VL per token, stacked to 20480 values, one linear
 * layer to 3072.)  Runs once per prompt, outside the sampling loop.  Requires
 * txt_feat_dim > 0 and 1 <= n_txt <= max_tokens. */
int dit_text_features(dit_ctx *ctx, const float *feat, int n_txt, float *txt, void *stream);

/* dit_forward for a flow-map model (flow_map = 1): the call also receives the time t_target
 * its step jumps to, whose embedding (temb_tgt) is added to every conditioning row
 * ("FLUX.3 Image Klein in Diffusers", "Modulation pro Token-Typ, Flow-Map-Destillation und
 * 4D-RoPE": the distilled checkpoint gets the target timestep through its own embedding,
 * added to every token's modulation).  dit_forward and dit_forward_cfg fail on a flow-map
 * context; dit_denoise and dit_denoise_cfg pass t_{i+1} as the target of step i. */
int dit_forward_flow(dit_ctx *ctx, const float *lat, const float *ref_lat, const float *txt,
                     int n_txt, int gh, int gw, int rgh, int rgw, float t, float t_target,
                     float *v, void *stream);

/* Classifier-free guidance: one call of the transformer on two sequences at once, the
 * conditional text txt and the unconditional text txt_uncond (both dev fp32 [n_txt, D]), each
 * with the same latents, references and time, and
 *   v = v_u + guidance * (v_c - v_u),
 * computed as guidance * v_c + (1 - guidance) * v_u, conditional branch first.
 * (Guidance scale: the C tool's generation parameters, hakusoku FLUX.2-klein-4B article,
 * "CライブラリAPI"; the non-distilled base checkpoint samples with guidance 3.5, we0.ai
 * "FLUX 3 Image Klein" article, checkpoint table.  The combination is the standard one of
 * classifier-free guidance; the pages print no formula.)
 * The two sequences are stacked as one batch of 2 (n_txt + gh*gw + rgh*rgw rows each), so
 * max_tokens must cover twice the sequence.  Each sequence attends only to itself.
 * guidance must be finite; other arguments as in dit_forward. */
int dit_forward_cfg(dit_ctx *ctx, const float *lat, const float *ref_lat, const float *txt,
                    const float *txt_uncond, int n_txt, int gh, int gw, int rgh, int rgw,
                    float t, float guidance, float *v, void *stream);

/* dit_denoise with the guided velocity of dit_forward_cfg at every step:
 * lat <- lat + (t_i - t_{i+1}) * (guidance * v_c + (1 - guidance) * v_u). */
int dit_denoise_cfg(dit_ctx *ctx, float *lat, const float *txt, const float *txt_uncond,
                    int n_txt, int gh, int gw, const float *ref_lat, int rgh, int rgw,
                    int n_steps, float guidance, int64_t seed, void *stream);

/* One generation request for dit_forward_ex / dit_denoise_ex: the inputs besides the
 * latents, in one place, so that guidance, several reference images and image-to-image
 * combine freely.  D, C as above. */
typedef struct {
  const float *txt;         /* dev fp32 [n_txt, D] text embeddings (conditional branch) */
  const float *txt_uncond;  /* dev fp32 [n_txt, D] unconditional text, or NULL: no guidance */
  int n_txt;
  float guidance;           /* guidance scale g when txt_uncond != NULL (as dit_forward_cfg) */
  int gh, gw;               /* image token grid (16x16 px per token) */
  const float *ref_lat;     /* dev fp32 [sum_k rows_k * cols_k, C]: the latents of the reference
                             * images one after another, or NULL with n_refs = 0 */
  int n_refs;               /* 0..10 reference images; reference k (from 0) sits at sequence
                             * coordinate l = -(k+1) on the image's (h, w) grid */
  const int *ref_grids;     /* host int [n_refs][2]: (rows, cols) of each reference */
} dit_request;
/* ("Up to ten reference images": we0.ai "FLUX 3 Image Klein" article, model summary; each
 * keeps its own size and gets l = -(k+1): "FLUX.3 Image Klein in Diffusers", sections
 * "Zweistufiger Transformer und Tokenisierung im Detail" and "Modulation pro Token-Typ,
 * Flow-Map-Destillation und 4D-RoPE".) */

/* One transformer call for a request at time t; t_target is read by flow-map models only
 * (the step's target time, as dit_forward_flow).  With guidance v = g v_c + (1 - g) v_u.
 * max_tokens must cover n_txt + gh*gw + all reference tokens, twice with guidance. */
int dit_forward_ex(dit_ctx *ctx, const dit_request *request, const float *lat, float t,
                   float t_target, float *v, void *stream);

/* Sampling for a request: n_steps Euler steps on t_i = 1 - i/n_steps, of which the last
 * floor(n_steps * strength) run.
 *   strength = 1: text-to-image.  lat is the starting noise: drawn from seed when seed >= 0,
 *     else copied from noise when noise != NULL, else used as it is.
 *   0 < strength < 1: image-to-image ("-t, --strength", 0.0-1.0, default 0.75, hakusoku
 *     FLUX.2-klein-4B article, "コマンドラインオプション"; strength in the C API's generation
 *     parameters).  lat holds the clean latents of the input image.  They are moved to
 *     t_s = floor(n_steps * strength) / n_steps on the straight path to the noise:
 *       lat = t_s * noise + (1 - t_s) * lat,
 *     with noise from the noise argument (dev fp32 [gh*gw, C]) or, when it is NULL, drawn
 *     from seed (then seed >= 0 is required).  n_steps * strength >= 1 is required.
 * lat dev fp32 [gh*gw, C] in/out. */
int dit_denoise_ex(dit_ctx *ctx, const dit_request *request, float *lat, int n_steps,
                   float strength, const float *noise, int64_t seed, void *stream);

/* Fill dst (dev fp32, n elements) with the N(0,1) noise dit_denoise draws for seed. */
int dit_fill_noise(float *dst, int64_t n, int64_t seed, void *stream);

/* Row-wise FP8 building blocks of DIT_FP8, on caller-owned device buffers (no context):
 * dit_quantize_rows_fp8: scale[r] = max_c |x[r][c]| / 448 (fp32), q[r][c] = E4M3 code of
 *   x[r][c] * (448 / max_c |x[r][c]|) (fp32 product, clamped to +-448), rounded to nearest
 *   even; a zero row gets scale 0 and codes 0.  x dev fp32 [rows][ldx], q dev uint8
 *   [rows][ldq], scale dev fp32 [rows]; cols <= 16384, cols, ldx, ldq multiples of 8.
 * dit_gemm_fp8: y[i][j] = sx[i] * sw[j] * sum_k qx[i][k] * qw[j][k] (fp32), the E4M3 MFMA
 *   product: qx dev uint8 [m][ldx] (rows readable up to m rounded up to 256), sx [m],
 *   qw dev uint8 [n][ldw], sw [n], y dev fp32 [m][ldy]; n % 256 == 0, k % 128 == 0, ldx and
 *   ldw multiples of 16, ldy of 4.  The MFMA truncates products more than about 12 bits
 *   below the largest one of its group of k, so results differ from the exact sum by a few
 *   units of 2^-12 of the largest products.
 * Both return 0 once the work is queued on stream; DIT_EINVAL for a NULL buffer, a negative
 * row count or a stride out of the ranges above (ldx, ldq >= cols; ldx, ldw >= k; ldy >= n),
 * DIT_EUNSUPPORTED for n or k that are not multiples of 256 and 128, DIT_EHIP when a launch
 * fails; the message is in dit_get_error().  rows = 0 or m = 0 is no work. */
int dit_quantize_rows_fp8(const float *x, int rows, int cols, int ldx, uint8_t *q, int ldq,
                          float *scale, void *stream);
int dit_gemm_fp8(const uint8_t *qx, const float *sx, int m, int ldx, const uint8_t *qw,
                 const float *sw, int n, int ldw, int k, float *y, int ldy, void *stream);

/* dit_gemm_fp8 for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): same arguments, checks, return codes
 * and result up to fp32 summation order.  It allocates nothing; in exchange, launches whose
 * 256 x 256 tiles fill under half of the compute units cut k into slices (as the library's
 * block projections do) whose fp32 partial tiles live in a file-scope device array of the
 * library, 32 MiB (128 partial tiles) per device, held until the process ends.  The slice
 * count is capped to what the array holds, so no size is rejected for want of room.  Every
 * call on one device shares that device's array: calls that overlap on one device (several
 * streams, several threads) race and must be serialised by the caller. */
int dit_gemm_fp8_static(const uint8_t *qx, const float *sx, int m, int ldx, const uint8_t *qw,
                        const float *sw, int n, int ldw, int k, float *y, int ldy, void *stream);

/* Workspace buffer of the last call, for inspection after the stream has finished:
 * "xm" (LayerNorm+modulation output, [N, D]), "qkv" ([N, 3D], q and k after RMSNorm and
 * RoPE; v only on the fp32 path), "vt" (16-bit and FP8 paths: V transposed, [H * 128 rows of
 * one head's dim][token'], where every 32 tokens are stored in the order 0-3, 16-19, 4-7,
 * 20-23, 8-11, 24-27, 12-15, 28-31, then zeros; NULL on the fp32 path), "cat" ([N, D+F],
 * attention output || SwiGLU output), "mod" (fp32
 * [M][3][R]: distinct modulation projection in order of first use (blocks in order, sets in
 * order), conditioning row, shift || scale || gate; R = 3D, or 6D with double_wiring = 1,
 * whose stream-block rows hold both halves), "x" (fp32 [N, D], the
 * residual stream of dit_forward / dit_denoise after the last block).  *dtype receives
 * the element type (compute type for xm, qkv, cat; DIT_F32 for mod and x; with DIT_FP8, xm
 * holds E4M3 codes (DIT_FP8) and qkv, cat are DIT_F16); *row_stride the
 * elements per row.  NULL for an unknown name. */
const void *dit_debug_buffer(dit_ctx *ctx, const char *name, int *dtype, int64_t *row_stride);

/* Per-kernel timing, for benchmarks.  dit_profile_start makes the following calls record a
 * hipEvent on their stream before and after each kernel launch (up to max_launches launches;
 * later ones are not timed).  dit_profile_stop ends recording and waits for the last event.
 * dit_profile_get sums, over the recorded launches of one kernel class, the elapsed time (ms),
 * the launch count, and the algorithmic work the library attributes to them: FLOPs (GEMMs,
 * attention: 4 * D per attended query-key pair) and HBM bytes (memory-bound kernels).
 * Kernel classes: "ln_modulate", "linear1", "qk_norm_rope", "attention", "linear2",
 * "conditioning", "embed", "final". */
int dit_profile_start(dit_ctx *ctx, int max_launches);
/* Restrict the timed launches to a comma-separated list of kernel classes (for example
 * "linear1"), so that a benchmark can time one class with few events in the stream; NULL or ""
 * selects every class.  Unknown names: DIT_EINVAL, selection unchanged. */
int dit_profile_select(dit_ctx *ctx, const char *kernels);
int dit_profile_stop(dit_ctx *ctx);
int dit_profile_get(dit_ctx *ctx, const char *kernel, double *ms, int64_t *launches,
                    double *flops, double *bytes);

/* Sustained matrix-core rate of the current device, the measured denominator beside the
 * published peak: two waves on every SIMD of every compute unit run iters x 8 independent
 * v_mfma_f32_16x16x32 of the compute type (DIT_F16 or DIT_BF16, the form the block kernels
 * use) on register operands.  *tflops = executed flops / event-timed duration; *ghz = the
 * clock that rate implies at one such MFMA per 16 cycles per SIMD (derived, not a counter
 * reading).  Allocates and frees a few bytes of device memory and synchronises the stream: a
 * benchmark tool, not for use inside a timed region.  1 <= iters <= 2^24 (10^5 takes about
 * 14 ms).  DIT_EINVAL for other arguments, DIT_EHIP on a HIP failure. */
int dit_mfma_rate(int compute, int iters, double *tflops, double *ghz, void *stream);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *dit_get_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
