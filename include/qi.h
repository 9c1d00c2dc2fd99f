/*
 * qi.h -- C ABI of the MI355X (gfx950) single-stream DiT denoising step with
 * block-causal attention and exact text-K/V reuse.
 *
 * Pages cited (by title and section):
 *   [PORT] "Qwen-Image-2.1 port" knowledge page of the coreai-model-zoo: the
 *          pieces table, DiT row (32 single-stream blocks, one modulation
 *          Linear shared by all blocks with rows for the sampled t and t = 0,
 *          ZeroCenterRMSNorm text projection, SwiGLU x3, 3-axis interleaved
 *          RoPE 16/56/56, block-causal attention as two SDPA calls).
 *   [HOST] "Host contract -- RGBA-Image-2.1 (Core AI port of Qwen-Image-2.1)":
 *          s.1 The graphs (the DiT signature), s.4 Sequence layout and RoPE,
 *          s.6 Sampler.
 *   [MLX]  "Qwen-Image-2.1 on MLX, faster and exact": "Text K/V reuse (exact,
 *          on by default)".
 *
 * Conventions for every entry point:
 *   - bf16 values travel as uint16_t bit patterns; fp32 as float.
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary host memory.  The caller owns every buffer; the
 *     library allocates nothing per call and keeps no mutable global state
 *     beyond the optional kernel-timing facility at the end of this header
 *     and the static per-GPU scratch of qi_dit_step_noalloc.
 *   - Linear weights use the [out, in] row-major layout, so each projection is
 *     y = x W^T.  Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without synchronising.
 *   - Every argument is validated on the host before anything is enqueued; a
 *     failed check returns a negative qi_status and enqueues nothing.  A HIP
 *     launch error returns QI_ERR_HIP; faults inside kernels surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI.
 */
#ifndef QI_H_
#define QI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qi_status;
#define QI_OK 0
#define QI_ERR_NULL (-1)        /* a required pointer is NULL */
#define QI_ERR_SHAPE (-2)       /* inconsistent dimensions */
#define QI_ERR_RANGE (-3)       /* a size outside its supported range */
#define QI_ERR_ALIGN (-4)       /* a device pointer not 16-byte aligned */
#define QI_ERR_WORKSPACE (-5)   /* workspace smaller than qi_workspace_bytes */
#define QI_ERR_CACHE (-6)       /* K/V cache invalid or made for another shape */
#define QI_ERR_HIP (-7)         /* a HIP runtime call or launch failed */
#define QI_ERR_UNSUPPORTED (-8) /* a valid request this library does not handle */

/* Pass kinds of one block.  JOINT runs the [text L | image N] sequence (step 1
 * of a render, or full recompute); IMAGE_ONLY runs the N image rows against
 * text K/V cached from a joint pass ([MLX] "Text K/V reuse"). */
#define QI_MODE_JOINT 0
#define QI_MODE_IMAGE_ONLY 1

/* Model dimensions.  head_dim must be 128 and heads = hidden / 128 ([PORT] DiT
 * row: 32 heads x 128 at hidden 4096).  hidden % 256 == 0 (256..8192),
 * ffn % 64 == 0, txt_dim % 256 == 0 (256..8192), 1 <= n_blocks <= 256. */
typedef struct {
  int32_t hidden, heads, head_dim, ffn, n_blocks, txt_dim;
} qi_dims;

/* Device weights of one block (bf16 as uint16, norms fp32).
 *   w_qkv  [3H, H]: rows [0,H) q, [H,2H) k, [2H,3H) v; head h owns rows h*128..
 *   w_o    [H, H]
 *   w_gu   [2F, H]: rows [0,F) gate (SiLU), [F,2F) up
 *   w_down [H, F]
 *   norm1, norm2 [H] fp32 RMSNorm weights. */
typedef struct {
  const uint16_t *w_qkv, *w_o, *w_gu, *w_down;
  const float *norm1, *norm2;
} qi_block_w;

/* Device weights of the whole DiT.  `blocks` is a HOST array of n_blocks
 * qi_block_w.  w_mod [4H, H] + b_mod [4H]: the one modulation Linear shared by
 * every block; w_img [H, 64] + b_img [H]: img-in; txt_norm [D] (zero-centred
 * weight), w_txt [H, D] + b_txt [H]: text projection; norm_out [H], w_out
 * [64, H] + b_out [64]: proj_out. */
typedef struct {
  const qi_block_w *blocks;
  const uint16_t *w_mod; const float *b_mod;
  const uint16_t *w_img; const float *b_img;
  const float *txt_norm; const uint16_t *w_txt; const float *b_txt;
  const float *norm_out; const uint16_t *w_out; const float *b_out;
} qi_model_w;

/* Text K/V cache ([MLX] "Text K/V reuse": 2 x blocks x tokens x hidden bf16).
 * kv is device memory of qi_kv_cache_bytes(dims, L) bytes.  Block b's slot
 * starts at kv + b * qi_kv_slot_elems(dims, L) and holds
 *   K  [heads][L][128]          (RoPE applied)
 *   Vt [heads][128][Lp]         (V transposed, Lp = L rounded up to 64;
 *                                columns >= L are never read as values)
 * `valid` is set to 1 by qi_text_kv_capture; L, n_blocks and hidden must match
 * the step that reads it. */
typedef struct {
  uint16_t *kv;
  int32_t L, n_blocks, hidden, valid;
} qi_kv_cache;

/* Status text (static string). */
const char *qi_status_str(qi_status s);
/* Library version string (static). */
const char *qi_version(void);

/* ---------------------------------------------------------------- host tables */

/* One RoPE axis table ([HOST] s.4): rows for positions -1024..8191 (row p+1024),
 * column k the angle p * 1/10000^(2k/d), each step rounded to fp32, cos/sin of
 * the fp32 angle evaluated in float64 and rounded once.  d in {16, 56} (any even
 * d in 2..128 is accepted).  cos_out, sin_out: host [9216][d/2]. */
qi_status qi_rope_axis_table(int32_t d, float *cos_out, float *sin_out);

/* Per-token RoPE rows ([HOST] s.4): text token i -> position (i, i, i); image
 * token (y, x), index y*w + x -> (L, y - (h - h/2), x - (w - w/2)); a token's 64
 * values are its axis-0 (8), axis-1 (28) and axis-2 (28) rows concatenated.
 * Host outputs: txt_cos/txt_sin [L][64], img_cos/img_sin [h*w][64].
 * Errors: QI_ERR_NULL; QI_ERR_RANGE if L < 0, h or w < 1, or a position falls
 * outside -1024..8191. */
qi_status qi_rope_tables(int32_t L, int32_t h, int32_t w, float *txt_cos, float *txt_sin,
                         float *img_cos, float *img_sin);

/* FlowMatch Euler schedule ([HOST] s.6): sigmas = linspace(1, 1/steps, steps),
 * exponential shift with mu = N m + b (base_shift 0.5 at 256 tokens, max_shift
 * 0.9 at 8192), terminal stretch to 0.02, timesteps = sigmas * 1000, then
 * sigmas ++ [0].  Each array operation in fp32.  Host outputs: sigmas
 * [steps+1], timesteps [steps].  The DiT's timestep input for step i is
 * timesteps[i] / 1000 in fp32.  Errors: QI_ERR_NULL; QI_ERR_RANGE if steps < 2
 * or n_img_tokens < 1. */
qi_status qi_flow_sigmas(int32_t steps, int32_t n_img_tokens, float *sigmas, float *timesteps);

/* ---------------------------------------------------------------- sizes */

/* Workspace bytes qi_dit_step / qi_text_kv_capture / qi_dit_block_fwd need for
 * a joint pass over L text and N image tokens (enough for an image-only pass
 * too).  0 if the dims are invalid. */
size_t qi_workspace_bytes(const qi_dims *d, int32_t L, int32_t N);
/* Elements (uint16) of one block's cache slot, and bytes of the whole cache. */
size_t qi_kv_slot_elems(const qi_dims *d, int32_t L);
size_t qi_kv_cache_bytes(const qi_dims *d, int32_t L);

/* ---------------------------------------------------------------- the step */

/* One single-stream block ([PORT] DiT row), in place on the fp32 residual
 * stream x [rows][H], rows = L + N (JOINT, text rows first) or N (IMAGE_ONLY):
 *   h  = bf16(RMSNorm(x; norm1) * (1 + scale1[row]))
 *   q,k,v = h W_qkv^T; RoPE on q, k (adjacent pairs 2k, 2k+1 rotated by the
 *          row's cos/sin[k]); rounded once to bf16
 *   o  = block-causal attention: a text row i sees text keys 0..i; an image
 *        row sees every text key and every image key; scale 1/sqrt(128)
 *   x += gate1[row] * (o W_o^T)
 *   h2 = bf16(RMSNorm(x; norm2) * (1 + scale2[row]))
 *   x += gate2[row] * ((SiLU(h2 Wg^T) * (h2 Wu^T)) W_down^T)
 * mod: device fp32 [2][4H]; row 0 is the t = 0 row (text rows), row 1 the
 * sampled-t row (image rows); each row is (scale1, gate1, scale2, gate2).
 * cos, sin: device fp32 [rows][64], the rows' RoPE values in row order.
 * kv_txt: this block's cache slot (layout of qi_kv_cache) or NULL.  JOINT: if
 * non-NULL, the text rows' K/V are written there (capture), else into the
 * workspace.  IMAGE_ONLY: required, read.
 * Ranges: 1 <= L <= 512, 1 <= N <= 16384 (the DiT's L axis and the 2048^2
 * token count of [PORT]).
 * Errors: NULL, SHAPE, RANGE, ALIGN, WORKSPACE (ws_bytes < qi_workspace_bytes),
 * HIP. */
qi_status qi_dit_block_fwd(const qi_dims *d, const qi_block_w *w, int32_t L, int32_t N,
                           int32_t mode, float *x, const float *mod, const float *cos,
                           const float *sin, uint16_t *kv_txt, void *ws, size_t ws_bytes,
                           void *stream);

/* One DiT forward, the DiT graph of [HOST] s.1: img_tokens [N][64], txt_feats
 * [L][txt_dim] (device fp32), timestep t (host fp32, already divided by 1000),
 * txt_cos/txt_sin [L][64], img_cos/img_sin [N][64] (device fp32) -> vel [N][64]
 * (device fp32).
 *   modulation rows m(0), m(t) = W_mod e(tau) + b_mod with e(tau) the width-H
 *     sinusoid [cos | sin](1000 tau 10000^(-j/(H/2)));
 *   x_txt = ZeroCenterRMSNorm(txt_feats) W_txt^T + b_txt;  x_img = img_tokens
 *     W_img^T + b_img;
 *   n_blocks blocks (qi_dit_block_fwd);
 *   vel = RMSNorm(x_img; norm_out) W_out^T + b_out.
 * cache NULL: joint pass (full recompute; txt_feats required).  cache valid:
 * image rows only, text K/V read from the cache (txt_feats, txt_cos, txt_sin
 * may be NULL).  The image rows of both give bit-identical vel.
 * Errors: as qi_dit_block_fwd; QI_ERR_CACHE if the cache is not valid or was
 * made for another L, n_blocks or hidden. */
qi_status qi_dit_step(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N,
                      const float *img_tokens, const float *txt_feats, float timestep,
                      const float *txt_cos, const float *txt_sin, const float *img_cos,
                      const float *img_sin, const qi_kv_cache *cache, float *vel, void *ws,
                      size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): qi_dit_step
 * with its workspace taken from a static scratch array inside the library
 * instead of a caller buffer.  Same arguments, same kernels and bit-identical
 * results as qi_dit_step, minus ws / ws_bytes.  The scratch is one
 * QI_NOALLOC_SCRATCH_BYTES (160 MiB) array per GPU, held from the library's
 * first use on that GPU until the process ends; its device address is looked
 * up once per device (hipGetSymbolAddress, the calling thread's current
 * device).  The call allocates nothing and clears nothing (no kernel of the
 * step reads workspace it has not written in the same call).  Every call on
 * one GPU uses the same scratch: calls that may overlap on one GPU (two
 * streams, two threads) race and must be serialised by the caller.
 * Limit: qi_workspace_bytes(d, L, N) <= QI_NOALLOC_SCRATCH_BYTES, e.g. the
 * 384^2 step (hidden 4096, L 494, N 576, 138 MiB) fits, the 1024^2 step does
 * not.  Errors: as qi_dit_step; QI_ERR_WORKSPACE when the request needs more
 * scratch than that (checked before anything else is done), QI_ERR_HIP if the
 * scratch address cannot be obtained. */
#define QI_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)
qi_status qi_dit_step_noalloc(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N,
                              const float *img_tokens, const float *txt_feats, float timestep,
                              const float *txt_cos, const float *txt_sin, const float *img_cos,
                              const float *img_sin, const qi_kv_cache *cache, float *vel, void *stream);

/* Step 1 of a render with reuse ([MLX] "Text K/V reuse"): the joint pass of
 * qi_dit_step that also writes every block's text K/V into cache->kv, then sets
 * cache->L, n_blocks, hidden and valid = 1.  vel may be NULL (the step-1 vel is
 * then not written).  Errors: as qi_dit_step; QI_ERR_NULL if cache or
 * cache->kv is NULL. */
qi_status qi_text_kv_capture(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N,
                             const float *img_tokens, const float *txt_feats, float timestep,
                             const float *txt_cos, const float *txt_sin, const float *img_cos,
                             const float *img_sin, qi_kv_cache *cache, float *vel, void *ws,
                             size_t ws_bytes, void *stream);

/* Euler update of the FlowMatch sampler ([HOST] s.6), in place on device fp32
 * x[n]: x = x + (sigma_next - sigma_cur) * vel, the difference computed in fp32
 * on the host, then a fp32 multiply and a fp32 add per element (no fused
 * multiply-add).  n = 0 is a no-op.  Errors: NULL, RANGE (n < 0), ALIGN, HIP. */
qi_status qi_euler_update(float *x, const float *vel, float sigma_cur, float sigma_next,
                          int64_t n, void *stream);

/* DPM++ 2M sampler coefficients ([MLX] "Optional modes" names the sampler;
 * the method is DPM-Solver++(2M), Lu et al. 2022, the multistep second-order
 * data-prediction solver, written for the flow x = (1 - sigma) x0 + sigma eps
 * with alpha = 1 - sigma, lambda = log(alpha / sigma), x0 = x - sigma v).  One
 * step sigma_cur -> sigma_next: x_next = a x - b D with a = sigma_next /
 * sigma_cur, b = alpha_next (e^-h - 1), h = lambda_next - lambda_cur; D = x0
 * (first order) or c1 x0 - c2 x0_prev with c2 = 1 / (2 r), r = h_prev / h,
 * c1 = 1 + c2 (second order).  First order when has_prev = 0, after sigma_prev
 * = 1 (r infinite) and at the final step (sigma_next = 0: a = 0, b = -1).
 * Host, double precision: coef[4] = {a, b, c1, c2}.  Returns the order (1 or
 * 2), or QI_ERR_NULL, or QI_ERR_RANGE unless 0 < sigma_cur <= 1, 0 <=
 * sigma_next < sigma_cur and (without a previous step) sigma_cur < sigma_prev
 * <= 1. */
qi_status qi_dpmpp_2m_coeffs(int32_t has_prev, float sigma_prev, float sigma_cur, float sigma_next,
                             double *coef);

/* One DPM++ 2M update on the device, in place on fp32 x[n] (same sigmas as the
 * Euler sampler, qi_flow_sigmas): p = sigma_cur vel, x0 = x - p, D = x0 or
 * c1 x0 - c2 x0_prev, x = a x - b D, each a separately rounded fp32 operation
 * in that order with the coefficients of qi_dpmpp_2m_coeffs rounded once to
 * fp32; x0 is written to x0_prev (device fp32 [n]) for the next step, which
 * passes has_prev = 1 and this step's sigma_cur as sigma_prev.  n = 0 is a
 * no-op.  Errors: NULL, RANGE, HIP. */
qi_status qi_dpmpp_2m_update(float *x, const float *vel, float *x0_prev, int32_t has_prev,
                             float sigma_prev, float sigma_cur, float sigma_next, int64_t n,
                             void *stream);

/* ---------------------------------------------------------------- true CFG */

/* Workspace bytes qi_dit_step_cfg needs (0 for invalid dims or N). */
size_t qi_cfg_workspace_bytes(const qi_dims *d, int32_t N);

/* One image-only step of true classifier-free guidance with reuse ([MLX]
 * "Optional modes": a second forward per step, on the negative prompt; "Text
 * K/V reuse": the negative prompt's K/V in a second slot).  Both branches run
 * through every block together as 2N image rows: branch 0 (positive prompt)
 * reads its text K/V from cache_pos, branch 1 (negative prompt) from
 * cache_neg, each captured by qi_text_kv_capture with its own prompt (the two
 * L may differ).  Each branch's vel is bit-identical to qi_dit_step on that
 * branch's cache alone (and so to its full joint recompute).
 *   img_tokens: device fp32 [N][64], the same latents for both branches;
 *   img_cos, img_sin: device fp32 [2][N][64], branch b's image RoPE rows (they
 *     depend on the branch's L, see qi_rope_tables);
 *   vel: device fp32 [2][N][64] out, [pos | neg].
 * Combine with qi_euler_update_cfg.  Errors: NULL, SHAPE, RANGE, ALIGN,
 * WORKSPACE (ws_bytes < qi_cfg_workspace_bytes), CACHE (a cache not valid,
 * made for another n_blocks or hidden, or both caches the same buffer), HIP. */
qi_status qi_dit_step_cfg(const qi_dims *d, const qi_model_w *w, int32_t N,
                          const float *img_tokens, float timestep, const float *img_cos,
                          const float *img_sin, const qi_kv_cache *cache_pos,
                          const qi_kv_cache *cache_neg, float *vel, void *ws, size_t ws_bytes,
                          void *stream);

/* The Euler update with the guidance combination fused in ([MLX] "Optional
 * modes", noise = neg + g (pos - neg); [HOST] s.6 for the update): in place on
 * device fp32 x[n], with vel = [pos | neg] (2n floats),
 *   x = x + (sigma_next - sigma_cur) * (neg + g * (pos - neg)),
 * the sigma difference computed in fp32 on the host and every other operation
 * a separately rounded fp32 operation in the order written (no fused
 * multiply-add).  n = 0 is a no-op.  Errors: NULL, RANGE (n < 0, guidance not
 * finite), ALIGN, HIP. */
qi_status qi_euler_update_cfg(float *x, const float *vel, float guidance, float sigma_cur,
                              float sigma_next, int64_t n, void *stream);

/* ---------------------------------------------------------------- first-block cache */

/* Device bytes of a first-block-cache buffer for N image rows (0 for invalid
 * dims or N).  The caller allocates it (16-byte aligned) and calls
 * qi_fbc_reset before the first step of a render. */
size_t qi_fbc_bytes(const qi_dims *d, int32_t N);

/* Marks the buffer's cached residuals invalid and zeroes its counts (one small
 * kernel on the stream; no memset, so it may sit in a captured graph).
 * Errors: NULL, ALIGN, WORKSPACE (fbc_bytes too small for the state), HIP. */
qi_status qi_fbc_reset(void *fbc, size_t fbc_bytes, void *stream);

/* An image-only step with the first-block cache ([MLX] "Optional modes",
 * Fast mode; the option table's threshold is 0.08).  Block 0 always runs.
 * Its residual r0 = x1 - x0 (x0 after the embed, x1 after block 0) is
 * compared with the one cached at the last step that ran every block:
 *   change = sum |r0 - r0_cached| / sum |r0_cached|  (over all image rows and
 *   features; fp32 differences, float64 sums in a fixed order).
 * If the cache is valid and change < threshold, blocks 1..n_blocks-1 are
 * skipped and x = x1 + rem_cached; otherwise they run, and r0 and their
 * residual rem = x_out - x1 are cached.  The decision is taken on the device:
 * the kernels of blocks 1.. read a device flag and return at once when the
 * step is skipped, so the loop needs no host synchronisation.  Approximate:
 * a skipped step differs from the exact step.  Other arguments as qi_dit_step
 * with a valid cache (txt inputs not needed).  threshold 0 never skips.
 * Errors: as qi_dit_step; NULL (fbc or cache NULL), RANGE (threshold negative
 * or not finite), WORKSPACE (fbc_bytes < qi_fbc_bytes), CACHE. */
qi_status qi_dit_step_fbc(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N,
                          const float *img_tokens, float timestep, const float *img_cos,
                          const float *img_sin, const qi_kv_cache *cache, float threshold,
                          void *fbc, size_t fbc_bytes, float *vel, void *ws, size_t ws_bytes,
                          void *stream);

/* Reporting only (it synchronises the stream): the steps seen since the last
 * reset, how many skipped blocks 1.., and the change the last decision saw
 * (+inf when the cache was not valid).  Errors: NULL, ALIGN, HIP. */
qi_status qi_fbc_stats(const void *fbc, int32_t *n_steps, int32_t *n_skipped, float *last_change,
                       void *stream);

/* ---------------------------------------------------------------- text encoder */

/* The text encoder of the port page's pieces table ("Text encoder" row: the
 * Qwen3-VL-8B text stack) and of the host contract s.1 and s.3: input_ids
 * [L] -> hidden [L][hidden], the residual stream after the last layer with no
 * final norm; bf16 weights, fp32 compute (the page's "<|im_start|> tokens
 * need fp32 compute" paragraph).  Per layer (Qwen3 decoder layer):
 *   h = RMSNorm(x; in_norm); q, k, v = h W_qkv^T split [heads | kv | kv] x 128;
 *   q, k = RoPE(RMSNorm_head(q; q_norm)), RoPE(RMSNorm_head(k; k_norm))
 *     (rotate-half: feature i pairs with i + 64, angle p theta^(-2i/128));
 *   o = causal GQA attention (query head h reads kv head h / (heads/kv_heads),
 *     scale 1/sqrt(128)); x += o W_o^T;
 *   h = RMSNorm(x; post_norm); x += (SiLU(h Wg^T) * (h Wu^T)) W_down^T;
 * RMSNorm eps 1e-6.  Sizes of the page: hidden 4096, heads 32, kv_heads 8,
 * head_dim 128, ffn 12288, n_layers 36. */
typedef struct {
  int32_t hidden, heads, kv_heads, head_dim, ffn, n_layers, vocab;
} qi_enc_dims;

typedef struct {
  const uint16_t *w_qkv;          /* [(heads + 2 kv_heads) * 128][hidden] bf16: q rows, k rows, v rows */
  const float *q_norm, *k_norm;   /* [128] */
  const uint16_t *w_o;            /* [hidden][heads * 128] */
  const uint16_t *w_gu;           /* [2 ffn][hidden]: gate rows then up rows */
  const uint16_t *w_down;         /* [hidden][ffn] */
  const float *in_norm, *post_norm; /* [hidden] */
} qi_enc_layer_w;

typedef struct {
  const qi_enc_layer_w *layers;   /* host array [n_layers] of device pointers */
  const uint16_t *embed;          /* [vocab][hidden] bf16 */
} qi_enc_model_w;

/* Host fp32 RoPE rows of positions 0..L-1: cos, sin [L][64] with angle
 * p * theta^(-2i/128), each step rounded to fp32 (the exponent 2i/128, the
 * power -- correctly rounded --, its reciprocal, the product with p) and cos /
 * sin correctly rounded.  Errors: NULL, RANGE (L < 1, theta <= 1). */
qi_status qi_enc_rope_table(int32_t L, float theta, float *cos, float *sin);

/* Workspace bytes of qi_text_encoder_fwd (0 for invalid dims or L). */
size_t qi_enc_workspace_bytes(const qi_enc_dims *d, int32_t L);

/* One encoder forward.  ids: device int32 [L] (an id outside 0..vocab-1 gives
 * a NaN row); cos, sin: device fp32 [L][64] from qi_enc_rope_table; hidden:
 * device fp32 [L][hidden] out.  Causal: the first L' outputs do not depend on
 * later tokens (bit for bit).  Ranges: 1 <= L <= 512; head_dim 128; hidden %
 * 256 == 0; heads % kv_heads == 0; ffn % 64 == 0; every weight matrix under
 * 2 GiB (it is addressed with 32-bit byte offsets).  Errors: NULL, SHAPE,
 * RANGE, ALIGN, WORKSPACE, HIP. */
qi_status qi_text_encoder_fwd(const qi_enc_dims *d, const qi_enc_model_w *w, const int32_t *ids,
                              int32_t L, const float *cos, const float *sin, float *hidden, void *ws,
                              size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- components */

/* The shared modulation rows alone: mod [2][4H] (device fp32) = W_mod e(0) +
 * b_mod and W_mod e(t) + b_mod ([PORT] DiT row).  Errors: NULL, RANGE, ALIGN,
 * HIP. */
qi_status qi_modulation(const qi_dims *d, const uint16_t *w_mod, const float *b_mod,
                        float timestep, float *mod, void *stream);

/* Block-causal attention alone ([PORT] DiT row; [MLX] "Text K/V reuse"), bf16:
 *   q_txt [heads][L][128], k_txt [heads][L][128], vt_txt [heads][128][Lp]
 *   q_img [heads][N][128], k_img [heads][N][128], vt_img [heads][128][Np]
 * (Lp, Np = L, N rounded up to 64; vt holds V transposed) ->
 *   o [rows][heads*128] bf16, rows = L + N (JOINT: text rows 0..L-1, image rows
 *   L..) or N (IMAGE_ONLY: q_txt unused, may be NULL; image rows 0..N-1).
 * Text row i attends causally to text keys 0..i; image rows attend to all L
 * text keys then all N image keys; softmax in fp32 with scale 1/sqrt(128).
 * Errors: NULL, RANGE (heads < 1 or > 64, L < 1 or > 512, N < 1 or > 16384), ALIGN,
 * HIP. */
qi_status qi_block_causal_attention(int32_t heads, int32_t L, int32_t N, int32_t mode,
                                    const uint16_t *q_txt, const uint16_t *k_txt,
                                    const uint16_t *vt_txt, const uint16_t *q_img,
                                    const uint16_t *k_img, const uint16_t *vt_img, uint16_t *o,
                                    void *stream);

/* The bf16 MFMA GEMM of the block projections, with an fp32 store epilogue:
 * C [M][N] (device fp32) = A [M][K] W^T (+ bias [N] if non-NULL), A and W bf16
 * (W in [N][K] layout).  M >= 1, N % 128 == 0, K % 64 == 0.  Errors: NULL,
 * RANGE, ALIGN, HIP. */
qi_status qi_linear_bf16(int32_t M, int32_t N, int32_t K, const uint16_t *A, const uint16_t *W,
                         const float *bias, float *C, void *stream);

/* ---------------------------------------------------------------- kernel timing */

/* Kernel kinds reported by the timing facility. */
#define QI_KERNEL_MODULATION 0   /* shared modulation GEMV (+ time embedding) */
#define QI_KERNEL_TXT_NORM 1     /* ZeroCenterRMSNorm of the text features */
#define QI_KERNEL_GEMM_TXT 2     /* text projection GEMM (and qi_linear_bf16) */
#define QI_KERNEL_IMG_EMBED 3    /* img-in Linear 64 -> H */
#define QI_KERNEL_NORM_MOD 4     /* RMSNorm with modulation (two per block) */
#define QI_KERNEL_GEMM_QKV 5     /* QKV GEMM + RoPE epilogue */
#define QI_KERNEL_ATTENTION 6    /* block-causal attention */
#define QI_KERNEL_GEMM_O 7       /* output projection + gated residual */
#define QI_KERNEL_GEMM_GATE_UP 8 /* gate/up GEMM + SwiGLU */
#define QI_KERNEL_GEMM_DOWN 9    /* down GEMM + gated residual */
#define QI_KERNEL_HEAD 10        /* final RMSNorm + proj_out */
#define QI_KERNEL_EULER 11       /* fp32 Euler update (and the DPM++ 2M update) */
#define QI_KERNEL_ENC_GEMM 12    /* text encoder: fp32-activation GEMMs */
#define QI_KERNEL_ENC_ATTN 13    /* text encoder: fp32 attention */
#define QI_KERNEL_ENC_MISC 14    /* text encoder: embed, norms, q/k prep */
#define QI_KERNEL_SPLITK_REDUCE 15 /* residual update of a K-split O-proj / down GEMM */
#define QI_KERNEL_KINDS 16

/* Name of a kernel kind (static string, "?" if out of range). */
const char *qi_kernel_kind_name(int32_t kind);

/* Start timing: from now on every kernel the library launches is bracketed by
 * two HIP events recorded on the stream it is launched on, for at most
 * max_launches launches (later ones are counted as dropped).  Creates the event
 * pool on first use (the only allocation the library makes; the pool lives
 * until the process ends).  Not meant for graph capture.  Errors: RANGE, HIP. */
qi_status qi_timing_begin(int32_t max_launches);

/* Stop timing, wait for the last recorded event, and report per kind the total
 * milliseconds and the number of launches: ms_total[QI_KERNEL_KINDS],
 * launches[QI_KERNEL_KINDS] (host arrays); dropped (may be NULL) receives the
 * launches that did not fit the pool.  Errors: NULL, HIP. */
qi_status qi_timing_end(double *ms_total, int64_t *launches, int64_t *dropped);

#ifdef __cplusplus
}
#endif

#endif /* QI_H_ */
