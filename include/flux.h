/*
 * flux.h - C ABI of libflux, an MI355X (gfx950) forward pass of the FLUX.2-style MMDiT
 * denoiser: double-stream block, single-stream block and the full denoiser step.
 *
 * Sources of the operations (the "pages"):
 *   [TRACE] "FLUX.2 Klein 9B Base 宏观架构" shape trace (flux-vis), sections 1-4
 *   [DIFF]  "Diffusers 中 Flux2Transformer2DModel 全面解析" (trdm.cn), sections
 *           模型配置参数全解, 前向传播输入输出约定, 双流块, 单流块, 激活函数与 FFN
 *   [KLEIN] "FLUX.2 [klein]" research note (zhao9797.github.io), section 模型架构
 *   [SDPA]  "Transformer架构解析FLUX.2-klein-base-9b-nvfp4" (kwkr.cn), section 2
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or retains them; scratch memory is the caller's `workspace`
 *     (size from the matching *_workspace_size query, 256-byte aligned).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default
 *     stream).  Nothing is synchronised.  Overlapping calls on different streams must
 *     use different workspaces.
 *   - Only kernels (and, for guided sampling, device-to-device copies) are enqueued, so
 *     the calls can be captured into a HIP graph on `stream`; make one call of each kind
 *     outside the capture first (the first launch of a kernel configuration sets its
 *     LDS limit).  Pointers are baked into the graph: keep the buffers alive and at the
 *     same addresses while it is replayed.
 *   - Arguments are validated before anything is enqueued: a non-OK status means no
 *     work was enqueued, and flux_last_error() returns a message (thread-local).
 *   - A HIP launch/runtime error reported while enqueuing returns FLUX_EHIP.  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Linear weights are stored [out, in] row-major (y = x W^T), no biases.  Every
 *     activation / weight pointer and leading dimension must be 16-byte aligned.
 *   - Storage type: `dtype` FLUX_BF16 = bfloat16 (compute: bf16 MFMA, fp32 accumulate);
 *     FLUX_F32 = float32 everywhere (fp32 compute).  QK-norm scales, timesteps and
 *     modulation vectors are always float32.  With FLUX_BF16, `precision` (below) selects
 *     how the block linears' operands are stored: bf16, bf16 hi + lo pairs, or binary16.
 */
#ifndef FLUX_H
#define FLUX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status of every int-returning entry point: 0 on success, a negative code on error. */
typedef enum {
  FLUX_OK = 0,
  FLUX_EINVAL = -1,     /* NULL pointer, non-positive size, unsupported value        */
  FLUX_ESHAPE = -2,     /* inconsistent dimensions (dim != heads*head_dim, ...)      */
  FLUX_EDTYPE = -3,     /* unknown dtype                                             */
  FLUX_EALIGN = -4,     /* pointer or leading dimension not 16-byte aligned          */
  FLUX_EWORKSPACE = -5, /* workspace NULL / too small / not 256-byte aligned         */
  FLUX_EHIP = -6        /* HIP runtime error while enqueuing                         */
} flux_status;

/* FLUX_F16 (IEEE binary16) is never a cfg->dtype: it is the storage of the block linears'
 * operands under FLUX_PRECISION_F16 (below). */
typedef enum { FLUX_BF16 = 0, FLUX_F32 = 1, FLUX_F16 = 2 } flux_dtype;

/* Operand precision of the bf16 path (flux_cfg.precision).
 *   FLUX_PRECISION_BF16  every MFMA operand is stored in bf16 (fp32 accumulation).
 *   FLUX_PRECISION_SPLIT the LayerNorm + modulate outputs (the inputs of the QKV, MLP-in and
 *                        fused linear1 projections) and the SwiGLU outputs (the inputs of
 *                        MLP-out and of linear2's MLP part) are carried as bf16 hi + lo
 *                        pairs (hi = bf16(v), lo = bf16(v - hi)) and multiplied against the
 *                        same weights twice: those products are exact to fp32 accumulation
 *                        and take twice the MFMA work.  Through the 32 blocks of the
 *                        Klein-9B step (D 4096) the bf16 rounding of these two operands is
 *                        amplified more than any other; carrying them removes most of the
 *                        step's error against the exact forward.
 *   FLUX_PRECISION_F16   the operands of the block linears are IEEE binary16 (fp16 MFMA,
 *                        fp32 accumulation): the LayerNorm + modulate outputs, the
 *                        attention output and the SwiGLU outputs are stored in binary16,
 *                        and the block linears' weights (double blocks: qkv, out, mlp_in,
 *                        mlp_out; single blocks: linear1, linear2) must be given in
 *                        binary16 (the caller converts the bf16 weights once: exact for
 *                        |w| in [2^-14, 65504], an absolute error of at most 2^-25 below).
 *                        Binary16 keeps 3 more mantissa bits than bf16, so these roundings
 *                        shrink 8x at the same MFMA rate; values must stay below 65504 in
 *                        magnitude.  q / k / v, the attention probabilities, the
 *                        embedders, the modulation and the output head stay bf16.
 * Every mode projects the step's final LayerNorm output as a hi + lo pair.  FLUX_F32
 * workloads take FLUX_PRECISION_BF16 only (their operands are fp32 already).
 * The operation-level entry points follow the block: under FLUX_PRECISION_F16,
 * flux_layernorm_modulate writes binary16, flux_attention writes a binary16 O, and
 * flux_linear takes binary16 x and w (a SwiGLU y in binary16). */
typedef enum {
  FLUX_PRECISION_BF16 = 0,
  FLUX_PRECISION_SPLIT = 1,
  FLUX_PRECISION_F16 = 2
} flux_precision;

/* Model hyper-parameters ([DIFF] 模型配置参数全解; [KLEIN] config table).
 * head_dim must be 128; dim = heads * head_dim; axes_dim are the per-axis RoPE widths
 * (even, summing to head_dim; the pages use 32,32,32,32); rope_theta 2000; eps 1e-6.
 * in_channels / context_dim / n_double / n_single are used by the step only.
 * FLUX_PRECISION_SPLIT needs dtype FLUX_BF16 and mlp_hidden a multiple of 64;
 * FLUX_PRECISION_F16 needs dtype FLUX_BF16. */
typedef struct {
  int32_t dim;
  int32_t heads;
  int32_t head_dim;
  int32_t mlp_hidden;
  int32_t axes_dim[4];
  float rope_theta;
  float eps;
  int32_t in_channels;
  int32_t context_dim;
  int32_t n_double;
  int32_t n_single;
  int32_t dtype;     /* flux_dtype */
  int32_t precision; /* flux_precision (0 = FLUX_PRECISION_BF16) */
} flux_cfg;

/* Timestep MLPEmbedder: temb = w2 silu(w1 sinusoid(1000 t)); w1 [D,256], w2 [D,D]. */
typedef struct {
  const void* w1;
  const void* w2;
} flux_temb_weights;

/* One stream of a double block ([DIFF] 双流块):
 *   qkv [3D, D] rows q | k | v (head-major inside each of q, k, v);  out [D, D];
 *   mlp_in [2H, D] rows gate | up;  mlp_out [D, H];  q_norm, k_norm [head_dim] fp32. */
typedef struct {
  const void* qkv;
  const void* out;
  const void* mlp_in;
  const void* mlp_out;
  const float* q_norm;
  const float* k_norm;
} flux_stream_weights;

/* Double-stream block: mod_img / mod_txt [6D, D] give per stream the chunks
 * (shift1, scale1, gate1, shift2, scale2, gate2) from silu(temb). */
typedef struct {
  flux_temb_weights temb;
  const void* mod_img;
  const void* mod_txt;
  flux_stream_weights img;
  flux_stream_weights txt;
} flux_double_weights;

/* Single-stream block ([DIFF] 单流块): mod [3D, D] -> (shift, scale, gate);
 * linear1 [3D+2H, D] rows q | k | v | gate | up;  linear2 [D, D+H] columns attn | mlp. */
typedef struct {
  flux_temb_weights temb;
  const void* mod;
  const void* linear1;
  const void* linear2;
  const float* q_norm;
  const float* k_norm;
} flux_single_weights;

/* Whole denoiser ([TRACE] section 3).  img_in [D, in_channels]; txt_in [D, context_dim];
 * model-level modulation shared by all blocks of a kind: mod_double_img/_txt [6D, D],
 * mod_single [3D, D], mod_final [2D, D] -> (shift, scale); proj_out [in_channels, D].
 * double_blocks[n_double] / single_blocks[n_single] are HOST arrays of per-block
 * weights whose temb / mod fields are ignored (the step shares its own). */
typedef struct {
  const void* img_in;
  const void* txt_in;
  flux_temb_weights temb;
  const void* mod_double_img;
  const void* mod_double_txt;
  const void* mod_single;
  const void* mod_final;
  const void* proj_out;
  const flux_double_weights* double_blocks;
  const flux_single_weights* single_blocks;
} flux_model_weights;

/* Last error message of the calling thread ("" if none). */
const char* flux_last_error(void);

/* Library version string. */
const char* flux_version(void);

/* ---------------------------------------------------------------------------------
 * Measurement hook (per-launch kernel durations inside a running workload)
 *
 * flux_timing_begin(site, max_launches) creates 2*max_launches HIP events and arms `site`:
 * from then on every launch of that site that this process enqueues (from any block or
 * step call) is bracketed by an event pair recorded on the launch's own stream, so the
 * timed calls create nothing (the reference-only forward of flux_ref_cache_fill is not
 * timed).  flux_timing_end waits for the recorded events, returns the
 * number of timed launches and their mean duration in microseconds, disarms the site and
 * destroys the events.  One site is armed at a time per process; begin while armed
 * discards the previous arming.  Errors: FLUX_EINVAL for an unknown site, a capacity
 * outside [1, 65536], NULL outputs, or more launches than the capacity (then nothing is
 * returned); FLUX_EHIP if event creation or timing fails.
 * ------------------------------------------------------------------------------- */
typedef enum {
  FLUX_SITE_SINGLE_QKV = 1,       /* single block: linear1 q|k|v part (QKV epilogue) */
  FLUX_SITE_SINGLE_MLP_IN = 2,    /* single block: linear1 gate|up part (SwiGLU epilogue) */
  FLUX_SITE_SINGLE_ATTENTION = 3, /* single block: joint attention (with its key-split merge) */
  FLUX_SITE_SINGLE_LINEAR2 = 4,   /* single block: linear2 + gated residual (with its split-K
                                     reduce) */
  FLUX_SITE_DOUBLE_QKV = 5,       /* double block: QKV projection (both streams, one launch) */
  FLUX_SITE_DOUBLE_ATTENTION = 6, /* double block: joint attention (with its merge) */
  FLUX_SITE_DOUBLE_OUT = 7,       /* double block: out-proj + gated residual (both streams) */
  FLUX_SITE_DOUBLE_MLP_IN = 8,    /* double block: MLP-in + SwiGLU (both streams) */
  FLUX_SITE_DOUBLE_MLP_OUT = 9    /* double block: MLP-out + gated residual (both streams) */
} flux_timing_site;
int flux_timing_begin(int site, int max_launches);
int flux_timing_end(int* launches, double* mean_us);

/* ---------------------------------------------------------------------------------
 * Blocks and step
 * ------------------------------------------------------------------------------- */

/* Double-stream block ([TRACE] section 4; [DIFF] 双流块 Flux2TransformerBlock).
 *   t        device float[batch], timestep in [0,1] (multiplied by 1000 inside)
 *   img      device [batch, n_img, dim] (dtype);  txt device [batch, n_txt, dim]
 *   img_ids  device int32 [n_img, 4];  txt_ids device int32 [n_txt, 4]  (shared by batch)
 *   img_out, txt_out  device outputs, same shapes; may alias img / txt.
 * The joint sequence is [txt ; img] (text first).  n_txt may be 0. */
size_t flux_double_block_workspace_size(const flux_cfg* cfg, int batch, int n_img, int n_txt);
int flux_double_block_fwd(const flux_cfg* cfg, const flux_double_weights* w, const float* t,
                          int batch, int n_img, int n_txt, const void* img, const void* txt,
                          const int32_t* img_ids, const int32_t* txt_ids, void* img_out,
                          void* txt_out, void* workspace, size_t workspace_bytes, void* stream);

/* Single-stream block ([TRACE] section 4; [DIFF] 单流块 Flux2SingleTransformerBlock):
 * merges [txt ; img], LayerNorm+modulate, linear1 -> q,k,v and SwiGLU(gate,up), joint
 * attention, linear2 on [attn | mlp], gated residual; splits back.  Arguments as for the
 * double block. */
size_t flux_single_block_workspace_size(const flux_cfg* cfg, int batch, int n_img, int n_txt);
int flux_single_block_fwd(const flux_cfg* cfg, const flux_single_weights* w, const float* t,
                          int batch, int n_img, int n_txt, const void* img, const void* txt,
                          const int32_t* img_ids, const int32_t* txt_ids, void* img_out,
                          void* txt_out, void* workspace, size_t workspace_bytes, void* stream);

/* Full denoiser step ([TRACE] section 3; [DIFF] 前向传播输入输出约定):
 *   x    device [batch, n_img, in_channels] (dtype), packed noisy latent tokens
 *   ctx  device [batch, n_txt, context_dim] (dtype), text condition
 *   t    device float[batch] in [0,1];  guidance must be NULL (no guidance embedder)
 *   out  device float32 [batch, n_img, in_channels]
 * Runs timestep embedding and all modulations once, the stems, n_double double blocks,
 * n_single single blocks, the final LayerNorm+modulate and proj_out.  The residual
 * stream is kept in float32 between blocks. */
size_t flux_denoiser_step_workspace_size(const flux_cfg* cfg, int batch, int n_img, int n_txt);
int flux_denoiser_step(const flux_cfg* cfg, const flux_model_weights* w, const float* t,
                       const float* guidance, int batch, int n_img, int n_txt, const void* x,
                       const void* ctx, const int32_t* img_ids, const int32_t* txt_ids,
                       float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Sampling loop: rectified-flow Euler steps of the denoiser from a noise latent
 * ([KLEIN] 训练方法: latent rectified flow, 4 steps for the distilled model, 50 steps with
 * the two forwards of classifier-free guidance for the base model; [DIFF] pipeline call
 * chain: packed latents with 4-D ids, a flow-matching Euler scheduler calling the
 * transformer once per step; [KLEIN] Visual tokenizer / VAE: 2x2 patchify of the latent).
 *
 *   x_0 = pack(noise);  x_{i+1} = x_i + (sigmas[i+1] - sigmas[i]) * v_i;  out = unpack(x_n)
 *
 * v_i is the step's output at x_i (rounded to cfg->dtype as the step's input) with
 * t = sigmas[i].  With ctx_uncond, each step is one batch-2*batch forward over
 * [ctx ; ctx_uncond] and v_i = v_u + guidance_scale * (v_c - v_u); without it the scale is
 * ignored.  Position ids are generated: image token (r, c) of the (latent_h/2) x
 * (latent_w/2) grid -> (0, r, c, 0) row-major, text token i -> (0, 0, 0, i).
 *   sigmas      HOST float[n_steps + 1], finite and strictly decreasing (t of each level;
 *               the step multiplies by 1000); NULL: the uniform grid 1 - i / n_steps
 *   noise       device fp32 [batch, in_channels/4, latent_h, latent_w] (latent_h, latent_w
 *               even); the state stays fp32 between steps
 *   ctx, ctx_uncond  device [batch, n_txt, context_dim] (cfg->dtype); ctx_uncond may be NULL
 *   latents_out device fp32 [batch, in_channels/4, latent_h, latent_w]; may alias noise
 *   workspace   flux_denoise_workspace_size(cfg, batch, latent_h, latent_w, n_txt,
 *               ctx_uncond != NULL) bytes, 256-byte aligned
 * The weights are those of flux_denoiser_step.  Errors (nothing enqueued): FLUX_EINVAL
 * (NULL pointers, n_steps outside [1, 10000], sigmas not finite or not decreasing,
 * guidance without text, non-finite scale), FLUX_ESHAPE (odd latent sides, in_channels not
 * a multiple of 8), FLUX_EALIGN, FLUX_EWORKSPACE, and the step's own errors. */
size_t flux_denoise_workspace_size(const flux_cfg* cfg, int batch, int latent_h, int latent_w,
                                   int n_txt, int guided);
int flux_denoise(const flux_cfg* cfg, const flux_model_weights* w, int n_steps,
                 const float* sigmas, float guidance_scale, int batch, int latent_h, int latent_w,
                 int n_txt, const float* noise, const void* ctx, const void* ctx_uncond,
                 float* latents_out, void* workspace, size_t workspace_bytes, void* stream);

/* Reference-image K/V cache ([DIFF] 参考图 KV 缓存机制: per-block cache of the reference
 * tokens' K/V after RoPE; extract mode runs [txt, ref, img] with reference tokens attending
 * only to reference tokens, modulated at the fixed timestep 0; cached mode runs [txt, img]
 * with the cached reference K/V among the keys; [KLEIN] Infra, KV 缓存: step 0 extracts,
 * later steps reuse).  Since reference tokens see only reference tokens at a fixed
 * timestep, their K/V do not depend on the noisy image, the text or t, so the extract step
 * is flux_ref_cache_fill followed by flux_denoiser_step_cached, with identical results.
 *
 * cache: device memory of flux_ref_cache_size(cfg, batch, n_ref) bytes, 256-byte aligned,
 * owned by the caller; one slot per block (double blocks, then single blocks), each holding
 * the reference tokens' q | k rows [batch * n_ref, 2 * dim] (k after RMSNorm + RoPE) and
 * their values transposed [batch * dim, n_ref rounded up to 64] (cfg->dtype).
 *
 * flux_ref_cache_fill: the reference-only forward.
 *   ref_x   device [batch, n_ref, in_channels] (cfg->dtype): packed reference latents
 *   ref_ids device int32 [n_ref, 4] (shared by the batch; flux_denoise_refs uses
 *           (1 + j, r, c, 0) for reference j)
 *   workspace flux_ref_cache_fill_workspace_size(cfg, batch, n_ref) bytes, 256-byte aligned
 * flux_denoiser_step_cached: flux_denoiser_step (same arguments and workspace size, without
 *   guidance) whose attention in every block also covers the cache's n_ref reference keys.
 * Errors (nothing enqueued): FLUX_EINVAL, FLUX_ESHAPE, FLUX_EALIGN, FLUX_EWORKSPACE (also for
 * a cache smaller than flux_ref_cache_size), and the step's own errors. */
size_t flux_ref_cache_size(const flux_cfg* cfg, int batch, int n_ref);
size_t flux_ref_cache_fill_workspace_size(const flux_cfg* cfg, int batch, int n_ref);
int flux_ref_cache_fill(const flux_cfg* cfg, const flux_model_weights* w, int batch, int n_ref,
                        const void* ref_x, const int32_t* ref_ids, void* cache, size_t cache_bytes,
                        void* workspace, size_t workspace_bytes, void* stream);
int flux_denoiser_step_cached(const flux_cfg* cfg, const flux_model_weights* w, const float* t,
                              int batch, int n_img, int n_txt, int n_ref, const void* x,
                              const void* ctx, const int32_t* img_ids, const int32_t* txt_ids,
                              const void* cache, size_t cache_bytes, float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Sampling conditioned on reference latents (the editing path of the pages' KV variant):
 * flux_denoise without guidance, where every step also attends to the reference tokens.
 *   refs  device fp32 [batch, n_refs, in_channels/4, ref_h, ref_w] (ref_h, ref_w even);
 *         reference j is packed like the noise and gets ids (1 + j, r, c, 0)
 *   use_cache  1: the cache is filled once, before the first step (extract, then cached);
 *              0: it is filled again before every step (the references recomputed each step;
 *              same result, bit for bit)
 *   workspace flux_denoise_refs_workspace_size(...) bytes (it holds the cache)
 * Errors as flux_denoise, and FLUX_EINVAL for n_refs <= 0. */
size_t flux_denoise_refs_workspace_size(const flux_cfg* cfg, int batch, int latent_h,
                                        int latent_w, int n_txt, int n_refs, int ref_h,
                                        int ref_w);
int flux_denoise_refs(const flux_cfg* cfg, const flux_model_weights* w, int n_steps,
                      const float* sigmas, int batch, int latent_h, int latent_w, int n_txt,
                      const float* noise, const void* ctx, int n_refs, int ref_h, int ref_w,
                      const float* refs, int use_cache, float* latents_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* 2x2 latent packing used by flux_denoise ([KLEIN] Visual tokenizer / VAE):
 * tokens[b, r * (W/2) + c, 4 ch + 2 ph + pw] = z[b, ch, 2 r + ph, 2 c + pw].
 *   z       device fp32 [batch, channels, H, W] (H, W even);  tokens device fp32
 *           [batch, (H/2)(W/2), 4 channels].  Errors: FLUX_EINVAL, FLUX_ESHAPE, FLUX_EALIGN. */
int flux_pack_latents(int batch, int channels, int H, int W, const float* z, float* tokens,
                      void* stream);
int flux_unpack_latents(int batch, int channels, int H, int W, const float* tokens, float* z,
                        void* stream);

/* Position ids of a generation ([DIFF] 位置 id): img_ids device int32 [grid_h * grid_w, 4]
 * = (0, r, c, 0) row-major; txt_ids device int32 [n_txt, 4] = (0, 0, 0, i) (may be NULL
 * when n_txt == 0).  Errors: FLUX_EINVAL, FLUX_ESHAPE, FLUX_EALIGN. */
int flux_generation_ids(int grid_h, int grid_w, int n_txt, int32_t* img_ids, int32_t* txt_ids,
                        void* stream);

/* ---------------------------------------------------------------------------------
 * Single operations of the hot path (each is one kernel, or a short fixed sequence,
 * of the blocks above; exported so each can be checked and timed on its own).
 * ------------------------------------------------------------------------------- */

/* RoPE position table ([DIFF] 位置 id 的维度): pos_out device int32 [n_txt+n_img, P]
 * where P = head_dim/2 pairs; row j is joint token j of [txt ; img]; pair p takes the id
 * of the axis whose dims contain 2p.  Integer work, bit-exact. */
int flux_rope_positions(const flux_cfg* cfg, const int32_t* txt_ids, const int32_t* img_ids,
                        int n_txt, int n_img, int32_t* pos_out, void* stream);

/* Modulation vectors ([DIFF] 双流块 / 单流块 AdaLN; [KLEIN] 条件注入):
 * out[b, :] = w_mod silu(w2 silu(w1 sinusoid(1000 t[b])))  -> device float [batch, n_out].
 * w_mod [n_out, dim] (dtype).  Workspace from flux_modulation_workspace_size. */
size_t flux_modulation_workspace_size(const flux_cfg* cfg, int batch);
int flux_modulation(const flux_cfg* cfg, const flux_temb_weights* temb, const void* w_mod,
                    int n_out, const float* t, int batch, float* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* LayerNorm (no affine, eps = cfg->eps) + modulate (1 + scale) x_hat + shift, per row
 * ([DIFF] 双流块 AdaLN pre-norm).  x: device [rows, dim] of x_dtype (FLUX_BF16/FLUX_F32);
 * shift, scale: device float [batch, dim] where row r uses batch r / rows_per_batch;
 * y: device [rows, dim] of cfg->dtype (binary16 under FLUX_PRECISION_F16). */
int flux_layernorm_modulate(const flux_cfg* cfg, int rows, int rows_per_batch, const void* x,
                            int x_dtype, const float* shift, const float* scale, void* y,
                            void* stream);

/* Per-head RMSNorm (eps = cfg->eps, scales gamma) then 4-axis RoPE, in place
 * ([DIFF] 双流块 norm_q/norm_k; 位置 id 的维度; [KLEIN] theta 2000).
 * q, k: device [batch, n_txt+n_img, ld] (cfg->dtype) holding head h of token j at
 * column h*head_dim of row j; the joint order is [txt ; img].  Rows j < n_txt use
 * (q_norm_txt, k_norm_txt), the others (q_norm_img, k_norm_img) (device float [128]).
 * ids as for the blocks.  Workspace from flux_qk_norm_rope_workspace_size. */
size_t flux_qk_norm_rope_workspace_size(const flux_cfg* cfg, int n_txt, int n_img);
int flux_qk_norm_rope(const flux_cfg* cfg, int batch, int n_txt, int n_img, void* q, void* k,
                      int64_t ld, const float* q_norm_txt, const float* k_norm_txt,
                      const float* q_norm_img, const float* k_norm_img,
                      const int32_t* txt_ids, const int32_t* img_ids, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Joint attention O = softmax(Q K^T / sqrt(head_dim)) V per head over the whole
 * sequence, no mask ([SDPA]; [TRACE] Joint multi-head attention).
 * q, k, v: device [batch, seq, ld_in] (cfg->dtype), head h at columns
 * [h*head_dim, (h+1)*head_dim); o: device [batch, seq, ld_out] (cfg->dtype; binary16 under
 * FLUX_PRECISION_F16).  The workspace (size from
 * flux_attention_workspace_size) receives V transposed, the layout the kernel reads, and
 * the fp32 partial outputs of query blocks whose keys are split over several workgroups
 * (merged in a fixed order, so results are deterministic). */
size_t flux_attention_workspace_size(const flux_cfg* cfg, int batch, int seq);
int flux_attention(const flux_cfg* cfg, int batch, int seq, const void* q, const void* k,
                   const void* v, int64_t ld_in, void* o, int64_t ld_out, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Linear layer y = x W^T with an optional fused epilogue ([DIFF] 双流块 / 单流块 / 激活函数
 * 与 FFN):
 *   FLUX_EPI_STORE   y[m, n] = acc                                  (y: dtype y_dtype)
 *   FLUX_EPI_SWIGLU  W has 2*n_half rows [gate | up]; y[m, j] = silu(acc_gate) * acc_up
 *                    for j < n_half (pass n = 2*n_half)             (y: operand dtype)
 *   FLUX_EPI_GATED_RESIDUAL
 *                    y[m, n] = resid[m, n] + gate[m / rows_per_batch, n] * acc
 *                    (resid, y: dtype y_dtype; gate device float [batch, n])
 * x: device [m, ldx], w: device [n, ldw] of the operand dtype: cfg->dtype, or binary16 under
 * FLUX_PRECISION_F16 (fp16 MFMA); k = reduction size. */
typedef enum {
  FLUX_EPI_STORE = 0,
  FLUX_EPI_SWIGLU = 1,
  FLUX_EPI_GATED_RESIDUAL = 2
} flux_epilogue;
/* FP8 (E4M3) linear layer ([KLEIN] Infra, 量化: the pages report FP8 releases and speed-ups;
 * the recipe is this library's reading).  Codes are OCP E4M3 bytes (bias 7, largest finite
 * 448, no infinities).
 *
 * flux_quantize_fp8_rows: per-row quantization of x [rows, ldx] (x_dtype FLUX_BF16 or
 *   FLUX_F32, device): with a = amax(|x[r, :cols]|), the dequantization scale is
 *   scales[r] = a / 448 and the codes are q[r, c] = E4M3(x[r, c] * m) with the multiplier
 *   m = 448 / a (both fp32, correctly rounded; scales[r] = m = 1 for an all-zero row): the
 *   product x * m is rounded to fp32, then to E4M3 by round to nearest even, saturating at
 *   448 (device bytes [rows, ldq]).  x * m may differ from x / scales[r] in the last fp32
 *   bit, which can move a code; the multiplier form is the one the hardware conversion
 *   takes.  Activation rows and weight rows (output channels) are quantized the same way.
 *   Errors: FLUX_EINVAL, FLUX_EDTYPE, FLUX_ESHAPE.
 * flux_linear_fp8: y = sa[m] sw[n] sum_k dec(qa[m, k]) dec(qw[n, k]) (fp32 accumulation)
 *   followed by the epilogue of flux_linear (STORE, SWIGLU with bf16 output, GATED_RESIDUAL
 *   with gate_bs = n).  qa device [m, lda] bytes, qw device [n, ldw] bytes (lda, ldw >= k,
 *   multiples of 16; operands under 4 GiB), sa device float [m], sw device float [n];
 *   k % 128 == 0.  workspace as flux_linear.  Errors: FLUX_EINVAL, FLUX_ESHAPE, FLUX_EALIGN,
 *   FLUX_EDTYPE, FLUX_EWORKSPACE. */
int flux_quantize_fp8_rows(int rows, int cols, const void* x, int x_dtype, int64_t ldx, void* q,
                           int64_t ldq, float* scales, void* stream);
int flux_linear_fp8(const flux_cfg* cfg, int epilogue, int m, int n, int k, const void* qa,
                    int64_t lda, const float* sa, const void* qw, int64_t ldw, const float* sw,
                    void* y, int64_t ldy, int y_dtype, const void* resid, int64_t ldr,
                    const float* gate, int rows_per_batch, void* workspace,
                    size_t workspace_bytes, void* stream);

/* workspace: NULL, or flux_linear_workspace_size() bytes (256-byte aligned) of scratch that
 * lets the large-tile path split the last partial round of output tiles along K (fp32
 * partials reduced in a fixed order, so results stay deterministic). */
size_t flux_linear_workspace_size(void);
int flux_linear(const flux_cfg* cfg, int epilogue, int m, int n, int k, const void* x,
                int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy, int y_dtype,
                const void* resid, int64_t ldr, const float* gate, int rows_per_batch,
                void* workspace, size_t workspace_bytes, void* stream);

/* flux_linear for callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation with the split-K
 * scratch taken from a fixed device array inside the library instead of a workspace.  The
 * array holds flux_linear_workspace_size() bytes (64 MiB), the most the tile planner ever
 * uses, so every shape flux_linear accepts fits and results equal flux_linear's with a
 * workspace bit for bit; each device holds its own copy from its first call until the
 * process ends.  The call allocates nothing (no hipMalloc / hipFree, no allocating library
 * routine).  Every call on a device shares that device's array: calls that may overlap on
 * one device (different streams, or host threads) race and must be serialised by the
 * caller.  Errors: those of flux_linear, and FLUX_EHIP if the array's device address cannot
 * be resolved. */
int flux_linear_noalloc(const flux_cfg* cfg, int epilogue, int m, int n, int k, const void* x,
                        int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy,
                        int y_dtype, const void* resid, int64_t ldr, const float* gate,
                        int rows_per_batch, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUX_H */
