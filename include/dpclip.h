/*
 * dpclip.h -- C ABI of libdpclip.so: the DP-SGD per-sample gradient clipping
 * hot path on AMD Instinct MI355X (gfx950).
 *
 * Conventions (all entry points):
 *  - Sizes are int64_t and must be >= 1. Tensors are device pointers to
 *    contiguous row-major arrays, last dimension fastest. A and G share one
 *    number type (dp_dtype). A, G and the workspace must be 16-byte aligned;
 *    float vectors 4-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream). All device work is
 *    enqueued asynchronously on it; nothing is synchronised. The caller keeps
 *    every buffer alive until the stream has passed the call.
 *  - The caller owns every buffer, including the workspace. The library keeps
 *    no pointer after returning. Its only global state is the fixed scratch
 *    array of dp_ghost_norm_clip_layers_noalloc (with its per-device
 *    address); calls are re-entrant. A workspace serves one call at a time: calls that
 *    may run concurrently (different streams) need distinct workspaces.
 *    Identical inputs give bitwise-identical outputs (fixed-order reductions,
 *    no floating-point atomics).
 *  - Every argument is validated before any HIP call. A failed validation
 *    returns its code and touches nothing. HIP launch failures return
 *    DP_ERR_HIP; no usable device returns DP_ERR_NO_DEVICE.
 *  - Calls may be captured into a HIP graph and replayed: they enqueue kernel
 *    launches only (no memset, copy or allocation), and a call's kernels read
 *    from the workspace only what the same call wrote there before. Buffers captured by
 *    pointer keep their addresses across replays, as graphs require.
 *
 * Page keys used in the comments:
 *  FPC  "Scaling up Differentially Private Deep Learning with Fast Per-Example
 *       Gradient Clipping"
 *  TTP  "Three Tools for Practical Differential Privacy"
 *  SEDP "Scalable and Efficient Training of Large Convolutional Neural Networks
 *       with Differential Privacy"
 *  DDP  "Privacy-Preserving Deep Learning: A Deep Dive into DP-SGD"
 */
#ifndef DPCLIP_H
#define DPCLIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DP_ABI_VERSION 3

typedef int32_t dp_status;
#define DP_OK 0
#define DP_ERR_NULL 1      /* a required pointer is NULL */
#define DP_ERR_SHAPE 2     /* a size is < 1 or a size product overflows the supported range */
#define DP_ERR_DTYPE 3     /* unknown dp_dtype */
#define DP_ERR_VALUE 4     /* a scalar is out of range (C, sigma, denom, alpha, beta, mode, kappa, ...) */
#define DP_ERR_WORKSPACE 5 /* workspace smaller than dp_workspace_bytes() */
#define DP_ERR_HIP 6       /* a HIP call or kernel launch failed */
#define DP_ERR_NO_DEVICE 7 /* no gfx950 device is current */
#define DP_ERR_ALIGN 8     /* a pointer is not aligned as required */

typedef int32_t dp_dtype;
#define DP_F32 0
#define DP_BF16 1

typedef int32_t dp_mode;
#define DP_MODE_MIXED 0    /* layerwise decision (SEDP Sec. 4, rule (4.1)) */
#define DP_MODE_GHOST 1    /* always the ghost norm (SEDP 'ghost' mode, App. E) */
#define DP_MODE_EXPLICIT 2 /* always per-sample instantiation */
#define DP_MODE_TIME 3     /* layerwise decision by matrix-core work per sample: explicit when
                              2*T*d*p + 2*d*p < T*(T+1)*(d+p) + 2*T*T (SEDP App. C costs, the
                              ghost Grams' unique entries), else ghost; kappa is not used */

#define DP_PATH_GHOST 1    /* <A_i A_i^T, G_i G_i^T> on per-sample Gram tiles */
#define DP_PATH_EXPLICIT 2 /* ||A_i^T G_i||_F^2 from per-sample gradient tiles */
#define DP_PATH_T1 3       /* T == 1 closed form ||a_i||^2 ||g_i||^2 */

/*
 * Per-example squared gradient norm of ONE layer (weight, plus bias when
 * has_bias != 0), without materialising per-example gradients in memory.
 *
 * Defines: SEDP eq. (2.4)/(2.6) per-sample gradient g_i = A_i^T G_i,
 * eq. (2.7) ghost norm ||g_i||_F^2 = <A_i A_i^T, G_i G_i^T>, Sec. 4 layerwise
 * decision; FPC eq. (6) (outer product for T = 1) and the bias gradient
 * b_i = sum_t G_i[t, :].
 *
 *  A        [B, T, d] layer inputs (for a conv: the unfolded U(a_i), d = C_in*kH*kW).
 *  G        [B, T, p] output gradients dL/ds_i (for a conv: F^-1, spatial flattened).
 *  dtype    DP_F32 or DP_BF16 (both tensors); accumulation is fp32.
 *  mode     DP_MODE_*; kappa >= 1: MIXED takes the explicit path when
 *           p*d < kappa*T*T, else ghost (tie -> ghost); TIME compares the
 *           per-sample work of both paths; T == 1 takes the closed form
 *           unless mode is EXPLICIT.
 *  workspace, ws_bytes  device scratch of at least dp_workspace_bytes(...)
 *           bytes (may be NULL when that is 0). Its contents on entry are
 *           ignored and on return undefined. When a sample spans several
 *           tile workgroups, each stores its partial there and a small
 *           finish kernel on the same stream folds them (no workgroup waits
 *           for another). DP_ERR_SHAPE when a sample would span more than
 *           65535 tiles (explicit path with d*p beyond ~1e9).
 *  sqnorm   [B] fp32 device: overwritten (accumulate == 0) or incremented
 *           (accumulate != 0) by the layer's squared norms, so several layers
 *           can be summed in call order into one global norm.
 *  path_out host int (may be NULL): receives DP_PATH_* actually taken.
 */
dp_status dp_ghost_norm(void* stream, const void* A, const void* G, dp_dtype dtype,
                        int64_t B, int64_t T, int64_t d, int64_t p, int32_t has_bias,
                        dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes,
                        float* sqnorm, int32_t accumulate, int32_t* path_out);

/* One layer of a dp_ghost_norm_layers call. */
typedef struct dp_layer {
  const void* A;     /* [B, T, d] layer inputs, as in dp_ghost_norm */
  const void* G;     /* [B, T, p] output gradients */
  int64_t T, d, p;
  int32_t has_bias;
  int32_t reserved;  /* must be 0 */
} dp_layer;

/*
 * Per-example squared gradient norm over several layers,
 * N_i^2 = sum_l n_{i,l}^2: the norm of the whole per-sample gradient that
 * the clip factor of SEDP eq. (2.1) (and FPC's clip_c) is taken of, with each
 * layer's n_{i,l}^2 as in dp_ghost_norm.
 *
 * The result is bitwise the one of dp_ghost_norm called on layers[0],
 * layers[1], ... in that order (one stream, one workspace), the first call
 * with `accumulate` and the others with accumulate = 1. Runs of up to 8
 * consecutive layers that take the same ghost kernel (the tiled kernel with
 * one tile size, or the direct-to-LDS bf16 engine: T > 64, d and p multiples
 * of 64) share a launch, whose Gram tiles fill the GPU together (a small
 * layer alone leaves most compute units idle); the launch's finish kernel
 * adds each sample's tile partials and then the layers in order. Other
 * layers (closed form, explicit) run one launch each.
 *
 *  layers, n_layers  host array, 1 <= n_layers <= 4096; each layer as in
 *           dp_ghost_norm (A, G non-NULL and 16-byte aligned, shape limits),
 *           reserved == 0.
 *  dtype, B, mode, kappa  shared by all layers, as in dp_ghost_norm.
 *  workspace, ws_bytes  at least dp_layers_workspace_bytes(...) bytes (may be
 *           NULL when that is 0); contents as in dp_ghost_norm.
 *  sqnorm, accumulate   as in dp_ghost_norm.
 *  paths_out host int[n_layers] (may be NULL): DP_PATH_* of each layer.
 */
dp_status dp_ghost_norm_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype,
                               int64_t B, dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes,
                               float* sqnorm, int32_t accumulate, int32_t* paths_out);

/*
 * dp_ghost_norm_layers, and the clip factors of its result in the same pass:
 * c[b] and norm[b] (norm may be NULL) exactly as dp_clip_factors(sqnorm, B,
 * C, c, norm) would give them after the call (same fp32 operations), formed
 * by the kernel that finishes each sample's squared norm (by the clip kernel
 * after it when the last layer takes the T = 1 closed form). C finite, > 0.
 */
dp_status dp_ghost_norm_clip_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype,
                                    int64_t B, dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes,
                                    float* sqnorm, int32_t accumulate, float C, float* c, float* norm,
                                    int32_t* paths_out);

/*
 * dp_ghost_norm_clip_layers for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and bitwise the same results, with no
 * workspace argument. Its scratch (the norm kernels' tile partials) is a
 * fixed 4 MiB device array inside the library, one per GPU, held from the
 * first call on that GPU until the process ends; the call allocates no
 * memory (device or host) and makes no memset.
 *
 * Every call on one GPU shares that array: calls that may overlap on one GPU
 * (different streams, or one stream and a graph replay) race and give wrong
 * results; serialise them. Nothing in the array needs clearing between calls.
 *
 *  Arguments as in dp_ghost_norm_clip_layers, with n_layers <= 1024.
 *  DP_ERR_WORKSPACE when the layers would need more than 4 MiB of scratch
 *  (dp_layers_workspace_bytes covers it: B * tiles-per-sample * 4 bytes,
 *  e.g. 20 KB for eight GPT-2-large layers at B = 32).
 */
dp_status dp_ghost_norm_clip_layers_noalloc(void* stream, const dp_layer* layers, int32_t n_layers,
                                            dp_dtype dtype, int64_t B, dp_mode mode, int32_t kappa,
                                            float* sqnorm, int32_t accumulate, float C, float* c, float* norm,
                                            int32_t* paths_out);

/* Workspace bytes that dp_ghost_norm_layers (with this mode and kappa) and
 * dp_clipped_sum_noise_layers need for these layers (the larger of the two).
 * Returns 0 for invalid arguments (and when no workspace is needed). */
size_t dp_layers_workspace_bytes(const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B,
                                 dp_mode mode, int32_t kappa);

/*
 * Norms and clip factors from squared norms.
 *
 * Defines: FPC clip_c(z) = z if ||z|| <= c else c*z/||z||; SEDP App. C
 * C_i = min(R/||g_i||, 1); DDP g/max(1, ||g||/C).
 *
 *  sqnorm  [B] fp32 device (e.g. the sum over layers from dp_ghost_norm).
 *  C       clipping bound, finite and > 0 (host value).
 *  c       [B] fp32 device out: c_i = 1 when norm_i <= C, else C/norm_i.
 *  norm    [B] fp32 device out, may be NULL: norm_i = sqrt(sqnorm_i), with
 *          negative round-off clamped to 0. NaN propagates to norm_i and c_i;
 *          an infinite norm gives c_i = 0.
 */
dp_status dp_clip_factors(void* stream, const float* sqnorm, int64_t B, float C,
                          float* c, float* norm);

/*
 * Clipped, noised mean gradient of ONE layer.
 *
 * Defines: FPC the clipped sum with Gaussian noise added before the update
 * (re-weighted loss, Gaussian mechanism); SEDP eq. (2.1) and Sec. 3.2
 * (weighted gradient sum_i C_i g_i); DDP noisy aggregation.
 *
 *   out[m][n]   = (sum_b c[b] * sum_t A[b,t,m] G[b,t,n] + (sigma*C) * z_w[m][n]) * (1/denom)
 *   bias_out[n] = (sum_b c[b] * sum_t G[b,t,n]          + (sigma*C) * z_b[n])    * (1/denom)
 *
 *  in fp32: the sum accumulates in fp32 (products of the input dtype),
 *  sigma*C and 1/denom are each rounded to fp32 once, and the last two
 *  operations are an fp32 add of fl(sigma*C)*z and a multiply by fl(1/denom)
 *  (no division), so the noise term is reproducible bit for bit.
 *
 *  A, G, dtype, B, T, d, p  as in dp_ghost_norm.
 *  c        [B] fp32 device clip factors (any finite values).
 *  C, sigma bound and noise multiplier (C > 0, sigma >= 0, finite).
 *  denom    divisor (> 0, finite); B for the plain mean.
 *  seed, layer_id, step  select the noise: Philox4x32-10 + Box-Muller with
 *           key (seed lo32, seed hi32), four normals per counter block.
 *           z_w[m][n] is lane m%4 of the block at counter
 *           ((m/4)*p + n, 2*layer_id, step, 0) (4 consecutive rows of one
 *           column share a block); z_b[n] is lane n%4 of the block at
 *           (n/4, 2*layer_id+1, step, 0). ceil(d/4)*p must be < 2^32.
 *  workspace, ws_bytes  as in dp_ghost_norm.
 *  out      [d, p] fp32 device (= A^T G layout, the transpose of a torch
 *           weight.grad).
 *  bias_out [p] fp32 device, or NULL for a layer without bias.
 */
dp_status dp_clipped_sum_noise(void* stream, const void* A, const void* G, dp_dtype dtype,
                               int64_t B, int64_t T, int64_t d, int64_t p,
                               const float* c, float C, float sigma, float denom,
                               uint64_t seed, uint32_t layer_id, uint32_t step,
                               void* workspace, size_t ws_bytes,
                               float* out, float* bias_out);

/*
 * Clipped, noised mean gradients of several layers under one set of clip
 * factors (flat clipping: one c for every layer), each layer's output as
 * dp_clipped_sum_noise defines it, with noise stream layer_ids[l] (or l when
 * layer_ids is NULL).
 *
 * Layers that the bf16 direct-to-LDS engine takes (bf16, no bias, T a
 * multiple of 64, d and p multiples of 8) share kernel launches of up to 8
 * layers: one tile shape and a K split per layer chosen for the set, so that
 * the work items of all of them fill the GPU together; the partial tiles of
 * split layers are added by one reduce launch for the group after it, in
 * split order, with the noise and the mean (in a call with several shared
 * launches, by workgroups of the next launch that run on the CUs its last
 * round of work leaves idle; the partials of consecutive launches then take
 * two workspace regions in turn). Other layers
 * run one dp_clipped_sum_noise-like launch each. Results are deterministic
 * for a given set of layer shapes; the K split of a layer may differ from the
 * one a single-layer call picks, which changes the fp32 rounding of the sum
 * (the noise term is the same bit for bit).
 *
 *  layers, n_layers  as in dp_ghost_norm_layers.
 *  dtype, B          shared by all layers.
 *  c, C, sigma, denom, seed, step  as in dp_clipped_sum_noise (c: [B]).
 *  layer_ids         host uint32[n_layers] or NULL.
 *  workspace, ws_bytes  at least dp_layers_workspace_bytes(...) bytes.
 *  outs              host array of n_layers device pointers, outs[l] [d_l, p_l] fp32.
 *  bias_outs         host array of n_layers device pointers or NULL: entry l
 *                    ([p_l] fp32) is required when layers[l].has_bias and
 *                    ignored otherwise; NULL when no layer has a bias.
 */
dp_status dp_clipped_sum_noise_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype,
                                      int64_t B, const float* c, float C, float sigma, float denom, uint64_t seed,
                                      const uint32_t* layer_ids, uint32_t step, void* workspace, size_t ws_bytes,
                                      float* const* outs, float* const* bias_outs);

/*
 * Virtual step (gradient accumulation): a logical batch fed to the GPU as
 * several physical batches, each back-propagated before one update (SEDP,
 * Performance section: physical vs logical batch size; App. E, the virtual
 * step). Each physical batch's samples are clipped with their own factors;
 * the clipped sums add up over the logical batch and the noise and the mean
 * are applied once, by dp_noise_mean.
 *
 * dp_clipped_sum_accumulate: acc[d][p] = (accumulate ? acc : 0) + sum_b c[b] A_b^T G_b
 * (and bias_acc[p] with sum_b c[b] sum_t G_b[t] when bias_acc != NULL), in
 * fp32: the physical batch's clipped sum as dp_clipped_sum_noise forms it,
 * then one fp32 add per element. A, G, dtype, B, T, d, p, c as in
 * dp_clipped_sum_noise; workspace of at least
 * dp_accumulate_workspace_bytes(dtype, B, T, d, p, bias_acc != NULL) bytes
 * (with accumulate == 0, dp_workspace_bytes(...) suffice).
 */
size_t dp_accumulate_workspace_bytes(dp_dtype dtype, int64_t B, int64_t T, int64_t d, int64_t p, int32_t has_bias);
dp_status dp_clipped_sum_accumulate(void* stream, const void* A, const void* G, dp_dtype dtype,
                                    int64_t B, int64_t T, int64_t d, int64_t p, const float* c,
                                    void* workspace, size_t ws_bytes, float* acc, float* bias_acc,
                                    int32_t accumulate);

/*
 * dp_clipped_sum_accumulate_layers: the same for several layers under one c
 * (flat clipping): accs[l] (+)= the clipped sum of layer l over this physical
 * batch, formed as dp_clipped_sum_noise_layers forms it (shared launches,
 * then one fp32 add per element). layers, n_layers, dtype, B, c as in
 * dp_clipped_sum_noise_layers; accs / bias_accs like its outs / bias_outs.
 * Workspace: dp_layers_accumulate_workspace_bytes(...) bytes (with
 * accumulate == 0, dp_layers_workspace_bytes(...) suffice).
 */
size_t dp_layers_accumulate_workspace_bytes(const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B);
dp_status dp_clipped_sum_accumulate_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype,
                                           int64_t B, const float* c, void* workspace, size_t ws_bytes,
                                           float* const* accs, float* const* bias_accs, int32_t accumulate);

/*
 * dp_noise_mean: out[m][n] = (acc[m][n] + (sigma*C) * z_w[m][n]) * (1/denom),
 * bias_out[n] likewise with z_b[n], the noise of dp_clipped_sum_noise
 * (same seed, layer_id, step -> same z, bit for bit; same fp32 operation
 * order). denom is the logical batch size for the plain mean. out may be acc
 * and bias_out may be bias_acc (each element is read before it is written).
 * bias_acc and bias_out are both NULL or both set.
 */
dp_status dp_noise_mean(void* stream, const float* acc, const float* bias_acc, int64_t d, int64_t p, float C,
                        float sigma, float denom, uint64_t seed, uint32_t layer_id, uint32_t step,
                        float* out, float* bias_out);

/*
 * One update of the adaptive per-layer clipping bound of TTP:
 *
 *   C_l2   = init ? mean_b(norm[b]) : beta * C_prev
 *   C_next = alpha / B * ( sum_b min(norm[b], C_l2) + sigma_l2 * C_l2 * z )
 *
 * where min(n, C_l2) = n / max(1, n / C_l2) is TTP's clip(||y||) and z is the
 * normal of counter (0, 2*layer_id, step, 1) under key (seed lo32, seed hi32),
 * lane 0. By convention `step` is the index t of the bound C_t being produced.
 *
 *  norm     [B] fp32 device per-example norms of the layer (previous step).
 *           With init != 0, C_l2 is their plain mean with no noise added, so
 *           they must come from a data-independent batch: TTP initialises
 *           C_l2,0 from one iteration on random noise. Norms of private
 *           training data there would make C_l2 and the noise scale
 *           sigma_l2 * C_l2 depend on that data without protection.
 *  C_prev   previous bound (host); must be finite and > 0 unless init != 0.
 *  alpha, beta > 0, sigma_l2 >= 0, finite.
 *  C_next   fp32 device scalar out; C_l2_out fp32 device scalar out (may be NULL).
 */
dp_status dp_adaptive_threshold(void* stream, const float* norm, int64_t B, float C_prev,
                                float alpha, float beta, float sigma_l2, int32_t init,
                                uint64_t seed, uint32_t layer_id, uint32_t step,
                                float* C_next, float* C_l2_out);

/*
 * Convolution layers from their folded input (implicit unfolding).
 *
 * SEDP Sec. 2.2 writes a 2-D convolution as a product with the unfolded
 * input U(a_i): one row per output position (T = H_out*W_out rows), one
 * column per (input channel, kernel row, kernel column), so d = C_in*kH*kW.
 * The entry points below take the folded input a [B, C_in, H, W] instead of
 * U(a) [B, T, d] and form U(a)'s rows on chip, element by element:
 *
 *   U(a)[b][t = ho*W_out + wo][f = (ci*kH + i)*kW + j]
 *       = a[b][ci][ho*stride_h - pad_h + i*dil_h][wo*stride_w - pad_w + j*dil_w]
 *         (0 where that position lies in the zero padding),
 *   H_out = (H + 2*pad_h - dil_h*(kH-1) - 1) / stride_h + 1, likewise W_out,
 *
 * which is torch's unfold (and conv2d, groups = 1) layout. The unfolded input
 * is never written to memory: a conv layer reads a, not kH*kW/(stride_h*stride_w)
 * times as much. Results are those of dp_ghost_norm / dp_clipped_sum_noise on
 * U(a) up to fp32 summation order.
 */
typedef struct dp_conv2d {
  int64_t C_in, H, W;          /* folded input geometry */
  int64_t kh, kw;              /* kernel size, >= 1 */
  int64_t stride_h, stride_w;  /* >= 1 */
  int64_t pad_h, pad_w;        /* zero padding, >= 0 */
  int64_t dil_h, dil_w;        /* dilation, >= 1 */
} dp_conv2d;

/*
 * dp_conv_norm: dp_ghost_norm of the layer (U(a), G).
 *
 *  a        [B, C_in, H, W] folded input, dtype as G, 4-byte aligned (fp32)
 *           or 2-byte aligned (bf16); (C_in+2)*(H+2*pad_h)*(W+2*pad_w) < 2^31.
 *  G        [B, T, p] output gradients (T = H_out*W_out, spatial positions
 *           row-major), 16-byte aligned.
 *  conv     host geometry; H_out, W_out >= 1; every size below 2^31.
 *  dtype, B, p, has_bias, mode, kappa, sqnorm, accumulate  as in dp_ghost_norm,
 *           with T and d of U(a). The path rule is dp_ghost_norm's; a T = 1
 *           layer takes the ghost path (the closed form reads U(a) rows).
 *  workspace, ws_bytes  at least dp_conv_workspace_bytes(...) bytes.
 *  path_out host int (may be NULL): DP_PATH_* taken.
 */
dp_status dp_conv_norm(void* stream, const void* a, const void* G, const dp_conv2d* conv, dp_dtype dtype,
                       int64_t B, int64_t p, int32_t has_bias, dp_mode mode, int32_t kappa,
                       void* workspace, size_t ws_bytes, float* sqnorm, int32_t accumulate, int32_t* path_out);

/*
 * dp_conv_clipped_sum_noise: dp_clipped_sum_noise of the layer (U(a), G):
 * out [d, p] fp32 with d = C_in*kH*kW in U(a)'s column order (torch's
 * weight.grad [p, C_in, kH, kW] transposed), bias_out [p] or NULL; c, C,
 * sigma, denom, seed, layer_id, step and the noise as in dp_clipped_sum_noise.
 * a, G, conv, dtype, B, p as in dp_conv_norm.
 */
dp_status dp_conv_clipped_sum_noise(void* stream, const void* a, const void* G, const dp_conv2d* conv,
                                    dp_dtype dtype, int64_t B, int64_t p, const float* c, float C, float sigma,
                                    float denom, uint64_t seed, uint32_t layer_id, uint32_t step,
                                    void* workspace, size_t ws_bytes, float* out, float* bias_out);

/*
 * dp_unfold2d: U(a) [B, T, d] itself, written to U in the layout above (dtype
 * of a; row t of sample b at U + (b*T + t)*d elements), for callers that run
 * the unfolded path (dp_ghost_norm[_layers], dp_clipped_sum_noise[_layers])
 * on a layer they hold folded, sharing launches with other layers. The
 * conv-as-linear unfolding of SEDP Sec. 2.2, eqs. (2.5)-(2.6) (FPC Alg. 3
 * works on the same unfolded patches). Every element is copied or set to 0:
 * U equals torch's unfold(a).transpose(1, 2) bit for bit.
 *
 *  a, conv, dtype, B  as in dp_conv_norm.
 *  U        [B, T, d] device buffer of the caller (B*T*d elements of dtype),
 *           16-byte aligned; T*d < 2^31.
 */
dp_status dp_unfold2d(void* stream, const void* a, const dp_conv2d* conv, dp_dtype dtype, int64_t B, void* U);

/* Workspace bytes that dp_conv_norm (with this mode and kappa) and
 * dp_conv_clipped_sum_noise need for this layer (the larger of the two).
 * Returns 0 for invalid arguments. */
size_t dp_conv_workspace_bytes(const dp_conv2d* conv, dp_dtype dtype, int64_t B, int64_t p, int32_t has_bias,
                               dp_mode mode, int32_t kappa);

/* Workspace bytes that dp_ghost_norm and dp_clipped_sum_noise need for this
 * layer shape (the larger of the two). Returns 0 for invalid arguments. */
size_t dp_workspace_bytes(dp_dtype dtype, int64_t B, int64_t T, int64_t d, int64_t p,
                          dp_mode mode, int32_t kappa);

/* The DP_PATH_* that dp_ghost_norm takes for this shape, or -1 for invalid
 * arguments. Pure host function. */
int32_t dp_choose_path(int64_t T, int64_t d, int64_t p, dp_mode mode, int32_t kappa);

/* Static string naming a status code. */
const char* dp_status_string(dp_status status);

/* DP_ABI_VERSION of the loaded library. */
int32_t dp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DPCLIP_H */
