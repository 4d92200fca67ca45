/*
 * vae.h - C ABI of libvae_mi355x: the tiled, halo-extended decode of a causal 3-D video VAE on one
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes what these pages describe:
 *   [P1] "[TRTLLM-14029][feat] LTX-2 tile-parallel VAE decode" (NVIDIA/TensorRT-LLM PR #15753)
 *   [P2] "[Feature] Support VAE tiling parallel encode for LTX-2" (vllm-project/vllm-omni PR #4831)
 *   [P4] "Add tiled VAE parallelism & extended model support" (xdit-project/DistVAE PR #14)
 *   [P5] "[TRTLLM-14123][feat] add ParallelVAE_TrtllmWan for native Wan VAE" (TensorRT-LLM PR #16066)
 * Each declaration below names the passage that defines its operation.
 *
 * Conventions for every call
 *  - Layout: activations are dense NDHWC (channels fastest), addressed with 64-bit offsets.
 *    Conv weights are [Cout][kt=3][kh=3][kw=3][Cin]. Bias, gamma and beta are fp32 vectors.
 *  - Dtypes: VAE_DTYPE_BF16 (bfloat16 storage, fp32 arithmetic) or VAE_DTYPE_F32.
 *    VAE_DTYPE_F16 (IEEE binary16 storage, 11 significant bits) is accepted only where a call
 *    says so: as a conv input on the MFMA path, as the conv output of a 2-byte input, as a
 *    GroupNorm output, and by vae_upsample (a copy). It is the operand hand-off of convs whose
 *    input needs more than bf16's 8 significant bits (see vae_conv3d_causal).
 *  - Ownership: the caller owns every buffer. Device buffers are passed as raw device pointers;
 *    the library never allocates or frees device memory. It never synchronises the stream,
 *    except in the setup calls that read a result back (fp16 weight packing checks its range;
 *    vae_decode_status and vae_decoder_get_timing read results), each saying so. It keeps no
 *    pointer after a call returns, except the weight pointers held by a decoder object, which
 *    must outlive that object.
 *  - Streams: every device call is asynchronous and enqueued on `stream` (a hipStream_t passed as
 *    void*, NULL = the default stream). vae_tile_split is host-only and synchronous.
 *  - Errors: every call returns a vae_status_t. On failure nothing is enqueued, and
 *    vae_last_error() / vae_last_error_info() describe the cause for the calling thread. No C++
 *    exception crosses this boundary.
 *  - Boxes: half-open [t0,t1) x [h0,h1) x [w0,w1) in the grid of the tensor they refer to;
 *    NULL means the whole tensor.
 */
#ifndef VAE_MI355X_H
#define VAE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define VAE_API __attribute__((visibility("default")))
#else
#define VAE_API
#endif

typedef void* vae_stream_t; /* a hipStream_t */

typedef enum {
    VAE_OK = 0,
    VAE_ERR_INVALID_ARG = 1,  /* malformed arguments: null pointers, mismatched shapes/dtypes */
    VAE_ERR_UNSUPPORTED = 2,  /* well-formed but outside what the library computes; see info */
    VAE_ERR_HIP = 3,          /* a HIP runtime call failed */
    VAE_ERR_WORKSPACE = 4     /* workspace missing or smaller than the size query returned */
} vae_status_t;

enum { VAE_DTYPE_BF16 = 1, VAE_DTYPE_F32 = 2, VAE_DTYPE_F16 = 3 };

typedef struct vae_tensor {
    void* data;       /* device pointer, NDHWC dense */
    int32_t dtype;    /* VAE_DTYPE_* */
    int32_t reserved; /* set to 0 */
    int64_t n, t, h, w, c;
} vae_tensor_t;

typedef struct vae_box {
    int32_t t0, t1, h0, h1, w0, w1;
} vae_box_t;

/* Structured details of the last failure (P4, commit on rectangular tile plans: callers get the
 * numbers instead of parsing error text). Unused fields are -1. */
typedef struct vae_error_info {
    int32_t status;            /* vae_status_t of the failure */
    int32_t axis;              /* 0 = N, 1 = T, 2 = H, 3 = W, 4 = C */
    int64_t extent;            /* the offending extent */
    int64_t required_multiple; /* a divisor the extent must have */
    int64_t min_width;         /* the smallest extent that would be accepted */
} vae_error_info_t;

/* Thread-local text of the last failure on this thread ("" after success). */
VAE_API const char* vae_last_error(void);
/* Copies the structured details of the last failure on this thread. */
VAE_API vae_status_t vae_last_error_info(vae_error_info_t* info);
/* Library version, major * 10000 + minor * 100 + patch. */
VAE_API int32_t vae_version(void);

/* ------------------------------------------------------------------------------------------ */
/* Causal Conv3d                                                                              */
/* ------------------------------------------------------------------------------------------ */
/*
 * y[n,t,h,w,o] = bias[o] + residual[n,t,h,w,o]
 *              + sum_{c,a,p,q} W[o,a,p,q,c] * x[n, max(t+a-2, 0), h+p-1, w+q-1, c]
 * with zeros where h+p-1 or w+q-1 leaves the image. Kernel 3x3x3, stride 1.
 *
 * Sources:
 *  - causal temporal padding repeats frame 0 on an axis that is never split (P4, commits on the
 *    LTX-2 and HunyuanVideo decoder adapters);
 *  - spatial padding is zero only at true image borders; a patch's halo rows come from its
 *    neighbours (P4, commit on how the direct path pads a patch);
 *  - halos are read in place in channels-last layout, never concatenated (P5, Description).
 *
 * The output positions computed are those in `out_box` (in y's grid; NULL = all). The inputs read
 * are out_box grown by one row/column on each side (the halo) and by two frames back, clamped to
 * the tensor. Such a box is one patch of a patch-halo decode.
 *
 * Arguments:
 *  x: [N,T,H,W,Cin] input (device), bf16, fp32, or fp16 (MFMA path only).
 *  weight: [Cout][3][3][3][Cin] (device) of dtype weight_dtype.
 *  bias: [Cout] fp32 (device), or NULL.
 *  residual: tensor of y's shape and dtype added to the result, or NULL. It may alias y. When y
 *            is bf16 or fp16 the residual may also be fp32 (a residual stream kept in fp32; the
 *            sum is rounded once, at the store).
 *  y: [N,T,H,W,Cout] output, bf16 or fp32; fp16 when x is bf16 or fp16 (MFMA path). It must
 *     not overlap x.
 *  flags: 0, or a combination of VAE_CONV_SPLIT_FP32 and one of
 *         VAE_CONV_PACKED_WEIGHTS (weight is the fragment-packed copy written by
 *         vae_conv_weight_pack; MFMA path, bf16 or fp32 x) or
 *         VAE_CONV_PACKED_F16_WEIGHTS (weight is the fp16 copy written by
 *         vae_conv_weight_pack_f16; fp16 x only).
 * bf16 weights with Cin % 32 == 0 and Cout % 4 == 0 run on the matrix cores (MFMA). Products
 * accumulate in fp32. An fp32 x is rounded to bf16 (nearest-even) as the operand, or, with
 * VAE_CONV_SPLIT_FP32, applied as two bf16 operands hi = bf16(x) and lo = bf16(x - hi). The split
 * keeps about 16 significant bits of x and costs twice the matrix-core work. An fp16 x is applied
 * as fp16 operands at the bf16 rate: the bf16 weights are converted exactly, scaled by 2^10 into
 * fp16's normal range (|w| must stay below 64), and the fp32 sums are scaled back by 2^-10, which
 * is exact. Every other case runs on a direct fp32-accumulating path, where the split flag changes
 * nothing.
 */
enum { VAE_CONV_SPLIT_FP32 = 1, VAE_CONV_PACKED_WEIGHTS = 2, VAE_CONV_PACKED_F16_WEIGHTS = 4,
       VAE_CONV_SPLIT_K = 8 };
VAE_API vae_status_t vae_conv3d_causal(const vae_tensor_t* x, const void* weight,
                                       int32_t weight_dtype, const float* bias,
                                       const vae_tensor_t* residual, vae_tensor_t* y,
                                       const vae_box_t* out_box, int32_t flags,
                                       vae_stream_t stream);

/* Causal Conv3d with work fused into its input and output stages: a nearest upsampling of its
 * input, a depth-to-space of the result, and the statistics of a GroupNorm that will read the
 * result.
 *
 * Input upsampling (in_up_sh, in_up_sw; 0 or 1 = none; powers of two up to 16). The conv reads
 * the nearest upsampling of x, u[t, h, w] = x[t, h / in_up_sh, w / in_up_sw], straight from x while
 * its input tile is staged; u is never written. The input grid below is then u's
 * [N, T, H * in_up_sh, W * in_up_sw], and zero padding applies at u's borders. This is exactly
 * vae_upsample(VAE_UPSAMPLE_NEAREST) followed by the conv, without writing and re-reading u (the
 * spatial upsampler of Wan-style decoders is a nearest upsampling followed by a conv).
 *
 * The conv is the one vae_conv3d_causal computes over out_box (in the input grid, NULL = all),
 * with Cout = y.c * st * sh * sw output channels.
 *
 * Depth-to-space (d2s_st, d2s_sh, d2s_sw; all 0 = none). Conv output channel
 * ((dt*sh + dh)*sw + dw)*C + c at (t, h, w) is written to channel c of y at
 * (st*t + dt - (st-1), sh*h + dh, sw*w + dw). Positions whose frame is below 0 are dropped (the
 * causal upsampler's first st-1 frames). y is [N, st*T-(st-1), sh*H, sw*W, C]. This is exactly
 * what vae_upsample(VAE_UPSAMPLE_D2S) does to the conv output, without writing and re-reading
 * that output. The upsampler moves channels into space (P4, LTX-2 decoder adapter commit).
 *
 * GroupNorm statistics (gn_groups > 0). gn_mean_rstd receives [N][gn_groups][2] fp32: the mean
 * of each (sample, group) of y's channels over the part of y this call writes, and
 * 1/sqrt(var + gn_eps). var is the biased variance about that global mean (divide by the count),
 * the statistic a patch-parallel GroupNorm must reproduce (P4, PatchGroupNorm commit). The
 * statistics are those of y as stored (after any rounding to bf16, after the residual).
 *  - On the MFMA path, with 4, 8, 16 or 32 channels per group (and C % 32 == 0 with a
 *    depth-to-space), the conv's epilogue forms (count, mean, M2) per output block and group
 *    while the outputs are in registers. These are merged with Chan's update in a fixed order:
 *    fp32 within a block, fp64 across blocks. y is not read again.
 *  - Other shapes run a separate statistics pass over y, with the same result up to rounding.
 *
 * Arguments:
 *  residual: as for vae_conv3d_causal (y's shape; y's dtype, or fp32), or NULL.
 *  ws / ws_bytes: device scratch of vae_conv3d_causal_fused_workspace() bytes, 16-byte aligned,
 *  owned by the caller (unused without statistics or a split over K). Its contents are
 *  undefined afterwards.
 *
 * VAE_CONV_SPLIT_K (this call only; flags of vae_conv3d_causal must not hold it): when the MFMA
 * launch over out_box would give fewer than two workgroups per compute unit (512 on the chip's
 * 256; a small box, such as one patch of the first decoder stages), the conv splits its K
 * dimension (the input-channel chunks) up to 4 ways. One launch stores each split's fp32 partial sums in ws, after the
 * statistics partials; a second adds them in split order and runs the epilogue. The result is
 * deterministic and differs from the unsplit conv only in the order of the fp32 additions. The
 * workspace query includes those bytes when the flag is given. A launch with Cout >= 128 and
 * fewer than 256 workgroups also takes 64-wide output-channel tiles instead of 128, for twice the
 * workgroups before the split: the conv's sums are the same, and its statistics partials cover
 * 128 positions each instead of 256.
 *
 * Input GroupNorm + SiLU (in_scale_shift non-NULL): the conv reads silu(x * scale_c + shift_c)
 * instead of x, with [N][Cin][2] fp32 (scale, shift) per (sample, input channel) as
 * vae_groupnorm_scale_shift writes them (device, 16-byte aligned). Each value is formed as its
 * input tile is staged and rounded to the operand type (bf16; fp16 with
 * VAE_CONV_PACKED_F16_WEIGHTS), exactly as vae_groupnorm_apply would have stored it: the result
 * equals vae_groupnorm_apply into a bf16 (fp16) tensor followed by the conv, without writing and
 * re-reading that tensor. The zero padding at the image borders pads the normalised tensor. The
 * pages name the fusion of the norm and SiLU into neighbouring kernels as a decode speed-up (P5,
 * conversation on the native Wan VAE's kernel fusions). Needs the MFMA path with packed weights
 * and no VAE_CONV_SPLIT_FP32:
 * x fp32 with VAE_CONV_PACKED_WEIGHTS or VAE_CONV_PACKED_F16_WEIGHTS, or x fp16 with
 * VAE_CONV_PACKED_WEIGHTS (UNSUPPORTED otherwise).
 *
 * Errors: those of vae_conv3d_causal; INVALID_ARG when y's shape does not match the factors;
 * UNSUPPORTED for a depth-to-space or an input upsampling off the MFMA path, for an input
 * upsampling factor that is not a power of two, for a channel count not divisible by gn_groups,
 * or for a shape vae_groupnorm_stats refuses; INVALID_ARG for gn_eps < 0, a NULL
 * gn_mean_rstd or an empty box with statistics; WORKSPACE for a short ws.
 */
typedef struct vae_conv_fused {
    const vae_tensor_t* x;
    const void* weight;             /* [Cout][3][3][3][Cin], device */
    int32_t weight_dtype;
    int32_t flags;                  /* as for vae_conv3d_causal, plus VAE_CONV_SPLIT_K */
    const float* bias;              /* [Cout] fp32, device, or NULL */
    const vae_tensor_t* residual;
    vae_tensor_t* y;
    const vae_box_t* out_box;
    int32_t d2s_st, d2s_sh, d2s_sw;
    int32_t gn_groups;              /* 0: no statistics */
    float gn_eps;
    float* gn_mean_rstd;            /* device, N * gn_groups * 2 floats */
    void* ws;
    size_t ws_bytes;
    int32_t in_up_sh, in_up_sw;     /* nearest upsampling of x read by the conv; 0 = none */
    const float* in_scale_shift;    /* input GroupNorm + SiLU, [N][Cin][2] fp32, device; or NULL */
} vae_conv_fused_t;
VAE_API vae_status_t vae_conv3d_causal_fused_workspace(const vae_conv_fused_t* args,
                                                       size_t* bytes);
VAE_API vae_status_t vae_conv3d_causal_fused(const vae_conv_fused_t* args, vae_stream_t stream);

/* Fragment-packed copy of bf16 conv weights, for the MFMA path. Layout:
 * [ceil(Cout/32)][27 taps][Cin/32][2][32][2][8], i.e. output channels in tiles of 32 and input
 * channels in chunks of 32, ordered so that each 16-byte matrix-core operand fragment of a
 * wavefront is one contiguous 1 KB read. Cout is padded to a multiple of 32 with zeros; requires
 * Cin % 32 == 0. The caller owns `packed` (device, vae_conv_weight_pack_size bytes).
 * Layout-only: the packed convolution computes exactly what the standard layout does. */
VAE_API vae_status_t vae_conv_weight_pack_size(int32_t cout, int32_t cin, size_t* bytes);
VAE_API vae_status_t vae_conv_weight_pack(const void* weight, int32_t cout, int32_t cin,
                                          void* packed, vae_stream_t stream);
/* The same layout with every bf16 weight converted to fp16 after scaling by 2^10 (exact for
 * |w| < 64; magnitudes below 2^-24 lose bits as fp16 subnormals). It is the weight operand of an
 * fp16 x (VAE_CONV_PACKED_F16_WEIGHTS). Same size as vae_conv_weight_pack_size. The call checks
 * the range: a weight of magnitude 64 or more (or not finite) would overflow fp16, and the call
 * returns VAE_ERR_UNSUPPORTED (the packed buffer is then not to be used). The check reads a
 * device flag back, so this setup call synchronises `stream`; concurrent checked packs in one
 * process are serialised. */
VAE_API vae_status_t vae_conv_weight_pack_f16(const void* weight, int32_t cout, int32_t cin,
                                              void* packed, vae_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Strided causal Conv3d (an encoder's bare downsampler)                                     */
/* ------------------------------------------------------------------------------------------ */
/*
 * y[n,t,h,w,o] = bias[o] + residual[n,t,h,w,o]
 *              + sum_{c,a,p,q} W[o,a,p,q,c] * x[n, max(st*t+a-2, 0), sh*h+p-pt, sw*w+q-pl, c]
 * with zeros where a row or column leaves the image. Kernel 3x3x3; strides st, sh, sw >= 1.
 * pad = VAE_PAD_AROUND: one zero row and column on every side (pt = pl = 1; LTX-2's bare strided
 * conv); VAE_PAD_AFTER: none before the image, one after (pt = pl = 0; the Wan / Qwen-Image
 * downsampler pads (0, 1, 0, 1) and strides 2). P4, LTX-2 and Qwen-Image/Wan encoder commit
 * messages. The temporal axis is causal, as for vae_conv3d_causal: T frames become
 * (T - 1) / st + 1.
 *
 * Arguments:
 *  x: [N,T,H,W,Cin] (device), bf16, fp32 or fp16.
 *  weight: [Cout][3][3][3][Cin] of weight_dtype, or with VAE_CONV_PACKED_WEIGHTS (bf16 x) /
 *          VAE_CONV_PACKED_F16_WEIGHTS (fp16 x) the packed copy of vae_conv_weight_pack(_f16).
 *  y: [N, (T-1)/st+1, (H+pt+pb-3)/sh+1, (W+pl+pr-3)/sw+1, Cout] (device), bf16, fp32 or fp16
 *     (fp16 only on the matrix-core path); it must not overlap x. residual (or NULL) has y's
 *     shape, y's dtype or fp32.
 *  out_box: the positions of y computed (NULL = all); its input footprint is read in place, so a
 *           box is one patch of a patch-halo encode.
 * Packed weights with a bf16 or fp16 x, Cin % 32 == 0, Cout % 4 == 0, st and sh = sw in {1, 2}
 * run on the matrix cores (fp32 accumulation; an fp16 x with fp16 weights scaled by 2^10, as for
 * vae_conv3d_causal). Standard-layout weights run on a direct fp32-accumulating path.
 * Errors: INVALID_ARG for shapes that do not match, strides < 1, an unknown pad or flags;
 * UNSUPPORTED for packed weights or fp16 tensors off the matrix-core conditions.
 */
enum { VAE_PAD_AROUND = 0, VAE_PAD_AFTER = 1 };
VAE_API vae_status_t vae_conv3d_causal_strided(const vae_tensor_t* x, const void* weight,
                                               int32_t weight_dtype, const float* bias,
                                               const vae_tensor_t* residual, vae_tensor_t* y,
                                               const vae_box_t* out_box, int32_t st, int32_t sh,
                                               int32_t sw, int32_t pad, int32_t flags,
                                               vae_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* GroupNorm (+SiLU) with statistics merged across patches                                    */
/* ------------------------------------------------------------------------------------------ */
/*
 * GroupNorm over a tensor that is cut into patches (boxes). The statistics are those of the whole
 * union of the boxes:
 *  - the global mean, and the variance about it divided by the count (biased);
 *  - not per-patch means and not Bessel's correction (P4, PatchGroupNorm commit message).
 * Each box reports (count, mean, M2) per (sample, group) over the positions it owns. The parts are
 * merged in box order with Chan et al.'s pairwise update:
 *  n = sum n_i;  mean = sum n_i mean_i / n;  M2 = sum (M2_i + n_i (mean_i - mean)^2).
 * Then y = act((x - mean) * rsqrt(M2/n + eps) * gamma + beta), with act = SiLU(z) = z / (1 + e^-z)
 * or the identity. Channel c belongs to group c / (C / groups).
 *
 * vae_groupnorm_silu performs stats, combine and apply in one call.
 *  boxes: the patches owning the statistics (n_boxes >= 1; NULL with n_boxes == 1 = whole tensor).
 *         The apply step writes y over every box.
 *  gamma, beta: [C] fp32 (device) or NULL (1 and 0).
 *  x: bf16, fp16 or fp32 (fp16: a conv output stored at half width inside a residual block).
 *  y: same shape as x; dtype bf16, fp32 or fp16 (it may differ from x: an fp32 activation
 *     normalised into the bf16 or fp16 operand of the next convolution). It may alias x when the
 *     dtypes match.
 *  ws: device scratch of at least vae_groupnorm_silu_workspace() bytes.
 * Partials are combined in a fixed order: results are bitwise reproducible run to run.
 */
VAE_API vae_status_t vae_groupnorm_silu_workspace(const vae_tensor_t* x, const vae_box_t* boxes,
                                                  int32_t n_boxes, int32_t groups, size_t* bytes);
VAE_API vae_status_t vae_groupnorm_silu(const vae_tensor_t* x, const vae_box_t* boxes,
                                        int32_t n_boxes, int32_t groups, float eps,
                                        const float* gamma, const float* beta, int32_t apply_silu,
                                        vae_tensor_t* y, void* ws, size_t ws_bytes,
                                        vae_stream_t stream);

/* vae_groupnorm_silu without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture into a graph, tight serving loops, harnesses that forbid
 * allocation). Same arguments and result: it runs the same kernels, bit for bit. Its scratch (the
 * partials and mean/rstd) is a fixed 8 MiB array in the library's device memory, one per GPU,
 * held until the process ends; its address is looked up on the first call on each device. A call
 * needing more (vae_groupnorm_silu_workspace() > 8 MiB: about N * groups * 3 * 8 bytes per
 * statistics block, at most 4096 blocks) is refused with VAE_ERR_UNSUPPORTED, info.extent = the
 * bytes needed and info.min_width = the bytes held. It allocates nothing and never
 * synchronises. Calls that overlap on one GPU (other streams, other host threads) share that
 * array and race; serialise them. Nothing in it needs clearing between calls: the statistics pass
 * writes every partial the merge reads. */
VAE_API vae_status_t vae_groupnorm_silu_noalloc(const vae_tensor_t* x, const vae_box_t* boxes,
                                                int32_t n_boxes, int32_t groups, float eps,
                                                const float* gamma, const float* beta,
                                                int32_t apply_silu, vae_tensor_t* y,
                                                vae_stream_t stream);

/* The same operation in three steps, for callers that move the per-box partials themselves.
 * vae_groupnorm_stats: per box, (count, mean, M2) as fp64 into part[n_boxes][N][groups][3]
 *   (device). ws is sized by vae_groupnorm_stats_workspace().
 * vae_groupnorm_combine: merges part[0..n_parts) in order and writes mean_rstd[N][groups][2]
 *   fp32 (mean, 1/sqrt(var + eps)) (device).
 * vae_groupnorm_apply: the normalise (+SiLU) step over `box` (NULL = whole) with given mean_rstd.
 */
VAE_API vae_status_t vae_groupnorm_stats_workspace(const vae_tensor_t* x, const vae_box_t* boxes,
                                                   int32_t n_boxes, int32_t groups, size_t* bytes);
VAE_API vae_status_t vae_groupnorm_stats(const vae_tensor_t* x, const vae_box_t* boxes,
                                         int32_t n_boxes, int32_t groups, double* part, void* ws,
                                         size_t ws_bytes, vae_stream_t stream);
VAE_API vae_status_t vae_groupnorm_combine(const double* part, int32_t n_parts, int32_t n,
                                           int32_t groups, float eps, float* mean_rstd,
                                           vae_stream_t stream);
VAE_API vae_status_t vae_groupnorm_apply(const vae_tensor_t* x, const vae_box_t* box,
                                         int32_t groups, const float* mean_rstd,
                                         const float* gamma, const float* beta,
                                         int32_t apply_silu, vae_tensor_t* y, vae_stream_t stream);

/* The normalise step as a per-channel affine map, for a conv that applies it while staging its
 * input (vae_conv_fused_t.in_scale_shift): scale_shift[N][channels][2] fp32 (device, 16-byte
 * aligned) receives, for channel c of group g = c / (channels / groups),
 *   scale = rstd[n][g] * gamma[c],  shift = beta[c] - mean[n][g] * scale
 * (gamma = NULL reads as 1, beta = NULL as 0), from mean_rstd[N][groups][2] as
 * vae_groupnorm_combine writes it. silu(x * scale + shift) is then exactly the value
 * vae_groupnorm_apply(apply_silu = 1) computes for x (P4, PatchGroupNorm commit: the global
 * mean and biased variance). INVALID_ARG for n < 0,
 * groups < 1, channels not a multiple of groups or of 8, a NULL mean_rstd or scale_shift, or a
 * misaligned scale_shift. */
VAE_API vae_status_t vae_groupnorm_scale_shift(const float* mean_rstd, int32_t n, int32_t channels,
                                               int32_t groups, const float* gamma,
                                               const float* beta, float* scale_shift,
                                               vae_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* RMS norm and frame attention (Wan-style decoders)                                          */
/* ------------------------------------------------------------------------------------------ */
/*
 * y = act(x / sqrt(mean_c(x^2) + eps) * gamma + beta) at every position, act = SiLU or the identity.
 * The norm reduces over the channels of one position only, so a patch-split decode needs no
 * statistics from other patches (P4, commit messages on the Qwen-Image / Wan adapters and on the
 * HunyuanVideo 1.5 encoder: RMS norms that reduce over channels need nothing sharded). The pages
 * give no formula; this is the root mean square of the channel vector with eps inside the root.
 *  x: bf16, fp16 or fp32, C % 8 == 0 and C / 8 dividing 256 (else UNSUPPORTED with info).
 *  gamma, beta: [C] fp32 (device) or NULL (1 and 0).
 *  y: x's shape; bf16, fp16 or fp32. It may alias x when the dtypes match.
 */
VAE_API vae_status_t vae_rmsnorm_silu(const vae_tensor_t* x, float eps, const float* gamma,
                                      const float* beta, int32_t apply_silu, vae_tensor_t* y,
                                      vae_stream_t stream);

/*
 * Single-head self-attention over the H*W positions of each frame (each sample and T index), plus
 * the residual: the mid-block attention of Wan-style decoders, which takes a frame whole, so a
 * patch-split decode gathers the frame around it (P4, commit message on the HunyuanVideo adapters;
 * P5, Description: the Wan attention block). The pages give no formula; the plainest reading:
 *   xn = rms_norm(x) with gamma/beta (no SiLU);  [q | k | v] = xn W_qkv^T + b_qkv;
 *   y = softmax(q k^T / sqrt(C)) v W_out^T + b_out + x   (softmax over the frame's positions).
 * Arithmetic: xn and the projections' operands bf16; q, k, v and the softmax weights fp16; every
 * product accumulates in fp32; the logits and y are fp32.
 *  x, y: fp32 [N,T,H,W,C], C % 32 == 0 and C / 8 dividing 256; y may alias x.
 *  w_qkv: bf16 [3C][C] (rows: q, then k, then v), b_qkv [3C] fp32 or NULL; w_out: bf16 [C][C],
 *  b_out [C] fp32 or NULL; gamma, beta: [C] fp32 or NULL. All device.
 *  ws: device scratch of vae_frame_attention_workspace() bytes (16-byte aligned); contents undefined
 *  afterwards. It holds about (8C + 6 H*W) * N*T*H*W bytes.
 */
VAE_API vae_status_t vae_frame_attention_workspace(const vae_tensor_t* x, size_t* bytes);
VAE_API vae_status_t vae_frame_attention(const vae_tensor_t* x, float eps, const float* gamma,
                                         const float* beta, const void* w_qkv,
                                         const float* b_qkv, const void* w_out,
                                         const float* b_out, vae_tensor_t* y, void* ws,
                                         size_t ws_bytes, vae_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Upsampling                                                                                 */
/* ------------------------------------------------------------------------------------------ */
/*
 * VAE_UPSAMPLE_NEAREST: y[t, sh*h+dh, sw*w+dw, c] = x[t, h, w, c]; requires st == 1.
 * VAE_UPSAMPLE_D2S: depth-to-space, one input position per output position (P4, LTX-2 decoder
 *   adapter commit): y[st*t+dt-(st-1), sh*h+dh, sw*w+dw, c] = x[t, h, w, ((dt*sh+dh)*sw+dw)*C + c],
 *   keeping only output frames >= 0. That is the causal drop of the first st-1 frames:
 *   T -> st*T - (st-1). The pages leave the channel order open; this one (sub-position slowest,
 *   channel fastest) makes every output row a contiguous slice of an input row. Any other fixed
 *   order is one permutation of the producing conv's output channels.
 * box: input positions to upsample (in x's grid; NULL = all). y must have the upsampled shape.
 * x and y have the same dtype and must not overlap.
 */
enum { VAE_UPSAMPLE_NEAREST = 1, VAE_UPSAMPLE_D2S = 2 };
VAE_API vae_status_t vae_upsample(const vae_tensor_t* x, const vae_box_t* box, int32_t mode,
                                  int32_t st, int32_t sh, int32_t sw, vae_tensor_t* y,
                                  vae_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Space-to-depth (the encoder's fold)                                                        */
/* ------------------------------------------------------------------------------------------ */
/*
 * The encoder's downsampling fold, the mirror of VAE_UPSAMPLE_D2S (P4, encoder commits: most
 * LTX-2 downsamplers fold space into channels after a stride-1 convolution, one input position
 * per output): st-1 copies of frame 0 go in front (causal), then
 *   y[t, h, w, ((dt*sh+dh)*sw+dw)*C + c] = x[max(st*t+dt-(st-1), 0), sh*h+dh, sw*w+dw, c].
 * T frames become (T + st - 1) / st; vae_upsample with VAE_UPSAMPLE_D2S and the same factors
 * gives x back.
 *  x: [N,T,H,W,C] with (T + st - 1) % st == 0, H % sh == 0, W % sw == 0 (else UNSUPPORTED with
 *     info); any dtype.
 *  y: [N, (T+st-1)/st, H/sh, W/sw, C*st*sh*sw], x's dtype; must not overlap x.
 */
VAE_API vae_status_t vae_space_to_depth(const vae_tensor_t* x, int32_t st, int32_t sh, int32_t sw,
                                        vae_tensor_t* y, vae_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Tile split / merge                                                                         */
/* ------------------------------------------------------------------------------------------ */
/*
 * Two ways to cut a decode:
 *  VAE_TILING_PATCH_HALO (mode A). The latent is cut into patches_h x patches_w bands. With L rows
 *    over p bands, the first L % p bands get one row more (P4, Patchify commit message). Every conv
 *    reads a one-row halo from the neighbouring patches, and GroupNorm merges per-patch statistics.
 *    The result equals the untiled decode up to float re-association.
 *  VAE_TILING_OVERLAP_BLEND (mode B). Tiles of tile_* latent rows start at 0, stride, 2*stride,
 *    ... < L, each min(tile, L - start) long. An axis no longer than its tile is not cut (P2, review
 *    thread: tile 512 / stride 448 px turns 576 into 512 + 128; 256 stays untiled). Each tile is
 *    decoded alone and blended with separable linear ramps (P1, Approach: a mask built from
 *    per-axis parts, a weight buffer, a divide). Where consecutive tiles overlap by E output
 *    samples, the later tile rises as (j+1)/(E+1) and the earlier one falls as (E-j)/(E+1),
 *    j = 0..E-1.
 *    Mode B also cuts T when tile_t > 0 (P1, Approach: the tiles overlap in space and in time).
 * Output boxes: spatial = latent box * scale. T is causal: a clip of n latent frames decodes to
 * 1 + (n-1)*scale_t frames, and the clip [t0, t1) lands on output frames
 * [t0*scale_t, (t1-1)*scale_t + 1), its single first frame standing for the last frame of latent
 * frame t0 in the whole decode (the pages do not say how temporal tiles line up; this is the
 * reading the causal decoder supports). With scale_t > 1, consecutive temporal tiles must share a
 * latent frame (stride_t < tile_t), or the scale_t - 1 frames before a tile's first frame would
 * come from no tile. Overlaps E are measured between neighbouring tiles' output spans.
 * Encoders (down_* > 1 = the plan's folds, scales 1, T whole): n, t, h, w are the input video's
 * extents, and tiles are cut on the output latent grid of (t + down_t - 1) / down_t frames,
 * h / down_h rows and w / down_w columns. Each tile's `latent` box is then its input-video box
 * (latent rows times the fold, all frames) and `out` its latent box.
 *  mode A: the bands are whole multiples of the fold (P4, encoder commit), i.e. the band rule over
 *    latent rows; the result equals the untiled encode.
 *  mode B: (P2: sample tiles 512 with stride 448 are 16 / 14 latent rows at a fold of 32, with
 *    per-tile latent shapes and a latent-space blend) the ramps run over the latent overlaps.
 * An encoder plan also runs untiled with patches 1 x 1 and no down_*.
 */
enum { VAE_TILING_PATCH_HALO = 1, VAE_TILING_OVERLAP_BLEND = 2 };

typedef struct vae_tiling_desc {
    int32_t mode;                        /* VAE_TILING_* */
    int32_t n, t, h, w;                  /* latent extents */
    int32_t scale_t, scale_h, scale_w;   /* latent -> output scale */
    int32_t patches_h, patches_w;        /* mode A grid */
    int32_t tile_h, tile_w;              /* mode B tile size, latent rows */
    int32_t stride_h, stride_w;          /* mode B tile stride, latent rows */
    int32_t tile_t, stride_t;            /* mode B temporal tiles, latent frames (0: T whole) */
    int32_t down_t, down_h, down_w;      /* an encoder's folds (0 or 1: none); see below */
} vae_tiling_desc_t;

typedef struct vae_tile {
    int32_t index, row, col;
    vae_box_t latent;                    /* latent grid */
    vae_box_t out;                       /* output grid */
    int32_t lead_t, lead_h, lead_w;      /* overlap with the previous tile, output samples */
    int32_t trail_t, trail_h, trail_w;   /* overlap with the next tile, output samples */
} vae_tile_t;

/* Host-only. tiles == NULL: *n_tiles receives the count. Otherwise up to `capacity` tiles, in
 * row-major order, are written and *n_tiles is the count. Refused (VAE_ERR_UNSUPPORTED, info
 * filled): a band that would be empty (a patch narrower than the one-row halo, P4,
 * calc_bottom_halo_width commit); a stride outside 1..tile; a temporal stride that is not below
 * the temporal tile while scale_t > 1 (info.axis = 1). Tiles come T-major, then H, then W; `row`
 * and `col` index the H and W tiles. */
VAE_API vae_status_t vae_tile_split(const vae_tiling_desc_t* desc, vae_tile_t* tiles,
                                    int32_t capacity, int32_t* n_tiles);

/* Blends one decoded tile into the full output. `out` accumulates (fp32):
 *   out[box] += w(t,h,w) * tile_out, with w = product of the tile's 1-D ramps.
 * flags: VAE_MERGE_ZERO zeroes all of `out` before this tile is added (give it to the first tile).
 *        VAE_MERGE_FINALIZE divides all of `out` by the summed weights after this tile is added
 *        (give it to the last tile). The sums come from the tile grid of `desc`, per axis.
 * tile_out: fp32 [N, out box extents, C]; out: fp32 [N, T_out, H_out, W_out, C].
 * This is the vae_tiling_desc_t / vae_tile_t returned by vae_tile_split for mode B. */
enum { VAE_MERGE_ZERO = 1, VAE_MERGE_FINALIZE = 2 };
VAE_API vae_status_t vae_tile_merge(const vae_tensor_t* tile_out, const vae_tile_t* tile,
                                    const vae_tiling_desc_t* desc, vae_tensor_t* out,
                                    int32_t flags, vae_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Whole decoder                                                                              */
/* ------------------------------------------------------------------------------------------ */
/*
 * A decoder is a layer plan plus device weight pointers. Each op reads and writes a channels-last
 * activation:
 *  VAE_OP_CONV    causal Conv3d cin -> cout (f32_out = 1 writes fp32: the last conv of a bf16 plan)
 *  VAE_OP_RES     residual block of width cin: GN+SiLU, conv, GN+SiLU, conv, plus the block input
 *  VAE_OP_GN_SILU GroupNorm + SiLU
 *  VAE_OP_D2S     depth-to-space (st, sh, sw) with the causal frame drop
 *  VAE_OP_NEAREST nearest spatial upsampling (sh, sw)
 *  VAE_OP_RES_RMS residual block of width cin with RMS norms (vae_rmsnorm_silu) for the GroupNorms
 *  VAE_OP_RMS_SILU RMS norm + SiLU
 *  VAE_OP_ATTN    single-head frame attention of width cin (vae_frame_attention), fp32 activations
 *  VAE_OP_S2D     space-to-depth fold (st, sh, sw) with the causal front copies of frame 0
 *                 (vae_space_to_depth): an encoder plan. Such a plan runs untiled, or tiled with
 *                 the tiling desc's down_* set to its folds; its input extents must fold evenly.
 *  VAE_OP_CONV_DOWN strided causal conv cin -> cout, strides (st, sh, sw), zero padding `pad`
 *                 (vae_conv3d_causal_strided): an encoder's downsampler. Its strides count as
 *                 folds of the plan (down_*), and its input's H and W must be whole strides.
 * Dtypes:
 *  - conv weights and GroupNorm outputs (the operands of the next conv) have the plan dtype;
 *  - conv outputs and the residual stream have act_dtype, which must be VAE_DTYPE_F32 (anything
 *    else is refused with VAE_ERR_UNSUPPORTED): with bf16 weights this keeps the bf16 rounding
 *    to the conv operands alone. Storing the activations in bf16 adds about 40 roundings on the
 *    way through the LTX-2-shaped plan and misses the 2e-2 max-abs bound of a bf16 decode;
 *  - the latent has the plan dtype, and the decoded output is fp32.
 * VAE_DECODE_SPLIT_FP32_OPERANDS goes further for convs that read an fp32 activation (the
 * upsampling convs read the fp32 residual stream): each such CONV runs with VAE_CONV_SPLIT_FP32
 * unless its no_split is set. A standalone GN_SILU followed by a splitting CONV writes fp32 for
 * it. The convs inside residual blocks keep one rounding of their GroupNorm operand.
 * VAE_DECODE_F16_OPERANDS (bf16 plans with fp32 activations; not with the split flag) gives
 * those same convs, i.e. every CONV that follows a RES, RES_RMS, GN_SILU, RMS_SILU, or a CONV
 * whose own input is bf16 or fp16 (possibly through its fused D2S and NEAREST ops, which copy),
 * fp16 operands instead: the producing op stores its output in
 * fp16 (one rounding to 11 significant bits) and the conv runs at the bf16 rate
 * (vae_conv3d_causal with an fp16 x). no_split does not apply to it. The flag also stores the
 * output of the first conv of each RES and RES_RMS block, which only its block's second norm
 * reads, in fp16 instead of fp32 (half the bytes written and read back). Activations must stay
 * below 65504 in magnitude in both places.
 * VAE_DECODE_NORM_IN_CONV: GroupNorm apply + SiLU is done by the conv that reads the norm's
 * output, while it stages its input (vae_conv_fused_t.in_scale_shift), wherever that conv runs
 * on the matrix cores with packed weights (vae_decoder_pack_weights) and without the fp32 split,
 * reading fp32 (or fp16 with bf16 weights): the first and second norm of every RES block and a
 * GN_SILU followed by a CONV. The normalised tensor is then never written; the results are the
 * same bit for bit. The norm's statistics still come from the producing conv's epilogue (or a
 * statistics pass). Off by default: on gfx950 those convs then stage through their tile buffer
 * instead of the faster frame ring (which has no registers left for the norm beside 128-channel
 * tiles), and the decode is slower overall than with separate normalise passes.
 * The parameter pointers come in plan order:
 *  conv, conv_down -> (weight, bias);
 *  GN or RMS -> (gamma, beta);
 *  res, res_rms -> norm, conv, norm, conv;
 *  attn -> (gamma, beta, w_qkv [3C][C] bf16, b_qkv [3C], w_out [C][C] bf16, b_out [C]).
 * bias, gamma and beta may be NULL.
 */
enum { VAE_OP_CONV = 1, VAE_OP_RES = 2, VAE_OP_GN_SILU = 3, VAE_OP_D2S = 4, VAE_OP_NEAREST = 5,
       VAE_OP_RES_RMS = 6, VAE_OP_RMS_SILU = 7, VAE_OP_ATTN = 8, VAE_OP_S2D = 9,
       VAE_OP_CONV_DOWN = 10 };

typedef struct vae_layer_desc {
    int32_t op;
    int32_t cin, cout;
    int32_t st, sh, sw;
    int32_t f32_out;
    int32_t no_split;  /* conv only: 1 = round an fp32 input to bf16 once even when the decoder
                          splits fp32 operands (VAE_DECODE_SPLIT_FP32_OPERANDS) */
    int32_t pad;       /* VAE_OP_CONV_DOWN: VAE_PAD_AROUND or VAE_PAD_AFTER; 0 otherwise */
} vae_layer_desc_t;

enum { VAE_DECODE_SPLIT_FP32_OPERANDS = 1, VAE_DECODE_F16_OPERANDS = 2,
       VAE_DECODE_NORM_IN_CONV = 4 };
typedef struct vae_decoder_spec {
    int32_t dtype;              /* weights and convolution operands: VAE_DTYPE_* */
    int32_t act_dtype;          /* activations stored between ops (conv outputs, residual
                                   stream): VAE_DTYPE_F32 */
    int32_t flags;              /* VAE_DECODE_SPLIT_FP32_OPERANDS or VAE_DECODE_F16_OPERANDS,
                                   plus VAE_DECODE_NORM_IN_CONV; or 0 */
    int32_t latent_channels;
    int32_t groups;
    float eps;
    int32_t n_layers;
    const vae_layer_desc_t* layers;
} vae_decoder_spec_t;

typedef struct vae_decoder vae_decoder_t;

/* Validates the plan and keeps a copy of it, along with the `n_ptrs` device pointers (no copy
 * of the weights themselves). */
VAE_API vae_status_t vae_decoder_create(const vae_decoder_spec_t* spec,
                                        const void* const* params, int32_t n_ptrs,
                                        vae_decoder_t** out);
VAE_API void vae_decoder_destroy(vae_decoder_t* dec);

/* Optional fragment-packed weights for the decoder's MFMA convs. The caller supplies a device
 * buffer of vae_decoder_packed_weight_size bytes, which must outlive the decoder. The pack is
 * enqueued on `stream`, and later decodes read the packed copies instead of the standard ones.
 * The results are identical; the packed copies are faster to load. The convs that take fp16
 * operands (VAE_DECODE_F16_OPERANDS) are packed as vae_conv_weight_pack_f16 does, with its range
 * check: a weight of magnitude 64 or more there is refused with VAE_ERR_UNSUPPORTED,
 * info.extent = the conv's index in plan order (counting every conv, residual blocks' two each),
 * and the decoder keeps its standard weights. With such convs the call synchronises `stream`. */
VAE_API vae_status_t vae_decoder_packed_weight_size(const vae_decoder_t* dec, size_t* bytes);
VAE_API vae_status_t vae_decoder_pack_weights(vae_decoder_t* dec, void* buf, size_t bytes,
                                              vae_stream_t stream);

/* How a patch-halo decode (mode A with more than one patch) launches its work on one GPU.
 *  VAE_LAUNCH_MERGED (the default): one launch per layer covers every patch box at once; each
 *    patch's halo is its neighbour's data read in place, and a GroupNorm's statistics come from
 *    the blocks of that one launch. The fastest way to run the whole decode on one device.
 *  VAE_LAUNCH_PER_PATCH: every conv, GroupNorm pass and upsampling is launched once per patch
 *    box, over that box only (its out_box), reading its halo in place: the work of one rank of a
 *    patch split (P4, commits on PatchConv3d, Patchify and PatchGroupNorm). A GroupNorm's
 *    statistics are formed per patch box as (count, mean, M2) and merged across the boxes with
 *    Chan's update in patch order before any box is normalised. The per-position RMS norm, the
 *    whole-frame attention and the space-to-depth fold stay one launch each. With timing on,
 *    each launch is recorded with its patch index in vae_op_timing_t.tile (-1: the merge of the
 *    statistics, shared by all patches).
 * Both give the untiled decode up to the rounding order of the statistics. The workspace size
 * depends on the setting: query it after setting it. Mode B ignores it.
 * Returns VAE_ERR_INVALID_ARG for another value. */
enum { VAE_LAUNCH_MERGED = 0, VAE_LAUNCH_PER_PATCH = 1 };
VAE_API vae_status_t vae_decoder_set_launch(vae_decoder_t* dec, int32_t launch);

/* Clip-by-clip decode ("[TRTLLM-14029][feat] LTX-2 tile-parallel VAE decode", Description: the
 * decode's overlapping spatial/temporal tiles of a causal decoder). With frames > 0 a mode A
 * decode of more than `frames` latent frames runs clip by clip: latent frames [0, frames),
 * [frames, 2 frames), ... (the last clip may be shorter), each through the whole plan, writing
 * its own output frames. Every causal conv keeps the last two frames of its input in the
 * workspace and reads them in front of the next clip's first frame, where the first clip reads
 * copies of its frame 0; a causal depth-to-space drops its leading frames in the first clip only.
 * The result is the whole decode's up to rounding order (the same arithmetic, frame for frame),
 * while every activation holds one clip: the workspace shrinks with the clip.
 * frames = 0 (the default) decodes all frames at once.
 * Refused (VAE_ERR_UNSUPPORTED) unless the plan is bf16 and every op is local in time: convs,
 * RMS norms, frame attention and upsamplings (a GroupNorm's statistics span every frame; a fold
 * that narrows time has no carry defined). At decode time a clip-by-clip decode takes N = 1 and
 * refuses a temporal depth-to-space not fused into a matrix-core conv (VAE_ERR_UNSUPPORTED).
 * Query the workspace after setting it. Mode B ignores it. */
VAE_API vae_status_t vae_decoder_set_clip_frames(vae_decoder_t* dec, int32_t frames);

/* Device scratch needed by vae_decode_tiled for this tiling (latent extents come from desc). */
VAE_API vae_status_t vae_decode_workspace_size(const vae_decoder_t* dec,
                                               const vae_tiling_desc_t* desc, size_t* bytes);

/*
 * Decodes `latent` ([N,T,H,W,latent_channels], the plan's dtype) into `out` (fp32, NDHWC).
 * mode A (patch-halo):
 *  - convs, upsampling and the final placement cover the patch boxes, and each patch's halo is
 *    its neighbour's data read in place; launched per layer or per patch box
 *    (vae_decoder_set_launch);
 *  - GroupNorm statistics are those of the whole tensor (the global mean and the biased
 *    variance), merged across patches per box with the per-patch launches.
 *  The result equals the untiled decode.
 * mode B (overlap-blend):
 *  - each tile is decoded alone, one tile in flight, with its own borders and statistics;
 *  - every tile is blended into `out` with vae_tile_merge's weights and normalised at the end.
 *  This is the serial tiled decode of P1.
 * desc's latent extents must match `latent`, and its scales the plan. ws must hold at least
 * vae_decode_workspace_size() bytes. All work goes on `stream`; per-tile host work is only
 * integer geometry, computed once per call.
 */
VAE_API vae_status_t vae_decode_tiled(const vae_decoder_t* dec, const vae_tensor_t* latent,
                                      const vae_tiling_desc_t* desc, vae_tensor_t* out, void* ws,
                                      size_t ws_bytes, vae_stream_t stream);

/* Status of the most recent vae_decode_tiled call that used `ws` (same decoder and tiling desc):
 * *flags = VAE_STATUS_NONFINITE when a GroupNorm's or RMS norm's statistics were not finite,
 * i.e. an activation became inf or NaN. The usual cause is a value past fp16's 65504 at an fp16
 * operand hand-off (VAE_DECODE_F16_OPERANDS): the output is then not to be trusted. 0 otherwise.
 * Each decode clears the word it sets (with a kernel, so a captured decode keeps the behaviour);
 * this call synchronises `stream` and reads the word back. */
enum { VAE_STATUS_NONFINITE = 1 };
VAE_API vae_status_t vae_decode_status(const vae_decoder_t* dec, const vae_tiling_desc_t* desc,
                                       const void* ws, size_t ws_bytes, int32_t* flags,
                                       vae_stream_t stream);

/* Per-op GPU timing of the most recent vae_decode_tiled call (events recorded on its stream).
 * Enabled with vae_decoder_set_timing(dec, 1); collecting waits for the last recorded event. */
enum { VAE_KIND_CONV = 1, VAE_KIND_GN = 2, VAE_KIND_UPSAMPLE = 3, VAE_KIND_MERGE = 4,
       VAE_KIND_OTHER = 5, VAE_KIND_RMS = 6, VAE_KIND_ATTN = 7 };
typedef struct vae_op_timing {
    int32_t kind;       /* VAE_KIND_* */
    int32_t layer;      /* index in the plan */
    int32_t tile;       /* tile index (mode B), patch index (per-patch launches) or -1 */
    int32_t reserved;
    double ms;          /* GPU time between the events around the op */
    double flops;       /* algorithmic flops (convs: 2 * 27 * Cin * Cout * positions) */
    double bytes;       /* algorithmic HBM bytes (streaming passes: bytes read + written) */
} vae_op_timing_t;
VAE_API vae_status_t vae_decoder_set_timing(vae_decoder_t* dec, int32_t enable);
VAE_API vae_status_t vae_decoder_get_timing(vae_decoder_t* dec, vae_op_timing_t* out,
                                            int32_t capacity, int32_t* n);

#ifdef __cplusplus
}
#endif
#endif /* VAE_MI355X_H */
