// Internal kernel launchers (not part of the C ABI). Every launcher assumes its arguments were
// validated by the ABI layer; it only enqueues work on `stream` and reports launch errors.
#pragma once

#include "common.h"
#include "tiling_math.h"

namespace vae {

constexpr int kMaxBoxes = 16;

struct BoxList {
    Box b[kMaxBoxes];
    int32_t n;
};

// ---- convolution ----
// Optional work fused into the MFMA conv's epilogue:
//  - depth-to-space (st, sh, sw), st = sh = sw = 1 for none: y is then the depth-to-space of the
//    conv output (channels y.c * st * sh * sw), with the causal drop of the first st-1 frames;
//  - GroupNorm partials of y as stored (gn_ws non-null): fp64 (count, mean, M2) per
//    [N][groups][slots]; conv_gn_slots() gives the slot count, or 0 when the shapes need the
//    separate statistics pass.
//  - a nearest upsampling of the input by (1 << lsh, 1 << lsw), read while the input tile is
//    staged: x is then the tensor before that upsampling, and every extent and box refers to the
//    upsampled grid.
// The partials of one launch fill slots [slot0, slot0 + conv_gn_slots(box)) of rows that are
// slot_stride slots long (0: the launch's own count), so that the launches of several patch
// boxes can share one array and be merged together.
// With `part` (conv_split_bytes(...) bytes of fp32 scratch) and splits > 1 the MFMA conv splits
// its K dimension `splits` ways: one launch stores each split's partial sums, a second adds them
// in split order and runs the epilogue (deterministic; the sums differ from the unsplit conv's
// only by the order of their fp32 additions).
struct ConvFuse {
    double* gn_ws;
    int32_t groups;
    int32_t st, sh, sw;
    int32_t lsh = 0, lsw = 0;
    int64_t slot0 = 0, slot_stride = 0;
    float* part = nullptr;
    int32_t splits = 1;
    // Frames of the depth-to-space output dropped before y's frame 0 (see MfmaArgs::tdrop);
    // -1: st - 1, the causal drop.
    int32_t tdrop = -1;
    // GroupNorm + SiLU of x applied while staging (MFMA path, packed weights): fp32 (scale,
    // shift) per (sample, input channel), [N][Cin][2]; the conv reads silu(x * scale + shift).
    const float* in_ab = nullptr;
};
vae_status_t launch_conv3d(const vae_tensor_t& x, const void* w, int32_t weight_dtype,
                           const float* bias, const vae_tensor_t* residual, const vae_tensor_t& y,
                           const Box& box, int32_t flags, hipStream_t stream,
                           const ConvFuse* fz = nullptr);
bool conv_uses_mfma(const vae_tensor_t& x, const vae_tensor_t& y, int32_t weight_dtype);
bool conv_uses_mfma_c(const vae_tensor_t& x, int64_t cout, int32_t weight_dtype);
// yc: channels of y; k = st * sh * sw of the fused depth-to-space (1 for none).
// fill: the launch may take narrower channel tiles to fill the chip (VAE_CONV_SPLIT_K).
int64_t conv_gn_slots(const vae_tensor_t& x, int64_t yc, int32_t weight_dtype, const Box& box,
                      int32_t groups, int32_t k, bool fill);
// Split over K for launches that would leave most of the chip idle (VAE_CONV_SPLIT_K): the number
// of splits worth making for a conv of x (its input grid) to `cout` channels over `box` (1: none),
// and the scratch bytes of that many splits. `split_fp32`: the conv applies an fp32 x as hi + lo.
int32_t conv_split_count(const vae_tensor_t& x, int64_t cout, int32_t weight_dtype, const Box& box,
                         bool split_fp32);
size_t conv_split_bytes(const vae_tensor_t& x, int64_t cout, const Box& box, int32_t splits);
// Fragment-packed bf16 weights (see conv3d.hip): element count and the packing kernel.
int64_t packed_weight_elems(int64_t cout, int64_t cin);
// to_f16: fp16(w * 2^10), the weight operand of fp16 inputs.
vae_status_t launch_pack_weights(const void* w, int32_t cout, int32_t cin, void* packed,
                                 hipStream_t stream, bool to_f16 = false);

// ---- strided conv (an encoder's bare downsampler) ----
// Strides (st, sh, sw) and the zero rows / columns before the image (pt top, pl left); the ones
// after it follow from y's extents.
struct StrideGeom {
    int32_t st, sh, sw, pt, pl;
};
// Whether the strided conv runs on the matrix cores: bf16 weights fragment-packed (bf16 or, for
// an fp16 x, fp16), a 2-byte x, Cin % 32 == 0, Cout % 4 == 0, strides 1 or 2 with sh == sw.
bool conv_strided_uses_mfma(const vae_tensor_t& x, int64_t cout, int32_t weight_dtype,
                            int32_t flags, const StrideGeom& g);
// Slots of the GroupNorm partials its epilogue gathers over `box` (of y), per (sample, group);
// 0 when the channel grouping does not allow it.
int64_t conv_strided_gn_slots(const vae_tensor_t& y, const Box& box, int32_t groups);
// `fz` may carry gn_ws (statistics of y as stored; matrix-core path only); its other fields are
// ignored.
vae_status_t launch_conv3d_strided(const vae_tensor_t& x, const void* w, int32_t weight_dtype,
                                   const float* bias, const vae_tensor_t* residual,
                                   const vae_tensor_t& y, const Box& box, const StrideGeom& g,
                                   int32_t flags, hipStream_t stream,
                                   const ConvFuse* fz = nullptr);

// ---- group norm ----
// Workspace: per-block partials of every box, fp64 [blocks][N][G][3].
size_t gn_stats_workspace(const vae_tensor_t& x, const BoxList& boxes, int32_t groups);
// Per-block partials -> per-box partials (part_out, optional) and mean/rstd (optional).
// `status` (optional, device): set to 1 when a group's statistics are not finite.
vae_status_t launch_gn_stats(const vae_tensor_t& x, const BoxList& boxes, int32_t groups,
                             double* ws, double* part_out, float* mean_rstd, float eps,
                             hipStream_t stream, uint32_t* status = nullptr);
vae_status_t launch_gn_combine(const double* part, int32_t n_parts, int32_t n, int32_t groups,
                               float eps, float* mean_rstd, hipStream_t stream,
                               uint32_t* status = nullptr);
// Partials [N][groups][slots][3] (as a fused conv writes them) -> mean/rstd [N][groups][2].
// Large slot counts are merged in two passes, the first in place over ws (whose contents are
// then spent).
vae_status_t launch_gn_finalize_slots(double* ws, int64_t slots, int32_t n, int32_t groups,
                                      float eps, float* mean_rstd, hipStream_t stream,
                                      uint32_t* status = nullptr);
// The apply step's per-(sample, channel) scale and shift, [N][C][2] fp32 (ConvFuse::in_ab).
vae_status_t launch_gn_scale_shift(const float* mean_rstd, int32_t n, int32_t c, int32_t groups,
                                   const float* gamma, const float* beta, float* ab,
                                   hipStream_t stream);
vae_status_t launch_gn_apply(const vae_tensor_t& x, const Box& box, int32_t groups,
                             const float* mean_rstd, const float* gamma, const float* beta,
                             bool silu, const vae_tensor_t& y, hipStream_t stream);
bool gn_shape_supported(const vae_tensor_t& x, int32_t groups);

// ---- RMS norm and frame attention (Wan-style decoders) ----
bool rms_shape_supported(int64_t c);
// y = x / sqrt(mean_c(x^2) + eps) * gamma + beta (+ SiLU) per position; x bf16/fp32, y any dtype.
// `status` (optional, device): set to 1 when a position's sum of squares is not finite.
vae_status_t launch_rms_norm(const vae_tensor_t& x, float eps, const float* gamma,
                             const float* beta, bool silu, const vae_tensor_t& y,
                             hipStream_t stream, uint32_t* status = nullptr);
bool attention_shape_supported(int64_t c);
size_t attention_workspace(const vae_tensor_t& x);
// Single-head attention over each frame's positions plus the residual; fp32 x and y (y may be
// x); bf16 weights w_qkv [3C][C] and w_out [C][C]; ws of attention_workspace(x) bytes.
vae_status_t launch_frame_attention(const vae_tensor_t& x, float eps, const float* gamma,
                                    const float* beta, const void* w_qkv, const float* b_qkv,
                                    const void* w_out, const float* b_out, const vae_tensor_t& y,
                                    void* ws, hipStream_t stream);

// ---- upsampling ----
vae_status_t launch_upsample(const vae_tensor_t& x, const Box& box, int32_t mode, int32_t st,
                             int32_t sh, int32_t sw, const vae_tensor_t& y, hipStream_t stream);

// ---- space-to-depth (encoder fold, causal front pad) ----
vae_status_t launch_space_to_depth(const vae_tensor_t& x, int32_t st, int32_t sh, int32_t sw,
                                   const vae_tensor_t& y, hipStream_t stream);

// ---- tiles ----
// A tile's overlaps with its neighbours along T, H and W (output samples).
struct MergeRamps {
    int32_t lead_t, trail_t, lead_h, trail_h, lead_w, trail_w;
    MergeRamps() = default;
    explicit MergeRamps(const vae_tile_t& t)
        : lead_t(t.lead_t), trail_t(t.trail_t), lead_h(t.lead_h), trail_h(t.trail_h),
          lead_w(t.lead_w), trail_w(t.trail_w) {}
};
vae_status_t launch_merge(const vae_tensor_t& tile_out, const Box& out_box, const MergeRamps& r,
                          const vae_tensor_t& out, hipStream_t stream);
vae_status_t launch_merge_finalize(const vae_tensor_t& out, const AxisTiling& at,
                                   const AxisTiling& ah, const AxisTiling& aw,
                                   hipStream_t stream);
vae_status_t launch_zero(void* p, int64_t bytes, hipStream_t stream);
// A device-to-device copy of `bytes` (16-byte aligned pointers and size), as a kernel.
vae_status_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);
// Copy x[:, box] (latent grid) into the dense tensor y (shape of the box).
vae_status_t launch_crop(const vae_tensor_t& x, const Box& box, const vae_tensor_t& y,
                         hipStream_t stream);

}  // namespace vae
