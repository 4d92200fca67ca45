// Causal Conv3d (3x3x3, stride 1) on channels-last (NDHWC) activations: dispatch, weight packing
// and the direct path.
//  - bf16 weights with Cin % 32 == 0 and Cout % 4 == 0 run on the matrix cores (conv3d_mfma.h);
//    fp16 inputs only run there.
//  - Otherwise a direct kernel computes one output per thread with fp32 accumulation.
#include <algorithm>
#include <mutex>

#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
// instantiated in conv3d_mfma_*.hip
#define VAE_MFMA_EXTERN(NT, TI, SPLIT)                                                         \
    extern template vae_status_t run_mfma_out<NT, TI, SPLIT>(                                 \
        const vae_tensor_t&, const void*, const float*, const vae_tensor_t*, const vae_tensor_t&, \
        const Box&, bool, const ConvFuse*, hipStream_t);
VAE_MFMA_EXTERN(128, uint16_t, false)
VAE_MFMA_EXTERN(128, float, false)
VAE_MFMA_EXTERN(128, float, true)
VAE_MFMA_EXTERN(64, uint16_t, false)
VAE_MFMA_EXTERN(64, float, false)
VAE_MFMA_EXTERN(64, float, true)
VAE_MFMA_EXTERN(128, _Float16, false)
VAE_MFMA_EXTERN(64, _Float16, false)
VAE_MFMA_EXTERN(32, uint16_t, false)
VAE_MFMA_EXTERN(32, float, false)
VAE_MFMA_EXTERN(32, float, true)
VAE_MFMA_EXTERN(32, _Float16, false)
VAE_MFMA_EXTERN(128, GnF32, false)
VAE_MFMA_EXTERN(64, GnF32, false)
VAE_MFMA_EXTERN(32, GnF32, false)
VAE_MFMA_EXTERN(128, GnF16, false)
VAE_MFMA_EXTERN(64, GnF16, false)
VAE_MFMA_EXTERN(32, GnF16, false)
VAE_MFMA_EXTERN(128, GnF32H, false)
VAE_MFMA_EXTERN(64, GnF32H, false)
VAE_MFMA_EXTERN(32, GnF32H, false)
#undef VAE_MFMA_EXTERN
}  // namespace mfma

namespace {
using namespace mfma;
// ------------------------------------------------------------------------------------------------
// Direct path: one thread per (output position, output channel).
// ------------------------------------------------------------------------------------------------
template <typename TX, typename TW, typename TO>
__global__ __launch_bounds__(256) void conv3d_direct_kernel(
    const TX* __restrict__ x, const TW* __restrict__ w, const float* __restrict__ bias,
    const TO* res, TO* y, int32_t N, int32_t T, int32_t H, int32_t W, int32_t cin, int32_t cout,
    Box box) {
    const int64_t total = (int64_t)N * box.volume() * cout;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int co = (int)(idx % cout);
    int64_t p = idx / cout;
    const int wl = (int)(p % box.bw());
    p /= box.bw();
    const int hl = (int)(p % box.bh());
    p /= box.bh();
    const int tl = (int)(p % box.bt());
    const int n = (int)(p / box.bt());
    const int t = box.t0 + tl, h = box.h0 + hl, ww = box.w0 + wl;
    float acc = bias ? bias[co] : 0.0f;
    const TX* xn = x + (int64_t)n * T * H * W * cin;
    for (int kt = 0; kt < 3; ++kt) {
        int ti = t + kt - 2;
        ti = ti < 0 ? 0 : ti;
        for (int kh = 0; kh < 3; ++kh) {
            int hi = h + kh - 1;
            if (hi < 0 || hi >= H) continue;
            for (int kw = 0; kw < 3; ++kw) {
                int wi = ww + kw - 1;
                if (wi < 0 || wi >= W) continue;
                const TX* xp = xn + ((int64_t)(ti * H + hi) * W + wi) * cin;
                const TW* wp = w + ((int64_t)co * 27 + (kt * 9 + kh * 3 + kw)) * cin;
                for (int c = 0; c < cin; ++c) acc += Elem<TX>::load(xp + c) * Elem<TW>::load(wp + c);
            }
        }
    }
    const int64_t o = ((((int64_t)n * T + t) * H + h) * W + ww) * cout + co;
    if (res) acc += Elem<TO>::load(res + o);
    Elem<TO>::store(y + o, acc);
}

// Output-block shapes (T x H x W = 256 positions; pick_block in conv3d_mfma.h). The launch picks
// the one that wastes the fewest MFMA rows on ragged block edges for the box: 16x22x40 takes
// 4x8x8 (9% waste instead of 31%), 31x44x80 takes 4x4x16, the larger stages take 2x8x16, and one
// width quarter of the first stages (10 or 20 columns) takes a narrow shape.
template <int NT>
vae_status_t run_mfma_in(const vae_tensor_t& x, const void* w, const float* bias,
                         const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                         bool split, bool packed, bool f16w, const ConvFuse* fz,
                         hipStream_t stream) {
    if (fz && fz->in_ab) {   // GroupNorm + SiLU while staging: bf16 or fp16 operands
        if (x.dtype == VAE_DTYPE_F32 && f16w)
            return run_mfma_out<NT, GnF32H, false>(x, w, bias, residual, y, box, packed, fz,
                                                   stream);
        if (x.dtype == VAE_DTYPE_F32)
            return run_mfma_out<NT, GnF32, false>(x, w, bias, residual, y, box, packed, fz,
                                                  stream);
        return run_mfma_out<NT, GnF16, false>(x, w, bias, residual, y, box, packed, fz, stream);
    }
    if (x.dtype == VAE_DTYPE_BF16)
        return run_mfma_out<NT, uint16_t, false>(x, w, bias, residual, y, box, packed, fz,
                                                 stream);
    if (x.dtype == VAE_DTYPE_F16)
        return run_mfma_out<NT, _Float16, false>(x, w, bias, residual, y, box, packed, fz,
                                                 stream);
    if (split)
        return run_mfma_out<NT, float, true>(x, w, bias, residual, y, box, packed, fz, stream);
    return run_mfma_out<NT, float, false>(x, w, bias, residual, y, box, packed, fz, stream);
}

// Fragment-packed weights: [Cout/32][27 taps][Cin/32 chunks][kk 2][32 co][khalf 2][8 ci] bf16,
// Cout padded to a multiple of 32 with zeros. One 32 (co) x 32 (ci) block per (tap, chunk) is
// 2 KB, ordered so that the 16-byte B fragment of lane l (column l % 32, k half l / 32) for
// k step kk sits at byte kk * 1024 + (l % 32) * 32 + (l / 32) * 16: one contiguous 1 KB read per
// fragment. With to_f16 each weight is stored as fp16(w * 2^10) instead (exact for |w| < 64).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ w,
                                                           uint16_t* __restrict__ p, int32_t cout,
                                                           int32_t cin, int64_t total,
                                                           int32_t to_f16, uint32_t* status) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int nch = cin / kCK;
    int64_t q = i;
    const int e = (int)(q % 8);
    q /= 8;
    const int khalf = (int)(q % 2);
    q /= 2;
    const int r = (int)(q % 32);
    q /= 32;
    const int kk = (int)(q % 2);
    q /= 2;
    const int chunk = (int)(q % nch);
    q /= nch;
    const int tap = (int)(q % 27);
    const int cot = (int)(q / 27);
    const int co = cot * 32 + r;
    const int ci = chunk * kCK + kk * 16 + khalf * 8 + e;
    const uint16_t b = co < cout ? w[((int64_t)co * 27 + tap) * cin + ci] : (uint16_t)0;
    if (to_f16) {
        // |w| * 2^10 must stay within fp16's 65504 (|w| < 64), and w must be finite
        const float sw = bf16_to_f32(b) * kF16WeightScale;
        if (status && !(fabsf(sw) <= 65504.0f)) *status = 1u;
        p[i] = f16_bits(sw);
    } else {
        p[i] = b;
    }
}

__global__ void clear_word_kernel(uint32_t* word) { *word = 0u; }

// The range flag of the fp16 packing, one per GPU (held until the process ends). In host code
// `pack_range_flag` stands for the variable, not its device address: kernels get the address
// hipGetSymbolAddress returns on that device.
__device__ __align__(16) uint32_t pack_range_flag[4];
constexpr int kMaxDevices = 64;
std::mutex pack_flag_mutex;                  // also serialises the checked packs of a process
uint32_t* pack_flag_ptr[kMaxDevices];

template <typename TX, typename TW, typename TO>
vae_status_t run_direct(const vae_tensor_t& x, const void* w, const float* bias,
                        const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                        hipStream_t stream) {
    int64_t total = x.n * box.volume() * y.c;
    int64_t blocks = ceil_div(total, 256);
    if (blocks > INT32_MAX) return fail(VAE_ERR_UNSUPPORTED, "conv3d: grid too large");
    hipLaunchKernelGGL((conv3d_direct_kernel<TX, TW, TO>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, static_cast<const TX*>(x.data), static_cast<const TW*>(w), bias,
                       residual ? static_cast<const TO*>(residual->data) : nullptr,
                       static_cast<TO*>(y.data), (int32_t)x.n, (int32_t)x.t, (int32_t)x.h,
                       (int32_t)x.w, (int32_t)x.c, (int32_t)y.c, box);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

template <typename TX, typename TW>
vae_status_t run_direct_out(const vae_tensor_t& x, const void* w, const float* bias,
                            const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                            hipStream_t stream) {
    if (y.dtype == VAE_DTYPE_F32)
        return run_direct<TX, TW, float>(x, w, bias, residual, y, box, stream);
    return run_direct<TX, TW, uint16_t>(x, w, bias, residual, y, box, stream);
}

}  // namespace

// Convs that run on the matrix cores: bf16 weights, Cin % 32 == 0, Cout % 4 == 0.
bool conv_uses_mfma_c(const vae_tensor_t& x, int64_t cout, int32_t weight_dtype) {
    return weight_dtype == VAE_DTYPE_BF16 && x.c % kCK == 0 && cout % 4 == 0;
}

// Output-channel tile of one launch: conv_nt's width, but with `fill` (a launch allowed to split
// over K to fill the chip) 64 where 128-wide tiles would give fewer than 256 workgroups, such as
// one patch's share of the first stages: twice the workgroups before any split over K, so half the
// split and half its partial sums. Measured on the 1x4 split's interior patch: its S0 convs 0.48
// -> 0.455 ms, conv_in 0.082 -> 0.069 ms.
static int launch_nt(int64_t n, int64_t cout, const Box& box, bool fill) {
    const int nt = conv_nt(cout);
    return fill && nt == 128 && conv_workgroups(n, cout, box) < 256 ? 64 : nt;
}

static int64_t launch_workgroups(int64_t n, int64_t cout, const Box& box, bool fill) {
    return conv_workgroups(n, cout, box) / ceil_div(cout, conv_nt(cout)) *
           ceil_div(cout, launch_nt(n, cout, box, fill));
}

int64_t conv_gn_slots(const vae_tensor_t& x, int64_t yc, int32_t weight_dtype, const Box& box,
                      int32_t groups, int32_t k, bool fill) {
    const int64_t cout = yc * k;
    if (!conv_uses_mfma_c(x, cout, weight_dtype) || groups < 1 || yc % groups) return 0;
    if (k > 1 && yc % 32) return 0;      // a wave's 32 channels share one sub-position
    const int64_t cpg = yc / groups;
    if (cpg % 4 || 32 % cpg) return 0;   // a lane's four channels, a wave's 32, hold whole groups
    const BlockDims& d = kBlockDims[pick_block(box)];
    const int nt = launch_nt(x.n, cout, box, fill);
    const int wm = nt == 128 ? wave_rows<128>() : nt == 64 ? wave_rows<64>() : wave_rows<32>();
    return k * ceil_div(box.bt(), d.tb) * ceil_div(box.bh(), d.hb) * ceil_div(box.bw(), d.wb) * wm;
}

// A launch of fewer than 512 workgroups leaves CUs idle or alone (256 CUs, two workgroups each
// when busy). Splitting K s ways multiplies the workgroups by s: s is the largest count (up to 4)
// that keeps the launch within one round of 512 workgroups, with at least two channel chunks per
// split.
int32_t conv_split_count(const vae_tensor_t& x, int64_t cout, int32_t weight_dtype, const Box& box,
                         bool split_fp32) {
    if (!conv_uses_mfma_c(x, cout, weight_dtype) || box.volume() == 0 || x.n == 0) return 1;
    const int64_t wgs = launch_workgroups(x.n, cout, box, true);
    const int64_t chunks = x.c / ((split_fp32 && x.dtype == VAE_DTYPE_F32) ? 16 : kCK);
    if (wgs >= 512) return 1;
    int64_t s = std::min<int64_t>({512 / wgs, chunks / 2, 4});
    return s >= 2 ? (int32_t)s : 1;
}

size_t conv_split_bytes(const vae_tensor_t& x, int64_t cout, const Box& box, int32_t splits) {
    if (splits <= 1) return 0;
    // one fp32 accumulator per (position of a 256-position block, channel of the tile)
    return (size_t)splits * (size_t)launch_workgroups(x.n, cout, box, true) * 256 *
           (size_t)launch_nt(x.n, cout, box, true) * sizeof(float);
}

int64_t packed_weight_elems(int64_t cout, int64_t cin) {
    return ceil_div(cout, 32) * 32 * 27 * cin;
}

vae_status_t launch_pack_weights(const void* w, int32_t cout, int32_t cin, void* packed,
                                 hipStream_t stream, bool to_f16) {
    const int64_t total = packed_weight_elems(cout, cin);
    if (!to_f16) {
        hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                           stream, static_cast<const uint16_t*>(w), static_cast<uint16_t*>(packed),
                           cout, cin, total, 0, (uint32_t*)nullptr);
        VAE_HIP_CHECK(hipGetLastError());
        return VAE_OK;
    }
    // fp16 packing checks the range: clear this device's flag, pack, read the flag back
    int dev = -1;
    VAE_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(VAE_ERR_UNSUPPORTED, "device index beyond the library's table");
    std::lock_guard<std::mutex> lock(pack_flag_mutex);
    if (!pack_flag_ptr[dev]) {
        void* p = nullptr;
        VAE_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(pack_range_flag)));
        if (!p) return fail(VAE_ERR_HIP, "hipGetSymbolAddress returned NULL for the range flag");
        pack_flag_ptr[dev] = static_cast<uint32_t*>(p);
    }
    uint32_t* flag = pack_flag_ptr[dev];
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, flag);
    VAE_HIP_CHECK(hipGetLastError());
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(w), static_cast<uint16_t*>(packed),
                       cout, cin, total, 1, flag);
    VAE_HIP_CHECK(hipGetLastError());
    uint32_t h = 0;
    VAE_HIP_CHECK(hipStreamSynchronize(stream));
    VAE_HIP_CHECK(hipMemcpy(&h, flag, sizeof(h), hipMemcpyDeviceToHost));
    if (h)
        return fail(VAE_ERR_UNSUPPORTED,
                    "fp16 weights: a weight of magnitude 64 or more (or not finite) overflows "
                    "fp16 at the 2^10 scale; use bf16 operands for this conv");
    return VAE_OK;
}

bool conv_uses_mfma(const vae_tensor_t& x, const vae_tensor_t& y, int32_t weight_dtype) {
    return conv_uses_mfma_c(x, y.c, weight_dtype);
}

vae_status_t launch_conv3d(const vae_tensor_t& x, const void* w, int32_t weight_dtype,
                           const float* bias, const vae_tensor_t* residual, const vae_tensor_t& y,
                           const Box& box, int32_t flags, hipStream_t stream, const ConvFuse* fz) {
    if (box.volume() == 0 || x.n == 0) return VAE_OK;
    const bool xf = x.dtype == VAE_DTYPE_F32;
    const bool split = (flags & VAE_CONV_SPLIT_FP32) != 0;
    const bool packed = (flags & (VAE_CONV_PACKED_WEIGHTS | VAE_CONV_PACKED_F16_WEIGHTS)) != 0;
    const bool f16w = (flags & VAE_CONV_PACKED_F16_WEIGHTS) != 0;
    const bool x16 = x.dtype == VAE_DTYPE_F16;
    const bool norm = fz && fz->in_ab;
    const int32_t k = fz ? fz->st * fz->sh * fz->sw : 1;
    const int64_t cout = y.c * k;
    if (norm) {
        // a normalised input: fp32 (bf16 or fp16 operands) or fp16 (bf16 operands), packed
        // weights, no split
        if (!packed || split || !conv_uses_mfma_c(x, cout, weight_dtype))
            return fail(VAE_ERR_UNSUPPORTED, "conv3d: an input GroupNorm needs the MFMA path with "
                                             "packed weights and no fp32 split");
        if (!xf && !(x16 && (flags & VAE_CONV_PACKED_WEIGHTS)))
            return fail(VAE_ERR_UNSUPPORTED, "conv3d: an input GroupNorm reads fp32, or fp16 "
                                             "with bf16-packed weights");
        if (reinterpret_cast<uintptr_t>(fz->in_ab) % 16)
            return fail(VAE_ERR_INVALID_ARG, "conv3d: the scale and shift must be 16-byte aligned");
    } else {
        if ((flags & VAE_CONV_PACKED_F16_WEIGHTS) && !x16)
            return fail(VAE_ERR_INVALID_ARG, "fp16-packed weights go with an fp16 input");
        if ((flags & VAE_CONV_PACKED_WEIGHTS) && x16)
            return fail(VAE_ERR_INVALID_ARG, "an fp16 input takes fp16-packed weights");
    }
    if (fz && (fz->lsh || fz->lsw) && !conv_uses_mfma_c(x, cout, weight_dtype))
        return fail(VAE_ERR_UNSUPPORTED, "conv3d: a folded nearest upsampling needs the MFMA path");
    if ((x16 || y.dtype == VAE_DTYPE_F16) && !conv_uses_mfma_c(x, cout, weight_dtype))
        return fail(VAE_ERR_UNSUPPORTED, "conv3d: fp16 tensors need the MFMA path");
    if (fz && k > 1 && !conv_uses_mfma_c(x, cout, weight_dtype))
        return fail(VAE_ERR_UNSUPPORTED, "conv3d: a fused depth-to-space needs the MFMA path");
    if (fz && fz->gn_ws && conv_gn_slots(x, y.c, weight_dtype, box, fz->groups, k, false) == 0)
        return fail(VAE_ERR_UNSUPPORTED, "conv3d: fused GroupNorm statistics need the MFMA path "
                                         "and 4, 8, 16 or 32 channels per group");
    if (fz && fz->part && fz->splits > 1 && !conv_uses_mfma_c(x, cout, weight_dtype))
        return fail(VAE_ERR_UNSUPPORTED, "conv3d: a split over K needs the MFMA path");
    if (conv_uses_mfma_c(x, cout, weight_dtype)) {
        // output-channel tile: 128 wide, or 64 / 32 for narrow outputs (conv_out's 48 or 12) and
        // for launches too small to fill the chip with 128-wide tiles
        switch (launch_nt(x.n, cout, box, (flags & VAE_CONV_SPLIT_K) != 0)) {
            case 128:
                return run_mfma_in<128>(x, w, bias, residual, y, box, split, packed, f16w, fz,
                                        stream);
            case 64:
                return run_mfma_in<64>(x, w, bias, residual, y, box, split, packed, f16w, fz,
                                       stream);
            default:
                return run_mfma_in<32>(x, w, bias, residual, y, box, split, packed, f16w, fz,
                                       stream);
        }
    }
    if (packed) return fail(VAE_ERR_UNSUPPORTED, "packed weights need the MFMA path");
    if (weight_dtype == VAE_DTYPE_F32)
        return xf ? run_direct_out<float, float>(x, w, bias, residual, y, box, stream)
                  : run_direct_out<uint16_t, float>(x, w, bias, residual, y, box, stream);
    return xf ? run_direct_out<float, uint16_t>(x, w, bias, residual, y, box, stream)
              : run_direct_out<uint16_t, uint16_t>(x, w, bias, residual, y, box, stream);
}

}  // namespace vae
