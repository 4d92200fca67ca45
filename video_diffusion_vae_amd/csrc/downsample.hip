// Space-to-depth downsampling of channels-last activations: the fold of an encoder.
//
// Encoder downsamplers that fold space into channels after a stride-1 convolution read one input
// position per output one ("Add tiled VAE parallelism & extended model support", encoder commit
// messages). The fold mirrors the decoder's depth-to-space: st-1 copies of frame 0 go in front
// (causal), and input (st*t + dt - (st-1), sh*h + dh, sw*w + dw, c) lands in output channel
// ((dt*sh + dh)*sw + dw)*C + c at (t, h, w); input frames below 0 read frame 0.
//
// One block handles one output row (t, h) and walks it in order: thread e writes output vector e
// of the row (V channels of one sub-position) and reads it from input row (st*t + dt - (st-1),
// sh*h + dh). Writes are fully contiguous. A wave's reads cover, for each sub-row, consecutive
// input columns, i.e. whole input lines spread over the wave (with 4 bf16 channels, the patchify
// of a padded video: 16 pieces of 8 bytes per output position, each line read once).
// When a 16-byte vector holds G = 2 whole sub-positions (C = 4 bf16/fp16 or 2 fp32 channels) and G
// divides sw, the sub-positions (dw, dw + 1) of one output vector are neighbouring columns of one
// input row, so the pair moves as one 16-byte vector.
#include "kernels.h"

namespace vae {
namespace {

constexpr int kThreads = 256;

// V elements per vector; G sub-positions per vector (1, or 2 with V = 2 * C)
template <typename T, int V, int G>
__global__ __launch_bounds__(kThreads) void space_to_depth_kernel(
    const T* __restrict__ x, T* __restrict__ y, int32_t xT, int32_t xH, int32_t xW, int32_t C,
    int32_t yT, int32_t yH, int32_t yW, int32_t st, int32_t sh, int32_t sw) {
    const int n = blockIdx.y;
    const int64_t row = blockIdx.x;                  // output row t * yH + h
    const int t = (int)(row / yH), h = (int)(row % yH);
    const int CV = G > 1 ? 1 : C / V;                // vectors per sub-position (group)
    const int kv = st * sh * sw * CV / G;            // vectors per output position
    const int seg = yW * kv;                         // vectors in the output row
    const int64_t xrow = (int64_t)xW * C;
    const T* xn = x + (int64_t)n * xT * xH * xrow;
    T* yr = y + ((int64_t)n * yT + t) * yH * (int64_t)yW * kv * V + (int64_t)h * yW * kv * V;
    for (int e = threadIdx.x; e < seg; e += kThreads) {
        const int wo = e / kv;
        const int j = e - wo * kv;
        const int pg = j / CV, cv = j - pg * CV;
        const int p = pg * G;                        // sub-position ((dt*sh + dh)*sw + dw)
        const int dw = p % sw, dh = (p / sw) % sh, dt = p / (sw * sh);
        int ti = st * t + dt - (st - 1);
        ti = ti < 0 ? 0 : ti;                        // the causal front copies of frame 0
        const T* src = xn + ((int64_t)ti * xH + sh * h + dh) * xrow +
                       (int64_t)(sw * wo + dw) * C + cv * V;
        T* dst = yr + (int64_t)e * V;
        if constexpr (V * sizeof(T) == 16) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else if constexpr (V * sizeof(T) == 8) {
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) dst[k] = src[k];
        }
    }
}

template <typename T, int V, int G = 1>
void launch(const vae_tensor_t& x, int32_t st, int32_t sh, int32_t sw, const vae_tensor_t& y,
            hipStream_t stream) {
    const dim3 grid((unsigned)(y.t * y.h), (unsigned)x.n);
    hipLaunchKernelGGL((space_to_depth_kernel<T, V, G>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(x.data), static_cast<T*>(y.data), (int32_t)x.t,
                       (int32_t)x.h, (int32_t)x.w, (int32_t)x.c, (int32_t)y.t, (int32_t)y.h,
                       (int32_t)y.w, st, sh, sw);
}

template <typename T>
void run(const vae_tensor_t& x, int32_t st, int32_t sh, int32_t sw, const vae_tensor_t& y,
         hipStream_t stream) {
    constexpr int V16 = 16 / sizeof(T), V8 = 8 / sizeof(T);
    if (x.c % V16 == 0) launch<T, V16>(x, st, sh, sw, y, stream);
    else if (2 * x.c == V16 && sw % 2 == 0) launch<T, V16, 2>(x, st, sh, sw, y, stream);
    else if (x.c % V8 == 0) launch<T, V8>(x, st, sh, sw, y, stream);
    else launch<T, 1>(x, st, sh, sw, y, stream);
}

}  // namespace

vae_status_t launch_space_to_depth(const vae_tensor_t& x, int32_t st, int32_t sh, int32_t sw,
                                   const vae_tensor_t& y, hipStream_t stream) {
    if (numel(y) == 0) return VAE_OK;
    // a copy: bf16 and fp16 move as 16-bit words
    if (x.dtype != VAE_DTYPE_F32) run<uint16_t>(x, st, sh, sw, y, stream);
    else run<float>(x, st, sh, sw, y, stream);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

}  // namespace vae
