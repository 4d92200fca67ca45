// Spatial/temporal upsampling of channels-last activations.
//
// Depth-to-space: one input position per output position. The upsampler moves channels into
// space ("Add tiled VAE parallelism & extended model support", LTX-2 decoder adapter commit
// message). Input channel ((dt*sh + dh)*sw + dw)*C + c goes to output channel c at
// (st*t + dt - (st-1), sh*h + dh, sw*w + dw); output frames below 0 are the causal drop. With the
// sub-position slowest, each output row is a contiguous C-channel slice of one input row, so every
// byte is read once and written once with 16-byte accesses.
// Nearest: out(t, sh*h+dh, sw*w+dw) = in(t, h, w).
//
// One block handles one (input row t,h; sub-row dt,dh) pair. It writes the contiguous output
// segment of row (st*t+dt-(st-1), sh*h+dh) that the box's columns cover.
#include "kernels.h"

namespace vae {
namespace {

constexpr int kThreads = 256;

template <typename T, int V>
__global__ __launch_bounds__(kThreads) void upsample_kernel(
    const T* __restrict__ x, T* __restrict__ y, int32_t xT, int32_t xH, int32_t xW, int32_t xC,
    int32_t yT, int32_t yH, int32_t yW, int32_t C, int32_t st, int32_t sh, int32_t sw,
    int32_t d2s, Box b) {
    const int n = blockIdx.z;
    const int64_t row = blockIdx.x;                  // input row of the box
    const int sub = blockIdx.y;                      // dt * sh + dh
    const int t = b.t0 + (int)(row / b.bh());
    const int h = b.h0 + (int)(row % b.bh());
    const int dt = sub / sh, dh = sub % sh;
    const int to = st * t + dt - (st - 1);
    if (to < 0) return;                              // causal drop of the first st-1 frames
    const int ho = sh * h + dh;
    const T* xr = x + ((((int64_t)n * xT + t) * xH + h) * xW + b.w0) * xC;
    T* yr = y + ((((int64_t)n * yT + to) * yH + ho) * yW + (int64_t)b.w0 * sw) * C;
    const int CV = C / V;
    const int seg = (int)b.bw() * sw * CV;           // output vectors in this segment
    for (int e = threadIdx.x; e < seg; e += kThreads) {
        const int cv = e % CV;
        const int wo = e / CV;                       // output column within the segment
        const int wl = wo / sw, dw = wo % sw;
        const int slice = d2s ? (sub * sw + dw) : 0;
        const T* src = xr + (int64_t)wl * xC + (int64_t)slice * C + cv * V;
        T* dst = yr + (int64_t)e * V;
        if (V * sizeof(T) == 16) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) dst[k] = src[k];
        }
    }
}

template <typename T>
vae_status_t run(const vae_tensor_t& x, const Box& b, int32_t mode, int32_t st, int32_t sh,
                 int32_t sw, const vae_tensor_t& y, hipStream_t stream) {
    dim3 grid((unsigned)(b.bt() * b.bh()), (unsigned)(st * sh), (unsigned)x.n);
    const int32_t d2s = mode == VAE_UPSAMPLE_D2S;
    constexpr int V16 = 16 / sizeof(T);
    if (y.c % V16 == 0)
        hipLaunchKernelGGL((upsample_kernel<T, V16>), grid, dim3(kThreads), 0, stream,
                           static_cast<const T*>(x.data), static_cast<T*>(y.data), (int32_t)x.t,
                           (int32_t)x.h, (int32_t)x.w, (int32_t)x.c, (int32_t)y.t, (int32_t)y.h,
                           (int32_t)y.w, (int32_t)y.c, st, sh, sw, d2s, b);
    else
        hipLaunchKernelGGL((upsample_kernel<T, 1>), grid, dim3(kThreads), 0, stream,
                           static_cast<const T*>(x.data), static_cast<T*>(y.data), (int32_t)x.t,
                           (int32_t)x.h, (int32_t)x.w, (int32_t)x.c, (int32_t)y.t, (int32_t)y.h,
                           (int32_t)y.w, (int32_t)y.c, st, sh, sw, d2s, b);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

}  // namespace

vae_status_t launch_upsample(const vae_tensor_t& x, const Box& box, int32_t mode, int32_t st,
                             int32_t sh, int32_t sw, const vae_tensor_t& y, hipStream_t stream) {
    if (box.volume() == 0 || x.n == 0) return VAE_OK;
    // a copy: bf16 and fp16 move as 16-bit words
    if (x.dtype != VAE_DTYPE_F32) return run<uint16_t>(x, box, mode, st, sh, sw, y, stream);
    return run<float>(x, box, mode, st, sh, sw, y, stream);
}

}  // namespace vae
