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
// The contiguous output segment of row (st*t+dt-(st-1), sh*h+dh) that the box's columns cover,
// for one (input row t,h; sub-row dt,dh) pair, is cut into slices of 512 vectors, one block each.
#include "kernels.h"

namespace vae {
namespace {

constexpr int kThreads = 256;
// Each block copies one slice of kSlice output vectors of a segment, kVecs per thread with all
// loads in flight: many short blocks keep more loads in flight across the chip than one block per
// segment looping over it.
constexpr int kVecs = 2;
constexpr int kSlice = kVecs * kThreads;

template <typename T, int V>
__global__ __launch_bounds__(kThreads) void upsample_kernel(
    const T* __restrict__ x, T* __restrict__ y, int32_t xT, int32_t xH, int32_t xW, int32_t xC,
    int32_t yT, int32_t yH, int32_t yW, int32_t C, int32_t st, int32_t sh, int32_t sw,
    int32_t d2s, Box b, int32_t slices) {
    const int n = blockIdx.z;
    const int64_t row = blockIdx.x / slices;         // input row of the box
    const int part = (int)(blockIdx.x - row * slices);
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
    const int e0 = part * kSlice, e1 = e0 + kSlice < seg ? e0 + kSlice : seg;
    // source of channel vector cv of output column wo (within the segment)
    auto src_at = [&](int cv, int wo) {
        const int wl = wo / sw, dw = wo - wl * sw;
        const int slice = d2s ? (sub * sw + dw) : 0;
        return xr + (int64_t)wl * xC + (int64_t)slice * C + cv * V;
    };
    auto src_of = [&](int e) { return src_at(e % CV, e / CV); };
    if constexpr (V * sizeof(T) == 16) {
        // When CV divides the block (every decoder width), a thread keeps one channel vector and
        // its columns step by kThreads / CV: no division by CV per vector.
        const bool fixed = kThreads % CV == 0;
        const int cv_t = fixed ? (int)threadIdx.x % CV : 0;
        const int wo_t = fixed ? (e0 + (int)threadIdx.x) / CV : 0;
        const int wstep = fixed ? kThreads / CV : 0;
        uint4 v[kVecs];
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            const int e = e0 + (int)threadIdx.x + u * kThreads;
            if (e < e1)
                v[u] = *reinterpret_cast<const uint4*>(fixed ? src_at(cv_t, wo_t + u * wstep)
                                                              : src_of(e));
        }
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            const int e = e0 + (int)threadIdx.x + u * kThreads;
            if (e < e1) *reinterpret_cast<uint4*>(yr + (int64_t)e * V) = v[u];
        }
    } else {
        for (int e = e0 + (int)threadIdx.x; e < e1; e += kThreads) {
            const T* src = src_of(e);
            T* dst = yr + (int64_t)e * V;
#pragma unroll
            for (int k = 0; k < V; ++k) dst[k] = src[k];
        }
    }
}

template <typename T>
vae_status_t run(const vae_tensor_t& x, const Box& b, int32_t mode, int32_t st, int32_t sh,
                 int32_t sw, const vae_tensor_t& y, hipStream_t stream) {
    constexpr int V16 = 16 / sizeof(T);
    const int64_t vec = y.c % V16 == 0 ? V16 : 1;            // elements per vector
    const int64_t seg = b.bw() * sw * (y.c / vec);           // output vectors per segment
    const int32_t slices = (int32_t)ceil_div(seg, (int64_t)kSlice);
    if (b.bt() * b.bh() * slices > INT32_MAX || st * sh > 65535 || x.n > 65535)
        return fail(VAE_ERR_UNSUPPORTED, "upsample: grid too large");
    dim3 grid((unsigned)(b.bt() * b.bh() * slices), (unsigned)(st * sh), (unsigned)x.n);
    const int32_t d2s = mode == VAE_UPSAMPLE_D2S;
    if (vec == V16)
        hipLaunchKernelGGL((upsample_kernel<T, V16>), grid, dim3(kThreads), 0, stream,
                           static_cast<const T*>(x.data), static_cast<T*>(y.data), (int32_t)x.t,
                           (int32_t)x.h, (int32_t)x.w, (int32_t)x.c, (int32_t)y.t, (int32_t)y.h,
                           (int32_t)y.w, (int32_t)y.c, st, sh, sw, d2s, b, slices);
    else
        hipLaunchKernelGGL((upsample_kernel<T, 1>), grid, dim3(kThreads), 0, stream,
                           static_cast<const T*>(x.data), static_cast<T*>(y.data), (int32_t)x.t,
                           (int32_t)x.h, (int32_t)x.w, (int32_t)x.c, (int32_t)y.t, (int32_t)y.h,
                           (int32_t)y.w, (int32_t)y.c, st, sh, sw, d2s, b, slices);
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
