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
// upsample_kernel (nearest, and depth-to-space with vectors that do not divide C): one block per
// (input row t,h; sub-row dt,dh) pair writes the contiguous output segment of row
// (st*t+dt-(st-1), sh*h+dh) that the box's columns cover. d2s_rows_kernel (depth-to-space with
// 16-byte vectors) goes by input rows instead: contiguous reads, writes in runs of sw*C.
#include "kernels.h"

namespace vae {
namespace {

constexpr int kThreads = 256;
// a 16-byte vector as the nontemporal load and store builtins take it
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// Depth-to-space by input rows: one block per slice of 512 16-byte vectors of an input row
// segment (two per thread, both loads in flight). The reads are contiguous; each vector goes to
// its output position, so the writes come in runs of sw * C elements (one output row segment of
// one sub-row per input position). Every byte is touched once, so loads and stores carry the
// nontemporal hint (S2 -> S3 fp32: 1.27-1.31 -> 1.11-1.13 ms per call; one vector or four per
// thread instead of two measured the same).
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void d2s_rows_kernel(
    const T* __restrict__ x, T* __restrict__ y, int32_t xT, int32_t xH, int32_t xW, int32_t xC,
    int32_t yT, int32_t yH, int32_t yW, int32_t C, int32_t st, int32_t sh, int32_t sw, Box b,
    int32_t slices) {
    constexpr int kVecs = 2;
    const int n = blockIdx.y;
    const int64_t row = blockIdx.x / slices;
    const int part = (int)(blockIdx.x - row * slices);
    const int t = b.t0 + (int)(row / b.bh());
    const int h = b.h0 + (int)(row % b.bh());
    const T* xr = x + ((((int64_t)n * xT + t) * xH + h) * xW + b.w0) * xC;
    const int XV = xC / V, CV = C / V;
    const int seg = (int)b.bw() * XV;                // input vectors in this row segment
    u32x4_t v[kVecs];
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
        const int e = part * kVecs * kThreads + u * kThreads + (int)threadIdx.x;
        if (e < seg)
            v[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(xr + (int64_t)e * V));
    }
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
        const int e = part * kVecs * kThreads + u * kThreads + (int)threadIdx.x;
        if (e >= seg) continue;
        const int wl = e / XV, j = e - wl * XV;      // input column, vector within the position
        const int p = j / CV, cv = j - p * CV;       // sub-position ((dt*sh + dh)*sw + dw)
        const int dw = p % sw, dh = (p / sw) % sh, dt = p / (sw * sh);
        const int to = st * t + dt - (st - 1);
        if (to < 0) continue;                        // causal drop of the first st-1 frames
        const int64_t o = ((((int64_t)n * yT + to) * yH + sh * h + dh) * yW +
                           (int64_t)sw * (b.w0 + wl) + dw) * C + cv * V;
        __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(y + o));
    }
}

template <typename T>
vae_status_t run(const vae_tensor_t& x, const Box& b, int32_t mode, int32_t st, int32_t sh,
                 int32_t sw, const vae_tensor_t& y, hipStream_t stream) {
    constexpr int V16 = 16 / sizeof(T);
    // by input rows when its writes come in runs of at least a 128-byte line (sw * C elements)
    if (mode == VAE_UPSAMPLE_D2S && y.c % V16 == 0 && sw * y.c * (int64_t)sizeof(T) >= 128) {
        const int64_t seg = b.bw() * (x.c / V16);
        const int64_t slices = ceil_div(seg, (int64_t)(2 * kThreads));
        if (b.bt() * b.bh() * slices <= INT32_MAX && x.n <= 65535) {
            const dim3 g2((unsigned)(b.bt() * b.bh() * slices), (unsigned)x.n);
            hipLaunchKernelGGL((d2s_rows_kernel<T, V16>), g2, dim3(kThreads), 0, stream,
                               static_cast<const T*>(x.data), static_cast<T*>(y.data),
                               (int32_t)x.t, (int32_t)x.h, (int32_t)x.w, (int32_t)x.c,
                               (int32_t)y.t, (int32_t)y.h, (int32_t)y.w, (int32_t)y.c, st, sh, sw,
                               b, (int32_t)slices);
            VAE_HIP_CHECK(hipGetLastError());
            return VAE_OK;
        }
    }
    dim3 grid((unsigned)(b.bt() * b.bh()), (unsigned)(st * sh), (unsigned)x.n);
    const int32_t d2s = mode == VAE_UPSAMPLE_D2S;
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
