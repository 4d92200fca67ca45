// Overlap-blend merge of decoded tiles, and small helpers (zero fill, latent crop).
//
// The serial tiled decode blends each tile into a full-size buffer with a mask assembled from
// per-axis parts, keeps the summed weights, and divides at the end ("[TRTLLM-14029][feat] LTX-2
// tile-parallel VAE decode", Approach). Building that mask on the host and copying it over per
// tile left the GPU about half idle, so here the mask is never materialised:
//  - each kernel evaluates the separable ramps from the tile's overlaps while it streams;
//  - the final divide evaluates the per-axis weight sums from the tile grid itself.
// All passes go over contiguous rows (fixed n, t, h) of fp32 NDHWC data.
#include <algorithm>

#include "kernels.h"

namespace vae {
namespace {

constexpr int kThreads = 256;

// Weight of tile row (tl, hl): ramp_t(tl) * ramp_h(hl).
__device__ inline float row_weight(const MergeRamps& m, const Box& b, int tl, int hl) {
    return ramp_weight(tl, (int)b.bt(), m.lead_t, m.trail_t) *
           ramp_weight(hl, (int)b.bh(), m.lead_h, m.trail_h);
}

// grid (tile rows bt*bh, N). out[box] += w * tile; w = ramp_t(t) * ramp_h(h) * ramp_w(w).
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ tile,
                                                         float* __restrict__ out, int32_t oT,
                                                         int32_t oH, int32_t oW, int32_t C, Box b,
                                                         MergeRamps m) {
    const int n = blockIdx.y;
    const int64_t r = blockIdx.x;
    const int tl = (int)(r / b.bh()), hl = (int)(r % b.bh());
    const float wh = row_weight(m, b, tl, hl);
    const float* src = tile + (((int64_t)n * b.bt() + tl) * b.bh() + hl) * b.bw() * C;
    float* dst = out + ((((int64_t)n * oT + b.t0 + tl) * oH + b.h0 + hl) * oW + b.w0) * C;
    const int seg = (int)b.bw() * C;
    for (int e = threadIdx.x; e < seg; e += kThreads) {
        const int wl = e / C;
        dst[e] += wh * ramp_weight(wl, (int)b.bw(), m.lead_w, m.trail_w) * src[e];
    }
}

// grid (rows oT*oH, N). out /= S_t(t) * S_h(h) * S_w(w).
__global__ __launch_bounds__(kThreads) void merge_finalize_kernel(float* __restrict__ out,
                                                                  int32_t oT, int32_t oH,
                                                                  int32_t oW, int32_t C,
                                                                  AxisTiling at, AxisTiling ah,
                                                                  AxisTiling aw) {
    const int n = blockIdx.y;
    const int64_t r = blockIdx.x;
    const float sh = axis_weight_sum(at, (int)(r / oH)) * axis_weight_sum(ah, (int)(r % oH));
    float* row = out + ((int64_t)n * oT * oH + r) * oW * C;
    const int seg = oW * C;
    for (int e = threadIdx.x; e < seg; e += kThreads) {
        const float s = sh * axis_weight_sum(aw, e / C);
        row[e] /= s;
    }
}

// The same two passes, each block streaming several rows. The per-column factor (the W ramp of
// the tile, or the W weight sum of the output) is evaluated once per block into LDS instead of
// once per element. With VEC, rows are read and written as float4: every row starts on a
// 16-byte boundary, and element 4e + k lies in column (4e + k) / C. The arithmetic per element
// is that of the kernels above.
// One block per row, up to the grid limit: many short blocks keep more loads in flight across the
// chip than a few that loop over rows (the column table costs each block a few ramp evaluations
// per thread, no memory traffic).
// The tile, read once, and the finalize's one read and write of each output element carry the
// nontemporal hint (merge + finalize of a 720p decode: 1.52-1.53 -> 1.43-1.44 ms). The merge's
// read-modify-write of the output stays cached: overlapping tiles come back to the same rows,
// and the hint there measured slower (1.46-1.48 ms).
constexpr int64_t kRowBlocks = INT32_MAX;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 nt_load4(const float4* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void nt_store4(float4* p, float4 v) {
    const f32x4_t u = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(u, reinterpret_cast<f32x4_t*>(p));
}
constexpr int kMaxLdsColumns = 8192;       // per-column factors kept in LDS (32 KB)

template <bool VEC>
__global__ __launch_bounds__(kThreads) void merge_rows_kernel(const float* __restrict__ tile,
                                                              float* __restrict__ out, int32_t oT,
                                                              int32_t oH, int32_t oW, int32_t C,
                                                              Box b, MergeRamps m) {
    extern __shared__ float col[];          // ramp_w of each tile column
    const int bw = (int)b.bw(), bh = (int)b.bh();
    for (int i = threadIdx.x; i < bw; i += kThreads) col[i] = ramp_weight(i, bw, m.lead_w, m.trail_w);
    __syncthreads();
    const int n = blockIdx.y;
    const int64_t rows = b.bt() * bh;
    const int seg = bw * C;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int tl = (int)(r / bh), hl = (int)(r % bh);
        const float wh = row_weight(m, b, tl, hl);
        const float* src = tile + (((int64_t)n * b.bt() + tl) * bh + hl) * (int64_t)seg;
        float* dst = out + ((((int64_t)n * oT + b.t0 + tl) * oH + b.h0 + hl) * oW + b.w0) * C;
        if constexpr (VEC) {
            const float4* s4 = reinterpret_cast<const float4*>(src);
            float4* d4 = reinterpret_cast<float4*>(dst);
            for (int e4 = threadIdx.x; e4 < seg / 4; e4 += kThreads) {
                int wl = (4 * e4) / C, rem = 4 * e4 - wl * C;
                const float4 sv = nt_load4(s4 + e4);
                float4 dv = d4[e4];
                float* dp = &dv.x;
                const float* sp = &sv.x;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    dp[k] += wh * col[wl] * sp[k];
                    if (++rem == C) {
                        rem = 0;
                        ++wl;
                    }
                }
                d4[e4] = dv;
            }
        } else {
            for (int e = threadIdx.x; e < seg; e += kThreads) dst[e] += wh * col[e / C] * src[e];
        }
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void merge_finalize_rows_kernel(float* __restrict__ out,
                                                                       int32_t oT, int32_t oH,
                                                                       int32_t oW, int32_t C,
                                                                       AxisTiling at,
                                                                       AxisTiling ah,
                                                                       AxisTiling aw) {
    extern __shared__ float col[];          // S_w of each output column
    for (int i = threadIdx.x; i < oW; i += kThreads) col[i] = axis_weight_sum(aw, i);
    __syncthreads();
    const int n = blockIdx.y;
    const int64_t rows = (int64_t)oT * oH;
    const int seg = oW * C;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float sh = axis_weight_sum(at, (int)(r / oH)) * axis_weight_sum(ah, (int)(r % oH));
        float* row = out + ((int64_t)n * rows + r) * seg;
        if constexpr (VEC) {
            float4* r4 = reinterpret_cast<float4*>(row);
            for (int e4 = threadIdx.x; e4 < seg / 4; e4 += kThreads) {
                int wl = (4 * e4) / C, rem = 4 * e4 - wl * C;
                float4 v = nt_load4(r4 + e4);
                float* vp = &v.x;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    vp[k] /= sh * col[wl];
                    if (++rem == C) {
                        rem = 0;
                        ++wl;
                    }
                }
                nt_store4(r4 + e4, v);
            }
        } else {
            for (int e = threadIdx.x; e < seg; e += kThreads) row[e] /= sh * col[e / C];
        }
    }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(uint4* p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kThreads)
        p[i] = make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(64) void zero_tail_kernel(uint8_t* p, int64_t n) {
    if ((int64_t)threadIdx.x < n) p[threadIdx.x] = 0;
}

// dst[i] = src[i] for n 16-byte words; the ranges must not overlap.
__global__ __launch_bounds__(kThreads) void copy_kernel(uint4* __restrict__ dst,
                                                        const uint4* __restrict__ src, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kThreads)
        dst[i] = src[i];
}

// grid (box rows, N): copy one contiguous row segment of bytes.
__global__ __launch_bounds__(kThreads) void crop_kernel(const uint8_t* __restrict__ x,
                                                        uint8_t* __restrict__ y, int32_t T,
                                                        int32_t H, int32_t W, int64_t pos_bytes,
                                                        Box b) {
    const int n = blockIdx.y;
    const int64_t r = blockIdx.x;
    const int tl = (int)(r / b.bh()), hl = (int)(r % b.bh());
    const uint8_t* src =
        x + ((((int64_t)n * T + b.t0 + tl) * H + b.h0 + hl) * W + b.w0) * pos_bytes;
    uint8_t* dst = y + (((int64_t)n * b.bt() + tl) * b.bh() + hl) * b.bw() * pos_bytes;
    const int64_t seg = b.bw() * pos_bytes;
    if (seg % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0) {
        for (int64_t e = threadIdx.x; e < seg / 16; e += kThreads)
            reinterpret_cast<uint4*>(dst)[e] = reinterpret_cast<const uint4*>(src)[e];
    } else {
        for (int64_t e = threadIdx.x; e < seg; e += kThreads) dst[e] = src[e];
    }
}

}  // namespace

vae_status_t launch_merge(const vae_tensor_t& tile_out, const Box& b, const MergeRamps& m,
                          const vae_tensor_t& out, hipStream_t stream) {
    if (b.volume() == 0 || out.n == 0) return VAE_OK;
    const float* tp = static_cast<const float*>(tile_out.data);
    float* op = static_cast<float*>(out.data);
    if (b.bw() <= kMaxLdsColumns) {
        const int64_t rows = b.bt() * b.bh();
        const dim3 grid((unsigned)std::min<int64_t>(rows, kRowBlocks), (unsigned)out.n);
        const size_t lds = (size_t)b.bw() * sizeof(float);
        const bool vec = (b.bw() * out.c) % 4 == 0 && (b.w0 * out.c) % 4 == 0 &&
                         (out.w * out.c) % 4 == 0 && (uintptr_t)tp % 16 == 0 &&
                         (uintptr_t)op % 16 == 0;
        if (vec)
            hipLaunchKernelGGL(merge_rows_kernel<true>, grid, dim3(kThreads), lds, stream, tp, op,
                               (int32_t)out.t, (int32_t)out.h, (int32_t)out.w, (int32_t)out.c, b,
                               m);
        else
            hipLaunchKernelGGL(merge_rows_kernel<false>, grid, dim3(kThreads), lds, stream, tp, op,
                               (int32_t)out.t, (int32_t)out.h, (int32_t)out.w, (int32_t)out.c, b,
                               m);
        VAE_HIP_CHECK(hipGetLastError());
        return VAE_OK;
    }
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(b.bt() * b.bh()), (unsigned)out.n),
                       dim3(kThreads), 0, stream, static_cast<const float*>(tile_out.data),
                       static_cast<float*>(out.data), (int32_t)out.t, (int32_t)out.h,
                       (int32_t)out.w, (int32_t)out.c, b, m);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

vae_status_t launch_merge_finalize(const vae_tensor_t& out, const AxisTiling& at,
                                   const AxisTiling& ah, const AxisTiling& aw,
                                   hipStream_t stream) {
    if (numel(out) == 0) return VAE_OK;
    float* op = static_cast<float*>(out.data);
    if (out.w <= kMaxLdsColumns) {
        const int64_t rows = out.t * out.h;
        const dim3 grid((unsigned)std::min<int64_t>(rows, kRowBlocks), (unsigned)out.n);
        const size_t lds = (size_t)out.w * sizeof(float);
        if ((out.w * out.c) % 4 == 0 && (uintptr_t)op % 16 == 0)
            hipLaunchKernelGGL(merge_finalize_rows_kernel<true>, grid, dim3(kThreads), lds, stream,
                               op, (int32_t)out.t, (int32_t)out.h, (int32_t)out.w, (int32_t)out.c,
                               at, ah, aw);
        else
            hipLaunchKernelGGL(merge_finalize_rows_kernel<false>, grid, dim3(kThreads), lds,
                               stream, op, (int32_t)out.t, (int32_t)out.h, (int32_t)out.w,
                               (int32_t)out.c, at, ah, aw);
        VAE_HIP_CHECK(hipGetLastError());
        return VAE_OK;
    }
    hipLaunchKernelGGL(merge_finalize_kernel, dim3((unsigned)(out.t * out.h), (unsigned)out.n),
                       dim3(kThreads), 0, stream, static_cast<float*>(out.data), (int32_t)out.t,
                       (int32_t)out.h, (int32_t)out.w, (int32_t)out.c, at, ah, aw);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

vae_status_t launch_zero(void* p, int64_t bytes, hipStream_t stream) {
    if (bytes <= 0) return VAE_OK;
    if ((uintptr_t)p % 16 != 0) return fail(VAE_ERR_INVALID_ARG, "zero: pointer not 16-byte aligned");
    const int64_t n16 = bytes / 16;
    if (n16 > 0) {
        int64_t blocks = ceil_div(n16, kThreads);
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           static_cast<uint4*>(p), n16);
        VAE_HIP_CHECK(hipGetLastError());
    }
    if (bytes % 16) {
        hipLaunchKernelGGL(zero_tail_kernel, dim3(1), dim3(64), 0, stream,
                           static_cast<uint8_t*>(p) + n16 * 16, bytes % 16);
        VAE_HIP_CHECK(hipGetLastError());
    }
    return VAE_OK;
}

vae_status_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
    if (bytes <= 0) return VAE_OK;
    if ((uintptr_t)dst % 16 || (uintptr_t)src % 16 || bytes % 16)
        return fail(VAE_ERR_INVALID_ARG, "copy: pointers and size must be 16-byte multiples");
    const int64_t n16 = bytes / 16;
    const int64_t blocks = std::min<int64_t>(ceil_div(n16, kThreads), 65536);
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

vae_status_t launch_crop(const vae_tensor_t& x, const Box& b, const vae_tensor_t& y,
                         hipStream_t stream) {
    if (b.volume() == 0 || x.n == 0) return VAE_OK;
    hipLaunchKernelGGL(crop_kernel, dim3((unsigned)(b.bt() * b.bh()), (unsigned)x.n),
                       dim3(kThreads), 0, stream, static_cast<const uint8_t*>(x.data),
                       static_cast<uint8_t*>(y.data), (int32_t)x.t, (int32_t)x.h, (int32_t)x.w,
                       x.c * elem_size(x.dtype), b);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

}  // namespace vae
