// RMS normalisation over the channels of each position (+ SiLU): the norm of Wan-style decoders.
//
// y = x / sqrt(mean_c(x^2) + eps) * gamma + beta, then optionally SiLU. The norm reduces over the
// channels of one position only, so a patch-split decode needs no statistics exchange ("Add tiled
// VAE parallelism & extended model support", commit messages on the Qwen-Image / Wan adapters and on
// the HunyuanVideo 1.5 encoder: RMS norms that reduce over channels need nothing sharded).
//
// NDHWC puts a position's C channels in one contiguous run. Each thread owns 8 consecutive
// channels of one position (one 16-byte load for bf16, two for fp32); the C / 8 threads of a
// position sum their squares with lane shuffles, and through LDS when a position spans two waves
// (C = 1024 or 2048). A block of 256 threads covers 256 / (C / 8) positions per step, and each
// thread loads its channels of two steps before reducing any, so that both loads are in flight.
#include <algorithm>

#include "kernels.h"

namespace vae {
namespace {

constexpr int kThreads = 256;
// One block per kUnroll block steps (up to the grid limit): many short blocks keep more loads in
// flight across the chip than a few that loop. Their set-up is one (gamma, beta) pair per thread
// into an LDS table. Measured over the Wan-shaped 720p decode's RMS norms: 10.65 ms with 8192
// looping blocks (four steps in flight), 11.1 ms short blocks with (gamma, beta) loaded per
// thread, 9.85 ms with the table, 9.77 ms with two steps per block, 11.0 ms with one. Filling the
// table after the block's activation loads are issued (one memory latency instead of two, which
// is what the GroupNorm apply needed) measured slower here: 9.76-9.88 -> 10.41-10.43 ms. The
// fp16-output instances hold 80 registers (6 waves per SIMD); bounding them to 8 waves spills
// (12.5 ms), to 7 waves changes nothing (9.81-9.83 ms). Stores carry the nontemporal hint
// (9.82-9.85 -> 9.62-9.69 ms); on the loads it made the pass slower (10.03-10.08 ms), as on both.
constexpr int64_t kMaxBlocks = INT32_MAX;
constexpr int kMaxC = 2048;                  // C / 8 <= 256 threads per position
constexpr int kUnroll = 2;          // block steps (positions per thread) in flight at once

// Elem<T>::store with the nontemporal hint (the backend merges a thread's 8 into 16-byte stores)
__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(_Float16* p, float v) {
    __builtin_nontemporal_store((_Float16)v, p);
}
__device__ __forceinline__ void store_nt(uint16_t* p, float v) {
    __builtin_nontemporal_store(f32_to_bf16(v), p);
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kThreads) void rms_norm_kernel(const TI* __restrict__ x,
                                                            TO* __restrict__ y, int64_t positions,
                                                            int32_t C, float eps,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta,
                                                            int32_t silu, uint32_t* status) {
    __shared__ float part[kUnroll][kThreads / 64];         // one partial per wave and position
    __shared__ float2 gb[kMaxC];                           // (gamma, beta) per channel
    const int tpp = C / 8;                                 // threads per position
    const int ppb = kThreads / tpp;                        // positions per block step
    const int tid = threadIdx.x;
    const int slot = tid / tpp, c0 = (tid % tpp) * 8;
    const int lane = tid & 63, wave = tid >> 6;
    for (int c = tid; c < C; c += kThreads)
        gb[c] = make_float2(gamma ? gamma[c] : 1.0f, beta ? beta[c] : 0.0f);
    __syncthreads();
    float sc[8], sh[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float2 q = gb[c0 + k];
        sc[k] = q.x;
        sh[k] = q.y;
    }
    // kUnroll block steps at a time: all their loads are in flight before the first reduction
    const int64_t step = (int64_t)ppb * kUnroll;
    for (int64_t p0 = (int64_t)blockIdx.x * step; p0 < positions; p0 += (int64_t)gridDim.x * step) {
        float v[kUnroll][8];
        bool valid[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t p = p0 + u * ppb + slot;
            valid[u] = p < positions;
            const TI* src = x + (valid[u] ? p : 0) * C + c0;
#pragma unroll
            for (int k = 0; k < 8; ++k) v[u][k] = Elem<TI>::load(src + k);
        }
        float ss[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            ss[u] = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) ss[u] = fmaf(v[u][k], v[u][k], ss[u]);
        }
        // sum over the position's threads: within the wave, then across the two waves of a
        // position when tpp = 128 or 256
        const int span = tpp < 64 ? tpp : 64;
        for (int off = 1; off < span; off <<= 1)
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) ss[u] += __shfl_xor(ss[u], off);
        if (tpp > 64) {
            if (lane == 0)
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) part[u][wave] = ss[u];
            __syncthreads();
            const int w0 = (tid / tpp) * (tpp / 64);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float t = 0.0f;
                for (int w = 0; w < tpp / 64; ++w) t += part[u][w0 + w];
                ss[u] = t;
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            // a non-finite sum of squares: an input value was inf or NaN (e.g. an activation
            // past fp16's 65504 at an fp16 operand hand-off)
            if (status && valid[u] && !isfinite(ss[u])) *status = 1u;
            const float r = 1.0f / sqrtf(ss[u] / (float)C + eps);
            if (valid[u]) {
                TO* dst = y + (p0 + u * ppb + slot) * C + c0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    float z = fmaf(v[u][k] * r, sc[k], sh[k]);
                    if (silu) z = z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
                    store_nt(dst + k, z);
                }
            }
        }
    }
}

template <typename TI, typename TO>
void rms_launch(const vae_tensor_t& x, float eps, const float* gamma, const float* beta, bool silu,
                const vae_tensor_t& y, hipStream_t stream, uint32_t* status) {
    const int64_t positions = vae::positions(x);
    const int ppb = kThreads / (int)(x.c / 8);
    const int64_t blocks =
        std::min<int64_t>(ceil_div(positions, (int64_t)ppb * kUnroll), kMaxBlocks);
    hipLaunchKernelGGL((rms_norm_kernel<TI, TO>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const TI*>(x.data), static_cast<TO*>(y.data), positions,
                       (int32_t)x.c, eps, gamma, beta, (int32_t)silu, status);
}

template <typename TI>
void rms_out(const vae_tensor_t& x, float eps, const float* gamma, const float* beta, bool silu,
             const vae_tensor_t& y, hipStream_t stream, uint32_t* status) {
    if (y.dtype == VAE_DTYPE_F32)
        rms_launch<TI, float>(x, eps, gamma, beta, silu, y, stream, status);
    else if (y.dtype == VAE_DTYPE_F16)
        rms_launch<TI, _Float16>(x, eps, gamma, beta, silu, y, stream, status);
    else
        rms_launch<TI, uint16_t>(x, eps, gamma, beta, silu, y, stream, status);
}

}  // namespace

bool rms_shape_supported(int64_t c) {
    return c >= 8 && c % 8 == 0 && c / 8 <= kThreads && kThreads % (c / 8) == 0;
}

vae_status_t launch_rms_norm(const vae_tensor_t& x, float eps, const float* gamma,
                             const float* beta, bool silu, const vae_tensor_t& y,
                             hipStream_t stream, uint32_t* status) {
    if (numel(x) == 0) return VAE_OK;
    if (!rms_shape_supported(x.c))
        return fail(VAE_ERR_UNSUPPORTED, "rms norm needs C % 8 == 0 and C / 8 dividing 256", 4,
                    x.c, 8);
    if (x.dtype == VAE_DTYPE_F32) rms_out<float>(x, eps, gamma, beta, silu, y, stream, status);
    else if (x.dtype == VAE_DTYPE_F16)
        rms_out<_Float16>(x, eps, gamma, beta, silu, y, stream, status);
    else rms_out<uint16_t>(x, eps, gamma, beta, silu, y, stream, status);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

}  // namespace vae
