// Internal helpers shared by the library's translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "vae.h"

namespace vae {

// ------------------------------------------------------------------------------------------------
// bfloat16 storage. Values are kept as raw uint16_t and converted by bit manipulation, so the
// rounding is exactly round-to-nearest-even on every store.
// ------------------------------------------------------------------------------------------------
__host__ __device__ inline float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__host__ __device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
    static constexpr int kVec = 8;  // elements per 16-byte vector
};
// IEEE binary16 storage (the fp16 operand hand-off). Conversions round to nearest even.
template <> struct Elem<_Float16> {
    static __device__ __forceinline__ float load(const _Float16* p) { return (float)*p; }
    static __device__ __forceinline__ void store(_Float16* p, float v) { *p = (_Float16)v; }
    static constexpr int kVec = 8;
};
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
    static constexpr int kVec = 4;
};

// GroupNorm apply as a per-channel affine map, and the SiLU after it. Every kernel that applies a
// GroupNorm (the normalise pass, the convs that normalise while staging) goes through these two,
// so that their results agree bit for bit: explicit fused multiply-adds leave the compiler no
// contraction to choose.
__host__ __device__ inline void gn_scale_shift_of(float mean, float rstd, float gamma, float beta,
                                                  float& scale, float& shift) {
    scale = rstd * gamma;
    shift = fmaf(-mean, scale, beta);
}
__device__ __forceinline__ float gn_silu_apply(float x, float scale, float shift) {
    const float z = fmaf(x, scale, shift);
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
// v as an fp32 value the compiler must produce: a narrowing that follows is then a second
// rounding of it, never folded with the operation that made v into one mixed-precision fma
// (v_fma_mixlo_f16 rounds the exact product once). An empty asm statement, no instruction.
__device__ __forceinline__ float materialise_f32(float v) {
    asm("" : "+v"(v));
    return v;
}

// ------------------------------------------------------------------------------------------------
// Error state (thread-local), filled by the ABI layer.
// ------------------------------------------------------------------------------------------------
struct ErrorState {
    std::string text;
    vae_error_info_t info{VAE_OK, -1, -1, -1, -1};
};
ErrorState& error_state();

vae_status_t fail(vae_status_t st, const std::string& msg, int32_t axis = -1, int64_t extent = -1,
                  int64_t multiple = -1, int64_t min_width = -1);
void clear_error();

#define VAE_HIP_CHECK(expr)                                                                  \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess)                                                                \
            return ::vae::fail(VAE_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    } while (0)

#define VAE_TRY(expr)                          \
    do {                                       \
        vae_status_t s_ = (expr);              \
        if (s_ != VAE_OK) return s_;           \
    } while (0)

// ------------------------------------------------------------------------------------------------
// Shapes
// ------------------------------------------------------------------------------------------------
struct Box {
    int32_t t0, t1, h0, h1, w0, w1;
    __host__ __device__ int64_t bt() const { return t1 - t0; }
    __host__ __device__ int64_t bh() const { return h1 - h0; }
    __host__ __device__ int64_t bw() const { return w1 - w0; }
    __host__ __device__ int64_t volume() const { return bt() * bh() * bw(); }
};

inline Box whole_box(const vae_tensor_t& x) {
    return Box{0, (int32_t)x.t, 0, (int32_t)x.h, 0, (int32_t)x.w};
}
inline Box to_box(const vae_box_t* b, const vae_tensor_t& x) {
    return b ? Box{b->t0, b->t1, b->h0, b->h1, b->w0, b->w1} : whole_box(x);
}
inline int64_t elem_size(int32_t dtype) { return dtype == VAE_DTYPE_F32 ? 4 : 2; }
inline int64_t positions(const vae_tensor_t& x) { return x.n * x.t * x.h * x.w; }
inline int64_t numel(const vae_tensor_t& x) { return positions(x) * x.c; }

inline hipStream_t as_stream(vae_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace vae
