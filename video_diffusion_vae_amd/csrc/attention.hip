// Single-head self-attention over the positions of each frame, with its residual: the mid-block
// attention of Wan-style decoders. It takes each frame whole, so a patch-split decode gathers the
// frame around it ("Add tiled VAE parallelism & extended model support", commit message on the
// HunyuanVideo adapters; the Wan attention block of "[TRTLLM-14123][feat] add
// ParallelVAE_TrtllmWan for native Wan VAE", Description). On one GPU every patch lives in the same
// tensor, so the block simply runs over the whole tensor.
//
//   xn = rms_norm(x)                          bf16 [P, C]
//   [q | k] = xn W_qk^T + b_qk                fp16 [P, 2C]     (one GEMM over all positions)
//   v^T = W_v xn^T + b_v, per frame           fp16 [F][C][HWp] (so that A v reads K-contiguous rows)
//   s = q k^T / sqrt(C), per frame            fp32 [F][HW][HWp]
//   a = softmax(s) along each row             fp16 [F][HW][HWp]
//   o = a v, per frame                        bf16 [P, C]
//   y = o W_out^T + b_out + x                 fp32 [P, C]
// P = N*T*H*W positions, F = N*T frames, HW = H*W positions per frame, HWp = HW rounded up to 8.
//
// Every product is one batched "NT" GEMM on the matrix cores: C[b][m][n] = alpha *
// sum_k A[b][m][k] B[b][n][k] (+ bias, + residual), A and B both K-contiguous, which is what
// channels-last activations and [out][in] weights already are. 128 x 128 tiles, 4 waves of 64 x 64
// (2 x 2 MFMA 32x32x16 tiles each), K in steps of 64 through two LDS buffers: the next step's
// global loads are in flight while the 16 MFMAs per wave of the current one run. Rows past M or N
// read a valid row and are never stored; K elements past K are zero-filled in LDS.
#include <algorithm>
#include <cmath>

#include "conv3d_mfma.h"

namespace vae {
namespace {

using mfma::bf16x8_t;
using mfma::f32x16_t;
using mfma::mfma_step;

constexpr int kThreads = 256;
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitch = kBK + 8;     // halves per LDS row (144 bytes, an odd number of 16-byte
                                    // units): conflict-free 16-byte fragment reads
constexpr int kUnits = kBM * kBK / 8 / kThreads;   // 16-byte units per thread per operand

struct GemmArgs {
    const uint16_t* a;   // 2-byte operands (bf16 or fp16 bits)
    const uint16_t* b;
    void* c;
    const float* bias_n;   // per output column, or null
    const float* bias_m;   // per output row, or null
    const float* res;      // fp32 residual [b][m][ldr], or null
    int32_t M, N, K;
    int64_t lda, ldb, ldc, ldr;
    int64_t sa, sb, sc, sr;   // batch strides (elements)
    float alpha;
};

template <bool F16, typename TO>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kPitch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int bz = blockIdx.z;
    const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
    const uint16_t* A = g.a + (int64_t)bz * g.sa;
    const uint16_t* B = g.b + (int64_t)bz * g.sb;

    // staging: each thread moves kUnits 16-byte units of A and of B per K step
    uint4 ra[kUnits], rb[kUnits];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kUnits; ++i) {
            const int u = tid + i * kThreads;
            const int row = u / (kBK / 8), kc = (u % (kBK / 8)) * 8;
            const int k = k0 + kc;
            const int ma = std::min(m0 + row, g.M - 1), nb = std::min(n0 + row, g.N - 1);
            uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
            if (k < g.K) {
                va = *reinterpret_cast<const uint4*>(A + (int64_t)ma * g.lda + k);
                vb = *reinterpret_cast<const uint4*>(B + (int64_t)nb * g.ldb + k);
                if (k + 8 > g.K) {   // a partial unit at the end of K: zero the tail
                    // per 32-bit word, keep the halves whose k is inside K (static indices only,
                    // so the unit stays in registers)
                    auto keep = [&](int e) {
                        return (k + e < g.K ? 0xffffu : 0u) |
                               (k + e + 1 < g.K ? 0xffff0000u : 0u);
                    };
                    const uint32_t m0 = keep(0), m1 = keep(2), m2 = keep(4), m3 = keep(6);
                    va.x &= m0; va.y &= m1; va.z &= m2; va.w &= m3;
                    vb.x &= m0; vb.y &= m1; vb.z &= m2; vb.w &= m3;
                }
            }
            ra[i] = va;
            rb[i] = vb;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kUnits; ++i) {
            const int u = tid + i * kThreads;
            const int row = u / (kBK / 8), kc = (u % (kBK / 8)) * 8;
            *reinterpret_cast<uint4*>(&As[buf][row * kPitch + kc]) = ra[i];
            *reinterpret_cast<uint4*>(&Bs[buf][row * kPitch + kc]) = rb[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (g.K + kBK - 1) / kBK;
    load(0);
    store(0);
    __syncthreads();
    const int lrow = lane & 31, khalf = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + lrow;
                af[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][r * kPitch + kk * 16 + khalf * 8]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn * 64 + j * 32 + lrow;
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][r * kPitch + kk * 16 + khalf * 8]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma_step<F16>(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane l holds column l % 32 of each 32x32 tile; register r holds row
    // (r / 4) * 8 + (l / 32) * 4 + r % 4
    TO* C = static_cast<TO*>(g.c) + (int64_t)bz * g.sc;
    const float* R = g.res ? g.res + (int64_t)bz * g.sr : nullptr;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + lrow;
            if (n >= g.N) continue;
            const float bn = g.bias_n ? g.bias_n[n] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
                if (m >= g.M) continue;
                float v = acc[i][j][r] * g.alpha + bn;
                if (g.bias_m) v += g.bias_m[m];
                if (R) v += R[(int64_t)m * g.ldr + n];
                Elem<TO>::store(C + (int64_t)m * g.ldc + n, v);
            }
        }
}

template <bool F16, typename TO>
vae_status_t gemm(const GemmArgs& g, int batch, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0 || batch <= 0) return VAE_OK;
    const dim3 grid((unsigned)ceil_div(g.N, kBN), (unsigned)ceil_div(g.M, kBM), (unsigned)batch);
    hipLaunchKernelGGL((gemm_nt_kernel<F16, TO>), grid, dim3(kThreads), 0, s, g);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

// Row softmax: s [rows][ld] fp32 (first `len` columns) -> p [rows][ld] fp16.
__global__ __launch_bounds__(kThreads) void softmax_rows_kernel(const float* __restrict__ s,
                                                                _Float16* __restrict__ p,
                                                                int32_t len, int64_t ld) {
    __shared__ float red[kThreads / 64];
    const float* row = s + (int64_t)blockIdx.x * ld;
    _Float16* out = p + (int64_t)blockIdx.x * ld;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float mx = -INFINITY;
    for (int i = tid; i < len; i += kThreads) mx = fmaxf(mx, row[i]);
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.0f;
    for (int i = tid; i < len; i += kThreads) sum += expf(row[i] - mx);
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sum;
    for (int i = tid; i < len; i += kThreads) out[i] = (_Float16)(expf(row[i] - mx) * inv);
}

struct AttnLayout {
    int64_t P, F, HW, HWp, C;
    size_t xn, qk, vt, s, p, o, total;
};

AttnLayout attn_layout(const vae_tensor_t& x) {
    AttnLayout L{};
    L.P = positions(x);
    L.F = x.n * x.t;
    L.HW = x.h * x.w;
    L.HWp = (L.HW + 7) / 8 * 8;
    L.C = x.c;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes, 256);
        return at;
    };
    L.xn = take((size_t)L.P * L.C * 2);
    L.qk = take((size_t)L.P * 2 * L.C * 2);
    L.vt = take((size_t)L.F * L.C * L.HWp * 2);
    L.s = take((size_t)L.F * L.HW * L.HWp * 4);
    L.p = take((size_t)L.F * L.HW * L.HWp * 2);
    L.o = take((size_t)L.P * L.C * 2);
    L.total = off;
    return L;
}

}  // namespace

bool attention_shape_supported(int64_t c) { return c % 32 == 0 && rms_shape_supported(c); }

size_t attention_workspace(const vae_tensor_t& x) { return attn_layout(x).total; }

vae_status_t launch_frame_attention(const vae_tensor_t& x, float eps, const float* gamma,
                                    const float* beta, const void* w_qkv, const float* b_qkv,
                                    const void* w_out, const float* b_out, const vae_tensor_t& y,
                                    void* ws, hipStream_t s) {
    if (numel(x) == 0) return VAE_OK;
    if (!attention_shape_supported(x.c))
        return fail(VAE_ERR_UNSUPPORTED, "attention needs C % 32 == 0 and C / 8 dividing 256", 4,
                    x.c, 32);
    if (x.dtype != VAE_DTYPE_F32 || y.dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_UNSUPPORTED, "attention reads and writes fp32 activations");
    const AttnLayout L = attn_layout(x);
    if (L.HW > INT32_MAX || L.P > INT32_MAX)
        return fail(VAE_ERR_UNSUPPORTED, "attention: too many positions");
    uint8_t* w = static_cast<uint8_t*>(ws);
    uint16_t* xn = reinterpret_cast<uint16_t*>(w + L.xn);
    uint16_t* qk = reinterpret_cast<uint16_t*>(w + L.qk);
    uint16_t* vt = reinterpret_cast<uint16_t*>(w + L.vt);
    float* sc = reinterpret_cast<float*>(w + L.s);
    _Float16* pr = reinterpret_cast<_Float16*>(w + L.p);
    uint16_t* o = reinterpret_cast<uint16_t*>(w + L.o);
    const int32_t C = (int32_t)L.C, HW = (int32_t)L.HW;
    const uint16_t* wq = static_cast<const uint16_t*>(w_qkv);

    vae_tensor_t xnt = x;
    xnt.data = xn;
    xnt.dtype = VAE_DTYPE_BF16;
    VAE_TRY(launch_rms_norm(x, eps, gamma, beta, false, xnt, s));

    GemmArgs g{};
    // [q | k] = xn W_qk^T + b_qk over all positions
    g = GemmArgs{xn, wq, qk, b_qkv, nullptr, nullptr, (int32_t)L.P, 2 * C, C, C, C, 2 * C, 0,
                 0, 0, 0, 0, 1.0f};
    VAE_TRY((gemm<false, _Float16>(g, 1, s)));
    // v^T = W_v xn^T + b_v per frame: M = C (rows of W_v), N = HW positions
    g = GemmArgs{wq + (int64_t)2 * C * C, xn, vt, nullptr, b_qkv ? b_qkv + 2 * C : nullptr,
                 nullptr, C, HW, C, C, C, L.HWp, 0, 0, (int64_t)HW * C, (int64_t)C * L.HWp, 0,
                 1.0f};
    VAE_TRY((gemm<false, _Float16>(g, (int)L.F, s)));
    // s = q k^T / sqrt(C) per frame
    g = GemmArgs{qk, qk + C, sc, nullptr, nullptr, nullptr, HW, HW, C, 2 * C, 2 * C, L.HWp, 0,
                 (int64_t)HW * 2 * C, (int64_t)HW * 2 * C, (int64_t)HW * L.HWp, 0,
                 1.0f / std::sqrt((float)C)};
    VAE_TRY((gemm<true, float>(g, (int)L.F, s)));
    hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)(L.F * L.HW)), dim3(kThreads), 0, s, sc,
                       pr, HW, L.HWp);
    VAE_HIP_CHECK(hipGetLastError());
    // o = a v per frame: A = a [HW][HWp], B = v^T [C][HWp], K = HW
    g = GemmArgs{reinterpret_cast<const uint16_t*>(pr), vt, o, nullptr, nullptr, nullptr, HW, C,
                 HW, L.HWp, L.HWp, C, 0, (int64_t)HW * L.HWp, (int64_t)C * L.HWp, (int64_t)HW * C,
                 0, 1.0f};
    VAE_TRY((gemm<true, uint16_t>(g, (int)L.F, s)));
    // y = o W_out^T + b_out + x
    g = GemmArgs{o, static_cast<const uint16_t*>(w_out), y.data, b_out, nullptr,
                 static_cast<const float*>(x.data), (int32_t)L.P, C, C, C, C, C, C, 0, 0, 0, 0,
                 1.0f};
    return gemm<false, float>(g, 1, s);
}

}  // namespace vae
