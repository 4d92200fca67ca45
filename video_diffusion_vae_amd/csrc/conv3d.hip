// Causal Conv3d (3x3x3, stride 1) on channels-last (NDHWC) activations.
//
// bf16 weights: implicit GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//  - GEMM view: M = output positions, N = Cout, K = 27 * Cin, ordered (channel chunk, tap).
//  - One workgroup computes a 2 x 8 x 16 (T x H x W) block of 256 output positions for NT
//    output channels.
//  - For each 32-channel chunk it stages the block's input tile in LDS once: 4 x 10 x 18 positions
//    x 32 channels, i.e. the block, its one-row halo on each spatial side, and the two earlier
//    frames. All 27 taps then read their A operands from that tile at shifted offsets. The halo
//    and the causal frame clamp are thus resolved while the tile is loaded: the halo is the
//    neighbouring data of the same tensor, read in place; rows outside the image become zeros; a
//    frame index below 0 reads frame 0. The pages motivate this: a halo built by concatenation
//    cost 1.31x ("[TRTLLM-14123][feat] add ParallelVAE_TrtllmWan for native Wan VAE",
//    Description).
//  - fp32 inputs are rounded to bf16 (nearest-even) as they are staged, because MFMA operands are
//    bf16. Accumulation is fp32. With the split flag an fp32 input is applied as two bf16
//    operands, hi = bf16(x) and lo = bf16(x - hi). The K loop visits every channel chunk twice,
//    about 16 significant bits of x reach the matrix cores, and the MFMA work doubles.
//  - The weights of the next tap are prefetched into registers while the current tap runs, and
//    double-buffered in LDS.
//  - LDS rows are padded from 64 to 80 bytes, so the 16-byte operand reads of 8 consecutive
//    lanes hit 8 distinct 16-byte bank groups.
//  - Epilogue: each wave parks one 32 x WN accumulator tile at a time in LDS (reusing the input
//    tile), then every lane writes four consecutive channels with one 16-byte (fp32) or 8-byte
//    (bf16) store. Bias and residual are added on the way.
//  - Workgroups are ordered output-channel tile slowest, and remapped so that each XCD (the
//    hardware deals workgroup i to XCD i % 8) runs a contiguous range of them. An XCD then keeps
//    one weight slice in its own L2 while it streams input blocks.
// fp32 weights, or Cin % 32 != 0, or Cout % 4 != 0: a direct kernel, one thread per output.
#include "kernels.h"

namespace vae {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kTB = 2, kHB = 8, kWB = 16;            // output block (T, H, W)
constexpr int kHT = kTB + 2, kHH = kHB + 2, kHW = kWB + 2;
constexpr int kHaloPos = kHT * kHH * kHW;            // 720 input positions per block
constexpr int kCK = 32;                              // input channels per LDS chunk
constexpr int kRow = kCK * 2 + 16;                   // padded LDS row, bytes
constexpr int kThreads = 256;
constexpr int kXcds = 8;

struct MfmaArgs {
    const void* x;
    const uint16_t* w;
    const float* bias;
    const void* res;
    void* y;
    int32_t T, H, W, cin, cout;
    Box box;
    int32_t nbt, nbh, nbw;   // blocks along each box axis
    int32_t n_mblocks;       // N * nbt * nbh * nbw
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    int per = total / kXcds;
    int full = per * kXcds;
    if (bid >= full) return bid;
    return (bid % kXcds) * per + bid / kXcds;
}

// 8 input channels starting at p, as 8 bf16 in one 16-byte word.
template <typename TI> __device__ __forceinline__ uint4 load8(const TI* p);
template <> __device__ __forceinline__ uint4 load8<uint16_t>(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
template <> __device__ __forceinline__ uint4 load8<float>(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    uint4 r;
    r.x = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
    r.y = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
    r.z = (uint32_t)f32_to_bf16(b.x) | ((uint32_t)f32_to_bf16(b.y) << 16);
    r.w = (uint32_t)f32_to_bf16(b.z) | ((uint32_t)f32_to_bf16(b.w) << 16);
    return r;
}

// The low half of the hi + lo bf16 split of 8 fp32 values: bf16(x - bf16(x)).
__device__ __forceinline__ uint16_t lo_bf16(float x) {
    return f32_to_bf16(x - bf16_to_f32(f32_to_bf16(x)));
}
template <typename TI> __device__ __forceinline__ uint4 load8_lo(const TI* p);
template <> __device__ __forceinline__ uint4 load8_lo<uint16_t>(const uint16_t*) {
    return make_uint4(0, 0, 0, 0);
}
template <> __device__ __forceinline__ uint4 load8_lo<float>(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    uint4 r;
    r.x = (uint32_t)lo_bf16(a.x) | ((uint32_t)lo_bf16(a.y) << 16);
    r.y = (uint32_t)lo_bf16(a.z) | ((uint32_t)lo_bf16(a.w) << 16);
    r.z = (uint32_t)lo_bf16(b.x) | ((uint32_t)lo_bf16(b.y) << 16);
    r.w = (uint32_t)lo_bf16(b.z) | ((uint32_t)lo_bf16(b.w) << 16);
    return r;
}

template <typename TO> __device__ __forceinline__ void load4(const TO* p, float* v);
template <> __device__ __forceinline__ void load4<float>(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
template <> __device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float* v) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_to_f32((uint16_t)(a.x & 0xffff)); v[1] = bf16_to_f32((uint16_t)(a.x >> 16));
    v[2] = bf16_to_f32((uint16_t)(a.y & 0xffff)); v[3] = bf16_to_f32((uint16_t)(a.y >> 16));
}
template <typename TO> __device__ __forceinline__ void store4(TO* p, const float* v);
template <> __device__ __forceinline__ void store4<float>(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float* v) {
    uint2 a;
    a.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    a.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = a;
}

template <int NT, typename TI, typename TO, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void conv3d_mfma_kernel(MfmaArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t halo[kHaloPos * kRow];
    __shared__ __attribute__((aligned(16))) uint8_t bbuf[2][NT * kRow];

    constexpr int WN = NT / 2;        // output channels per wave
    constexpr int NJ = WN / 32;       // 32-wide MFMA column tiles per wave
    constexpr int BU = NT * 4 / kThreads;  // 16-byte weight units per thread per tap

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = logical / a.n_mblocks;
    int mb = logical - nt * a.n_mblocks;
    const int bw_i = mb % a.nbw;
    mb /= a.nbw;
    const int bh_i = mb % a.nbh;
    mb /= a.nbh;
    const int bt_i = mb % a.nbt;
    const int n = mb / a.nbt;
    const int t_blk = a.box.t0 + bt_i * kTB;
    const int h_blk = a.box.h0 + bh_i * kHB;
    const int w_blk = a.box.w0 + bw_i * kWB;
    const int n_blk = nt * NT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave >> 1;     // frame of the block this wave computes
    const int wave_n = wave & 1;
    const int lrow = lane & 31;
    const int khalf = lane >> 5;      // which 8 of the 16 k values this lane feeds

    const int64_t cin = a.cin;
    const TI* xn = static_cast<const TI*>(a.x) + (int64_t)n * a.T * a.H * a.W * cin;

    f32x16_t acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // halo position of this lane's output row for sub-tile 0, tap (0,0,0)
    const int a_base = (wave_m * kHH + (lrow >> 4)) * kHW + (lrow & 15);

    uint4 breg[BU];
    auto load_b = [&](int tap, int c0) {
#pragma unroll
        for (int k = 0; k < BU; ++k) {
            int u = tid + k * kThreads;
            int row = u >> 2, g = u & 3;
            int co = n_blk + row;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (co < a.cout)
                v = *reinterpret_cast<const uint4*>(a.w + ((int64_t)co * 27 + tap) * cin + c0 + g * 8);
            breg[k] = v;
        }
    };
    auto store_b = [&](int buf) {
#pragma unroll
        for (int k = 0; k < BU; ++k) {
            int u = tid + k * kThreads;
            int row = u >> 2, g = u & 3;
            *reinterpret_cast<uint4*>(&bbuf[buf][row * kRow + g * 16]) = breg[k];
        }
    };

    const int n_passes = (a.cin / kCK) * (SPLIT ? 2 : 1);
    for (int kc = 0; kc < n_passes; ++kc) {
        const int c0 = (SPLIT ? (kc >> 1) : kc) * kCK;
        const bool lo = SPLIT && (kc & 1);
        __syncthreads();  // the previous chunk's LDS reads are done
        for (int u = tid; u < kHaloPos * 4; u += kThreads) {
            int pos = u >> 2, g = u & 3;
            int f = pos / (kHH * kHW);
            int rem = pos - f * (kHH * kHW);
            int r = rem / kHW;
            int c = rem - r * kHW;
            int tg = t_blk - 2 + f;
            tg = tg < 0 ? 0 : tg;                      // causal: frames before 0 read frame 0
            int hg = h_blk - 1 + r, wg = w_blk - 1 + c;
            uint4 v = make_uint4(0, 0, 0, 0);          // outside the image: zero padding
            if (tg < a.T && hg >= 0 && hg < a.H && wg >= 0 && wg < a.W) {
                const TI* src = xn + ((int64_t)(tg * a.H + hg) * a.W + wg) * cin + c0 + g * 8;
                v = lo ? load8_lo<TI>(src) : load8<TI>(src);
            }
            *reinterpret_cast<uint4*>(&halo[pos * kRow + g * 16]) = v;
        }
        load_b(0, c0);
        store_b(0);
        __syncthreads();

        for (int tap = 0; tap < 27; ++tap) {
            if (tap + 1 < 27) load_b(tap + 1, c0);
            const int kt = tap / 9, kh = (tap / 3) % 3, kw = tap % 3;
            const uint8_t* bb = bbuf[tap & 1];
            const int a_tap = a_base + (kt * kHH + kh) * kHW + kw;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int goff = (kk * 2 + khalf) * 16;
                bf16x8_t bf[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    bf[j] = *reinterpret_cast<const bf16x8_t*>(
                        bb + (wave_n * WN + j * 32 + lrow) * kRow + goff);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(
                        &halo[(a_tap + i * 2 * kHW) * kRow + goff]);
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[j], acc[i][j],
                                                                            0, 0, 0);
                }
            }
            if (tap + 1 < 27) store_b((tap + 1) & 1);
            __syncthreads();
        }
    }

    // Epilogue. In a 32x32 accumulator tile, lane l holds column l % 32 and register r holds
    // row (r / 4) * 8 + (l / 32) * 4 + r % 4. Each wave parks one 32 x WN sub-tile at a time in
    // its own slice of the (now idle) input tile, then reads rows back four channels per lane.
    constexpr int EP = WN + 4;                      // padded staging row, floats
    constexpr int LPR = WN / 4;                     // lanes per staged row
    constexpr int RPP = 64 / LPR;                   // rows per pass
    static_assert(4 * 32 * EP * 4 <= kHaloPos * kRow, "epilogue staging must fit the input tile");
    float* ep = reinterpret_cast<float*>(halo) + wave * (32 * EP);
    const TO* res = static_cast<const TO*>(a.res);
    TO* y = static_cast<TO*>(a.y);
    const int t = t_blk + wave_m;
    const int c4 = (lane % LPR) * 4;
    const int co = n_blk + wave_n * WN + c4;
    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a.bias)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (co + k < a.cout) bv[k] = a.bias[co + k];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ep[((r >> 2) * 8 + khalf * 4 + (r & 3)) * EP + j * 32 + lrow] = acc[i][j][r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int pass = 0; pass < 32 / RPP; ++pass) {
            const int row = pass * RPP + lane / LPR;
            const int m = i * 32 + row;
            const int h = h_blk + (m >> 4), w = w_blk + (m & 15);
            if (t < a.box.t1 && h < a.box.h1 && w < a.box.w1 && co < a.cout) {
                float v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = ep[row * EP + c4 + k] + bv[k];
                const int64_t o = ((((int64_t)n * a.T + t) * a.H + h) * a.W + w) * a.cout + co;
                if (co + 4 <= a.cout) {
                    if (res) {
                        float rv[4];
                        load4<TO>(res + o, rv);
#pragma unroll
                        for (int k = 0; k < 4; ++k) v[k] += rv[k];
                    }
                    store4<TO>(y + o, v);
                } else {
                    for (int k = 0; co + k < a.cout; ++k) {
                        float vk = v[k];
                        if (res) vk += Elem<TO>::load(res + o + k);
                        Elem<TO>::store(y + o + k, vk);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

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

template <int NT, typename TI, typename TO, bool SPLIT>
vae_status_t run_mfma(const vae_tensor_t& x, const void* w, const float* bias,
                      const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                      hipStream_t stream) {
    MfmaArgs a;
    a.x = x.data;
    a.w = static_cast<const uint16_t*>(w);
    a.bias = bias;
    a.res = residual ? residual->data : nullptr;
    a.y = y.data;
    a.T = (int32_t)x.t;
    a.H = (int32_t)x.h;
    a.W = (int32_t)x.w;
    a.cin = (int32_t)x.c;
    a.cout = (int32_t)y.c;
    a.box = box;
    a.nbt = (int32_t)ceil_div(box.bt(), kTB);
    a.nbh = (int32_t)ceil_div(box.bh(), kHB);
    a.nbw = (int32_t)ceil_div(box.bw(), kWB);
    int64_t mblocks = x.n * (int64_t)a.nbt * a.nbh * a.nbw;
    int64_t total = mblocks * ceil_div(y.c, NT);
    if (total > INT32_MAX) return fail(VAE_ERR_UNSUPPORTED, "conv3d: grid too large");
    a.n_mblocks = (int32_t)mblocks;
    hipLaunchKernelGGL((conv3d_mfma_kernel<NT, TI, TO, SPLIT>), dim3((unsigned)total),
                       dim3(kThreads), 0, stream, a);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

template <int NT, typename TI, bool SPLIT>
vae_status_t run_mfma_out(const vae_tensor_t& x, const void* w, const float* bias,
                          const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                          hipStream_t stream) {
    if (y.dtype == VAE_DTYPE_F32)
        return run_mfma<NT, TI, float, SPLIT>(x, w, bias, residual, y, box, stream);
    return run_mfma<NT, TI, uint16_t, SPLIT>(x, w, bias, residual, y, box, stream);
}

template <int NT>
vae_status_t run_mfma_in(const vae_tensor_t& x, const void* w, const float* bias,
                         const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                         bool split, hipStream_t stream) {
    if (x.dtype == VAE_DTYPE_BF16)
        return run_mfma_out<NT, uint16_t, false>(x, w, bias, residual, y, box, stream);
    if (split) return run_mfma_out<NT, float, true>(x, w, bias, residual, y, box, stream);
    return run_mfma_out<NT, float, false>(x, w, bias, residual, y, box, stream);
}

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

bool conv_uses_mfma(const vae_tensor_t& x, const vae_tensor_t& y, int32_t weight_dtype) {
    return weight_dtype == VAE_DTYPE_BF16 && x.c % kCK == 0 && y.c % 4 == 0;
}

vae_status_t launch_conv3d(const vae_tensor_t& x, const void* w, int32_t weight_dtype,
                           const float* bias, const vae_tensor_t* residual, const vae_tensor_t& y,
                           const Box& box, int32_t flags, hipStream_t stream) {
    if (box.volume() == 0 || x.n == 0) return VAE_OK;
    const bool xf = x.dtype == VAE_DTYPE_F32;
    const bool split = (flags & VAE_CONV_SPLIT_FP32) != 0;
    if (conv_uses_mfma(x, y, weight_dtype)) {
        if (y.c >= 128) return run_mfma_in<128>(x, w, bias, residual, y, box, split, stream);
        return run_mfma_in<64>(x, w, bias, residual, y, box, split, stream);
    }
    if (weight_dtype == VAE_DTYPE_F32)
        return xf ? run_direct_out<float, float>(x, w, bias, residual, y, box, stream)
                  : run_direct_out<uint16_t, float>(x, w, bias, residual, y, box, stream);
    return xf ? run_direct_out<float, uint16_t>(x, w, bias, residual, y, box, stream)
              : run_direct_out<uint16_t, uint16_t>(x, w, bias, residual, y, box, stream);
}

}  // namespace vae
