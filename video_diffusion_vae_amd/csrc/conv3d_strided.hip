// Strided causal Conv3d: the bare downsampler of an encoder. One of the LTX-2 encoder's downsample
// kinds is a plain strided convolution, and the Wan / Qwen-Image encoder pads (0, 1, 0, 1) and then
// strides 2 ("Add tiled VAE parallelism & extended model support", LTX-2 and Qwen-Image/Wan encoder
// commit messages).
//
//   y[n, t, h, w, o] = bias[o] + sum_{a,p,q,c} W[o, a, p, q, c] *
//                      x[n, max(st*t + a - 2, 0), sh*h + p - pt, sw*w + q - pl, c]
// with zeros where a row or column leaves the image; pt / pl are the zero rows / columns before
// the image (1 with padding around it, 0 with padding after it only). T frames become
// (T - 1) / st + 1; H rows become (H + pt + pb - 3) / sh + 1.
//
// Matrix-core path (bf16 or fp16 x, fragment-packed weights, Cin % 32 == 0):
//  - implicit GEMM over output blocks of 2 x 8 x 8 positions, or 2 x 4 x 8 with 128-wide channel
//    tiles (the stride multiplies the input footprint: 5 x 17 x 17 or 5 x 9 x 17 positions at
//    stride 2), 4 waves, NT output channels per workgroup;
//  - per 32-channel chunk the block's input footprint is staged in LDS (halo rows read in place,
//    causal frames clamped, zeros outside the image), 80 bytes per position; lane l of a fragment
//    read takes output column l % 8 at input column 2 * (l % 8), 160 bytes apart, so 8 lanes hit
//    8 distinct 16-byte bank groups;
//  - a 2 x 8 x 8 block's stride-2 footprint fills 116 KB of LDS (one workgroup per CU), a 2 x 4 x 8
//    block's 61 KB (two per CU, one staging while the other computes). All of a chunk's staging
//    loads are issued before the first is written, so a chunk waits about one memory latency;
//  - weights and the epilogue (bias, residual, GroupNorm partials) as in conv3d_mfma.h.
// Everything else runs on a direct kernel, one thread per output, fp32 accumulation.
#include <algorithm>

#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
namespace {

// Output block per workgroup: 2 x 8 x 8 (128 positions), or 2 x 4 x 8 (64) at NT = 128. The
// smaller block's stride-2 footprint (61 KB of LDS) lets two workgroups share a CU, so one stages
// while the other computes; with 128-wide channel tiles each still runs two MFMA tiles per wave.
constexpr int kSTB = 2, kSWB = 8;
constexpr int strided_hb(int nt) { return nt == 128 ? 4 : 8; }

template <int ST, int SS, int HB>
struct StridedShape {
    static constexpr int FT = (kSTB - 1) * ST + 3;   // input frames staged per block
    static constexpr int FH = (HB - 1) * SS + 3;
    static constexpr int FW = (kSWB - 1) * SS + 3;
    static constexpr int kPos = FT * FH * FW;
    static constexpr int kBytes = kPos * kRow;
};

struct StridedArgs {
    MfmaArgs e;            // the output side as the epilogue reads it (no depth-to-space)
    int32_t xT, xH, xW;    // input extents
    int32_t pt, pl;        // zero rows and columns before the image
};

template <int NT, typename TI, typename TO, int ST, int SS>
__global__ __launch_bounds__(kMfmaThreads, NT == 128 ? 2 : 1)
void conv3d_strided_kernel(StridedArgs sa) {
    constexpr int HB = strided_hb(NT);
    using S = StridedShape<ST, SS, HB>;
    const MfmaArgs& a = sa.e;
    constexpr bool F16 = std::is_same<TI, _Float16>::value;
    constexpr int TB = kSTB, WB = kSWB;
    constexpr int WNN = NT / 32;
    constexpr int WM = kMfmaWaves / WNN;
    constexpr int MW = TB * HB * WB / WM;
    constexpr int MI = MW / 32;
    constexpr int PD = 2, NB = PD + 1;
    constexpr int UNITS = S::kPos * 4;                   // 8-channel staging units per chunk
    constexpr int NU = (UNITS + kMfmaThreads - 1) / kMfmaThreads;
    static_assert(MI >= 1 && WNN * WM == kMfmaWaves, "wave grid");
    static_assert(kMfmaWaves * 32 * kEp * 4 <= S::kBytes, "epilogue staging must fit the tile");
    __shared__ __attribute__((aligned(16))) uint8_t tile[S::kBytes];

    const int logical = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, gridDim.x));
    const int nt = __builtin_amdgcn_readfirstlane(logical / a.n_mblocks);
    int mb = logical - nt * a.n_mblocks;
    const int bw_i = mb % a.nbw;
    mb /= a.nbw;
    const int bh_i = mb % a.nbh;
    mb /= a.nbh;
    const int bt_i = mb % a.nbt;
    const int n = mb / a.nbt;
    const int t_blk = a.box.t0 + bt_i * TB;
    const int h_blk = a.box.h0 + bh_i * HB;
    const int w_blk = a.box.w0 + bw_i * WB;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave / WNN;
    const int wave_n = wave % WNN;
    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    const int64_t cin = a.cin;
    const TI* xn = static_cast<const TI*>(a.x) + (int64_t)n * sa.xT * sa.xH * sa.xW * cin;

    f32x16_t acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    // LDS byte offset of this lane's A row (tap 0,0,0): output (tb, hb, wb) reads the footprint
    // from (ST * tb, SS * hb, SS * wb)
    int a_off[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int m = wave_m * MW + i * 32 + lrow;
        const int tb = m / (HB * WB), hb = (m / WB) % HB, wb = m % WB;
        a_off[i] = ((ST * tb * S::FH + SS * hb) * S::FW + SS * wb) * kRow + khalf * 16;
    }
    // fragment-packed weights: the 64 lanes of a fragment read 1 KB contiguously
    const int nch = a.cin / kCK;
    const int co_tile = nt * NT + wave_n * 32;
    const uint16_t* b_ptr = a.w + (int64_t)(co_tile < a.cout ? co_tile >> 5 : 0) * 27 * nch * 1024 +
                            lrow * 16 + khalf * 8;
    uint4 bq[NB][2];
    auto load_b = [&](int buf, int tap, int c0) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            bq[buf][kk] = *reinterpret_cast<const uint4*>(
                b_ptr + ((int64_t)tap * nch + (c0 >> 5)) * 1024 + kk * 512);
    };

    const int t_org = ST * t_blk - 2;           // first staged frame (before the causal clamp)
    const int h_org = SS * h_blk - sa.pt;
    const int w_org = SS * w_blk - sa.pl;
    for (int kc = 0; kc < nch; ++kc) {
        const int c0 = kc * kCK;
#pragma unroll
        for (int t = 0; t < PD; ++t) load_b(t, t, c0);
        __syncthreads();                        // the previous chunk's LDS reads are done
        // all of the chunk's loads first, then all LDS writes
        uint4 v[NU];
        uint32_t in_img = 0;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            int u = tid + i * kMfmaThreads;
            u = u < UNITS ? u : UNITS - 1;      // surplus lanes repeat the last unit
            const int p = u >> 2, g = u & 3;
            const int ft = p / (S::FH * S::FW), fr = p % (S::FH * S::FW);
            const int fh = fr / S::FW, fw = fr % S::FW;
            int tg = t_org + ft;
            tg = tg < 0 ? 0 : (tg >= sa.xT ? sa.xT - 1 : tg);   // causal clamp; past T unused
            const int hg = h_org + fh, wg = w_org + fw;
            const bool in = (unsigned)hg < (unsigned)sa.xH && (unsigned)wg < (unsigned)sa.xW;
            const int hc = hg < 0 ? 0 : (hg >= sa.xH ? sa.xH - 1 : hg);
            const int wc = wg < 0 ? 0 : (wg >= sa.xW ? sa.xW - 1 : wg);
            v[i] = *reinterpret_cast<const uint4*>(
                xn + ((int64_t)(tg * sa.xH + hc) * sa.xW + wc) * cin + c0 + g * 8);
            in_img |= in ? (1u << i) : 0u;
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = tid + i * kMfmaThreads;
            if (u < UNITS)
                *reinterpret_cast<uint4*>(&tile[(u >> 2) * kRow + (u & 3) * 16]) =
                    ((in_img >> i) & 1u) ? v[i] : make_uint4(0, 0, 0, 0);
        }
        __syncthreads();

        bf16x8_t af[2][MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[0][i] = *reinterpret_cast<const bf16x8_t*>(&tile[a_off[i]]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int step = 0; step < 54; ++step) {
            const int tap = step >> 1, kk = step & 1;
            if (kk == 0 && tap + PD < 27) load_b((tap + PD) % NB, tap + PD, c0);
            if (step + 1 < 54) {
                const int nt2 = (step + 1) >> 1, nk = (step + 1) & 1;
                const int kt = nt2 / 9, kh = (nt2 / 3) % 3, kw = nt2 % 3;
                const int off = ((kt * S::FH + kh) * S::FW + kw) * kRow + nk * 32;
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    af[(step + 1) & 1][i] =
                        *reinterpret_cast<const bf16x8_t*>(&tile[a_off[i] + off]);
            }
            const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, bq[tap % NB][kk]);
#pragma unroll
            for (int i = 0; i < MI; ++i) acc[i] = mfma_step<F16>(af[step & 1][i], bf, acc[i]);
            if (kk == 0 && tap + PD < 27) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (step + 1 < 54) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (F16) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] *= kF16WeightUnscale;
    }
    __syncthreads();   // the tile is reused for the epilogue
    conv_epilogue<TO, HB, WB, MI, MW, WM>(a, acc, reinterpret_cast<float*>(tile) + wave * 32 * kEp,
                                          n, t_blk, h_blk, w_blk, bt_i, bh_i, bw_i, co_tile, lane,
                                          wave_m);
}

// One thread per (output position, output channel), fp32 accumulation.
template <typename TX, typename TW, typename TO>
__global__ __launch_bounds__(256) void conv3d_strided_direct_kernel(
    const TX* __restrict__ x, const TW* __restrict__ w, const float* __restrict__ bias,
    const TO* res, TO* y, int32_t N, int32_t xT, int32_t xH, int32_t xW, int32_t yT, int32_t yH,
    int32_t yW, int32_t cin, int32_t cout, int32_t st, int32_t sh, int32_t sw, int32_t pt,
    int32_t pl, Box box) {
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
    const TX* xn = x + (int64_t)n * xT * xH * xW * cin;
    for (int kt = 0; kt < 3; ++kt) {
        const int ti = std::max(st * t + kt - 2, 0);
        for (int kh = 0; kh < 3; ++kh) {
            const int hi = sh * h + kh - pt;
            if (hi < 0 || hi >= xH) continue;
            for (int kw = 0; kw < 3; ++kw) {
                const int wi = sw * ww + kw - pl;
                if (wi < 0 || wi >= xW) continue;
                const TX* xp = xn + ((int64_t)(ti * xH + hi) * xW + wi) * cin;
                const TW* wp = w + ((int64_t)co * 27 + (kt * 9 + kh * 3 + kw)) * cin;
                for (int c = 0; c < cin; ++c) acc += Elem<TX>::load(xp + c) * Elem<TW>::load(wp + c);
            }
        }
    }
    const int64_t o = ((((int64_t)n * yT + t) * yH + h) * yW + ww) * cout + co;
    if (res) acc += Elem<TO>::load(res + o);
    Elem<TO>::store(y + o, acc);
}

template <typename TX, typename TW, typename TO>
vae_status_t run_strided_direct(const vae_tensor_t& x, const void* w, const float* bias,
                                const vae_tensor_t* res, const vae_tensor_t& y, const Box& box,
                                const StrideGeom& g, hipStream_t stream) {
    const int64_t blocks = ceil_div(x.n * box.volume() * y.c, 256);
    if (blocks > INT32_MAX) return fail(VAE_ERR_UNSUPPORTED, "strided conv: grid too large");
    hipLaunchKernelGGL((conv3d_strided_direct_kernel<TX, TW, TO>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, static_cast<const TX*>(x.data),
                       static_cast<const TW*>(w), bias,
                       res ? static_cast<const TO*>(res->data) : nullptr, static_cast<TO*>(y.data),
                       (int32_t)x.n, (int32_t)x.t, (int32_t)x.h, (int32_t)x.w, (int32_t)y.t,
                       (int32_t)y.h, (int32_t)y.w, (int32_t)x.c, (int32_t)y.c, g.st, g.sh, g.sw,
                       g.pt, g.pl, box);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

template <typename TX, typename TW>
vae_status_t run_strided_direct_out(const vae_tensor_t& x, const void* w, const float* bias,
                                    const vae_tensor_t* res, const vae_tensor_t& y, const Box& box,
                                    const StrideGeom& g, hipStream_t stream) {
    if (y.dtype == VAE_DTYPE_F32)
        return run_strided_direct<TX, TW, float>(x, w, bias, res, y, box, g, stream);
    return run_strided_direct<TX, TW, uint16_t>(x, w, bias, res, y, box, g, stream);
}

template <int NT, typename TI, typename TO, int ST, int SS>
vae_status_t run_strided_mfma(const vae_tensor_t& x, const void* w, const float* bias,
                              const vae_tensor_t* res, const vae_tensor_t& y, const Box& box,
                              const StrideGeom& g, const ConvFuse* fz, hipStream_t stream) {
    StridedArgs sa{};
    MfmaArgs& a = sa.e;
    a.x = x.data;
    a.w = static_cast<const uint16_t*>(w);
    a.bias = bias;
    a.res = res ? res->data : nullptr;
    a.res_f32 = res && res->dtype == VAE_DTYPE_F32 && y.dtype != VAE_DTYPE_F32;
    a.y = y.data;
    a.T = (int32_t)y.t;
    a.H = (int32_t)y.h;
    a.W = (int32_t)y.w;
    a.cin = (int32_t)x.c;
    a.cout = (int32_t)y.c;
    a.zc = (int32_t)y.c;
    a.st = a.sh = a.sw = 1;
    a.tdrop = 0;
    a.yT = (int32_t)y.t;
    a.yH = (int32_t)y.h;
    a.yW = (int32_t)y.w;
    a.box = box;
    a.nbt = (int32_t)ceil_div(box.bt(), kSTB);
    a.nbh = (int32_t)ceil_div(box.bh(), strided_hb(NT));
    a.nbw = (int32_t)ceil_div(box.bw(), kSWB);
    const int64_t mblocks = x.n * (int64_t)a.nbt * a.nbh * a.nbw;
    const int64_t total = mblocks * ceil_div(a.cout, NT);
    if (total > INT32_MAX) return fail(VAE_ERR_UNSUPPORTED, "strided conv: grid too large");
    a.n_mblocks = (int32_t)mblocks;
    a.stats = fz ? fz->gn_ws : nullptr;
    a.groups = a.stats ? fz->groups : 1;
    // partial slots [slot0, slot0 + own) of rows slot_stride long (see ConvFuse)
    const int64_t own = (int64_t)a.nbt * a.nbh * a.nbw * wave_rows<NT>();
    const int64_t stride = fz && fz->slot_stride ? fz->slot_stride : own;
    if (a.stats && (fz->slot0 < 0 || fz->slot0 + own > stride || stride > INT32_MAX))
        return fail(VAE_ERR_INVALID_ARG, "strided conv: GroupNorm slot range outside its row");
    a.nslots = (int32_t)stride;
    a.slot0 = fz ? (int32_t)fz->slot0 : 0;
    a.splits = 1;
    sa.xT = (int32_t)x.t;
    sa.xH = (int32_t)x.h;
    sa.xW = (int32_t)x.w;
    sa.pt = g.pt;
    sa.pl = g.pl;
    hipLaunchKernelGGL((conv3d_strided_kernel<NT, TI, TO, ST, SS>), dim3((unsigned)total),
                       dim3(kMfmaThreads), 0, stream, sa);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

template <int NT, typename TI, typename TO>
vae_status_t run_strided_strides(const vae_tensor_t& x, const void* w, const float* bias,
                                 const vae_tensor_t* res, const vae_tensor_t& y, const Box& box,
                                 const StrideGeom& g, const ConvFuse* fz, hipStream_t stream) {
    if (g.st == 2 && g.sh == 2)
        return run_strided_mfma<NT, TI, TO, 2, 2>(x, w, bias, res, y, box, g, fz, stream);
    if (g.st == 1 && g.sh == 2)
        return run_strided_mfma<NT, TI, TO, 1, 2>(x, w, bias, res, y, box, g, fz, stream);
    if (g.st == 2 && g.sh == 1)
        return run_strided_mfma<NT, TI, TO, 2, 1>(x, w, bias, res, y, box, g, fz, stream);
    return run_strided_mfma<NT, TI, TO, 1, 1>(x, w, bias, res, y, box, g, fz, stream);
}

template <int NT, typename TI>
vae_status_t run_strided_out(const vae_tensor_t& x, const void* w, const float* bias,
                             const vae_tensor_t* res, const vae_tensor_t& y, const Box& box,
                             const StrideGeom& g, const ConvFuse* fz, hipStream_t stream) {
    if (y.dtype == VAE_DTYPE_F32)
        return run_strided_strides<NT, TI, float>(x, w, bias, res, y, box, g, fz, stream);
    if (y.dtype == VAE_DTYPE_F16)
        return run_strided_strides<NT, TI, _Float16>(x, w, bias, res, y, box, g, fz, stream);
    return run_strided_strides<NT, TI, uint16_t>(x, w, bias, res, y, box, g, fz, stream);
}

template <typename TI>
vae_status_t run_strided_nt(const vae_tensor_t& x, const void* w, const float* bias,
                            const vae_tensor_t* res, const vae_tensor_t& y, const Box& box,
                            const StrideGeom& g, const ConvFuse* fz, hipStream_t stream) {
    switch (conv_nt(y.c)) {
        case 128: return run_strided_out<128, TI>(x, w, bias, res, y, box, g, fz, stream);
        case 64: return run_strided_out<64, TI>(x, w, bias, res, y, box, g, fz, stream);
        default: return run_strided_out<32, TI>(x, w, bias, res, y, box, g, fz, stream);
    }
}

}  // namespace
}  // namespace mfma

using namespace mfma;

bool conv_strided_uses_mfma(const vae_tensor_t& x, int64_t cout, int32_t weight_dtype,
                            int32_t flags, const StrideGeom& g) {
    return weight_dtype == VAE_DTYPE_BF16 && x.c % kCK == 0 && cout % 4 == 0 &&
           (flags & (VAE_CONV_PACKED_WEIGHTS | VAE_CONV_PACKED_F16_WEIGHTS)) &&
           x.dtype != VAE_DTYPE_F32 && g.sh == g.sw && g.st >= 1 && g.st <= 2 && g.sh >= 1 &&
           g.sh <= 2;
}

int64_t conv_strided_gn_slots(const vae_tensor_t& y, const Box& box, int32_t groups) {
    if (groups < 1 || y.c % groups) return 0;
    const int64_t cpg = y.c / groups;
    if (cpg % 4 || 32 % cpg) return 0;
    const int wm = y.c >= 128 ? wave_rows<128>() : y.c > 32 ? wave_rows<64>() : wave_rows<32>();
    return ceil_div(box.bt(), kSTB) * ceil_div(box.bh(), strided_hb(conv_nt(y.c))) *
           ceil_div(box.bw(), kSWB) * wm;
}

vae_status_t launch_conv3d_strided(const vae_tensor_t& x, const void* w, int32_t weight_dtype,
                                   const float* bias, const vae_tensor_t* residual,
                                   const vae_tensor_t& y, const Box& box, const StrideGeom& g,
                                   int32_t flags, hipStream_t stream, const ConvFuse* fz) {
    if (box.volume() == 0 || x.n == 0) return VAE_OK;
    if (conv_strided_uses_mfma(x, y.c, weight_dtype, flags, g)) {
        if ((x.dtype == VAE_DTYPE_F16) != ((flags & VAE_CONV_PACKED_F16_WEIGHTS) != 0))
            return fail(VAE_ERR_INVALID_ARG,
                        "strided conv: an fp16 x takes fp16-packed weights, a bf16 x bf16-packed");
        if (fz && fz->gn_ws && conv_strided_gn_slots(y, box, fz->groups) == 0)
            return fail(VAE_ERR_UNSUPPORTED, "strided conv: fused statistics need 4, 8, 16 or 32 "
                                             "channels per group");
        if (x.dtype == VAE_DTYPE_F16)
            return run_strided_nt<_Float16>(x, w, bias, residual, y, box, g, fz, stream);
        return run_strided_nt<uint16_t>(x, w, bias, residual, y, box, g, fz, stream);
    }
    if (flags & (VAE_CONV_PACKED_WEIGHTS | VAE_CONV_PACKED_F16_WEIGHTS))
        return fail(VAE_ERR_UNSUPPORTED,
                    "strided conv: packed weights need a bf16 or fp16 x, Cin % 32 == 0, "
                    "Cout % 4 == 0, strides of 1 or 2 and sh == sw");
    if (fz && fz->gn_ws)
        return fail(VAE_ERR_UNSUPPORTED, "strided conv: fused statistics need the MFMA path");
    if (x.dtype == VAE_DTYPE_F16 || y.dtype == VAE_DTYPE_F16)
        return fail(VAE_ERR_UNSUPPORTED, "strided conv: fp16 tensors need the MFMA path");
    const bool xf = x.dtype == VAE_DTYPE_F32;
    if (weight_dtype == VAE_DTYPE_F32)
        return xf ? run_strided_direct_out<float, float>(x, w, bias, residual, y, box, g, stream)
                  : run_strided_direct_out<uint16_t, float>(x, w, bias, residual, y, box, g,
                                                            stream);
    return xf ? run_strided_direct_out<float, uint16_t>(x, w, bias, residual, y, box, g, stream)
              : run_strided_direct_out<uint16_t, uint16_t>(x, w, bias, residual, y, box, g,
                                                           stream);
}

}  // namespace vae
