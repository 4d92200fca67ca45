// Causal Conv3d on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, or _f16 for fp16 inputs):
// the kernel and its launch templates. Each (NT, input type, split) combination is instantiated in a source file of its
// own (conv3d_mfma_*.hip), so that they compile in parallel.
//
// Implicit GEMM:
//  - GEMM view: M = output positions, N = Cout, K = 27 * Cin, ordered (channel chunk, tap).
//  - One workgroup (4 waves) computes a block of 256 output positions for NT output channels
//    (NT = 128; 64 or 32 for narrow outputs, whose waves then split the positions 2 or 4 ways).
//    The block is TB x HB x WB positions (2x8x16, 4x8x8 or 4x4x16, whichever pads the box least).
//    Each wave owns 32 output channels and 256 * 32 / NT positions (32x32 MFMA tiles): at NT = 128
//    a wave covers all 256 positions. Each weight fragment it loads then feeds eight MFMAs. Its
//    128 accumulator registers allow two waves per SIMD, i.e. two workgroups per CU, so one
//    workgroup's tile staging overlaps the other's MFMA work.
//  - Input (A operand). For each 32-channel chunk the block's input tile is staged in LDS once:
//    (TB+2) x (HB+2) x (WB+2) positions x 32 channels, i.e. the block, a one-row halo on each
//    spatial side, and the two earlier frames. All 27 taps read their A fragments from that tile
//    at shifted offsets. The halo and the causal frame clamp are resolved while the tile is
//    loaded: the halo is the neighbouring data of the same tensor, read in place; rows outside
//    the image become zeros; a frame index below 0 reads frame 0. The pages motivate this: a halo
//    built by concatenation cost 1.31x ("[TRTLLM-14123][feat] add ParallelVAE_TrtllmWan for native
//    Wan VAE", Description). LDS rows are padded from 64 to 80 bytes, so the 16-byte reads of
//    8 consecutive lanes hit 8 distinct 16-byte bank groups.
//  - Weights (B operand). They go straight from global memory (L2-resident per XCD) into
//    registers in MFMA fragment order, prefetched two taps ahead. The tap loop therefore has no
//    barriers and LDS carries only A.
//  - fp32 inputs are rounded to bf16 (nearest-even) as they are staged, because MFMA operands are
//    bf16. Accumulation is fp32. With the split flag an fp32 input is applied as two bf16
//    operands, hi = bf16(x) and lo = bf16(x - hi), so about 16 significant bits of x reach the
//    matrix cores and the MFMA work doubles. A chunk then holds 16 channels: its LDS row carries
//    their hi halves in the first 32 bytes and their lo halves in the next 32. The two k steps of
//    a tap read hi and lo against the same weight fragment. Each fp32 value is loaded once, and
//    the weight loads per MFMA halve.
//  - fp16 inputs (the operand hand-off of convs that read an fp32 stream) stage as they are and
//    run v_mfma_f32_32x32x16_f16 at the bf16 rate: 11 significant bits of x reach the matrix
//    cores, against 8 for bf16 and 16 for the split at twice the work. The bf16 weights become
//    fp16 exactly after a 2^10 scale (packed that way ahead of time, or converted as each
//    fragment is used with the standard layout); the sums are scaled back by 2^-10 before the
//    epilogue, which is exact.
//  - A GroupNorm + SiLU of the input can be applied while staging: the conv then reads the
//    norm's input x (fp32 or fp16) and stages bf16(silu(x * scale_c + shift_c)) (or fp16, for a
//    conv on fp16 operands), with a per-(sample, channel) scale and shift formed from the norm's
//    statistics, gamma and beta. The operand is the value a separate normalisation pass would have
//    stored, computed the same way, so the result is the same; the normalised tensor is never
//    written or read back. Image padding stays zero (it pads the normalised tensor).
//  - Epilogue. Where a wave's 32 channels are 32 consecutive channels of y (Cout and y's channel
//    count multiples of 32), each lane stores its accumulator registers directly: one channel at
//    16 positions, two runs of 32 channels per store instruction. Otherwise each wave parks one
//    32 x 32 tile at a time in LDS (reusing the input tile) and every lane writes four
//    consecutive channels with one 16-byte (fp32) or 8-byte (bf16) store. Bias, residual,
//    depth-to-space placement and GroupNorm partials are done on the way.
//  - Workgroups are ordered output-channel tile slowest, and remapped so that each XCD (the
//    hardware deals workgroup i to XCD i % 8) runs a contiguous range of them. An XCD then keeps
//    one weight slice in its own L2 while it streams input blocks.
#pragma once

#include <type_traits>

#include "kernels.h"

namespace vae {
namespace mfma {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// fp16 weight operands are the bf16 weights times 2^10 (exact for |w| < 64); the fp32 sums are
// multiplied by 2^-10 before the epilogue.
constexpr float kF16WeightScale = 1024.0f;
constexpr float kF16WeightUnscale = 1.0f / 1024.0f;

__host__ __device__ inline uint16_t f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// 8 bf16 weights (one B fragment of the standard layout) as 8 scaled fp16 weights.
__device__ __forceinline__ uint4 bf16x8_to_f16x8_scaled(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16) * kF16WeightScale;
        const float hi = __uint_as_float(w[i] & 0xffff0000u) * kF16WeightScale;
        o[i] = (uint32_t)f16_bits(lo) | ((uint32_t)f16_bits(hi) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// One 32x32x16 MFMA step; a and b carry 8 bf16 or 8 fp16 values.
template <bool F16>
__device__ __forceinline__ f32x16_t mfma_step(const bf16x8_t& a, const bf16x8_t& b,
                                              const f32x16_t& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kCK = 32;                              // input channels per LDS chunk
constexpr int kRow = kCK * 2 + 16;                   // padded LDS row, bytes
constexpr int kMfmaWaves = 4;                        // waves per workgroup
constexpr int kMfmaThreads = kMfmaWaves * 64;
constexpr int kXcds = 8;

struct MfmaArgs {
    const void* x;
    const uint16_t* w;
    const float* bias;
    const void* res;
    void* y;
    // The conv's input grid is T x H x W. With a nearest upsampling folded into the staging
    // (lsh, lsw = log2 of its factors, 0 = none), x holds the T x (H >> lsh) x (W >> lsw) tensor
    // and input position (h, w) reads x at (h >> lsh, w >> lsw).
    int32_t T, H, W, cin, cout;
    int32_t lsh, lsw;
    Box box;
    int32_t nbt, nbh, nbw;   // blocks along each box axis
    int32_t n_mblocks;       // N * nbt * nbh * nbw
    // Output mapping. y may be the depth-to-space (st, sh, sw) of the conv output: conv channel
    // ((dt*sh + dh)*sw + dw)*zc + c at (t, h, w) lands at channel c of y position
    // (st*t + dt - tdrop, sh*h + dh, sw*w + dw); frames below 0 are dropped. tdrop is st - 1 (the
    // causal drop of the first frames), plus st times the leading frames of an input whose
    // first frames are only causal context (a clip's carried frames). Identity: st = sh = sw = 1,
    // tdrop = 0 and zc = cout. The residual, if any, has y's shape.
    int32_t yT, yH, yW, zc, st, sh, sw, tdrop;
    int32_t res_f32;         // the residual is fp32 while y is bf16 or fp16 (a hand-off)
    // Optional GroupNorm partials of y as stored: fp64 (count, mean, M2) per (sample, group of
    // y's channels, slot), slot = slot0 + (sub-position * position blocks + block) * WM + wave
    // row, in rows of nslots slots per (sample, group). slot0 > 0 and nslots above this launch's
    // own count let several launches (one per patch box) fill one array.
    double* stats;
    int32_t groups, nslots, slot0;
    // Split over K. With splits > 1 the grid holds `splits` copies of the (channel tile, block)
    // grid, split s taking the input-channel chunks [s * chunks / splits, (s + 1) * chunks /
    // splits); each workgroup stores its raw fp32 accumulators to `part` and stops. Then
    // conv3d_reduce_kernel, with `reduce` = that array, adds the splits' accumulators in split
    // order and runs the epilogue. Layout: [split][tile][wave][MFMA tile][lane][16].
    int32_t splits;
    float* part;
    const float* reduce;
    // Input GroupNorm + SiLU applied while staging (input tags below): fp32 (scale, shift) per
    // (sample, input channel), [N][cin][2].
    const float* nab;
};

// Input kinds. A plain element type stages as it is (bf16, fp16) or rounded to bf16 (fp32). The
// tags read fp32 or fp16 and stage silu(x * scale + shift) as bf16 (GnF32, GnF16) or as fp16
// (GnF32H, for fp16 weights).
struct GnF32 {};
struct GnF16 {};
struct GnF32H {};
template <typename TI> struct InT {
    using raw = TI;                                       // element type in memory
    static constexpr bool f16op = std::is_same<TI, _Float16>::value;   // fp16 MFMA operands
    static constexpr bool norm = false;
};
template <> struct InT<GnF32> {
    using raw = float;
    static constexpr bool f16op = false;
    static constexpr bool norm = true;
};
template <> struct InT<GnF16> {
    using raw = _Float16;
    static constexpr bool f16op = false;
    static constexpr bool norm = true;
};
template <> struct InT<GnF32H> {
    using raw = float;
    static constexpr bool f16op = true;
    static constexpr bool norm = true;
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    int per = total / kXcds;
    int full = per * kXcds;
    if (bid >= full) return bid;
    return (bid % kXcds) * per + bid / kXcds;
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
template <> __device__ __forceinline__ void load4<_Float16>(const _Float16* p, float* v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = (float)p[k];
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

template <> __device__ __forceinline__ void store4<_Float16>(_Float16* p, const float* v) {
    uint2 a;
    a.x = (uint32_t)f16_bits(v[0]) | ((uint32_t)f16_bits(v[1]) << 16);
    a.y = (uint32_t)f16_bits(v[2]) | ((uint32_t)f16_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = a;
}

// The value an output element holds once stored.
template <typename TO> __device__ __forceinline__ float stored(float v);
template <> __device__ __forceinline__ float stored<float>(float v) { return v; }
template <> __device__ __forceinline__ float stored<uint16_t>(float v) {
    return bf16_to_f32(f32_to_bf16(v));
}
template <> __device__ __forceinline__ float stored<_Float16>(float v) {
    return (float)(_Float16)v;
}

// Chan's pairwise update of (count, mean, M2) with another partial, in fp32.
__device__ __forceinline__ void chan_merge_f32(float& n, float& mean, float& m2, float nb,
                                               float mb, float m2b) {
    const float t = n + nb;
    if (nb > 0.0f && n > 0.0f) {
        const float d = mb - mean;
        mean += d * (nb / t);
        m2 += m2b + d * d * (n * nb / t);
    } else if (nb > 0.0f) {
        mean = mb;
        m2 = m2b;
    }
    n = t;
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1, each a separate instantiation.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Raw input of one staging unit: 8 input channels (16 bytes of bf16, 32 of fp32).
template <typename TI> struct Raw8 {
    uint4 v[sizeof(TI) / 2];
};
template <typename TI> __device__ __forceinline__ Raw8<TI> load_raw8(const TI* p) {
    Raw8<TI> r;
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(TI) / 2); ++i) r.v[i] = q[i];
    return r;
}
// Operand granule(s) of a unit: bf16 as is; fp32 rounded to bf16, or split into hi and lo.
// A unit outside the image (in == false) is zero padding.
// Operand granule of a normalised unit: silu(x * sc + sh) for each of the 8 channels, rounded
// to bf16 (or fp16 with F16OP) exactly as the separate normalisation pass stores it.
template <typename TR, bool F16OP>
__device__ __forceinline__ uint4 norm_operand(const Raw8<TR>& r, bool in, const float (&sc)[8],
                                              const float (&sh)[8]) {
    float v[8];
    if constexpr (sizeof(TR) == 2) {
        const _Float16* h = reinterpret_cast<const _Float16*>(&r.v[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
    } else {
        const float* f = reinterpret_cast<const float*>(&r.v[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = f[i];
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float z0 = gn_silu_apply(v[2 * i], sc[2 * i], sh[2 * i]);
        const float z1 = gn_silu_apply(v[2 * i + 1], sc[2 * i + 1], sh[2 * i + 1]);
        if constexpr (F16OP)   // rounded to fp32 first, as the normalise pass stores it
            o[i] = (uint32_t)f16_bits(materialise_f32(z0)) |
                   ((uint32_t)f16_bits(materialise_f32(z1)) << 16);
        else
            o[i] = (uint32_t)f32_to_bf16(z0) | ((uint32_t)f32_to_bf16(z1) << 16);
    }
    return in ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(0, 0, 0, 0);
}

// norm_operand with the scale and shift read from LDS (tab: 8 channels' (scale, shift) pairs),
// two channels at a time, each read volatile so that it is issued where it is used.
template <typename TR, bool F16OP>
__device__ __forceinline__ uint4 norm_operand_lds(const Raw8<TR>& r, bool in, const float* tab) {
    float v[8];
    if constexpr (sizeof(TR) == 2) {
        const _Float16* h = reinterpret_cast<const _Float16*>(&r.v[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
    } else {
        const float* f = reinterpret_cast<const float*>(&r.v[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = f[i];
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 p = *reinterpret_cast<const volatile f32x4*>(tab + 4 * i);
        const float z0 = gn_silu_apply(v[2 * i], p.x, p.y);
        const float z1 = gn_silu_apply(v[2 * i + 1], p.z, p.w);
        if constexpr (F16OP)
            o[i] = (uint32_t)f16_bits(materialise_f32(z0)) |
                   ((uint32_t)f16_bits(materialise_f32(z1)) << 16);
        else
            o[i] = (uint32_t)f32_to_bf16(z0) | ((uint32_t)f32_to_bf16(z1) << 16);
    }
    return in ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(0, 0, 0, 0);
}

// This thread's scale and shift for 8 channels from c (of sample n): [N][cin][2] fp32.
__device__ __forceinline__ void load_norm8(const float* nab, int64_t n, int64_t cin, int c,
                                           float (&sc)[8], float (&sh)[8]) {
    const float4* q = reinterpret_cast<const float4*>(nab + (n * cin + c) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = q[i];
        sc[2 * i] = v.x;
        sh[2 * i] = v.y;
        sc[2 * i + 1] = v.z;
        sh[2 * i + 1] = v.w;
    }
}

template <typename TI, bool SPLIT>
__device__ __forceinline__ void to_operand(const Raw8<TI>& r, bool in, uint4& hi, uint4& lo) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    lo = z;
    if constexpr (sizeof(TI) == 2) {
        hi = in ? r.v[0] : z;
    } else {
        float v[8] = {__uint_as_float(r.v[0].x), __uint_as_float(r.v[0].y),
                      __uint_as_float(r.v[0].z), __uint_as_float(r.v[0].w),
                      __uint_as_float(r.v[1].x), __uint_as_float(r.v[1].y),
                      __uint_as_float(r.v[1].z), __uint_as_float(r.v[1].w)};
        uint32_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
            h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            if constexpr (SPLIT) {
                const uint16_t l0 = f32_to_bf16(v[2 * i] - bf16_to_f32(h0));
                const uint16_t l1 = f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1));
                l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
        }
        hi = in ? make_uint4(h[0], h[1], h[2], h[3]) : z;
        if constexpr (SPLIT) lo = in ? make_uint4(l[0], l[1], l[2], l[3]) : z;
    }
}

// Staged input tile: (TB+2) x (HB+2) rows of (WB+2) positions, 80 bytes per position. The row
// pitch is chosen for conflict-free 16-byte A-fragment reads. A fragment read covers
//  - 16 positions of one row plus 16 of the next (WB = 16), or
//  - 8 positions of each of four rows (WB = 8).
// Measured with the LDS bank-conflict counter on gfx950, such reads are conflict-free only when
// the row pitch is 0 mod 256 bytes (WB = 16) or 128 mod 256 bytes (WB = 8): the 16-byte reads of
// 8 consecutive lanes must land in 8 distinct 16-byte groups of a 256-byte line. The pitch is
// 1536 or 896 bytes. The same rule gives the narrow blocks theirs: 8 lanes read 4 positions of
// 2 rows (WB = 4; columns land in groups 0, 5, 10, 15, so the next row must shift them by 8:
// pitch 128 mod 256, 640 bytes) or 2 positions of 4 rows (WB = 2; groups 0, 5, shifted by 4 per
// row: pitch 64 mod 256, 320 bytes).
template <int TB, int HB, int WB>
struct BlockShape {
    static_assert(TB * HB * WB == 256, "a block is 256 output positions");
    static constexpr int HT = TB + 2, HH = HB + 2, HW = WB + 2;
    static constexpr int kPos = HT * HH * HW;       // input positions staged per chunk
    static constexpr int kPitch = WB == 16 ? 1536 : WB == 8 ? 896 : WB == 4 ? 640 : 320;
    static_assert(HW * kRow <= kPitch, "a row must fit its pitch");
    static constexpr int kBytes = HT * HH * kPitch;
};

// Epilogue of one block. In a 32x32 accumulator tile, lane l holds column l % 32 and register r
// holds row (r / 4) * 8 + (l / 32) * 4 + r % 4. Each wave parks one 32 x 32 tile at a time in its
// LDS slice `ep` (32 rows of kEp floats), then reads rows back four channels per lane: bias,
// residual, the store (optionally at its depth-to-space position) and GroupNorm partials.
constexpr int kEp = 32 + 4;                         // padded staging row, floats
template <typename TO, int HB, int WB, int MI, int MW, int WM>
__device__ __forceinline__ void conv_epilogue(const MfmaArgs& a, const f32x16_t (&acc)[MI],
                                              float* ep, int n, int t_blk, int h_blk, int w_blk,
                                              int bt_i, int bh_i, int bw_i, int co_tile, int lane,
                                              int wave_m) {
    constexpr int EP = kEp;
    constexpr int LPR = 8;                          // lanes per staged row
    constexpr int RPP = 64 / LPR;                   // rows per pass
    const int lrow = lane & 31, khalf = lane >> 5;
    const TO* res = static_cast<const TO*>(a.res);
    const float* res32 = static_cast<const float*>(a.res);   // when a.res_f32
    TO* y = static_cast<TO*>(a.y);
    const int c4 = (lane % LPR) * 4;
    const int co = co_tile + c4;
    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a.bias)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (co + k < a.cout) bv[k] = a.bias[co + k];
    // Where this lane's four channels go in y. The sw * zc conv channels of one (dt, dh) are
    // consecutive elements of one y row (dw, then c). When that count is a multiple of 4, a
    // lane's aligned four channels stay together and are stored as one vector; otherwise each
    // channel is placed on its own.
    const int rowc = a.sw * a.zc;
    const bool vec = rowc % 4 == 0;
    const int srow = co / rowc, rem = co - srow * rowc;
    const int sdh = srow % a.sh, sdt = srow / a.sh;
    const int sub = co / a.zc, cz = co - sub * a.zc;   // sub-position and channel of y
    auto y_off = [&](int t, int h, int w, int s_dt, int s_dh, int r) -> int64_t {
        const int to = a.st * t + s_dt - a.tdrop;
        if (to < 0) return -1;   // causal drop
        return ((((int64_t)n * a.yT + to) * a.yH + a.sh * h + s_dh) * a.yW + (int64_t)a.sw * w) *
                   a.zc + r;
    };
    // GroupNorm partials of this lane's four channels (one group): shifted sums, shift = the
    // lane's first stored value.
    float sn = 0.0f, sk = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ep[((r >> 2) * 8 + khalf * 4 + (r & 3)) * EP + lrow] = acc[i][r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int pass = 0; pass < 32 / RPP; ++pass) {
            const int row = pass * RPP + lane / LPR;
            const int m = wave_m * MW + i * 32 + row;
            const int t = t_blk + m / (HB * WB);
            const int h = h_blk + (m / WB) % HB, w = w_blk + m % WB;
            if (t < a.box.t1 && h < a.box.h1 && w < a.box.w1 && co < a.cout) {
                const int nv = a.cout - co < 4 ? a.cout - co : 4;
                float v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = ep[row * EP + c4 + k] + bv[k];
                if (vec) {
                    const int64_t o = y_off(t, h, w, sdt, sdh, rem);
                    if (o >= 0) {
                        if (nv == 4) {
                            if (res) {
                                float rv[4];
                                if (a.res_f32) load4<float>(res32 + o, rv);
                                else load4<TO>(res + o, rv);
#pragma unroll
                                for (int k = 0; k < 4; ++k) v[k] += rv[k];
                            }
                            store4<TO>(y + o, v);
                        } else {
                            for (int k = 0; k < nv; ++k) {
                                if (res)
                                    v[k] += a.res_f32 ? res32[o + k] : Elem<TO>::load(res + o + k);
                                Elem<TO>::store(y + o + k, v[k]);
                            }
                        }
                        if (a.stats) {
#pragma unroll
                            for (int k = 0; k < 4; ++k) {
                                if (k < nv) {
                                    const float q = stored<TO>(v[k]);
                                    sk = sn == 0.0f ? q : sk;
                                    const float d = q - sk;
                                    s1 += d;
                                    s2 = fmaf(d, d, s2);
                                    sn += 1.0f;
                                }
                            }
                        }
                    }
                } else {
                    for (int k = 0; k < nv; ++k) {
                        const int ck = co + k, rk = ck / rowc;
                        const int64_t o = y_off(t, h, w, rk / a.sh, rk % a.sh, ck - rk * rowc);
                        if (o < 0) continue;
                        if (res) v[k] += a.res_f32 ? res32[o] : Elem<TO>::load(res + o);
                        Elem<TO>::store(y + o, v[k]);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (a.stats) {
        // lane -> (count, mean, M2); then merge the 8 lanes that hold the same four channels
        // (lane ^ 8, 16, 32) and the lanes of one group (cpg / 4 neighbours), in a fixed order.
        float mean = 0.0f, m2 = 0.0f;
        if (sn > 0.0f) {
            const float mk = s1 / sn;
            mean = sk + mk;
            m2 = fmaxf(s2 - s1 * mk, 0.0f);
        }
        const int cpg = a.zc / a.groups;
#pragma unroll
        for (int off = 8; off < 64; off <<= 1) {
            const float nb = __shfl_xor(sn, off), mb = __shfl_xor(mean, off),
                        m2b = __shfl_xor(m2, off);
            chan_merge_f32(sn, mean, m2, nb, mb, m2b);
        }
        for (int off = 1; off < cpg / 4; off <<= 1) {
            const float nb = __shfl_xor(sn, off), mb = __shfl_xor(mean, off),
                        m2b = __shfl_xor(m2, off);
            chan_merge_f32(sn, mean, m2, nb, mb, m2b);
        }
        if (lane < LPR && lane % (cpg / 4) == 0 && co < a.cout) {
            const int g = cz / cpg;
            const int nblk = a.nbt * a.nbh * a.nbw;
            const int mb_local = (bt_i * a.nbh + bh_i) * a.nbw + bw_i;
            const int64_t slot = a.slot0 + ((int64_t)sub * nblk + mb_local) * WM + wave_m;
            double* o = a.stats + (((int64_t)n * a.groups + g) * a.nslots + slot) * 3;
            o[0] = sn;
            o[1] = mean;
            o[2] = m2;
        }
    }
}

// Epilogue straight from the accumulator registers, for outputs where a wave tile's 32 channels
// are 32 consecutive channels of one y position (zc and Cout multiples of 32): no LDS round trip.
// Lane l stores channel co_tile + l % 32 of the 16 positions its registers hold, so one store
// instruction writes two runs of 32 channels.
//
// The 16 rows of a lane's 32x32 tile, (r / 4) * 8 + (l / 32) * 4 + r % 4 past the tile's first
// row, lie in one frame of the block: with WB = 16 they are columns +0..3 and +8..11 of two
// consecutive rows, with WB = 8 columns +0..3 of four consecutive rows (the tile's first row is a
// multiple of 32, so no offset carries into the next row or frame). A y offset is then a uniform
// part (block, tile, register) plus a per-lane 32-bit part (channel, k half), which the stores
// take as a scalar base and a vector offset. MASKED = false is the case of a block entirely
// inside the box with no dropped frame: no per-position test.
template <bool MASKED, typename TO, int HB, int WB, int MI, int MW, int WM>
__device__ __forceinline__ void conv_epilogue_direct_tiles(
    const MfmaArgs& a, const f32x16_t (&acc)[MI], int n, int t_blk, int h_blk, int w_blk,
    int sub, int cz, float bv, int khalf, int wave_m, float& sn, float& sk, float& s1, float& s2) {
    static_assert(WB == 16 || WB == 8, "direct epilogue row pattern");
    static_assert(MW % 32 == 0, "tiles start at multiples of 32 rows");
    const int sdw = sub % a.sw, sdh = (sub / a.sw) % a.sh, sdt = sub / (a.sw * a.sh);
    const int64_t stride_t = (int64_t)a.st * a.yH * a.yW * a.zc;
    const int64_t stride_h = (int64_t)a.sh * a.yW * a.zc;
    const int64_t stride_w = (int64_t)a.sw * a.zc;
    const int to_blk = a.st * t_blk + sdt - a.tdrop;
    // uniform offset of the block's first position (at sub-position `sub`, channel 0 of y)
    const int64_t blk = ((((int64_t)n * a.yT + to_blk) * a.yH + (int64_t)a.sh * h_blk + sdh) *
                             a.yW + (int64_t)a.sw * w_blk + sdw) * a.zc;
    const uint32_t lane_b = (uint32_t)((khalf * 4 * stride_w + cz) * (int64_t)sizeof(TO));
    char* yb = reinterpret_cast<char*>(a.y);
    const char* rb = reinterpret_cast<const char*>(a.res);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int mi = wave_m * MW + i * 32;                 // uniform first row of the tile
        const int tl = mi / (HB * WB), hl = (mi / WB) % HB, wl = mi % WB;
        const int64_t di = blk + tl * stride_t + hl * stride_h + wl * stride_w;
        int64_t d[16];                                        // uniform, elements
        bool ok[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dh = WB == 16 ? r >> 3 : r >> 2;
            const int dw = WB == 16 ? ((r >> 2) & 1) * 8 + (r & 3) : r & 3;
            d[r] = di + dh * stride_h + dw * stride_w;
            ok[r] = !MASKED || (t_blk + tl < a.box.t1 && to_blk + a.st * tl >= 0 &&
                                h_blk + hl + dh < a.box.h1 &&
                                w_blk + wl + khalf * 4 + dw < a.box.w1);
        }
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = acc[i][r] + bv;
        if (rb) {
            // all 16 loads in flight at once; masked positions read the tensor's first element
            float rv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const char* q = rb + d[r] * (a.res_f32 ? 4 : (int64_t)sizeof(TO)) +
                                (a.res_f32 ? lane_b / sizeof(TO) * 4 : lane_b);
                if (MASKED && !ok[r]) q = rb;
                rv[r] = a.res_f32 ? *reinterpret_cast<const float*>(q)
                                  : Elem<TO>::load(reinterpret_cast<const TO*>(q));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] += rv[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (ok[r])
                Elem<TO>::store(reinterpret_cast<TO*>(yb + d[r] * (int64_t)sizeof(TO) + lane_b),
                                v[r]);
        if (a.stats) {
            // shifted sums of the values as stored; shift = this lane's first stored value
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float q = stored<TO>(v[r]);
                if (MASKED) {
                    sk = (sn == 0.0f && ok[r]) ? q : sk;
                    const float dq = ok[r] ? q - sk : 0.0f;
                    s1 += dq;
                    s2 = fmaf(dq, dq, s2);
                    sn += ok[r] ? 1.0f : 0.0f;
                } else {
                    if (i == 0 && r == 0) sk = q;
                    const float dq = q - sk;
                    s1 += dq;
                    s2 = fmaf(dq, dq, s2);
                }
            }
            if (!MASKED) sn += 16.0f;
        }
    }
}

template <typename TO, int TB, int HB, int WB, int MI, int MW, int WM>
__device__ __forceinline__ void conv_epilogue_direct(const MfmaArgs& a, const f32x16_t (&acc)[MI],
                                                     int n, int t_blk, int h_blk, int w_blk,
                                                     int bt_i, int bh_i, int bw_i, int co_tile,
                                                     int lane, int wave_m) {
    // Cout is a multiple of 32: a wave's 32 channels are all stored or all past Cout
    if (co_tile >= a.cout) return;
    const int lrow = lane & 31, khalf = lane >> 5;
    const int co = co_tile + lrow;
    const float bv = a.bias ? a.bias[co] : 0.0f;
    // the wave's 32 channels share one sub-position of the depth-to-space mapping
    const int sub = co_tile / a.zc, cz = co - sub * a.zc;
    const int sdt = sub / (a.sw * a.sh);
    float sn = 0.0f, sk = 0.0f, s1 = 0.0f, s2 = 0.0f;
    const bool inside = t_blk + TB <= a.box.t1 && h_blk + HB <= a.box.h1 &&
                        w_blk + WB <= a.box.w1 && a.st * t_blk + sdt - a.tdrop >= 0;
    if (inside)
        conv_epilogue_direct_tiles<false, TO, HB, WB, MI, MW, WM>(
            a, acc, n, t_blk, h_blk, w_blk, sub, cz, bv, khalf, wave_m, sn, sk, s1, s2);
    else
        conv_epilogue_direct_tiles<true, TO, HB, WB, MI, MW, WM>(
            a, acc, n, t_blk, h_blk, w_blk, sub, cz, bv, khalf, wave_m, sn, sk, s1, s2);
    if (a.stats) {
        // lane -> (count, mean, M2); merge the two lanes of one channel (lane ^ 32), then the
        // cpg lanes of one group, in a fixed order
        float mean = 0.0f, m2 = 0.0f;
        if (sn > 0.0f) {
            const float mk = s1 / sn;
            mean = sk + mk;
            m2 = fmaxf(s2 - s1 * mk, 0.0f);
        }
        const int cpg = a.zc / a.groups;
        for (int off = 32; off >= 1; off >>= 1) {
            if (off < 32 && off >= cpg) continue;
            const float nb = __shfl_xor(sn, off), mb = __shfl_xor(mean, off),
                        m2b = __shfl_xor(m2, off);
            chan_merge_f32(sn, mean, m2, nb, mb, m2b);
        }
        if (lane < 32 && lane % cpg == 0) {
            const int g = cz / cpg;
            const int nblk = a.nbt * a.nbh * a.nbw;
            const int mb_local = (bt_i * a.nbh + bh_i) * a.nbw + bw_i;
            const int64_t slot = a.slot0 + ((int64_t)sub * nblk + mb_local) * WM + wave_m;
            double* o = a.stats + (((int64_t)n * a.groups + g) * a.nslots + slot) * 3;
            o[0] = sn;
            o[1] = mean;
            o[2] = m2;
        }
    }
}

template <int NT, typename TI, typename TO, bool SPLIT, bool PACKED, int TB, int HB, int WB>
__global__ __launch_bounds__(kMfmaThreads, 2)
void conv3d_mfma_kernel(MfmaArgs a) {
    using S = BlockShape<TB, HB, WB>;
    using TR = typename InT<TI>::raw;                         // the input's element type
    constexpr bool F16 = InT<TI>::f16op;                      // fp16 operands
    constexpr bool NORM = InT<TI>::norm;                      // GroupNorm + SiLU while staging
    static_assert(!(F16 && SPLIT) && !(NORM && SPLIT), "fp16 or normalised inputs are not split");
    constexpr int HH = S::HH, HW = S::HW;
    constexpr int RP = S::kPitch;
    // With packed weights and bf16 (or split) operands the tile is staged through a ring of frame
    // slots (see below); otherwise through one tile buffer. The ring's extra registers fit two
    // waves per SIMD in those cases. Its schedule is written for blocks of 2 or 4 frames, and on
    // a narrow block (4 x 16 x 4) it needs more than half the registers of a SIMD: the narrow
    // blocks stage through the tile buffer. So does a normalised input of 4-byte values (twice
    // the raw registers of a 2-byte one), and any normalised input at NT = 128: the norm's
    // arithmetic needs registers that the ring leaves free only beside 64-channel tiles (at
    // NT = 128 it spills).
    constexpr bool ROLL = PACKED && (sizeof(TR) == 2 || SPLIT) && TB <= 4 && WB >= 8 &&
                          !(NORM && NT > 64);
    constexpr int NSP = TB == 2 ? 1 : 2;           // spare frame slots of the ring
    constexpr int NS = S::HT + NSP;                // frame slots of the ring
    constexpr int FB = HH * RP;                    // bytes of one frame slot
    constexpr int kSink = ROLL ? NS * FB : S::kBytes;   // 64 bytes absorbing padding units
    __shared__ __attribute__((aligned(16))) uint8_t halo[kSink + (ROLL ? 64 : 0)];
    // A normalised input on the ring: each chunk's (scale, shift) table (32 channels x 2 fp32)
    // in a ring of three, chunk c in slot c % 3, written two chunks ahead.
    __shared__ __attribute__((aligned(16))) float ntab[ROLL && NORM ? 3 * 64 : 1];

    // WNN waves across the NT output channels (32 each), WM across the 256 positions.
    constexpr int WNN = NT / 32;
    constexpr int WM = kMfmaWaves / WNN;
    constexpr int MW = 256 / WM;       // positions per wave
    constexpr int MI = MW / 32;        // 32-row MFMA tiles per wave
    constexpr int PD = 2;              // weight fragments are prefetched PD taps ahead
    constexpr int NB = PD + 1;
    static_assert(WNN * WM == kMfmaWaves && MI >= 1, "wave grid");

    // Uniform block indices, kept in scalar registers (readfirstlane): the vector registers are
    // all taken by the accumulators, fragments and staging.
    const int logical = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, gridDim.x));
    // a split launch holds `splits` copies of the (channel tile, block) grid, split slowest
    const int per_split = (int)gridDim.x / a.splits;
    const int split = __builtin_amdgcn_readfirstlane(logical / per_split);
    const int tile = __builtin_amdgcn_readfirstlane(logical - split * per_split);
    const int nt = __builtin_amdgcn_readfirstlane(tile / a.n_mblocks);
    // block order within a channel tile: T fastest, so that the workgroups an XCD runs at once
    // are temporal neighbours, which stage 2 of their TB + 2 frames in common (hits in its L2)
    int mb = tile - nt * a.n_mblocks;
    const int bt_i = mb % a.nbt;
    mb /= a.nbt;
    const int bw_i = mb % a.nbw;
    mb /= a.nbw;
    const int bh_i = mb % a.nbh;
    const int n = mb / a.nbh;
    const int t_blk = a.box.t0 + bt_i * TB;
    const int h_blk = a.box.h0 + bh_i * HB;
    const int w_blk = a.box.w0 + bw_i * WB;
    const int n_blk = nt * NT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave / WNN;    // which MW of the block's 256 positions
    const int wave_n = wave % WNN;    // which 32 of the NT output channels
    const int lrow = lane & 31;
    const int khalf = lane >> 5;      // which 8 of the 16 k values this lane feeds

    const int64_t cin = a.cin;
    const int xH = a.H >> a.lsh, xW = a.W >> a.lsw;      // x's own extents
    const TR* xn = static_cast<const TR*>(a.x) + (int64_t)n * a.T * xH * xW * cin;

    f32x16_t acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    // LDS byte offset of this lane's A row (tap 0,0,0) in each of the MI sub-tiles
    int a_off[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int m = wave_m * MW + i * 32 + lrow;
        const int tb = m / (HB * WB), hb = (m / WB) % HB, wb = m % WB;
        a_off[i] = (tb * HH + hb) * RP + wb * kRow + khalf * 16;
    }
    // This lane's weights: B column lrow of the wave's 32-channel tile, k half `khalf`.
    // Standard layout [Cout][27][Cin]: 16 bytes of one weight row per fragment.
    // Packed layout (see pack_weights_kernel): the 64 lanes of a fragment read 1 KB contiguously.
    const int nch = a.cin / kCK;
    const int co_tile = n_blk + wave_n * 32;
    const bool b_ok = PACKED ? co_tile < a.cout : co_tile + lrow < a.cout;
    const uint16_t* b_ptr =
        PACKED ? a.w + (int64_t)(b_ok ? co_tile >> 5 : 0) * 27 * nch * 1024 + lrow * 16 + khalf * 8
               : a.w + (int64_t)(b_ok ? co_tile + lrow : 0) * 27 * cin + khalf * 8;
    // Weight fragments per tap: one per k step, or one for both (hi and lo) with the split.
    constexpr int KB = SPLIT ? 1 : 2;
    uint4 bq[NB][KB];
    // The B operand as the MFMA takes it: packed fp16 weights are used as loaded; standard-layout
    // bf16 weights become scaled fp16 here, after their load has landed.
    auto b_operand = [&](const uint4& q) -> bf16x8_t {
        if constexpr (F16 && !PACKED) return __builtin_bit_cast(bf16x8_t, bf16x8_to_f16x8_scaled(q));
        else return __builtin_bit_cast(bf16x8_t, q);
    };
    auto load_b = [&](int buf, int tap, int c0) {
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            // split chunks are 16 channels: the k-step half of a packed 32-channel block
            const int half = SPLIT ? (c0 >> 4) & 1 : kk;
            const int64_t off = PACKED ? ((int64_t)tap * nch + (c0 >> 5)) * 1024 + half * 512
                                       : (int64_t)tap * cin + c0 + kk * 16;
            // Unconditional: b_ptr points at valid weights even for columns past Cout, whose
            // outputs are never stored. A branch here would split the tap loop into blocks the
            // scheduler cannot overlap, and force a full wait on every prefetch.
            bq[buf][kk] = *reinterpret_cast<const uint4*>(b_ptr + off);
        }
    };

    constexpr int CK = SPLIT ? 16 : kCK;       // input channels per staged chunk
    constexpr int UPP = SPLIT ? 2 : 4;         // staging units per position (8 channels each)
    const int n_chunks = a.cin / CK;
    // this workgroup's chunks [kc0, kc1): all of them, or its split's share
    const int kc0 = __builtin_amdgcn_readfirstlane((int)((int64_t)split * n_chunks / a.splits));
    const int kc1 =
        __builtin_amdgcn_readfirstlane((int)((int64_t)(split + 1) * n_chunks / a.splits));
    if constexpr (ROLL) {
        // Ring staging. The tile's HT = TB + 2 frames live in HT of NS = HT + NSP LDS frame
        // slots: frame f of chunk c is slot (b_c + f) mod NS, and b moves back by NSP slots per
        // chunk. Taps kt = 0, 1, 2 read frames kt .. kt + TB - 1, so frame 0's slot frees after
        // phase 0 and frame 1's after phase 1. While chunk c runs, the next chunk's frames are
        // loaded into registers and written into free slots:
        //  - frames 0 .. NSP - 1 into the spare slots (anytime);
        //  - frame NSP into frame 0's slot (after phase 0);
        //  - frame NSP + 1 into frame 1's slot (after phase 1);
        //  - the remaining NHOLD frames at the start of the next chunk, into slots its first phase
        //    does not read; they become visible at its phase-0 barrier.
        // One barrier per phase; no chunk waits for its own loads.
        constexpr int NIN = NSP + 2;                       // next frames written in the chunk
        constexpr int NHOLD = S::HT - NIN;                 // next frames held into the chunk
        static_assert(NHOLD == 1 || NHOLD == 2, "ring schedule");
        static_assert(NIN >= TB, "the next chunk's first phase must be staged in time");
        constexpr int FPOS = HH * HW;                     // positions per frame
        constexpr int FUN = FPOS * UPP;                   // staging units per frame
        constexpr int FST = (FUN + kMfmaThreads - 1) / kMfmaThreads;
        int fu_pos[FST], fu_lds[FST];
#pragma unroll
        for (int i = 0; i < FST; ++i) {
            int u = tid + i * kMfmaThreads;
            const bool valid = u < FUN;
            u = valid ? u : FUN - 1;
            const int pos = u / UPP, g = u % UPP;
            const int r = pos / HW, c = pos % HW;
            fu_pos[i] = r | (c << 8) | (g << 16) | (valid ? 0 : 1 << 30);
            fu_lds[i] = r * RP + c * kRow + g * 16;
        }
        Raw8<TR> fst[2][FST];                             // [1] only for a second held frame
        uint32_t fin[2] = {0, 0};                         // bit i: unit i inside the image
        auto frame_load = [&](int f, int c0, int reg) {
            int tg = t_blk - 2 + f;
            tg = tg < 0 ? 0 : (tg >= a.T ? a.T - 1 : tg);   // causal clamp; past T is not stored
#pragma unroll
            for (int i = 0; i < FST; ++i) {
                const int q = fu_pos[i];
                const int r = q & 255, c = (q >> 8) & 255, g = (q >> 16) & 3;
                const int hg = h_blk - 1 + r, wg = w_blk - 1 + c;
                const bool in = (unsigned)hg < (unsigned)a.H && (unsigned)wg < (unsigned)a.W;
                const int hc = hg < 0 ? 0 : (hg >= a.H ? a.H - 1 : hg);
                const int wc = wg < 0 ? 0 : (wg >= a.W ? a.W - 1 : wg);
                fst[reg][i] = load_raw8<TR>(xn + ((int64_t)(tg * xH + (hc >> a.lsh)) * xW +
                                                  (wc >> a.lsw)) * cin +
                                            c0 + g * 8);
                fin[reg] = in ? (fin[reg] | (1u << i)) : (fin[reg] & ~(1u << i));
            }
        };
        // with NORM: the table of chunk kc, and this thread's 8 channels of it (channel group
        // tid % 4 in every unit it stages)
        auto ntab_value = [&](int kc) {   // one table entry per lane of a wave; kc is clamped
            const int c = kc < kc1 ? kc : kc1 - 1;
            return a.nab[((int64_t)n * cin + (int64_t)c * CK) * 2 + (tid & 63)];
        };
        auto frame_write = [&](int slot, int reg, int kcf) {
            const float* tab = ntab + (kcf % 3) * 64 + (tid % UPP) * 16;
#pragma unroll
            for (int i = 0; i < FST; ++i) {
                uint4 hi, lo;
                if constexpr (NORM) {
                    // the table is read again for every unit, a channel pair at a time: only
                    // four of its values are live at once
                    hi = norm_operand_lds<TR, F16>(fst[reg][i], (fin[reg] >> i) & 1u, tab);
                    lo = hi;
                } else {
                    to_operand<TR, SPLIT>(fst[reg][i], (fin[reg] >> i) & 1u, hi, lo);
                }
                uint8_t* dst = (fu_pos[i] >> 30) ? halo + kSink : halo + slot * FB + fu_lds[i];
                *reinterpret_cast<uint4*>(dst) = hi;              // split: hi in bytes 0..31
                if constexpr (SPLIT) *reinterpret_cast<uint4*>(dst + 32) = lo;
            }
        };
        // A rows of this lane inside a frame, and the tile frame each of its MI tiles starts at
        int a_in[MI], tb_of[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int m = wave_m * MW + i * 32 + lrow;
            const int hb = (m / WB) % HB, wb = m % WB;
            a_in[i] = hb * RP + wb * kRow + khalf * 16;
            tb_of[i] = (wave_m * MW + i * 32) / (HB * WB);
        }

        // prologue: chunk 0 into slots 0 .. HT-1 (its held frames stay in registers too, so that
        // the first chunk's step-0 rewrite is harmless), the first weights in flight
        int b = 0;
        if constexpr (NORM) {   // the tables of the first two chunks (every wave writes the same)
            const float t0 = ntab_value(kc0), t1 = ntab_value(kc0 + 1);
            ntab[(kc0 % 3) * 64 + (tid & 63)] = t0;
            ntab[((kc0 + 1) % 3) * 64 + (tid & 63)] = t1;
            __syncthreads();
        }
#pragma unroll
        for (int f = 0; f < NIN; ++f) {
            frame_load(f, kc0 * CK, 0);
            frame_write(f, 0, kc0);
        }
#pragma unroll
        for (int h = 0; h < NHOLD; ++h) {
            frame_load(NIN + h, kc0 * CK, h);
            frame_write(NIN + h, h, kc0);
        }
#pragma unroll
        for (int t = 0; t < PD; ++t) load_b(t, t, kc0 * CK);
        __syncthreads();

        // step schedule: in-chunk frame k is loaded at LDK[k] and written at WRK[k] into slot
        // offset k - NSP; held frame h is loaded at HLD[h]
        constexpr int LDK[4] = {2, TB == 2 ? 20 : 10, TB == 2 ? 38 : 20, 38};
        constexpr int WRK[4] = {TB == 2 ? 14 : 8, TB == 2 ? 32 : 16, TB == 2 ? 48 : 30, 46};
        constexpr int HLD[2] = {TB == 2 ? 50 : 48, 50};
        // One chunk. NEXT: stage the next chunk's frames and fetch its first weights while this
        // one computes. The last chunk is a copy without those loads and writes.
        auto chunk = [&](int kc, auto next_c) {
            constexpr bool NEXT = decltype(next_c)::value;
            const int c0 = kc * CK;
            const int cn = (kc + 1) * CK;
            float ntv = 0.0f;                     // NORM: chunk kc + 2's table entry in flight
            auto slot = [&](int f) { return (b + f + 2 * NS) % NS; };
            int abase[MI];
            auto set_phase = [&](int kt) {
#pragma unroll
                for (int i = 0; i < MI; ++i) abase[i] = slot(tb_of[i] + kt) * FB + a_in[i];
            };
            set_phase(0);
            bf16x8_t af[2][MI];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                af[0][i] = *reinterpret_cast<const bf16x8_t*>(&halo[abase[i]]);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, 54>([&](auto step_c) {
                constexpr int step = decltype(step_c)::value;
                constexpr int tap = step >> 1, kk = step & 1;
                // phase ends: every wave is done with the phase's first frame
                if constexpr (step == 17 || step == 35) {
                    __syncthreads();
                    set_phase(step == 17 ? 1 : 2);
                }
                constexpr bool ldb = kk == 0 && (tap + PD < 27 || NEXT);
                if constexpr (ldb) {
                    if constexpr (tap + PD < 27) load_b((tap + PD) % NB, tap + PD, c0);
                    else load_b((tap + PD) % NB, tap + PD - 27, cn);
                }
                constexpr int ldk = !NEXT ? -1 : step == LDK[0] ? 0 : step == LDK[1] ? 1
                                  : step == LDK[2] ? 2 : (NIN > 3 && step == LDK[3]) ? 3 : -1;
                constexpr int wrk = !NEXT ? -1 : step == WRK[0] ? 0 : step == WRK[1] ? 1
                                  : step == WRK[2] ? 2 : (NIN > 3 && step == WRK[3]) ? 3 : -1;
                constexpr int hld = !NEXT ? -1 : step == HLD[0] ? 0
                                  : (NHOLD > 1 && step == HLD[1]) ? 1 : -1;
                if constexpr (step == 0) {
#pragma unroll
                    for (int h = 0; h < NHOLD; ++h) frame_write(slot(NIN + h), h, kc);
                }
                // NORM: the table of chunk kc + 2 is fetched early and written late in the chunk,
                // into the slot of chunk kc - 1 (read last at its step 0); the chunk's closing
                // barrier publishes it before chunk kc + 1 writes kc + 2's frames
                constexpr bool tld = NORM && NEXT && step == LDK[0];
                constexpr bool tst = NORM && NEXT && step == 40;
                if constexpr (tld) ntv = ntab_value(kc + 2);
                if constexpr (tst) ntab[((kc + 2) % 3) * 64 + (tid & 63)] = ntv;
                if constexpr (ldk >= 0) frame_load(ldk, cn, 0);
                if constexpr (wrk >= 0) frame_write(slot(wrk - NSP), 0, kc + 1);
                if constexpr (hld >= 0) frame_load(NIN + hld, cn, hld);
                if constexpr (step + 1 < 54) {
                    constexpr int nt = (step + 1) >> 1, nk = (step + 1) & 1;
                    constexpr int kh = (nt / 3) % 3, kw = nt % 3;
                    constexpr int off = kh * RP + kw * kRow + nk * 32;
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        af[(step + 1) & 1][i] =
                            *reinterpret_cast<const bf16x8_t*>(&halo[abase[i] + off]);
                }
                const bf16x8_t bf = b_operand(bq[tap % NB][SPLIT ? 0 : kk]);
#pragma unroll
                for (int i = 0; i < MI; ++i) acc[i] = mfma_step<F16>(af[step & 1][i], bf, acc[i]);
                constexpr int n_ld = (ldk >= 0) + (hld >= 0);
                constexpr int n_wr = (wrk >= 0) + (step == 0 ? NHOLD : 0);
                constexpr int n_tr = NORM ? 4 * FST * n_wr : 0;   // table reads of the writes
                if constexpr (ldb) __builtin_amdgcn_sched_group_barrier(0x020, KB, 0);
                if constexpr (n_ld > 0 || tld)
                    __builtin_amdgcn_sched_group_barrier(
                        0x020, n_ld * FST * (int)(sizeof(TR) / 2) + (tld ? 1 : 0), 0);
                if constexpr (tst) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                if constexpr (n_tr > 0) __builtin_amdgcn_sched_group_barrier(0x100, n_tr, 0);
                if constexpr (n_wr > 0)
                    __builtin_amdgcn_sched_group_barrier(0x200, n_wr * FST * (SPLIT ? 2 : 1), 0);
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if constexpr (step + 1 < 54) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            __syncthreads();   // chunk done: its later frames are free, the next chunk is staged
            b = (b + NS - NSP) % NS;
        };
        for (int kc = kc0; kc + 1 < kc1; ++kc) chunk(kc, std::true_type{});
        chunk(kc1 - 1, std::false_type{});
    } else {
        // Thread tid stages units tid + 256 k of each chunk's tile: unit_load issues a unit's load
        // (none outside the image: zero padding), unit_store converts it and writes it to LDS.
        constexpr int NUNIT = S::kPos * UPP;
        constexpr int NU = (NUNIT + kMfmaThreads - 1) / kMfmaThreads;
        auto unit_load = [&](int k, int c0x, Raw8<TR>& raw, bool& in, int& dst) {
            const int u = tid + k * kMfmaThreads;
            const bool valid = u < NUNIT;
            const int pos = (valid ? u : 0) / UPP, g = (valid ? u : 0) % UPP;
            const int f = pos / (HH * HW);
            const int rem = pos - f * (HH * HW);
            const int r = rem / HW;
            const int c = rem - r * HW;
            int tg = t_blk - 2 + f;
            tg = tg < 0 ? 0 : tg;                          // causal: frames before 0 read frame 0
            const int hg = h_blk - 1 + r, wg = w_blk - 1 + c;
            in = valid && tg < a.T && hg >= 0 && hg < a.H && wg >= 0 && wg < a.W;
            if (in)
                raw = load_raw8<TR>(xn + ((int64_t)(tg * xH + (hg >> a.lsh)) * xW + (wg >> a.lsw)) *
                                             cin + c0x + g * 8);
            dst = valid ? (f * HH + r) * RP + c * kRow + g * 16 : -1;
        };
        // sc, sh: the chunk's per-channel scale and shift of a normalised input (unused otherwise)
        auto unit_store = [&](const Raw8<TR>& raw, bool in, int dst, const auto& sc,
                              const auto& sh) {
            if (dst < 0) return;
            uint4 v, vl;
            if constexpr (NORM) {
                v = norm_operand<TR, F16>(raw, in, sc, sh);
                vl = v;
            } else {
                to_operand<TR, SPLIT>(raw, in, v, vl);
            }
            uint8_t* d = &halo[dst];
            *reinterpret_cast<uint4*>(d) = v;                  // split: hi in bytes 0..31 of the row
            if constexpr (SPLIT) *reinterpret_cast<uint4*>(d + 32) = vl;  // lo in bytes 32..63
        };
        // A chunk's units are loaded in rounds of BATCH, a round's loads all in flight before its
        // first write: one at a time, each unit would wait out a full memory latency. (Loading the
        // next chunk's whole tile into registers while this one computes measured the same.)
        constexpr int BATCH = (NT == 128 ? 4 : 8) / (int)(sizeof(TR) / 2);
        for (int kc = kc0; kc < kc1; ++kc) {
            const int c0 = kc * CK;
    #pragma unroll
            for (int t = 0; t < PD; ++t) load_b(t, t, c0);   // in flight while the tile is staged
            __syncthreads();              // the previous chunk's LDS reads are done
            float sc[NORM ? 8 : 1], sh[NORM ? 8 : 1];   // every unit of a thread: group tid % 4
            if constexpr (NORM) load_norm8(a.nab, n, cin, c0 + (tid % UPP) * 8, sc, sh);
            static_for<0, (NU + BATCH - 1) / BATCH>([&](auto round_c) {
                constexpr int R0 = decltype(round_c)::value * BATCH;
                constexpr int NR = NU - R0 < BATCH ? NU - R0 : BATCH;
                Raw8<TR> raw[NR] = {};
                bool inb[NR];
                int dst[NR];
#pragma unroll
                for (int k = 0; k < NR; ++k) unit_load(R0 + k, c0, raw[k], inb[k], dst[k]);
#pragma unroll
                for (int k = 0; k < NR; ++k) unit_store(raw[k], inb[k], dst[k], sc, sh);
            });
            __syncthreads();

            // 54 k steps (27 taps x 2). The A fragments of step s + 1 are read from LDS while the
            // MFMAs of step s run; the weights of tap + 1 are fetched during tap.
            bf16x8_t af[2][MI];
    #pragma unroll
            for (int i = 0; i < MI; ++i)
                af[0][i] = *reinterpret_cast<const bf16x8_t*>(&halo[a_off[i]]);
            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
            for (int step = 0; step < 54; ++step) {
                const int tap = step >> 1, kk = step & 1;
                if (kk == 0 && tap + PD < 27) load_b((tap + PD) % NB, tap + PD, c0);
                if (step + 1 < 54) {
                    const int nt = (step + 1) >> 1, nk = (step + 1) & 1;
                    const int kt = nt / 9, kh = (nt / 3) % 3, kw = nt % 3;
                    const int off = (kt * HH + kh) * RP + kw * kRow + nk * 32;
    #pragma unroll
                    for (int i = 0; i < MI; ++i)
                        af[(step + 1) & 1][i] =
                            *reinterpret_cast<const bf16x8_t*>(&halo[a_off[i] + off]);
                }
                const bf16x8_t bf = b_operand(bq[tap % NB][SPLIT ? 0 : kk]);
    #pragma unroll
                for (int i = 0; i < MI; ++i) acc[i] = mfma_step<F16>(af[step & 1][i], bf, acc[i]);
                // Each k step is its own scheduling island: the weight loads first, then the MFMAs
                // alternating with the next step's LDS reads, so that neither waits on the other.
                if (kk == 0 && tap + PD < 27) __builtin_amdgcn_sched_group_barrier(0x020, KB, 0);
    #pragma unroll
                for (int i = 0; i < MI; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (step + 1 < 54) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (a.part) {
        // one split of a split conv: store the raw sums for the reduce launch
        float* dst = a.part + (((int64_t)split * per_split + tile) * kMfmaWaves + wave) * MI * 1024 +
                     lane * 16;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            float4* q = reinterpret_cast<float4*>(dst + i * 1024);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                q[k] = make_float4(acc[i][4 * k], acc[i][4 * k + 1], acc[i][4 * k + 2],
                                   acc[i][4 * k + 3]);
        }
        return;
    }
    if constexpr (F16) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] *= kF16WeightUnscale;
    }
    // The narrow blocks (WB < 8) always take the staged epilogue: the direct one's register rows
    // follow the 8- and 16-wide patterns, and with them it would not fit beside the staging.
    if constexpr (WB >= 8) {
        if (a.zc % 32 == 0 && a.cout % 32 == 0) {
            conv_epilogue_direct<TO, TB, HB, WB, MI, MW, WM>(a, acc, n, t_blk, h_blk, w_blk, bt_i,
                                                             bh_i, bw_i, co_tile, lane, wave_m);
            return;
        }
    }
    __syncthreads();  // the input tile is reused for the epilogue

    // Epilogue: each wave stages through its own slice of the (now idle) input tile.
    static_assert(kMfmaWaves * 32 * kEp * 4 <= S::kBytes, "epilogue staging must fit the tile");
    conv_epilogue<TO, HB, WB, MI, MW, WM>(a, acc, reinterpret_cast<float*>(halo) + wave * 32 * kEp,
                                          n, t_blk, h_blk, w_blk, bt_i, bh_i, bw_i, co_tile, lane,
                                          wave_m);
}

// The second launch of a conv split over K: one workgroup per (channel tile, block) pair, with
// the wave roles of conv3d_mfma_kernel. It adds the splits' accumulators in split order, then
// runs the same epilogue. A kernel of its own, so that the main kernel's registers stay as they
// are.
template <int NT, typename TI, typename TO, int TB, int HB, int WB>
__global__ __launch_bounds__(kMfmaThreads, 2)
void conv3d_reduce_kernel(MfmaArgs a) {
    constexpr bool F16 = InT<TI>::f16op;
    constexpr int WNN = NT / 32;
    constexpr int WM = kMfmaWaves / WNN;
    constexpr int MW = 256 / WM;
    constexpr int MI = MW / 32;
    __shared__ __attribute__((aligned(16))) float ep[kMfmaWaves * 32 * kEp];
    const int tile = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, gridDim.x));
    const int nt = __builtin_amdgcn_readfirstlane(tile / a.n_mblocks);
    // block order within a channel tile: T fastest, so that the workgroups an XCD runs at once
    // are temporal neighbours, which stage 2 of their TB + 2 frames in common (hits in its L2)
    int mb = tile - nt * a.n_mblocks;
    const int bt_i = mb % a.nbt;
    mb /= a.nbt;
    const int bw_i = mb % a.nbw;
    mb /= a.nbw;
    const int bh_i = mb % a.nbh;
    const int n = mb / a.nbh;
    const int t_blk = a.box.t0 + bt_i * TB;
    const int h_blk = a.box.h0 + bh_i * HB;
    const int w_blk = a.box.w0 + bw_i * WB;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave / WNN;
    const int co_tile = nt * NT + (wave % WNN) * 32;
    f32x16_t acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    const int64_t per_split = gridDim.x;
    for (int sp = 0; sp < a.splits; ++sp) {
        const float* src =
            a.reduce + (((int64_t)sp * per_split + tile) * kMfmaWaves + wave) * MI * 1024 + lane * 16;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const float4* q = reinterpret_cast<const float4*>(src + i * 1024);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 v = q[k];
                acc[i][4 * k] += v.x;
                acc[i][4 * k + 1] += v.y;
                acc[i][4 * k + 2] += v.z;
                acc[i][4 * k + 3] += v.w;
            }
        }
    }
    if constexpr (F16) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] *= kF16WeightUnscale;
    }
    if constexpr (WB >= 8) {
        if (a.zc % 32 == 0 && a.cout % 32 == 0) {
            conv_epilogue_direct<TO, TB, HB, WB, MI, MW, WM>(a, acc, n, t_blk, h_blk, w_blk, bt_i,
                                                             bh_i, bw_i, co_tile, lane, wave_m);
            return;
        }
    }
    conv_epilogue<TO, HB, WB, MI, MW, WM>(a, acc, ep + wave * 32 * kEp, n, t_blk, h_blk, w_blk,
                                          bt_i, bh_i, bw_i, co_tile, lane, wave_m);
}

// Output-block shapes (T x H x W = 256 positions). The wide ones suit big boxes; the narrow ones
// (WB = 4 or 2, deep in T) fit boxes 10 or 20 positions wide, such as one width quarter of the
// 720p decode's first stages, where an 8- or 16-wide block wastes up to 43% of its rows.
enum BlockKind {
    kBlk2x8x16 = 0, kBlk4x8x8 = 1, kBlk4x4x16 = 2, kBlk4x16x4 = 3, kBlk16x4x4 = 4, kBlk16x8x2 = 5,
    kBlockKinds = 6
};

struct BlockDims {
    int tb, hb, wb;
};

constexpr BlockDims kBlockDims[kBlockKinds] = {{2, 8, 16}, {4, 8, 8}, {4, 4, 16},
                                               {4, 16, 4}, {16, 4, 4}, {16, 8, 2}};

inline int64_t padded_volume(const Box& b, int tb, int hb, int wb) {
    return ceil_div(b.bt(), tb) * tb * ceil_div(b.bh(), hb) * hb * ceil_div(b.bw(), wb) * wb;
}

// The shape that pads the box least. The narrow shapes, which stage without the ring, are
// charged 10% more, about what the ring gains. Ties keep the earlier shape.
inline BlockKind pick_block(const Box& b) {
    int best = 0;
    int64_t best_cost = INT64_MAX;
    for (int k = 0; k < kBlockKinds; ++k) {
        const BlockDims& d = kBlockDims[k];
        const int64_t cost = padded_volume(b, d.tb, d.hb, d.wb) * (d.wb >= 8 ? 10 : 11);
        if (cost < best_cost) {
            best = k;
            best_cost = cost;
        }
    }
    return (BlockKind)best;
}

template <int NT>
constexpr int wave_rows() {
    return kMfmaWaves / (NT / 32);
}

// Output-channel tile of a conv: 128 wide, or 64 / 32 for narrow outputs (conv_out's 48 or 12).
inline int conv_nt(int64_t cout) { return cout >= 128 ? 128 : cout > 32 ? 64 : 32; }

// Workgroups of one conv launch over `box` (all samples), before any split over K.
inline int64_t conv_workgroups(int64_t n, int64_t cout, const Box& box) {
    const BlockDims& d = kBlockDims[pick_block(box)];
    return n * ceil_div(box.bt(), d.tb) * ceil_div(box.bh(), d.hb) * ceil_div(box.bw(), d.wb) *
           ceil_div(cout, conv_nt(cout));
}

// The launch arguments every MFMA conv kernel shares, and the check that the box lies in the
// input grid and every value the grid stores lies in y (and in the residual, which has y's
// shape).
inline vae_status_t mfma_common_args(const vae_tensor_t& x, const void* w, const float* bias,
                                     const vae_tensor_t* residual, const vae_tensor_t& y,
                                     const Box& box, const ConvFuse* fz, MfmaArgs* out) {
    MfmaArgs& a = *out;
    a.x = x.data;
    a.w = static_cast<const uint16_t*>(w);
    a.bias = bias;
    a.res = residual ? residual->data : nullptr;
    a.res_f32 = residual && residual->dtype == VAE_DTYPE_F32 && y.dtype != VAE_DTYPE_F32;
    a.y = y.data;
    a.T = (int32_t)x.t;
    a.lsh = fz ? fz->lsh : 0;
    a.lsw = fz ? fz->lsw : 0;
    a.H = (int32_t)(x.h << a.lsh);
    a.W = (int32_t)(x.w << a.lsw);
    a.cin = (int32_t)x.c;
    a.st = fz ? fz->st : 1;
    a.sh = fz ? fz->sh : 1;
    a.sw = fz ? fz->sw : 1;
    a.tdrop = fz && fz->tdrop >= 0 ? fz->tdrop : a.st - 1;
    a.nab = fz ? fz->in_ab : nullptr;
    a.zc = (int32_t)y.c;
    a.cout = (int32_t)(y.c * a.st * a.sh * a.sw);
    a.yT = (int32_t)y.t;
    a.yH = (int32_t)y.h;
    a.yW = (int32_t)y.w;
    a.box = box;
    a.stats = nullptr;
    a.groups = 1;
    a.nslots = a.slot0 = 0;
    a.splits = 1;
    a.part = nullptr;
    a.reduce = nullptr;
    if (box.t0 < 0 || box.h0 < 0 || box.w0 < 0 || box.t1 > a.T || box.h1 > a.H ||
        box.w1 > a.W || (int64_t)a.st * box.t1 - a.tdrop > a.yT ||
        (int64_t)a.sh * box.h1 > a.yH || (int64_t)a.sw * box.w1 > a.yW || y.n != x.n ||
        (residual && (residual->n != y.n || residual->t != y.t || residual->h != y.h ||
                      residual->w != y.w || residual->c != y.c)))
        return fail(VAE_ERR_INVALID_ARG, "conv3d: box outside the input, or outputs outside y");
    return VAE_OK;
}

template <int NT, typename TI, typename TO, bool SPLIT, bool PACKED, int TB, int HB, int WB>
vae_status_t run_shape(const vae_tensor_t& x, const void* w, const float* bias,
                       const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                       const ConvFuse* fz, hipStream_t stream) {
    MfmaArgs a;
    VAE_TRY(mfma_common_args(x, w, bias, residual, y, box, fz, &a));
    if (InT<TI>::norm != (a.nab != nullptr))
        return fail(VAE_ERR_INVALID_ARG, "conv3d: input normalisation without its scale and shift");
    a.nbt = (int32_t)ceil_div(box.bt(), TB);
    a.nbh = (int32_t)ceil_div(box.bh(), HB);
    a.nbw = (int32_t)ceil_div(box.bw(), WB);
    int64_t mblocks = x.n * (int64_t)a.nbt * a.nbh * a.nbw;
    int64_t total = mblocks * ceil_div(a.cout, NT);
    if (total > INT32_MAX) return fail(VAE_ERR_UNSUPPORTED, "conv3d: grid too large");
    a.n_mblocks = (int32_t)mblocks;
    a.stats = fz ? fz->gn_ws : nullptr;
    a.groups = fz && fz->gn_ws ? fz->groups : 1;
    const int64_t own = (int64_t)(a.cout / a.zc) * a.nbt * a.nbh * a.nbw * wave_rows<NT>();
    const int64_t stride = fz && fz->slot_stride ? fz->slot_stride : own;
    if (a.stats && (fz->slot0 < 0 || fz->slot0 + own > stride || stride > INT32_MAX))
        return fail(VAE_ERR_INVALID_ARG, "conv3d: GroupNorm slot range outside its row");
    a.nslots = (int32_t)stride;
    a.slot0 = fz ? (int32_t)fz->slot0 : 0;
    a.splits = 1;
    a.part = nullptr;
    a.reduce = nullptr;
    const int32_t splits = fz && fz->part ? fz->splits : 1;
    if (splits > 1) {
        // split over K: `splits` times the grid store partial sums, then one launch adds them
        // and runs the epilogue
        if (splits > a.cin / (SPLIT ? 16 : kCK) || total * splits > INT32_MAX)
            return fail(VAE_ERR_INVALID_ARG, "conv3d: more K splits than channel chunks");
        a.splits = splits;
        a.part = fz->part;
        hipLaunchKernelGGL((conv3d_mfma_kernel<NT, TI, TO, SPLIT, PACKED, TB, HB, WB>),
                           dim3((unsigned)(total * splits)), dim3(kMfmaThreads), 0, stream, a);
        VAE_HIP_CHECK(hipGetLastError());
        a.part = nullptr;
        a.reduce = fz->part;
        hipLaunchKernelGGL((conv3d_reduce_kernel<NT, TI, TO, TB, HB, WB>), dim3((unsigned)total),
                           dim3(kMfmaThreads), 0, stream, a);
        VAE_HIP_CHECK(hipGetLastError());
        return VAE_OK;
    }
    hipLaunchKernelGGL((conv3d_mfma_kernel<NT, TI, TO, SPLIT, PACKED, TB, HB, WB>),
                       dim3((unsigned)total), dim3(kMfmaThreads), 0, stream, a);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

// The narrow block shapes, instantiated in translation units of their own
// (conv3d_mfma_*_narrow.hip) to keep the build parallel.
template <int NT, typename TI, typename TO, bool SPLIT, bool PACKED>
vae_status_t run_narrow(BlockKind kind, const vae_tensor_t& x, const void* w, const float* bias,
                        const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                        const ConvFuse* fz, hipStream_t stream) {
    switch (kind) {
        case kBlk4x16x4:
            return run_shape<NT, TI, TO, SPLIT, PACKED, 4, 16, 4>(x, w, bias, residual, y, box,
                                                                  fz, stream);
        case kBlk16x4x4:
            return run_shape<NT, TI, TO, SPLIT, PACKED, 16, 4, 4>(x, w, bias, residual, y, box,
                                                                  fz, stream);
        default:
            return run_shape<NT, TI, TO, SPLIT, PACKED, 16, 8, 2>(x, w, bias, residual, y, box,
                                                                  fz, stream);
    }
}

// Explicit instantiations of run_narrow for one (NT, input type, split): `extern` in the file that
// instantiates run_mfma_out, empty in the file that holds the narrow kernels.
#define VAE_NARROW_SIG(NT, TI, TO, SPLIT, PACKED)                                               \
    vae_status_t run_narrow<NT, TI, TO, SPLIT, PACKED>(                                        \
        BlockKind, const vae_tensor_t&, const void*, const float*, const vae_tensor_t*,        \
        const vae_tensor_t&, const Box&, const ConvFuse*, hipStream_t)
#define VAE_NARROW_INST(PREFIX, NT, TI, SPLIT)                                                  \
    PREFIX template VAE_NARROW_SIG(NT, TI, float, SPLIT, true);                                 \
    PREFIX template VAE_NARROW_SIG(NT, TI, float, SPLIT, false);                                \
    PREFIX template VAE_NARROW_SIG(NT, TI, uint16_t, SPLIT, true);                              \
    PREFIX template VAE_NARROW_SIG(NT, TI, uint16_t, SPLIT, false);
// fp16 outputs exist for 2-byte inputs only
#define VAE_NARROW_INST_F16(PREFIX, NT, TI, SPLIT)                                              \
    VAE_NARROW_INST(PREFIX, NT, TI, SPLIT)                                                      \
    PREFIX template VAE_NARROW_SIG(NT, TI, _Float16, SPLIT, true);                              \
    PREFIX template VAE_NARROW_SIG(NT, TI, _Float16, SPLIT, false);
// normalised inputs: packed weights, every output type
#define VAE_NARROW_INST_GN(PREFIX, NT, TI)                                                      \
    PREFIX template VAE_NARROW_SIG(NT, TI, float, false, true);                                 \
    PREFIX template VAE_NARROW_SIG(NT, TI, uint16_t, false, true);                              \
    PREFIX template VAE_NARROW_SIG(NT, TI, _Float16, false, true);

template <int NT, typename TI, typename TO, bool SPLIT, bool PACKED>
vae_status_t run_block(const vae_tensor_t& x, const void* w, const float* bias,
                       const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                       const ConvFuse* fz, hipStream_t stream) {
    const BlockKind kind = pick_block(box);
    switch (kind) {
        case kBlk4x8x8:
            return run_shape<NT, TI, TO, SPLIT, PACKED, 4, 8, 8>(x, w, bias, residual, y, box, fz,
                                                                 stream);
        case kBlk4x4x16:
            return run_shape<NT, TI, TO, SPLIT, PACKED, 4, 4, 16>(x, w, bias, residual, y, box,
                                                                  fz, stream);
        case kBlk2x8x16:
            return run_shape<NT, TI, TO, SPLIT, PACKED, 2, 8, 16>(x, w, bias, residual, y, box,
                                                                  fz, stream);
        default:
            return run_narrow<NT, TI, TO, SPLIT, PACKED>(kind, x, w, bias, residual, y, box, fz,
                                                         stream);
    }
}

template <int NT, typename TI, typename TO, bool SPLIT>
vae_status_t run_mfma(const vae_tensor_t& x, const void* w, const float* bias,
                      const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                      bool packed, const ConvFuse* fz, hipStream_t stream) {
    if constexpr (InT<TI>::norm) {   // normalising staging is built for packed weights only
        if (!packed) return fail(VAE_ERR_UNSUPPORTED, "conv3d: an input norm needs packed weights");
        return run_block<NT, TI, TO, SPLIT, true>(x, w, bias, residual, y, box, fz, stream);
    } else {
        if (packed)
            return run_block<NT, TI, TO, SPLIT, true>(x, w, bias, residual, y, box, fz, stream);
        return run_block<NT, TI, TO, SPLIT, false>(x, w, bias, residual, y, box, fz, stream);
    }
}

template <int NT, typename TI, bool SPLIT>
vae_status_t run_mfma_out(const vae_tensor_t& x, const void* w, const float* bias,
                          const vae_tensor_t* residual, const vae_tensor_t& y, const Box& box,
                          bool packed, const ConvFuse* fz, hipStream_t stream) {
    if (y.dtype == VAE_DTYPE_F32)
        return run_mfma<NT, TI, float, SPLIT>(x, w, bias, residual, y, box, packed, fz, stream);
    if (y.dtype == VAE_DTYPE_F16) {
        // fp16 outputs are the operand hand-off to an fp16-input conv, from a 2-byte input (or a
        // normalised one)
        if constexpr (sizeof(typename InT<TI>::raw) == 2 || InT<TI>::norm)
            return run_mfma<NT, TI, _Float16, SPLIT>(x, w, bias, residual, y, box, packed, fz,
                                                     stream);
        else
            return fail(VAE_ERR_UNSUPPORTED, "conv3d: an fp16 output needs a bf16 or fp16 input");
    }
    return run_mfma<NT, TI, uint16_t, SPLIT>(x, w, bias, residual, y, box, packed, fz, stream);
}

}  // namespace mfma
}  // namespace vae
