// GroupNorm (+SiLU) whose statistics are merged across patches.
//
// The statistics must be those of the whole tensor: the global mean, and the variance about it
// divided by the count. Per-patch means and Bessel's correction are both wrong ("Add tiled VAE
// parallelism & extended model support", PatchGroupNorm commit message). Three steps:
//  1. gn_stats_kernel. Each block streams a range of rows of one patch box. A "row" is the
//     positions of the box at fixed (n, t, h), which are contiguous in NDHWC. Every thread owns a
//     fixed 16-byte channel vector. Per channel it accumulates sums of (x - K) and (x - K)^2, where
//     the shift K is the first value it reads (the shifted-data variance algorithm; no division in
//     the loop, and robust to a large mean). At the end these become (count, mean, M2). The block
//     merges its threads into per-group partials (fp64, Chan) and writes them to its own slot: no
//     atomics.
//  2. gn_finalize_kernel. One block per (group, sample). It merges the block partials of each box
//     with Chan's pairwise update in a fixed order, then merges the boxes in box order. It writes
//     per-box (count, mean, M2) and (mean, rstd).
//  3. gn_apply_kernel. Streams rows again. Each thread folds (mean, rstd, gamma, beta) of its
//     channels into one scale and shift, so an element costs one FMA plus the SiLU. It may read
//     fp32 and write bf16 (the next convolution's operand).
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "kernels.h"

namespace vae {
namespace {

constexpr int kThreads = 256;
// 16- and 8-byte vectors as the nontemporal load and store builtins take them.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int64_t kElemsPerBlock = 1 << 18;   // target elements one stats block streams
constexpr int kMaxStatsBlocks = 4096;
constexpr int kUnroll = 4;

struct GnBoxes {
    Box b[kMaxBoxes];
    int32_t start[kMaxBoxes + 1];  // first block of each box; start[n] = total blocks
    int32_t n;
};

struct Moments {
    double n, mean, m2;
};

__device__ __forceinline__ void chan_merge(Moments& a, double nb, double mb, double m2b) {
    if (nb <= 0.0) return;
    if (a.n <= 0.0) {
        a.n = nb;
        a.mean = mb;
        a.m2 = m2b;
        return;
    }
    double n = a.n + nb;
    double d = mb - a.mean;
    a.mean += d * (nb / n);
    a.m2 += m2b + d * d * (a.n * nb / n);
    a.n = n;
}

// Sets *status (when given) if a group's statistics are not finite: an input value was inf or
// NaN, e.g. an activation past fp16's 65504 stored at an fp16 operand hand-off.
__device__ __forceinline__ void flag_nonfinite(uint32_t* status, double mean, double var) {
    if (status && !(isfinite(mean) && isfinite(var))) *status = 1u;
}

// Number of stats blocks per box for a given tensor.
int32_t blocks_for_box(const Box& b, int64_t c, int32_t n_boxes) {
    int64_t rows = b.bt() * b.bh();
    int64_t elems = b.volume() * c;
    int64_t nb = ceil_div(elems, kElemsPerBlock);
    int64_t cap = kMaxStatsBlocks / n_boxes;
    if (nb > cap) nb = cap;
    if (nb > rows) nb = rows;
    if (nb < 1) nb = 1;
    return (int32_t)nb;
}

GnBoxes make_boxes(const vae_tensor_t& x, const BoxList& bl) {
    GnBoxes g{};
    g.n = bl.n;
    int32_t s = 0;
    for (int i = 0; i < bl.n; ++i) {
        g.b[i] = bl.b[i];
        g.start[i] = s;
        s += blocks_for_box(bl.b[i], x.c, bl.n);
    }
    g.start[bl.n] = s;
    return g;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void gn_stats_kernel(const T* __restrict__ x, int32_t Tn,
                                                            int32_t H, int32_t W, int32_t C,
                                                            int32_t groups, GnBoxes boxes,
                                                            double* __restrict__ ws) {
    constexpr int V = Elem<T>::kVec;
    const int n = blockIdx.y;
    const int N = gridDim.y;
    const int blk = blockIdx.x;
    int bi = 0;
    while (bi + 1 < boxes.n && blk >= boxes.start[bi + 1]) ++bi;
    const Box b = boxes.b[bi];
    const int nb = boxes.start[bi + 1] - boxes.start[bi];
    const int local = blk - boxes.start[bi];
    const int64_t rows = b.bt() * b.bh();
    const int64_t r0 = rows * local / nb, r1 = rows * (local + 1) / nb;

    const int CV = C / V;                 // 16-byte vectors per position (divides 256)
    const int tid = threadIdx.x;
    const int seg = (int)b.bw() * CV;     // vectors per row
    float cnt = 0.0f;
    float shift[V], s1[V], s2[V];
#pragma unroll
    for (int k = 0; k < V; ++k) shift[k] = s1[k] = s2[k] = 0.0f;
    bool have_shift = false;

    for (int64_t r = r0; r < r1; ++r) {
        const int t = b.t0 + (int)(r / b.bh());
        const int h = b.h0 + (int)(r % b.bh());
        const T* row = x + ((((int64_t)n * Tn + t) * H + h) * W + b.w0) * C;
        int e = tid;
        if (!have_shift && e < seg) {
            const uint4 raw = *reinterpret_cast<const uint4*>(row + (int64_t)e * V);
            const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int k = 0; k < V; ++k) shift[k] = Elem<T>::load(v + k);
            have_shift = true;
        }
        for (; e + (kUnroll - 1) * kThreads < seg; e += kUnroll * kThreads) {
            uint4 raw[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                raw[u] = *reinterpret_cast<const uint4*>(row + (int64_t)(e + u * kThreads) * V);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const T* v = reinterpret_cast<const T*>(&raw[u]);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float d = Elem<T>::load(v + k) - shift[k];
                    s1[k] += d;
                    s2[k] = fmaf(d, d, s2[k]);
                }
            }
            cnt += (float)kUnroll;
        }
        for (; e < seg; e += kThreads) {
            const uint4 raw = *reinterpret_cast<const uint4*>(row + (int64_t)e * V);
            const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = Elem<T>::load(v + k) - shift[k];
                s1[k] += d;
                s2[k] = fmaf(d, d, s2[k]);
            }
            cnt += 1.0f;
        }
    }

    // per-channel (mean, M2) of this thread
    float mean[V], m2[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const float mk = cnt > 0.0f ? s1[k] / cnt : 0.0f;
        mean[k] = shift[k] + mk;
        m2[k] = fmaxf(s2[k] - s1[k] * mk, 0.0f);
    }

    // Per-thread group partials. Thread tid always sees channels [(tid % CV) * V, +V).
    const int cpg = C / groups;
    __shared__ float sp[kThreads][V][3];
    if (cpg <= V) {
#pragma unroll
        for (int q = 0; q < V; ++q) {
            if (q * cpg >= V) break;
            float gm = 0.0f;
            for (int k = 0; k < cpg; ++k) gm += mean[q * cpg + k];
            gm /= (float)cpg;
            float gm2 = 0.0f;
            for (int k = 0; k < cpg; ++k) {
                const float d = mean[q * cpg + k] - gm;
                gm2 += m2[q * cpg + k] + cnt * d * d;
            }
            sp[tid][q][0] = cnt * cpg;
            sp[tid][q][1] = gm;
            sp[tid][q][2] = gm2;
        }
    } else {
        float gm = 0.0f;
#pragma unroll
        for (int k = 0; k < V; ++k) gm += mean[k];
        gm /= (float)V;
        float gm2 = 0.0f;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const float d = mean[k] - gm;
            gm2 += m2[k] + cnt * d * d;
        }
        sp[tid][0][0] = cnt * V;
        sp[tid][0][1] = gm;
        sp[tid][0][2] = gm2;
    }
    __syncthreads();

    for (int g = tid; g < groups; g += kThreads) {
        Moments m{0.0, 0.0, 0.0};
        int v0, v1, slot;
        if (cpg <= V) {
            v0 = (g * cpg) / V;
            v1 = v0 + 1;
            slot = (g * cpg - v0 * V) / cpg;
        } else {
            v0 = (g * cpg) / V;
            v1 = ((g + 1) * cpg) / V;
            slot = 0;
        }
        for (int t2 = 0; t2 < kThreads; ++t2) {
            const int v = t2 % CV;
            if (v < v0 || v >= v1) continue;
            chan_merge(m, sp[t2][slot][0], sp[t2][slot][1], sp[t2][slot][2]);
        }
        double* o = ws + (((int64_t)blk * N + n) * groups + g) * 3;
        o[0] = m.n;
        o[1] = m.mean;
        o[2] = m.m2;
    }
}

// Merge (count, mean, M2) triples `src[i * stride]`, i in [lo, hi), over 256 threads in a fixed
// order; thread 0 returns the result.
__device__ Moments block_merge(const double* src, int64_t stride, int lo, int hi) {
    __shared__ double red[kThreads][3];
    Moments m{0.0, 0.0, 0.0};
    for (int i = lo + threadIdx.x; i < hi; i += kThreads) {
        const double* p = src + (int64_t)i * stride;
        chan_merge(m, p[0], p[1], p[2]);
    }
    red[threadIdx.x][0] = m.n;
    red[threadIdx.x][1] = m.mean;
    red[threadIdx.x][2] = m.m2;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            Moments a{red[threadIdx.x][0], red[threadIdx.x][1], red[threadIdx.x][2]};
            chan_merge(a, red[threadIdx.x + s][0], red[threadIdx.x + s][1],
                       red[threadIdx.x + s][2]);
            red[threadIdx.x][0] = a.n;
            red[threadIdx.x][1] = a.mean;
            red[threadIdx.x][2] = a.m2;
        }
        __syncthreads();
    }
    Moments r{red[0][0], red[0][1], red[0][2]};
    __syncthreads();
    return r;
}

// grid (groups, N). ws: [blocks][N][G][3]; part_out: [n_boxes][N][G][3].
__global__ __launch_bounds__(kThreads) void gn_finalize_kernel(const double* __restrict__ ws,
                                                               GnBoxes boxes, int32_t groups,
                                                               float eps, double* part_out,
                                                               float* mean_rstd,
                                                               uint32_t* status) {
    const int g = blockIdx.x, n = blockIdx.y, N = gridDim.y;
    const int64_t stride = (int64_t)N * groups * 3;
    const double* base = ws + ((int64_t)n * groups + g) * 3;
    Moments total{0.0, 0.0, 0.0};
    for (int bi = 0; bi < boxes.n; ++bi) {
        Moments m = block_merge(base, stride, boxes.start[bi], boxes.start[bi + 1]);
        if (threadIdx.x == 0) {
            if (part_out) {
                double* o = part_out + (((int64_t)bi * N + n) * groups + g) * 3;
                o[0] = m.n;
                o[1] = m.mean;
                o[2] = m.m2;
            }
            chan_merge(total, m.n, m.mean, m.m2);
        }
    }
    if (threadIdx.x == 0 && mean_rstd) {
        const double var = total.n > 0.0 ? total.m2 / total.n : 0.0;
        mean_rstd[((int64_t)n * groups + g) * 2] = (float)total.mean;
        mean_rstd[((int64_t)n * groups + g) * 2 + 1] = (float)(1.0 / sqrt(var + (double)eps));
        flag_nonfinite(status, total.mean, var);
    }
}

// Slot counts above this are merged in two passes: chunks of kSlotChunk slots, one block each, in
// place, then the chunk results. A conv epilogue leaves up to ~50k slots per (sample, group) at
// the 720p shapes; one block per group merging them all took ~27 us per GroupNorm.
constexpr int64_t kSlotChunk = 1024;

// grid (chunks, groups, N). Chunk c merges slots [c * L, min((c + 1) * L, slots)) of ws
// [N][G][slots][3] in a fixed order and writes the result over its first slot (only this block
// reads or writes the chunk).
__global__ __launch_bounds__(kThreads) void gn_slots_chunk_kernel(double* __restrict__ ws,
                                                                  int64_t slots, int32_t groups,
                                                                  int32_t L) {
    const int c = blockIdx.x, g = blockIdx.y, n = blockIdx.z;
    double* base = ws + ((int64_t)n * groups + g) * slots * 3;
    const int64_t lo = (int64_t)c * L;
    const int64_t hi = lo + L < slots ? lo + L : slots;
    const Moments m = block_merge(base, 3, (int)lo, (int)hi);
    if (threadIdx.x == 0) {
        base[lo * 3] = m.n;
        base[lo * 3 + 1] = m.mean;
        base[lo * 3 + 2] = m.m2;
    }
}

// grid (groups, N). ws: [N][G][slots][3], the layout a fused conv epilogue writes; merges `count`
// triples `stride` slots apart (every slot, or the first slot of every chunk).
__global__ __launch_bounds__(kThreads) void gn_finalize_slots_kernel(const double* __restrict__ ws,
                                                                     int64_t slots, int64_t stride,
                                                                     int32_t count, int32_t groups,
                                                                     float eps, float* mean_rstd,
                                                                     uint32_t* status) {
    const int g = blockIdx.x, n = blockIdx.y;
    const double* base = ws + ((int64_t)n * groups + g) * slots * 3;
    const Moments m = block_merge(base, 3 * stride, 0, count);
    if (threadIdx.x == 0) {
        const double var = m.n > 0.0 ? m.m2 / m.n : 0.0;
        mean_rstd[((int64_t)n * groups + g) * 2] = (float)m.mean;
        mean_rstd[((int64_t)n * groups + g) * 2 + 1] = (float)(1.0 / sqrt(var + (double)eps));
        flag_nonfinite(status, m.mean, var);
    }
}

// grid (groups, N). part: [n_parts][N][G][3].
__global__ __launch_bounds__(64) void gn_combine_kernel(const double* __restrict__ part,
                                                        int32_t n_parts, int32_t groups, float eps,
                                                        float* mean_rstd, uint32_t* status) {
    const int g = blockIdx.x, n = blockIdx.y, N = gridDim.y;
    Moments m{0.0, 0.0, 0.0};
    if (threadIdx.x == 0) {
        for (int i = 0; i < n_parts; ++i) {
            const double* p = part + (((int64_t)i * N + n) * groups + g) * 3;
            chan_merge(m, p[0], p[1], p[2]);
        }
        const double var = m.n > 0.0 ? m.m2 / m.n : 0.0;
        mean_rstd[((int64_t)n * groups + g) * 2] = (float)m.mean;
        mean_rstd[((int64_t)n * groups + g) * 2 + 1] = (float)(1.0 / sqrt(var + (double)eps));
        flag_nonfinite(status, m.mean, var);
    }
}

// grid (rows of the box x slices, N): each block takes one slice of a contiguous row segment,
// kApplyVec 16-byte vectors per thread (V input elements each), all loads in flight before the
// first use. Many short blocks keep more loads in flight across the chip than a few long ones. So
// that a short block's set-up stays small, its threads first fold (mean, rstd, gamma, beta) of all
// C channels into a (scale, shift) table in LDS, one channel each, while the slice's loads fly;
// then each thread reads its V channels' entries. The channel vector of a thread is fixed because
// CV divides 256 and slices start at multiples of 256 vectors. Measured at the 720p decode's S3
// shape (fp32 in, bf16 out, SiLU): 0.80 ms (6.5 TB/s) against 0.96 ms for one block per row
// looping over it; 4 vectors per thread 0.82 ms, 8 vectors 1.7 ms.
constexpr int kApplyVec = 2;
constexpr int kApplySlice = kApplyVec * kThreads;      // vectors per block
constexpr int kApplyMaxC = 2048;                       // 256 vectors of 8 2-byte channels

template <typename TI, typename TO>
__global__ __launch_bounds__(kThreads) void gn_apply_kernel(
    const TI* x, TO* y, int32_t Tn, int32_t H, int32_t W, int32_t C, int32_t groups, Box b,
    int32_t slices, const float* __restrict__ mean_rstd, const float* __restrict__ gamma,
    const float* __restrict__ beta, int32_t silu) {
    constexpr int V = Elem<TI>::kVec;
    __shared__ float2 tab[kApplyMaxC];
    const int n = blockIdx.y;
    const int64_t r = blockIdx.x / slices;
    const int part = (int)(blockIdx.x - r * slices);
    const int t = b.t0 + (int)(r / b.bh());
    const int h = b.h0 + (int)(r % b.bh());
    const int64_t off = ((((int64_t)n * Tn + t) * H + h) * W + b.w0) * C;
    const TI* xr = x + off;
    TO* yr = y + off;
    const int CV = C / V;
    const int seg = (int)b.bw() * CV;
    const int e0 = part * kApplySlice + (int)threadIdx.x;
    u32x4_t raw[kApplyVec];
#pragma unroll
    for (int u = 0; u < kApplyVec; ++u) {
        const int e = e0 + u * kThreads;
        if (e < seg)
            raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xr + (int64_t)e * V));
    }
    const int cpg = C / groups;
    const float* mr = mean_rstd + (int64_t)n * groups * 2;
    for (int c = threadIdx.x; c < C; c += kThreads) {
        const int g = c / cpg;
        float a, bb;
        gn_scale_shift_of(mr[2 * g], mr[2 * g + 1], gamma ? gamma[c] : 1.0f,
                          beta ? beta[c] : 0.0f, a, bb);
        tab[c] = make_float2(a, bb);
    }
    __syncthreads();
    const int c0 = (threadIdx.x % CV) * V;
    float sc[V], sh[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const float2 q = tab[c0 + k];
        sc[k] = q.x;
        sh[k] = q.y;
    }
    // Streaming accesses: x is read once and y is next read by another kernel, long after the
    // caches have turned over, so both go with the nontemporal hint (measured 3% faster at the
    // decode's fp32 -> bf16 shapes; the hint on the stores alone or the loads alone is slower
    // than on both: 5.02-5.05 and 5.19-5.24 ms per decode against 4.84-4.85 ms).
    auto apply = [&](int e, const u32x4_t& raw) {
        const TI* v = reinterpret_cast<const TI*>(&raw);
        TO out[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const float x = Elem<TI>::load(v + k);
            // fp32 first, then the store's rounding (as a conv that normalises while staging)
            Elem<TO>::store(out + k, materialise_f32(silu ? gn_silu_apply(x, sc[k], sh[k])
                                                          : fmaf(x, sc[k], sh[k])));
        }
        if constexpr (sizeof(TO) * V == 16) {
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(out),
                                        reinterpret_cast<u32x4_t*>(yr + (int64_t)e * V));
        } else if constexpr (sizeof(TO) * V == 8) {
            __builtin_nontemporal_store(*reinterpret_cast<const u32x2_t*>(out),
                                        reinterpret_cast<u32x2_t*>(yr + (int64_t)e * V));
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) yr[(int64_t)e * V + k] = out[k];
        }
    };
#pragma unroll
    for (int u = 0; u < kApplyVec; ++u) {
        const int e = e0 + u * kThreads;
        if (e < seg) apply(e, raw[u]);
    }
}

// One thread per (sample, channel): the apply kernel's scale and shift, stored for a conv that
// normalises its input while staging it ([N][C][2] fp32).
__global__ __launch_bounds__(kThreads) void gn_scale_shift_kernel(
    const float* __restrict__ mean_rstd, int32_t C, int32_t groups, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* __restrict__ ab, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= total) return;
    const int64_t n = i / C;
    const int c = (int)(i - n * C);
    const int g = c / (C / groups);
    const float* mr = mean_rstd + n * groups * 2;
    const float gm = gamma ? gamma[c] : 1.0f;
    const float bt = beta ? beta[c] : 0.0f;
    gn_scale_shift_of(mr[2 * g], mr[2 * g + 1], gm, bt, ab[2 * i], ab[2 * i + 1]);
}

template <typename TI, typename TO>
void apply_launch(const vae_tensor_t& x, const Box& box, int32_t groups, const float* mean_rstd,
                  const float* gamma, const float* beta, bool silu, const vae_tensor_t& y,
                  hipStream_t stream) {
    constexpr int V = Elem<TI>::kVec;
    const int64_t seg = box.bw() * (x.c / V);
    const int32_t slices = (int32_t)ceil_div(seg, (int64_t)kApplySlice);
    dim3 grid((unsigned)(box.bt() * box.bh() * slices), (unsigned)x.n);
    hipLaunchKernelGGL((gn_apply_kernel<TI, TO>), grid, dim3(kThreads), 0, stream,
                       static_cast<const TI*>(x.data), static_cast<TO*>(y.data), (int32_t)x.t,
                       (int32_t)x.h, (int32_t)x.w, (int32_t)x.c, groups, box, slices, mean_rstd,
                       gamma, beta, (int32_t)silu);
}

}  // namespace

bool gn_shape_supported(const vae_tensor_t& x, int32_t groups) {
    const int64_t V = elem_size(x.dtype) == 2 ? 8 : 4;
    if (groups <= 0 || x.c % groups != 0 || x.c % V != 0) return false;
    const int64_t cv = x.c / V;
    if (cv > kThreads || kThreads % cv != 0) return false;
    const int64_t cpg = x.c / groups;
    return (V % cpg == 0) || (cpg % V == 0);
}

size_t gn_stats_workspace(const vae_tensor_t& x, const BoxList& boxes, int32_t groups) {
    GnBoxes g = make_boxes(x, boxes);
    return (size_t)g.start[g.n] * (size_t)x.n * (size_t)groups * 3 * sizeof(double);
}

vae_status_t launch_gn_stats(const vae_tensor_t& x, const BoxList& boxes, int32_t groups,
                             double* ws, double* part_out, float* mean_rstd, float eps,
                             hipStream_t stream, uint32_t* status) {
    GnBoxes g = make_boxes(x, boxes);
    dim3 grid((unsigned)g.start[g.n], (unsigned)x.n);
    if (x.dtype == VAE_DTYPE_BF16)
        hipLaunchKernelGGL(gn_stats_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(x.data), (int32_t)x.t, (int32_t)x.h,
                           (int32_t)x.w, (int32_t)x.c, groups, g, ws);
    else if (x.dtype == VAE_DTYPE_F16)
        hipLaunchKernelGGL(gn_stats_kernel<_Float16>, grid, dim3(kThreads), 0, stream,
                           static_cast<const _Float16*>(x.data), (int32_t)x.t, (int32_t)x.h,
                           (int32_t)x.w, (int32_t)x.c, groups, g, ws);
    else
        hipLaunchKernelGGL(gn_stats_kernel<float>, grid, dim3(kThreads), 0, stream,
                           static_cast<const float*>(x.data), (int32_t)x.t, (int32_t)x.h,
                           (int32_t)x.w, (int32_t)x.c, groups, g, ws);
    VAE_HIP_CHECK(hipGetLastError());
    hipLaunchKernelGGL(gn_finalize_kernel, dim3((unsigned)groups, (unsigned)x.n), dim3(kThreads),
                       0, stream, ws, g, groups, eps, part_out, mean_rstd, status);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

vae_status_t launch_gn_combine(const double* part, int32_t n_parts, int32_t n, int32_t groups,
                               float eps, float* mean_rstd, hipStream_t stream,
                               uint32_t* status) {
    hipLaunchKernelGGL(gn_combine_kernel, dim3((unsigned)groups, (unsigned)n), dim3(64), 0, stream,
                       part, n_parts, groups, eps, mean_rstd, status);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

vae_status_t launch_gn_finalize_slots(double* ws, int64_t slots, int32_t n, int32_t groups,
                                      float eps, float* mean_rstd, hipStream_t stream,
                                      uint32_t* status) {
    if (slots > INT32_MAX) return fail(VAE_ERR_UNSUPPORTED, "too many statistics slots");
    if (slots <= kSlotChunk) {
        hipLaunchKernelGGL(gn_finalize_slots_kernel, dim3((unsigned)groups, (unsigned)n),
                           dim3(kThreads), 0, stream, ws, slots, (int64_t)1, (int32_t)slots,
                           groups, eps, mean_rstd, status);
        VAE_HIP_CHECK(hipGetLastError());
        return VAE_OK;
    }
    const int64_t chunks = ceil_div(slots, kSlotChunk);
    hipLaunchKernelGGL(gn_slots_chunk_kernel, dim3((unsigned)chunks, (unsigned)groups, (unsigned)n),
                       dim3(kThreads), 0, stream, ws, slots, groups, (int32_t)kSlotChunk);
    VAE_HIP_CHECK(hipGetLastError());
    hipLaunchKernelGGL(gn_finalize_slots_kernel, dim3((unsigned)groups, (unsigned)n),
                       dim3(kThreads), 0, stream, ws, slots, kSlotChunk, (int32_t)chunks, groups,
                       eps, mean_rstd, status);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

vae_status_t launch_gn_scale_shift(const float* mean_rstd, int32_t n, int32_t c, int32_t groups,
                                   const float* gamma, const float* beta, float* ab,
                                   hipStream_t stream) {
    const int64_t total = (int64_t)n * c;
    if (total == 0) return VAE_OK;
    hipLaunchKernelGGL(gn_scale_shift_kernel, dim3((unsigned)ceil_div(total, kThreads)),
                       dim3(kThreads), 0, stream, mean_rstd, c, groups, gamma, beta, ab, total);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

vae_status_t launch_gn_apply(const vae_tensor_t& x, const Box& box, int32_t groups,
                             const float* mean_rstd, const float* gamma, const float* beta,
                             bool silu, const vae_tensor_t& y, hipStream_t stream) {
    if (box.volume() == 0 || x.n == 0) return VAE_OK;
    // blocks of the launch (fp32 input: 4 elements per vector, the most slices)
    if (box.bt() * box.bh() * ceil_div(box.bw() * (x.c / 4), (int64_t)kApplySlice) > INT32_MAX ||
        x.n > 65535 || x.c > kApplyMaxC)
        return fail(VAE_ERR_UNSUPPORTED, "group norm apply: grid too large");
    const bool xb = x.dtype == VAE_DTYPE_BF16, yb = y.dtype == VAE_DTYPE_BF16;
    if (x.dtype == VAE_DTYPE_F16) {   // an fp16 conv output (the middle of a residual block)
        if (y.dtype == VAE_DTYPE_F16)
            apply_launch<_Float16, _Float16>(x, box, groups, mean_rstd, gamma, beta, silu, y,
                                             stream);
        else if (yb)
            apply_launch<_Float16, uint16_t>(x, box, groups, mean_rstd, gamma, beta, silu, y,
                                             stream);
        else
            apply_launch<_Float16, float>(x, box, groups, mean_rstd, gamma, beta, silu, y, stream);
    } else if (y.dtype == VAE_DTYPE_F16) {   // the fp16 operand of the next conv
        if (xb)
            apply_launch<uint16_t, _Float16>(x, box, groups, mean_rstd, gamma, beta, silu, y,
                                             stream);
        else
            apply_launch<float, _Float16>(x, box, groups, mean_rstd, gamma, beta, silu, y, stream);
    } else if (xb && yb)
        apply_launch<uint16_t, uint16_t>(x, box, groups, mean_rstd, gamma, beta, silu, y, stream);
    else if (xb)
        apply_launch<uint16_t, float>(x, box, groups, mean_rstd, gamma, beta, silu, y, stream);
    else if (yb)
        apply_launch<float, uint16_t>(x, box, groups, mean_rstd, gamma, beta, silu, y, stream);
    else
        apply_launch<float, float>(x, box, groups, mean_rstd, gamma, beta, silu, y, stream);
    VAE_HIP_CHECK(hipGetLastError());
    return VAE_OK;
}

}  // namespace vae
