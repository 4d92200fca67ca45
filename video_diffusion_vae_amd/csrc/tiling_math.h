// Tile-grid index maths used by the host split (vae_tile_split) and by the merge kernels.
//
// Overlap tiles along one axis of L latent rows: starts 0, s, 2s, ... < L, each min(tile, L-start)
// rows long. An axis with L <= tile is left whole ("[Feature] Support VAE tiling parallel encode for
// LTX-2", review thread). Blend ramps over the overlap E of consecutive tiles: the later tile
// rises as (j+1)/(E+1), the earlier falls as (E-j)/(E+1) ("[TRTLLM-14029][feat] LTX-2 tile-parallel
// VAE decode", Approach: a blend mask from per-axis parts, a weight buffer, a divide).
//
// Output spans. A spatial span of latent rows [s, s + n) decodes to [s * r, (s + n) * r). The
// temporal axis is causal: a clip of n latent frames decodes to 1 + (n - 1) * r frames, since its
// first latent frame yields one frame, and the clip [s, s + n) lands on output frames
// [s * r, (s + n - 1) * r + 1) (its single first frame stands for the last frame of latent frame s
// in the whole decode). Overlaps are taken between the output spans of neighbouring tiles.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace vae {

struct AxisTiling {
    int32_t length;  // latent rows
    int32_t tile;    // latent rows per tile (<= 0: the axis is not cut)
    int32_t stride;  // latent rows between tile starts
    int32_t scale;   // output samples per latent row
    int32_t causal;  // 1: the temporal axis of a causal decoder (see the output spans above)
};

__host__ __device__ inline bool axis_is_cut(const AxisTiling& a) {
    return a.tile > 0 && a.length > a.tile;
}

__host__ __device__ inline int32_t axis_count(const AxisTiling& a) {
    return axis_is_cut(a) ? (a.length + a.stride - 1) / a.stride : 1;
}

__host__ __device__ inline void axis_span(const AxisTiling& a, int32_t i, int32_t* start,
                                          int32_t* size) {
    if (!axis_is_cut(a)) {
        *start = 0;
        *size = a.length;
        return;
    }
    int32_t s = i * a.stride;
    int32_t rem = a.length - s;
    *start = s;
    *size = rem < a.tile ? rem : a.tile;
}

// Output span [*lo, *lo + *len) of tile i.
__host__ __device__ inline void axis_out_span(const AxisTiling& a, int32_t i, int32_t* lo,
                                              int32_t* len) {
    int32_t s, n;
    axis_span(a, i, &s, &n);
    *lo = s * a.scale;
    *len = a.causal ? 1 + (n - 1) * a.scale : n * a.scale;
}

// Overlap (output samples) of tile i with tile i-1 (lead) and with tile i+1 (trail).
__host__ __device__ inline int32_t axis_lead(const AxisTiling& a, int32_t i) {
    if (i <= 0) return 0;
    int32_t lo0, n0, lo1, n1;
    axis_out_span(a, i - 1, &lo0, &n0);
    axis_out_span(a, i, &lo1, &n1);
    const int32_t e = lo0 + n0 - lo1;
    return e > 0 ? e : 0;
}

__host__ __device__ inline int32_t axis_trail(const AxisTiling& a, int32_t i) {
    if (i + 1 >= axis_count(a)) return 0;
    int32_t lo0, n0, lo1, n1;
    axis_out_span(a, i, &lo0, &n0);
    axis_out_span(a, i + 1, &lo1, &n1);
    const int32_t e = lo0 + n0 - lo1;
    return e > 0 ? e : 0;
}

// Weight at sample j of a tile that is `size` output samples long.
__host__ __device__ inline float ramp_weight(int32_t j, int32_t size, int32_t lead, int32_t trail) {
    float w = 1.0f;
    if (j < lead) w *= (float)(j + 1) / (float)(lead + 1);
    if (size - j <= trail) w *= (float)(size - j) / (float)(trail + 1);
    return w;
}

// Sum over the tiles of this axis of their ramps at output sample x.
__host__ __device__ inline float axis_weight_sum(const AxisTiling& a, int32_t x) {
    float s = 0.0f;
    int32_t n = axis_count(a);
    for (int32_t i = 0; i < n; ++i) {
        int32_t lo, len;
        axis_out_span(a, i, &lo, &len);
        if (x >= lo && x < lo + len) s += ramp_weight(x - lo, len, axis_lead(a, i), axis_trail(a, i));
    }
    return s;
}

}  // namespace vae
