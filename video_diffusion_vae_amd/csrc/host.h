// Host-side helpers shared between the ABI layer and the decode executor (not part of the C ABI).
#pragma once

#include <vector>

#include "kernels.h"

namespace vae {

vae_status_t check_tensor(const vae_tensor_t* t, const char* name);
vae_status_t check_tiling(const vae_tiling_desc_t* d);
bool overlaps(const vae_tensor_t& a, const vae_tensor_t& b);
std::vector<vae_tile_t> make_tiles(const vae_tiling_desc_t& d);
int32_t out_frames(int32_t t, int32_t scale_t);
// A space-to-depth fold (st, sh, sw) of x: factors >= 1 and extents it divides (T causally).
vae_status_t check_fold(const vae_tensor_t& x, int32_t st, int32_t sh, int32_t sw);
// Whether a tiling desc is an encoder's (down_* > 1): its tile grid is on the output grid.
bool encodes(const vae_tiling_desc_t& d);
// Output extents of a tiling desc (decoder: scaled up, causal T; encoder: folded down).
void desc_out_extents(const vae_tiling_desc_t& d, int32_t* t, int32_t* h, int32_t* w);
// The T, H and W axes of a mode-B tiling (T causal).
void overlap_axes(const vae_tiling_desc_t& d, AxisTiling ax[3]);
size_t gn_full_workspace(const vae_tensor_t& x, const BoxList& bl, int32_t groups);

}  // namespace vae
