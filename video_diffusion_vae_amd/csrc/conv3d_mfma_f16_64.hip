// MFMA conv kernels for NT = 64, fp16 input (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST_F16(extern, 64, _Float16, false)
template vae_status_t run_mfma_out<64, _Float16, false>(const vae_tensor_t&, const void*, const float*,
                                                   const vae_tensor_t*, const vae_tensor_t&,
                                                   const Box&, bool, const ConvFuse*, hipStream_t);
}  // namespace mfma
}  // namespace vae
