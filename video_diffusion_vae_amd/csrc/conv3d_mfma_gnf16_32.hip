// MFMA conv kernels for NT = 32, fp16 input normalised to bf16 operands (a GroupNorm + SiLU
// applied while staging; see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST_GN(extern, 32, GnF16)
template vae_status_t run_mfma_out<32, GnF16, false>(const vae_tensor_t&, const void*,
                                                    const float*, const vae_tensor_t*,
                                                    const vae_tensor_t&, const Box&, bool,
                                                    const ConvFuse*, hipStream_t);
}  // namespace mfma
}  // namespace vae
