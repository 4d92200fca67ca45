// MFMA conv kernels with the narrow block shapes for NT = 32, bf16 input (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST_F16(, 32, uint16_t, false)
}  // namespace mfma
}  // namespace vae
