// MFMA conv kernels with the narrow block shapes for NT = 128, fp32 input (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST(, 128, float, false)
}  // namespace mfma
}  // namespace vae
