// MFMA conv kernels with the narrow block shapes for NT = 64,
// fp32 input split into bf16 hi + lo (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST(, 64, float, true)
}  // namespace mfma
}  // namespace vae
