// MFMA conv kernels with the narrow block shapes for NT = 32, fp32 input normalised to fp16
// operands (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST_GN(, 32, GnF32H)
}  // namespace mfma
}  // namespace vae
