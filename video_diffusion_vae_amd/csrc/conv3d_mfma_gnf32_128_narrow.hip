// MFMA conv kernels with the narrow block shapes for NT = 128, fp32 input normalised to bf16
// operands (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST_GN(, 128, GnF32)
}  // namespace mfma
}  // namespace vae
