// MFMA conv kernels with the narrow block shapes for NT = 64, fp16 input normalised to bf16
// operands (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST_GN(, 64, GnF16)
}  // namespace mfma
}  // namespace vae
