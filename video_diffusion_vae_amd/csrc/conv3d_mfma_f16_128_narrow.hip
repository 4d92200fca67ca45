// MFMA conv kernels with the narrow block shapes for NT = 128, fp16 input (see conv3d_mfma.h).
#include "conv3d_mfma.h"

namespace vae {
namespace mfma {
VAE_NARROW_INST_F16(, 128, _Float16, false)
}  // namespace mfma
}  // namespace vae
