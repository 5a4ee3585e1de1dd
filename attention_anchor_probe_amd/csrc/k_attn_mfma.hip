// bf16 MFMA attention kernels (gfx950), head_dim 128.
#include "acache_dev.h"
#include "acache_launch.h"

namespace acache {

bool mfma_supported(int dtype, int head_dim) { (void)dtype; (void)head_dim; return false; }
hipError_t launch_attn_mfma(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_colmass_mfma(const ColmassArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace acache
