// route_mfma_e64_noisy.hip -- instantiates the certified MFMA gate (route_mfma.h) for
// 64 padded experts, noisy gate (gate and noise columns).
#include "route_mfma.h"

namespace moe {
template hipError_t launch_fused_kk<64, true>(int, const FusedArgs&, hipStream_t);
}  // namespace moe
