// route_mfma_e256.hip -- instantiates the certified MFMA gate (route_mfma.h) for
// 256 padded experts, plain gate.
#include "route_mfma.h"

namespace moe {
template hipError_t launch_fused_kk<256, false>(int, const FusedArgs&, hipStream_t);
}  // namespace moe
