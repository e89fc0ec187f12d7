// route_mfma_e64.hip -- instantiates the certified MFMA gate (route_mfma.h) for
// 64 padded experts, plain gate.
#include "route_mfma.h"

namespace moe {
template hipError_t launch_fused_kk<64, false>(int, const FusedArgs&, hipStream_t);
}  // namespace moe
