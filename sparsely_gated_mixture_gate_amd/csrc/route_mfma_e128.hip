// route_mfma_e128.hip -- instantiates the certified MFMA gate (route_mfma.h) for
// 128 padded experts, plain gate.
#include "route_mfma.h"

namespace moe {
template hipError_t launch_fused_kk<128, false>(int, const FusedArgs&, hipStream_t);
}  // namespace moe
