// The grouped GEMMs for 3-bit codes (the templates of gemm_impl.h).
#include "gemm_impl.h"

namespace moe {

template hipError_t launch_gateup_gemm_bits<3>(const Ctx& c);
template hipError_t launch_down_gemm_bits<3>(const Ctx& c);

}  // namespace moe
