// The grouped GEMMs for 2-bit codes (the templates of gemm_impl.h).
#include "gemm_impl.h"

namespace moe {

template hipError_t launch_gateup_gemm_bits<2>(const Ctx& c);
template hipError_t launch_down_gemm_bits<2>(const Ctx& c);

}  // namespace moe
