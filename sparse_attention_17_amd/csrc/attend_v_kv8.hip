// attention over FP8 caches with a bf16 RoPE half, head dim 128
// (explicit instantiations of the attention templates; one translation unit
// per variant so that the library builds in parallel)
#include "attend_impl.hpp"

namespace csa {
template hipError_t attend_variant<bf16, 128, true>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
}  // namespace csa
