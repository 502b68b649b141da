// bf16 attention, head dim 128
// (explicit instantiations of the attention templates; one translation unit
// per variant so that the library builds in parallel)
#include "attend_impl.hpp"

namespace csa {
template hipError_t attend_variant<bf16, 128, false>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
template hipError_t combine_pair_variant<bf16, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, hipStream_t);
}  // namespace csa
