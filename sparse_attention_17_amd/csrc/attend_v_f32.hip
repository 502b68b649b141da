// fp32 attention, head dims 64 and 128
// (explicit instantiations of the attention templates; one translation unit
// per variant so that the library builds in parallel)
#include "attend_impl.hpp"

namespace csa {
template hipError_t attend_variant<float, 64, false>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
template hipError_t attend_variant<float, 128, false>(const AttendArgs&, const AttnGeom&, const AttendLaunch&, hipStream_t);
template hipError_t pair_variant<float, 64>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, int, hipStream_t);
template hipError_t pair_variant<float, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, int, hipStream_t);
template hipError_t combine_pair_variant<float, 64>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, hipStream_t);
template hipError_t combine_pair_variant<float, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, hipStream_t);
}  // namespace csa
