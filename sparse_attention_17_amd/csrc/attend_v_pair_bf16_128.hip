// bf16 layer-pair attention in one launch, head dim 128
// (explicit instantiations of the attention templates; one translation unit
// per variant so that the library builds in parallel)
#include "attend_impl.hpp"

namespace csa {
template hipError_t pair_variant<bf16, 128>(const AttendArgs&, const AttnGeom&, const AttendArgs&, const AttnGeom&, int, hipStream_t);
}  // namespace csa
