// kda_bwd.hip -- backward pass (placeholder while the forward is brought up).
#include "kda_internal.hpp"

namespace kda {
template <typename E, int DK, int DV>
hipError_t launch_bwd(const Args&, hipStream_t) { return hipErrorNotSupported; }
#define KDA_INST(E, DK, DV) template hipError_t launch_bwd<E, DK, DV>(const Args&, hipStream_t);
KDA_INST(bf16, 64, 64)
KDA_INST(bf16, 64, 128)
KDA_INST(bf16, 128, 64)
KDA_INST(bf16, 128, 128)
KDA_INST(float, 64, 64)
KDA_INST(float, 64, 128)
KDA_INST(float, 128, 64)
KDA_INST(float, 128, 128)
}  // namespace kda
