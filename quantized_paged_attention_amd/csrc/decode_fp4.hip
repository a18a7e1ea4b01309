// decode_fp4.hip -- placeholder until the FP4 D=256 kernel lands.
#include "uq_kernels.h"
namespace uq {
hipError_t launch_decode_fp4(const DecodeArgs&, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace uq
