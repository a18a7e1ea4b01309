// index_score.hip -- placeholder until the nvfp4 index scorer lands.
#include "uq_kernels.h"
namespace uq {
hipError_t launch_index_score(const IndexArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace uq
