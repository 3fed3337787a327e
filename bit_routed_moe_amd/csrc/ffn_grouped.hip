// Prefill expert FFN (bf16 path): grouped GEMM on the matrix cores.
#include "formats.hpp"
#include "launch.hpp"

namespace ds4 {

hipError_t launch_ffn_grouped_bf16(const FfnArgs&, bool, bool, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ds4
