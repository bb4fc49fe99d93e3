// gemm_inst_splitk8.hip -- split-K launchers for MXFP8 operands, every epilogue.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_splitk<kMXFP8, kEpiNone>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP8, kEpiBias>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP8, kEpiResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP8, kEpiBiasResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP8, kEpiBiasGelu>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP8, kEpiBiasGeluFp4>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP8, kEpiFp8>(const GemmArgs& g, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
