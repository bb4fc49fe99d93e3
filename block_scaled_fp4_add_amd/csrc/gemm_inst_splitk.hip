// gemm_inst_splitk.hip -- split-K launchers (decode schedule with K split across workgroups) for
// NVFP4 and MXFP4 operands, every epilogue (one compilation unit).
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_splitk<kNVFP4, kEpiNone>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBias>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBiasResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBiasGelu>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBiasGeluFp4>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiFp8>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiNone>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBias>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBiasResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBiasGelu>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBiasGeluFp4>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiFp8>(const GemmArgs& g, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
