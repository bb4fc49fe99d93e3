// gemm_inst_mx3.hip -- instantiates the GEMM launchers for MXFP4 with the FP8-output
// epilogue.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kMXFP4, kEpiFp8>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
