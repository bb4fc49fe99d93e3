// gemm_inst_nv3.hip -- instantiates the GEMM launchers for NVFP4 with the FP8-output
// epilogue.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kNVFP4, kEpiFp8>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
