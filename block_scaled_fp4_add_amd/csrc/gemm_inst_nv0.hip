// gemm_inst_nv0.hip -- instantiates the GEMM launchers for NVFP4 with the
// None and Bias epilogues (one compilation unit per pair).
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kNVFP4, kEpiNone>(const GemmArgs& g, int variant, hipStream_t s);
template hipError_t launch_fmt_epi<kNVFP4, kEpiBias>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
