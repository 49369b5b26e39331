// Launchers of the column-block weight kernels (one instance per op).
#include "colblock_kernels.hpp"
#include "launch.hpp"

namespace dsr {

hipError_t launch_colblock_rownorm(const TaskArgs<RownormTask>& args, int grid,
                                   hipStream_t stream) {
  colblock_kernel<ColOp::kFwd><<<grid, kColThreads, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_colblock_rownorm_backward(const TaskArgs<RownormGradTask>& args, int grid,
                                            hipStream_t stream) {
  colblock_kernel<ColOp::kBwd><<<grid, kColThreads, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_colblock_rescale(bool after_step, const TaskArgs<RescaleTask>& args, int grid,
                                   hipStream_t stream) {
  if (after_step)
    colblock_kernel<ColOp::kAfterStep><<<grid, kColThreads, 0, stream>>>(args);
  else
    colblock_kernel<ColOp::kProject><<<grid, kColThreads, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_colblock1_rownorm(const TaskArgs<RownormTask>& args, int grid,
                                    hipStream_t stream) {
  colblock1_kernel<ColOp::kFwd, kCol1KFwd, kCol1LanesFwd><<<grid, kColThreads, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_colblock1_rownorm_backward(const TaskArgs<RownormGradTask>& args, int grid,
                                             hipStream_t stream) {
  colblock1_kernel<ColOp::kBwd, kCol1KBwd, kCol1LanesBwd><<<grid, kColThreads, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_colblock1_rescale(bool after_step, const TaskArgs<RescaleTask>& args, int grid,
                                    hipStream_t stream) {
  if (after_step)
    colblock1_kernel<ColOp::kAfterStep, kCol1KRescale, kCol1LanesRescale><<<grid, kColThreads, 0, stream>>>(args);
  else
    colblock1_kernel<ColOp::kProject, kCol1KRescale, kCol1LanesRescale><<<grid, kColThreads, 0, stream>>>(args);
  return hipGetLastError();
}

}  // namespace dsr
