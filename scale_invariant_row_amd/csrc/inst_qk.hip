// q/k rows: RoPE, per-head L2, q scale (head_dim 128 or 256).
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

hipError_t launch_qk_rows_l2(int head_dim, const QkArgs& args, int grid, hipStream_t stream) {
  if (head_dim == 256)
    qk_rows_l2_kernel<256><<<grid, 256, 0, stream>>>(args);
  else if (head_dim == 128)
    qk_rows_l2_kernel<128><<<grid, 256, 0, stream>>>(args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsr
