// slerp_rows: one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V>
static hipError_t run(const void* res, const void* out, const float* alpha, void* h,
                      int64_t rows, int nvec, float eps, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  slerp_rows_kernel<G, V><<<grid, T, 0, stream>>>(
      (const u32x4_t*)res, (const u32x4_t*)out, (const f32x4_t*)alpha, (u32x4_t*)h, rows, nvec,
      eps);
  return hipGetLastError();
}

hipError_t launch_slerp_rows(Shape s, const void* res, const void* out, const float* alpha,
                             void* h, int64_t rows, int nvec, float eps, int grid,
                             hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 102: return run<1, 2>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 202: return run<2, 2>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 402: return run<4, 2>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 403: return run<4, 3>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 404: return run<4, 4>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 803: return run<8, 3>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 804: return run<8, 4>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 1603: return run<16, 3>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 1604: return run<16, 4>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 1605: return run<16, 5>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 1606: return run<16, 6>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 1607: return run<16, 7>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    case 1608: return run<16, 8>(res, out, alpha, h, rows, nvec, eps, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
