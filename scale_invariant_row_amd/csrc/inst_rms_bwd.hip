// rms_rows gradient (l2_rows' gradient kernel with the mean): one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V>
static hipError_t run(const void* x, const void* r, const void* dy, void* dx, int64_t rows,
                      int nvec, float eps, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  if (r != nullptr)
    l2_rows_backward_kernel<G, V, true, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, (const u32x4_t*)r, (const u32x4_t*)dy, (u32x4_t*)dx, rows, nvec, eps);
  else
    l2_rows_backward_kernel<G, V, false, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, nullptr, (const u32x4_t*)dy, (u32x4_t*)dx, rows, nvec, eps);
  return hipGetLastError();
}

hipError_t launch_rms_rows_backward(Shape s, const void* x, const void* r, const void* dy,
                                    void* dx, int64_t rows, int nvec, float eps, int grid,
                                    hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 102: return run<1, 2>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 202: return run<2, 2>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 402: return run<4, 2>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 403: return run<4, 3>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 404: return run<4, 4>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 803: return run<8, 3>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 804: return run<8, 4>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 1603: return run<16, 3>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 1604: return run<16, 4>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 1605: return run<16, 5>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 1606: return run<16, 6>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 1607: return run<16, 7>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    case 1608: return run<16, 8>(x, r, dy, dx, rows, nvec, eps, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
