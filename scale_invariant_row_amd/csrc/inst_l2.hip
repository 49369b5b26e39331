// l2_rows: one launcher over every kernel shape pick_shape() can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V>
static hipError_t run(const void* x, const void* r, void* y, int64_t rows, int nvec, float eps,
                      int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  if (r != nullptr)
    l2_rows_kernel<G, V, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, (const u32x4_t*)r, (u32x4_t*)y, rows, nvec, eps);
  else
    l2_rows_kernel<G, V, false><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, nullptr, (u32x4_t*)y, rows, nvec, eps);
  return hipGetLastError();
}

hipError_t launch_l2_rows(Shape s, const void* x, const void* r, void* y, int64_t rows,
                          int nvec, float eps, int grid, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1>(x, r, y, rows, nvec, eps, grid, stream);
    case 102: return run<1, 2>(x, r, y, rows, nvec, eps, grid, stream);
    case 103: return run<1, 3>(x, r, y, rows, nvec, eps, grid, stream);
    case 104: return run<1, 4>(x, r, y, rows, nvec, eps, grid, stream);
    case 105: return run<1, 5>(x, r, y, rows, nvec, eps, grid, stream);
    case 106: return run<1, 6>(x, r, y, rows, nvec, eps, grid, stream);
    case 107: return run<1, 7>(x, r, y, rows, nvec, eps, grid, stream);
    case 108: return run<1, 8>(x, r, y, rows, nvec, eps, grid, stream);
    case 205: return run<2, 5>(x, r, y, rows, nvec, eps, grid, stream);
    case 206: return run<2, 6>(x, r, y, rows, nvec, eps, grid, stream);
    case 207: return run<2, 7>(x, r, y, rows, nvec, eps, grid, stream);
    case 208: return run<2, 8>(x, r, y, rows, nvec, eps, grid, stream);
    case 405: return run<4, 5>(x, r, y, rows, nvec, eps, grid, stream);
    case 406: return run<4, 6>(x, r, y, rows, nvec, eps, grid, stream);
    case 407: return run<4, 7>(x, r, y, rows, nvec, eps, grid, stream);
    case 408: return run<4, 8>(x, r, y, rows, nvec, eps, grid, stream);
    case 805: return run<8, 5>(x, r, y, rows, nvec, eps, grid, stream);
    case 806: return run<8, 6>(x, r, y, rows, nvec, eps, grid, stream);
    case 807: return run<8, 7>(x, r, y, rows, nvec, eps, grid, stream);
    case 808: return run<8, 8>(x, r, y, rows, nvec, eps, grid, stream);
    case 1605: return run<16, 5>(x, r, y, rows, nvec, eps, grid, stream);
    case 1606: return run<16, 6>(x, r, y, rows, nvec, eps, grid, stream);
    case 1607: return run<16, 7>(x, r, y, rows, nvec, eps, grid, stream);
    case 1608: return run<16, 8>(x, r, y, rows, nvec, eps, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
