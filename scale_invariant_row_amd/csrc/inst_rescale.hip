// rescale method (projection; rescale after a step): one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V, bool RESCALE>
static hipError_t run(const RescaleArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rescale_kernel<G, V, RESCALE><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_rescale_project(Shape s, const RescaleArgs& args, int grid, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1, false>(args, grid, stream);
    case 102: return run<1, 2, false>(args, grid, stream);
    case 103: return run<1, 3, false>(args, grid, stream);
    case 104: return run<1, 4, false>(args, grid, stream);
    case 105: return run<1, 5, false>(args, grid, stream);
    case 106: return run<1, 6, false>(args, grid, stream);
    case 204: return run<2, 4, false>(args, grid, stream);
    case 205: return run<2, 5, false>(args, grid, stream);
    case 206: return run<2, 6, false>(args, grid, stream);
    case 404: return run<4, 4, false>(args, grid, stream);
    case 405: return run<4, 5, false>(args, grid, stream);
    case 406: return run<4, 6, false>(args, grid, stream);
    case 804: return run<8, 4, false>(args, grid, stream);
    case 805: return run<8, 5, false>(args, grid, stream);
    case 806: return run<8, 6, false>(args, grid, stream);
    case 1604: return run<16, 4, false>(args, grid, stream);
    case 1605: return run<16, 5, false>(args, grid, stream);
    case 1606: return run<16, 6, false>(args, grid, stream);
    case 1607: return run<16, 7, false>(args, grid, stream);
    case 1608: return run<16, 8, false>(args, grid, stream);
    case 1609: return run<16, 9, false>(args, grid, stream);
    case 1610: return run<16, 10, false>(args, grid, stream);
    case 1611: return run<16, 11, false>(args, grid, stream);
    case 1612: return run<16, 12, false>(args, grid, stream);
    case 1613: return run<16, 13, false>(args, grid, stream);
    case 1614: return run<16, 14, false>(args, grid, stream);
    case 1615: return run<16, 15, false>(args, grid, stream);
    case 1616: return run<16, 16, false>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rescale_after_step(Shape s, const RescaleArgs& args, int grid,
                                     hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1, true>(args, grid, stream);
    case 102: return run<1, 2, true>(args, grid, stream);
    case 103: return run<1, 3, true>(args, grid, stream);
    case 104: return run<1, 4, true>(args, grid, stream);
    case 105: return run<1, 5, true>(args, grid, stream);
    case 106: return run<1, 6, true>(args, grid, stream);
    case 204: return run<2, 4, true>(args, grid, stream);
    case 205: return run<2, 5, true>(args, grid, stream);
    case 206: return run<2, 6, true>(args, grid, stream);
    case 404: return run<4, 4, true>(args, grid, stream);
    case 405: return run<4, 5, true>(args, grid, stream);
    case 406: return run<4, 6, true>(args, grid, stream);
    case 804: return run<8, 4, true>(args, grid, stream);
    case 805: return run<8, 5, true>(args, grid, stream);
    case 806: return run<8, 6, true>(args, grid, stream);
    case 1604: return run<16, 4, true>(args, grid, stream);
    case 1605: return run<16, 5, true>(args, grid, stream);
    case 1606: return run<16, 6, true>(args, grid, stream);
    case 1607: return run<16, 7, true>(args, grid, stream);
    case 1608: return run<16, 8, true>(args, grid, stream);
    case 1609: return run<16, 9, true>(args, grid, stream);
    case 1610: return run<16, 10, true>(args, grid, stream);
    case 1611: return run<16, 11, true>(args, grid, stream);
    case 1612: return run<16, 12, true>(args, grid, stream);
    case 1613: return run<16, 13, true>(args, grid, stream);
    case 1614: return run<16, 14, true>(args, grid, stream);
    case 1615: return run<16, 15, true>(args, grid, stream);
    case 1616: return run<16, 16, true>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
