// weight rownorm+gain gradient: one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V>
static hipError_t run(const RownormGradArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rownorm_backward_kernel<G, V><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_rownorm_backward(Shape s, const RownormGradArgs& args, int grid,
                                   hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1>(args, grid, stream);
    case 102: return run<1, 2>(args, grid, stream);
    case 103: return run<1, 3>(args, grid, stream);
    case 104: return run<1, 4>(args, grid, stream);
    case 105: return run<1, 5>(args, grid, stream);
    case 106: return run<1, 6>(args, grid, stream);
    case 204: return run<2, 4>(args, grid, stream);
    case 205: return run<2, 5>(args, grid, stream);
    case 206: return run<2, 6>(args, grid, stream);
    case 404: return run<4, 4>(args, grid, stream);
    case 405: return run<4, 5>(args, grid, stream);
    case 406: return run<4, 6>(args, grid, stream);
    case 804: return run<8, 4>(args, grid, stream);
    case 805: return run<8, 5>(args, grid, stream);
    case 806: return run<8, 6>(args, grid, stream);
    case 1604: return run<16, 4>(args, grid, stream);
    case 1605: return run<16, 5>(args, grid, stream);
    case 1606: return run<16, 6>(args, grid, stream);
    case 1607: return run<16, 7>(args, grid, stream);
    case 1608: return run<16, 8>(args, grid, stream);
    case 1609: return run<16, 9>(args, grid, stream);
    case 1610: return run<16, 10>(args, grid, stream);
    case 1611: return run<16, 11>(args, grid, stream);
    case 1612: return run<16, 12>(args, grid, stream);
    case 1613: return run<16, 13>(args, grid, stream);
    case 1614: return run<16, 14>(args, grid, stream);
    case 1615: return run<16, 15>(args, grid, stream);
    case 1616: return run<16, 16>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
