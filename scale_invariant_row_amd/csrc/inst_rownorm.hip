// weight rownorm+gain: one launcher over every kernel shape pick_shape() can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V>
static hipError_t run(const RownormTask* tasks, int ntasks, int nitems, int grid,
                      hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rownorm_kernel<G, V><<<grid, T, 0, stream>>>(tasks, ntasks, nitems);
  return hipGetLastError();
}

hipError_t launch_rownorm(Shape s, const RownormTask* tasks, int ntasks, int nitems, int grid,
                          hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1>(tasks, ntasks, nitems, grid, stream);
    case 102: return run<1, 2>(tasks, ntasks, nitems, grid, stream);
    case 103: return run<1, 3>(tasks, ntasks, nitems, grid, stream);
    case 104: return run<1, 4>(tasks, ntasks, nitems, grid, stream);
    case 105: return run<1, 5>(tasks, ntasks, nitems, grid, stream);
    case 106: return run<1, 6>(tasks, ntasks, nitems, grid, stream);
    case 107: return run<1, 7>(tasks, ntasks, nitems, grid, stream);
    case 108: return run<1, 8>(tasks, ntasks, nitems, grid, stream);
    case 109: return run<1, 9>(tasks, ntasks, nitems, grid, stream);
    case 110: return run<1, 10>(tasks, ntasks, nitems, grid, stream);
    case 111: return run<1, 11>(tasks, ntasks, nitems, grid, stream);
    case 112: return run<1, 12>(tasks, ntasks, nitems, grid, stream);
    case 207: return run<2, 7>(tasks, ntasks, nitems, grid, stream);
    case 208: return run<2, 8>(tasks, ntasks, nitems, grid, stream);
    case 209: return run<2, 9>(tasks, ntasks, nitems, grid, stream);
    case 210: return run<2, 10>(tasks, ntasks, nitems, grid, stream);
    case 211: return run<2, 11>(tasks, ntasks, nitems, grid, stream);
    case 212: return run<2, 12>(tasks, ntasks, nitems, grid, stream);
    case 407: return run<4, 7>(tasks, ntasks, nitems, grid, stream);
    case 408: return run<4, 8>(tasks, ntasks, nitems, grid, stream);
    case 409: return run<4, 9>(tasks, ntasks, nitems, grid, stream);
    case 410: return run<4, 10>(tasks, ntasks, nitems, grid, stream);
    case 411: return run<4, 11>(tasks, ntasks, nitems, grid, stream);
    case 412: return run<4, 12>(tasks, ntasks, nitems, grid, stream);
    case 807: return run<8, 7>(tasks, ntasks, nitems, grid, stream);
    case 808: return run<8, 8>(tasks, ntasks, nitems, grid, stream);
    case 809: return run<8, 9>(tasks, ntasks, nitems, grid, stream);
    case 810: return run<8, 10>(tasks, ntasks, nitems, grid, stream);
    case 811: return run<8, 11>(tasks, ntasks, nitems, grid, stream);
    case 812: return run<8, 12>(tasks, ntasks, nitems, grid, stream);
    case 1607: return run<16, 7>(tasks, ntasks, nitems, grid, stream);
    case 1608: return run<16, 8>(tasks, ntasks, nitems, grid, stream);
    case 1609: return run<16, 9>(tasks, ntasks, nitems, grid, stream);
    case 1610: return run<16, 10>(tasks, ntasks, nitems, grid, stream);
    case 1611: return run<16, 11>(tasks, ntasks, nitems, grid, stream);
    case 1612: return run<16, 12>(tasks, ntasks, nitems, grid, stream);
    case 1613: return run<16, 13>(tasks, ntasks, nitems, grid, stream);
    case 1614: return run<16, 14>(tasks, ntasks, nitems, grid, stream);
    case 1615: return run<16, 15>(tasks, ntasks, nitems, grid, stream);
    case 1616: return run<16, 16>(tasks, ntasks, nitems, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
