// weight rownorm+gain gradient: one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V, int NE>
static hipError_t run(const RownormGradArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rownorm_backward_kernel<G, V, NE><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}


__global__ void __launch_bounds__(128) rownorm_backward_mixed_128(const RownormGradArgs args) {
  __shared__ GroupScratch<2> gs2;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x) {
    const RownormGradTask t = task_of(args, item, (int)(threadIdx.x & 63));
    switch (t.shape) {
      case 40204: rownorm_backward_item<2, 4, 4>(t, item, Geo<2>::per_item(), gs2, slot); break;
      case 40205: rownorm_backward_item<2, 5, 4>(t, item, Geo<2>::per_item(), gs2, slot); break;
      case 40206: rownorm_backward_item<2, 6, 4>(t, item, Geo<2>::per_item(), gs2, slot); break;
      case 10216: rownorm_backward_item<2, 16, 1>(t, item, Geo<2>::per_item(), gs2, slot); break;
      default: break;
    }
  }
}

__global__ void __launch_bounds__(256) rownorm_backward_mixed_256(const RownormGradArgs args) {
  __shared__ GroupScratch<1> gs1;
  __shared__ GroupScratch<4> gs4;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x) {
    const RownormGradTask t = task_of(args, item, (int)(threadIdx.x & 63));
    switch (t.shape) {
      case 40101: rownorm_backward_item<1, 1, 4>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40102: rownorm_backward_item<1, 2, 4>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40103: rownorm_backward_item<1, 3, 4>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40104: rownorm_backward_item<1, 4, 4>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40105: rownorm_backward_item<1, 5, 4>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40106: rownorm_backward_item<1, 6, 4>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40404: rownorm_backward_item<4, 4, 4>(t, item, Geo<4>::per_item(), gs4, slot); break;
      case 40405: rownorm_backward_item<4, 5, 4>(t, item, Geo<4>::per_item(), gs4, slot); break;
      case 40406: rownorm_backward_item<4, 6, 4>(t, item, Geo<4>::per_item(), gs4, slot); break;
      case 10101: rownorm_backward_item<1, 1, 1>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10102: rownorm_backward_item<1, 2, 1>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10104: rownorm_backward_item<1, 4, 1>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10108: rownorm_backward_item<1, 8, 1>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10116: rownorm_backward_item<1, 16, 1>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10416: rownorm_backward_item<4, 16, 1>(t, item, Geo<4>::per_item(), gs4, slot); break;
      default: break;
    }
  }
}

__global__ void __launch_bounds__(512) rownorm_backward_mixed_512(const RownormGradArgs args) {
  __shared__ GroupScratch<8> gs8;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x) {
    const RownormGradTask t = task_of(args, item, (int)(threadIdx.x & 63));
    switch (t.shape) {
      case 40804: rownorm_backward_item<8, 4, 4>(t, item, Geo<8>::per_item(), gs8, slot); break;
      case 40805: rownorm_backward_item<8, 5, 4>(t, item, Geo<8>::per_item(), gs8, slot); break;
      case 40806: rownorm_backward_item<8, 6, 4>(t, item, Geo<8>::per_item(), gs8, slot); break;
      case 10816: rownorm_backward_item<8, 16, 1>(t, item, Geo<8>::per_item(), gs8, slot); break;
      default: break;
    }
  }
}

// The classes of a ragged call that share a workgroup size, in one launch.
static hipError_t run_mixed(int threads, const RownormGradArgs& args, int grid, hipStream_t stream) {
  switch (threads) {
    case 128: rownorm_backward_mixed_128<<<grid, 128, 0, stream>>>(args); break;
    case 256: rownorm_backward_mixed_256<<<grid, 256, 0, stream>>>(args); break;
    case 512: rownorm_backward_mixed_512<<<grid, 512, 0, stream>>>(args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rownorm_backward(Shape s, const RownormGradArgs& args, int grid,
                                   hipStream_t stream) {
  if (s.mixed > 0) return run_mixed(s.mixed, args, grid, stream);
  switch (s.key()) {
    case 40101: return run<1, 1, 4>(args, grid, stream);
    case 40102: return run<1, 2, 4>(args, grid, stream);
    case 40103: return run<1, 3, 4>(args, grid, stream);
    case 40104: return run<1, 4, 4>(args, grid, stream);
    case 40105: return run<1, 5, 4>(args, grid, stream);
    case 40106: return run<1, 6, 4>(args, grid, stream);
    case 40204: return run<2, 4, 4>(args, grid, stream);
    case 40205: return run<2, 5, 4>(args, grid, stream);
    case 40206: return run<2, 6, 4>(args, grid, stream);
    case 40404: return run<4, 4, 4>(args, grid, stream);
    case 40405: return run<4, 5, 4>(args, grid, stream);
    case 40406: return run<4, 6, 4>(args, grid, stream);
    case 40804: return run<8, 4, 4>(args, grid, stream);
    case 40805: return run<8, 5, 4>(args, grid, stream);
    case 40806: return run<8, 6, 4>(args, grid, stream);
    case 41604: return run<16, 4, 4>(args, grid, stream);
    case 41605: return run<16, 5, 4>(args, grid, stream);
    case 41606: return run<16, 6, 4>(args, grid, stream);
    case 41607: return run<16, 7, 4>(args, grid, stream);
    case 41608: return run<16, 8, 4>(args, grid, stream);
    case 41609: return run<16, 9, 4>(args, grid, stream);
    case 41610: return run<16, 10, 4>(args, grid, stream);
    case 41611: return run<16, 11, 4>(args, grid, stream);
    case 41612: return run<16, 12, 4>(args, grid, stream);
    case 41613: return run<16, 13, 4>(args, grid, stream);
    case 41614: return run<16, 14, 4>(args, grid, stream);
    case 41615: return run<16, 15, 4>(args, grid, stream);
    case 41616: return run<16, 16, 4>(args, grid, stream);
    case 10101: return run<1, 1, 1>(args, grid, stream);
    case 10102: return run<1, 2, 1>(args, grid, stream);
    case 10104: return run<1, 4, 1>(args, grid, stream);
    case 10108: return run<1, 8, 1>(args, grid, stream);
    case 10116: return run<1, 16, 1>(args, grid, stream);
    case 10216: return run<2, 16, 1>(args, grid, stream);
    case 10416: return run<4, 16, 1>(args, grid, stream);
    case 10816: return run<8, 16, 1>(args, grid, stream);
    case 11616: return run<16, 16, 1>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
