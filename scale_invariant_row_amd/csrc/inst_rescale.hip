// rescale method (projection; rescale after a step): one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V, int NE, bool RESCALE>
static hipError_t run(const RescaleArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rescale_kernel<G, V, NE, RESCALE><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}


template <bool RESCALE>
__global__ void __launch_bounds__(128) rescale_mixed_128(const RescaleArgs args) {
  __shared__ GroupScratch<2> gs2;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x) {
    const RescaleTask t = task_of(args, item, (int)(threadIdx.x & 63));
    switch (t.shape) {
      case 40204: rescale_item<2, 4, 4, RESCALE>(t, item, Geo<2>::per_item(), gs2, slot); break;
      case 40205: rescale_item<2, 5, 4, RESCALE>(t, item, Geo<2>::per_item(), gs2, slot); break;
      case 40206: rescale_item<2, 6, 4, RESCALE>(t, item, Geo<2>::per_item(), gs2, slot); break;
      case 10216: rescale_item<2, 16, 1, RESCALE>(t, item, Geo<2>::per_item(), gs2, slot); break;
      default: break;
    }
  }
}

template <bool RESCALE>
__global__ void __launch_bounds__(256) rescale_mixed_256(const RescaleArgs args) {
  __shared__ GroupScratch<1> gs1;
  __shared__ GroupScratch<4> gs4;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x) {
    const RescaleTask t = task_of(args, item, (int)(threadIdx.x & 63));
    switch (t.shape) {
      case 40101: rescale_item<1, 1, 4, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40102: rescale_item<1, 2, 4, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40103: rescale_item<1, 3, 4, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40104: rescale_item<1, 4, 4, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40105: rescale_item<1, 5, 4, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40106: rescale_item<1, 6, 4, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 40404: rescale_item<4, 4, 4, RESCALE>(t, item, Geo<4>::per_item(), gs4, slot); break;
      case 40405: rescale_item<4, 5, 4, RESCALE>(t, item, Geo<4>::per_item(), gs4, slot); break;
      case 40406: rescale_item<4, 6, 4, RESCALE>(t, item, Geo<4>::per_item(), gs4, slot); break;
      case 10101: rescale_item<1, 1, 1, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10102: rescale_item<1, 2, 1, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10104: rescale_item<1, 4, 1, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10108: rescale_item<1, 8, 1, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10116: rescale_item<1, 16, 1, RESCALE>(t, item, Geo<1>::per_item(), gs1, slot); break;
      case 10416: rescale_item<4, 16, 1, RESCALE>(t, item, Geo<4>::per_item(), gs4, slot); break;
      default: break;
    }
  }
}

template <bool RESCALE>
__global__ void __launch_bounds__(512) rescale_mixed_512(const RescaleArgs args) {
  __shared__ GroupScratch<8> gs8;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x) {
    const RescaleTask t = task_of(args, item, (int)(threadIdx.x & 63));
    switch (t.shape) {
      case 40804: rescale_item<8, 4, 4, RESCALE>(t, item, Geo<8>::per_item(), gs8, slot); break;
      case 40805: rescale_item<8, 5, 4, RESCALE>(t, item, Geo<8>::per_item(), gs8, slot); break;
      case 40806: rescale_item<8, 6, 4, RESCALE>(t, item, Geo<8>::per_item(), gs8, slot); break;
      case 10816: rescale_item<8, 16, 1, RESCALE>(t, item, Geo<8>::per_item(), gs8, slot); break;
      default: break;
    }
  }
}

// The classes of a ragged call that share a workgroup size, in one launch.
template <bool RESCALE>
static hipError_t run_mixed(int threads, const RescaleArgs& args, int grid, hipStream_t stream) {
  switch (threads) {
    case 128: rescale_mixed_128<RESCALE><<<grid, 128, 0, stream>>>(args); break;
    case 256: rescale_mixed_256<RESCALE><<<grid, 256, 0, stream>>>(args); break;
    case 512: rescale_mixed_512<RESCALE><<<grid, 512, 0, stream>>>(args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rescale_project(Shape s, const RescaleArgs& args, int grid, hipStream_t stream) {
  if (s.mixed > 0) return run_mixed<false>(s.mixed, args, grid, stream);
  switch (s.key()) {
    case 40101: return run<1, 1, 4, false>(args, grid, stream);
    case 40102: return run<1, 2, 4, false>(args, grid, stream);
    case 40103: return run<1, 3, 4, false>(args, grid, stream);
    case 40104: return run<1, 4, 4, false>(args, grid, stream);
    case 40105: return run<1, 5, 4, false>(args, grid, stream);
    case 40106: return run<1, 6, 4, false>(args, grid, stream);
    case 40204: return run<2, 4, 4, false>(args, grid, stream);
    case 40205: return run<2, 5, 4, false>(args, grid, stream);
    case 40206: return run<2, 6, 4, false>(args, grid, stream);
    case 40404: return run<4, 4, 4, false>(args, grid, stream);
    case 40405: return run<4, 5, 4, false>(args, grid, stream);
    case 40406: return run<4, 6, 4, false>(args, grid, stream);
    case 40804: return run<8, 4, 4, false>(args, grid, stream);
    case 40805: return run<8, 5, 4, false>(args, grid, stream);
    case 40806: return run<8, 6, 4, false>(args, grid, stream);
    case 41604: return run<16, 4, 4, false>(args, grid, stream);
    case 41605: return run<16, 5, 4, false>(args, grid, stream);
    case 41606: return run<16, 6, 4, false>(args, grid, stream);
    case 41607: return run<16, 7, 4, false>(args, grid, stream);
    case 41608: return run<16, 8, 4, false>(args, grid, stream);
    case 41609: return run<16, 9, 4, false>(args, grid, stream);
    case 41610: return run<16, 10, 4, false>(args, grid, stream);
    case 41611: return run<16, 11, 4, false>(args, grid, stream);
    case 41612: return run<16, 12, 4, false>(args, grid, stream);
    case 41613: return run<16, 13, 4, false>(args, grid, stream);
    case 41614: return run<16, 14, 4, false>(args, grid, stream);
    case 41615: return run<16, 15, 4, false>(args, grid, stream);
    case 41616: return run<16, 16, 4, false>(args, grid, stream);
    case 10101: return run<1, 1, 1, false>(args, grid, stream);
    case 10102: return run<1, 2, 1, false>(args, grid, stream);
    case 10104: return run<1, 4, 1, false>(args, grid, stream);
    case 10108: return run<1, 8, 1, false>(args, grid, stream);
    case 10116: return run<1, 16, 1, false>(args, grid, stream);
    case 10216: return run<2, 16, 1, false>(args, grid, stream);
    case 10416: return run<4, 16, 1, false>(args, grid, stream);
    case 10816: return run<8, 16, 1, false>(args, grid, stream);
    case 11616: return run<16, 16, 1, false>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rescale_after_step(Shape s, const RescaleArgs& args, int grid,
                                     hipStream_t stream) {
  if (s.mixed > 0) return run_mixed<true>(s.mixed, args, grid, stream);
  switch (s.key()) {
    case 40101: return run<1, 1, 4, true>(args, grid, stream);
    case 40102: return run<1, 2, 4, true>(args, grid, stream);
    case 40103: return run<1, 3, 4, true>(args, grid, stream);
    case 40104: return run<1, 4, 4, true>(args, grid, stream);
    case 40105: return run<1, 5, 4, true>(args, grid, stream);
    case 40106: return run<1, 6, 4, true>(args, grid, stream);
    case 40204: return run<2, 4, 4, true>(args, grid, stream);
    case 40205: return run<2, 5, 4, true>(args, grid, stream);
    case 40206: return run<2, 6, 4, true>(args, grid, stream);
    case 40404: return run<4, 4, 4, true>(args, grid, stream);
    case 40405: return run<4, 5, 4, true>(args, grid, stream);
    case 40406: return run<4, 6, 4, true>(args, grid, stream);
    case 40804: return run<8, 4, 4, true>(args, grid, stream);
    case 40805: return run<8, 5, 4, true>(args, grid, stream);
    case 40806: return run<8, 6, 4, true>(args, grid, stream);
    case 41604: return run<16, 4, 4, true>(args, grid, stream);
    case 41605: return run<16, 5, 4, true>(args, grid, stream);
    case 41606: return run<16, 6, 4, true>(args, grid, stream);
    case 41607: return run<16, 7, 4, true>(args, grid, stream);
    case 41608: return run<16, 8, 4, true>(args, grid, stream);
    case 41609: return run<16, 9, 4, true>(args, grid, stream);
    case 41610: return run<16, 10, 4, true>(args, grid, stream);
    case 41611: return run<16, 11, 4, true>(args, grid, stream);
    case 41612: return run<16, 12, 4, true>(args, grid, stream);
    case 41613: return run<16, 13, 4, true>(args, grid, stream);
    case 41614: return run<16, 14, 4, true>(args, grid, stream);
    case 41615: return run<16, 15, 4, true>(args, grid, stream);
    case 41616: return run<16, 16, 4, true>(args, grid, stream);
    case 10101: return run<1, 1, 1, true>(args, grid, stream);
    case 10102: return run<1, 2, 1, true>(args, grid, stream);
    case 10104: return run<1, 4, 1, true>(args, grid, stream);
    case 10108: return run<1, 8, 1, true>(args, grid, stream);
    case 10116: return run<1, 16, 1, true>(args, grid, stream);
    case 10216: return run<2, 16, 1, true>(args, grid, stream);
    case 10416: return run<4, 16, 1, true>(args, grid, stream);
    case 10816: return run<8, 16, 1, true>(args, grid, stream);
    case 11616: return run<16, 16, 1, true>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
