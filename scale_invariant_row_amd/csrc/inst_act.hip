// gate and SwiGLU activation rows: one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {

template <int G, int V, Act A>
static hipError_t run(const void* in0, const void* in1, const float* s0, const float* s1, void* y,
                      int64_t rows, int nvec, float eps, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  act_l2_rows_kernel<G, V, A><<<grid, T, 0, stream>>>(
      (const u32x4_t*)in0, (const u32x4_t*)in1, (const f32x4_t*)s0, (const f32x4_t*)s1,
      (u32x4_t*)y, rows, nvec, eps);
  return hipGetLastError();
}

hipError_t launch_gate_l2_rows(Shape s, const void* o, const void* g, const float* sg, void* y,
                               int64_t rows, int nvec, float eps, int grid, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 102: return run<1, 2, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 202: return run<2, 2, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 402: return run<4, 2, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 802: return run<8, 2, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 1602: return run<16, 2, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 1603: return run<16, 3, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 1604: return run<16, 4, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 1605: return run<16, 5, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 1606: return run<16, 6, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 1607: return run<16, 7, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    case 1608: return run<16, 8, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_swiglu_l2_rows(Shape s, const void* g, const void* u, const float* sug,
                                 const float* suu, void* y, int64_t rows, int nvec, float eps,
                                 int grid, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run<1, 1, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 102: return run<1, 2, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 202: return run<2, 2, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 402: return run<4, 2, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 802: return run<8, 2, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 1602: return run<16, 2, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 1603: return run<16, 3, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 1604: return run<16, 4, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 1605: return run<16, 5, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 1606: return run<16, 6, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 1607: return run<16, 7, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    case 1608: return run<16, 8, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
