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

// SwiGLU: with at least kSiluTableRows rows per resident workgroup, a grid of
// the resident workgroups (each filling the silu table once, then looping
// over its rows); otherwise one workgroup per row group and the formula.
// The two give the same bits.
template <int G, int V>
static hipError_t run_swiglu(const void* g, const void* u, const float* sug, const float* suu,
                             void* y, int64_t rows, int nvec, float eps, int grid, int cus,
                             hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, swiglu_table_l2_rows_kernel<G, V>, T, 0) != hipSuccess)
      n = 0;
    return n;
  }();
  const int64_t units = (rows + Geo<G>::R - 1) / Geo<G>::R;
  const int64_t resident = (int64_t)cus * per_cu;
  if (per_cu > 0 && units >= (int64_t)kSiluTableRows * resident) {
    swiglu_table_l2_rows_kernel<G, V><<<(int)resident, T, 0, stream>>>(
        (const u32x4_t*)g, (const u32x4_t*)u, (const f32x4_t*)sug, (const f32x4_t*)suu,
        (u32x4_t*)y, rows, nvec, eps);
    return hipGetLastError();
  }
  return run<G, V, Act::kSwiglu>(g, u, sug, suu, y, rows, nvec, eps, grid, stream);
}

hipError_t launch_swiglu_l2_rows(Shape s, const void* g, const void* u, const float* sug,
                                 const float* suu, void* y, int64_t rows, int nvec, float eps,
                                 int grid, int cus, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
    case 101: return run_swiglu<1, 1>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 102: return run_swiglu<1, 2>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 202: return run_swiglu<2, 2>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 402: return run_swiglu<4, 2>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 802: return run_swiglu<8, 2>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 1602: return run_swiglu<16, 2>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 1603: return run_swiglu<16, 3>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 1604: return run_swiglu<16, 4>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 1605: return run_swiglu<16, 5>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 1606: return run_swiglu<16, 6>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 1607: return run_swiglu<16, 7>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    case 1608: return run_swiglu<16, 8>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
