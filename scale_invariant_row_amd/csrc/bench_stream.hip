// A plain read-2-write-1 stream over bf16 rows: the benchmark's reference
// for the bandwidth a kernel of l2_rows' launch shape can reach on this GPU.
// It has the same shape policy, grid, row-to-wave mapping, buffer resources
// and cache hints as l2_rows_kernel.  Where l2_rows normalises, it does one
// bitwise op per dword (y = x ^ r), so what remains is the memory traffic.
//
// Built into its own library (libdsbench.so) for bench.py and the tests (it
// also holds a check kernel the tests run); it is not part of the row library
// or its C ABI.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.hpp"
#include "row_kernels.hpp"

namespace dsr {

template <int G, int V>
__global__ void __launch_bounds__(Geo<G>::THREADS)
stream_rows_kernel(const u32x4_t* x, const u32x4_t* r, u32x4_t* y, int64_t rows, int nvec) {
  constexpr int R = Geo<G>::R;
  const Geo<G> geo;
  int off[V];
  geo.offsets(off, 16);
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  {
    const int64_t row = (int64_t)blockIdx.x * R + geo.rr;   // one row group per workgroup
    if (G == 1 && row >= rows) return;
    Bf16Row<V> a, b;
    a.load(RowBuf(x + row * nvec, row_bytes), off);
    b.load(RowBuf(r + row * nvec, row_bytes), off);
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) a.p[v][k] ^= b.p[v][k];
    a.store(RowBuf(y + row * nvec, row_bytes), off);
  }
}

template <int G, int V>
static hipError_t run(const void* x, const void* r, void* y, int64_t rows, int nvec, int grid,
                      hipStream_t stream) {
  stream_rows_kernel<G, V><<<grid, Geo<G>::THREADS, 0, stream>>>(
      (const u32x4_t*)x, (const u32x4_t*)r, (u32x4_t*)y, rows, nvec);
  return hipGetLastError();
}

}  // namespace dsr

// y = x ^ r over [rows, cols] bf16 rows (cols a multiple of 8, up to 8,192),
// with the launch l2_rows would use.  Returns 0, or -1 for an unsupported
// width, -2 for a runtime error.
extern "C" int dsb_stream_rows(const void* x, const void* r, void* y, int64_t rows,
                               int64_t cols, void* stream) {
  using namespace dsr;
  if (rows < 0 || cols < 8 || cols > 8192 || cols % 8 != 0) return -1;
  if (rows == 0) return 0;
  const int nvec = (int)(cols / 8);
  const Shape s = pick_bf16_shape(nvec);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -2;
  // as the row library launches l2_rows: one row group per workgroup, in
  // launches of at most 64 row groups per compute unit
  const int rpg = s.rows_per_block();
  const int64_t piece = (int64_t)cus * 64 * rpg;
  hipStream_t hs = (hipStream_t)stream;
  for (int64_t r0 = 0; r0 < rows; r0 += piece) {
    const int64_t n = std::min<int64_t>(piece, rows - r0);
    const int grid = (int)((n + rpg - 1) / rpg);
    const char* xp = (const char*)x + r0 * cols * 2;
    const char* rp = (const char*)r + r0 * cols * 2;
    char* yp = (char*)y + r0 * cols * 2;
    hipError_t e;
    switch (s.G * 100 + s.V) {
      case 101: e = run<1, 1>(xp, rp, yp, n, nvec, grid, hs); break;
      case 102: e = run<1, 2>(xp, rp, yp, n, nvec, grid, hs); break;
      case 202: e = run<2, 2>(xp, rp, yp, n, nvec, grid, hs); break;
      case 402: e = run<4, 2>(xp, rp, yp, n, nvec, grid, hs); break;
      case 403: e = run<4, 3>(xp, rp, yp, n, nvec, grid, hs); break;
      case 404: e = run<4, 4>(xp, rp, yp, n, nvec, grid, hs); break;
      default: return -1;
    }
    if (e != hipSuccess) return -2;
  }
  return 0;
}

// ------------------------------------------------- fp32 in, bf16 out (weights)
//
// The weight op's traffic without its arithmetic: fp32 rows read, each value
// rounded to bf16 and written, with the launch the weight rows of this width
// get (pick_rownorm_shape, items of R rows, one workgroup per item up to 64
// per compute unit, the rest grid-stride), the same buffer resources and
// cache hints.  The reference rate for the fp32 weight kernels, whose other
// traffic (gains and lengths, 8 bytes a row) is negligible.
namespace dsr {

template <int G, int V>
__global__ void __launch_bounds__(Geo<G>::THREADS)
stream_f32_rows_kernel(const float* x, uint16_t* y, int64_t rows, int cols, int64_t items) {
  constexpr int R = Geo<G>::R;
  const Geo<G> geo;
  int off[V];
  geo.offsets(off, 16);
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t row = item * R + geo.rr;
    if (G == 1 && row >= rows) break;       // a wave's rows only grow
    const RowBuf xb(x + row * cols, (uint32_t)cols * 4u);
    const RowBuf yb(y + row * cols, (uint32_t)cols * 2u);
    f32x4_t w[V];
#pragma unroll
    for (int v = 0; v < V; ++v) w[v] = xb.ld16f(off[v]);
#pragma unroll
    for (int v = 0; v < V; ++v)
      yb.st8(u32x2_t{pack_bf16(w[v].x, w[v].y), pack_bf16(w[v].z, w[v].w)}, off[v] / 2);
  }
}

template <int G, int V>
static hipError_t run_f32(const float* x, uint16_t* y, int64_t rows, int cols, int64_t items,
                          int grid, hipStream_t stream) {
  stream_f32_rows_kernel<G, V><<<grid, Geo<G>::THREADS, 0, stream>>>(x, y, rows, cols, items);
  return hipGetLastError();
}

}  // namespace dsr

// y = bf16(x) over [rows, cols] fp32 rows (cols a multiple of 4 whose weight
// shape is one of the cases below), with the launch the weight op uses for
// that width.  Returns 0, -1 for an unsupported width, -2 for a runtime error.
extern "C" int dsb_stream_f32_rows(const float* x, uint16_t* y, int64_t rows, int64_t cols,
                                   void* stream) {
  using namespace dsr;
  if (rows < 0 || cols < 4 || cols % 4 != 0 || cols > 65536) return -1;
  if (rows == 0) return 0;
  const Shape s = pick_rownorm_shape(cols / 4);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -2;
  const int rpg = s.rows_per_block();
  const int64_t items = (rows + rpg - 1) / rpg;
  const int grid = (int)std::min<int64_t>(items, (int64_t)cus * 64);
  const int c = (int)cols;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  switch (s.G * 100 + s.V) {
    case 101: e = run_f32<1, 1>(x, y, rows, c, items, grid, hs); break;
    case 102: e = run_f32<1, 2>(x, y, rows, c, items, grid, hs); break;
    case 103: e = run_f32<1, 3>(x, y, rows, c, items, grid, hs); break;
    case 104: e = run_f32<1, 4>(x, y, rows, c, items, grid, hs); break;
    case 105: e = run_f32<1, 5>(x, y, rows, c, items, grid, hs); break;
    case 106: e = run_f32<1, 6>(x, y, rows, c, items, grid, hs); break;
    case 204: e = run_f32<2, 4>(x, y, rows, c, items, grid, hs); break;
    case 205: e = run_f32<2, 5>(x, y, rows, c, items, grid, hs); break;
    case 206: e = run_f32<2, 6>(x, y, rows, c, items, grid, hs); break;
    case 404: e = run_f32<4, 4>(x, y, rows, c, items, grid, hs); break;
    case 405: e = run_f32<4, 5>(x, y, rows, c, items, grid, hs); break;
    case 406: e = run_f32<4, 6>(x, y, rows, c, items, grid, hs); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -2;
}

// ---------------------------------------------------------------- test kernel
//
// The gate's fast reciprocal against IEEE division over a range of fp32 bit
// patterns [first, first + count): counts the values where the two differ
// and keeps the smallest such pattern.  The test suite runs it over every b
// in [1, 2^126) and beyond.  `out` holds two uint32: the count (cleared by
// the caller) and the smallest differing pattern (set to ~0 by the caller).
namespace dsr {
__global__ void __launch_bounds__(256)
recip_check_kernel(uint32_t first, uint32_t count, uint32_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  uint32_t bad = 0, lowest = 0xffffffffu;
  // a 64-bit index: i + stride never wraps, so every lane's loop ends
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < count; i += stride) {
    const uint32_t bits = first + (uint32_t)i;
    const float b = __uint_as_float(bits);
    const float fast = recip_fast(b);
    const float ieee = 1.0f / b;
    if (__float_as_uint(fast) != __float_as_uint(ieee)) {
      ++bad;
      lowest = min(lowest, bits);
    }
  }
  if (bad) {
    atomicAdd(&out[0], bad);
    atomicMin(&out[1], lowest);
  }
}
}  // namespace dsr

// Runs the check over [first, first + count) (count > 0, first + count <=
// 2^32) on `stream`; out: device memory as above.  Returns 0, or -2 for a
// runtime error.
extern "C" int dsb_recip_check(uint32_t first, uint32_t count, uint32_t* out, void* stream) {
  if (count == 0 || (uint64_t)first + count > (1ull << 32)) return -1;
  dsr::recip_check_kernel<<<4096, 256, 0, (hipStream_t)stream>>>(first, count, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
