// Host-side launchers of the row kernels (one translation unit per op).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsr {

struct RownormArgs;

// Kernel shape: G waves per row, V 16-byte vectors per lane.
struct Shape {
  int G = 0;
  int V = 0;
  int rows_per_block() const { return G == 1 ? 4 : 1; }
  int threads() const { return 64 * G * rows_per_block(); }
  bool ok() const { return G > 0; }
};

// Largest V per lane for each op (registers hold the whole row): the shape is
// the smallest G in {1, 2, 4, 8, 16} whose V = ceil(vectors / (64 G)) fits.
// Measured on MI355X: rows spread over more, lighter waves (V <= 2) stream
// best for bf16 rows from 1,024 to 8,192 wide; only rows wider than 16,384
// fall back to G = 16 with up to 8 vectors per lane.
constexpr int kVmaxL2 = 2;
constexpr int kVmaxSlerp = 2;
constexpr int kVmaxRownorm = 6;
constexpr int kVmaxWide = 16;     // G = 16 may go up to here (DS_MAX_COLS fp32 rows)

// Shape for a row of `vectors` 16-byte vectors; a function of the width only.
inline Shape pick_shape(int64_t vectors, int vmax) {
  for (int G = 1; G <= 16; G *= 2) {
    int64_t V = (vectors + 64 * G - 1) / (64 * G);
    if (V <= vmax || (G == 16 && V <= kVmaxWide)) return Shape{G, (int)V};
  }
  return Shape{};
}

hipError_t launch_l2_rows(Shape s, const void* x, const void* r, void* y, int64_t rows,
                          int nvec, float eps, int grid, hipStream_t stream);
hipError_t launch_slerp_rows(Shape s, const void* res, const void* out, const float* alpha,
                             void* h, int64_t rows, int nvec, float eps, int grid,
                             hipStream_t stream);
hipError_t launch_rownorm(Shape s, const RownormArgs& args, int grid, hipStream_t stream);

}  // namespace dsr
