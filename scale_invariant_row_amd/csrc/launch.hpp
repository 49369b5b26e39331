// Host-side launchers of the row kernels (one translation unit per op).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsr {

template <class Task>
struct TaskArgs;
struct RownormTask;
struct RownormGradTask;
struct QkArgs;
struct RescaleTask;

// Kernel shape: G waves per row, V vectors per lane, NE values per vector
// (the fp32 weight kernels: 4 for 16-byte vectors, 1 for single elements;
// every other kernel uses 16-byte vectors).
// A column-block weight (its rows spread over the stored rows) instead runs
// one 1024-thread workgroup per tile of `units` adjacent rows; `col1` > 0
// (K * 100 + LANES) picks the seg-1 kernel whose tiles are single-pass where
// the matrix fits and two-pass elsewhere (its tile width varies with the
// matrix, so its launches group by col1 alone).  A launch with `mixed` > 0
// runs the ragged weight kernels' mixed-shape kernel of that workgroup size:
// each task carries its own row shape.
struct Shape {
  int G = 0;
  int V = 0;
  int NE = 4;
  int units = 0;
  int col1 = 0;
  int mixed = 0;
  int rows_per_block() const { return units > 0 ? units : (G == 1 ? 4 : 1); }
  int threads() const { return mixed > 0 ? mixed : units > 0 ? 1024 : 64 * G * rows_per_block(); }
  bool ok() const { return G > 0 || units > 0; }
  int key() const {
    return col1 > 0 ? 2000000 + col1 : units > 0 ? 1000000 + units : NE * 10000 + G * 100 + V;
  }
};

// Mixed-shape launches of the ragged weight calls (measured on MI355X): the
// small classes of contiguous rows that share a workgroup size of at most
// kMaxMixedThreads run in one launch, so their short kernels' fixed
// latencies overlap (ResNet-50's 54 weights: 36 instead of 60 us forward);
// a class of at least kMixedItemsPerCu items per compute unit streams at its
// own kernel's speed and keeps its own launch (GPT-2's 48 linears lost 8% in
// the gradient when their two classes shared one).
constexpr int kMaxMixedThreads = 512;
constexpr int kMixedItemsPerCu = 32;

// Column-block tiles: 64 / seg rows of seg values per stored row.
constexpr int kMaxSeg = 64;
inline Shape colblock_shape(int64_t seg) {
  Shape s{};
  if (seg >= 1 && seg <= kMaxSeg) s.units = (int)(64 / seg);
  return s;
}

// Single-pass column blocks (seg 1): a tile of 4 LANES adjacent units, each
// lane holding K 16-byte vectors of W (and of the second input), so the
// workgroup holds 1024 K / LANES stored rows.  Per op: the forward and the
// gradient 64-unit tiles (K = 12: W takes 48 VGPRs, the gradient's bf16
// dW_eff 24 more), so every stream moves whole 128-byte lines; the rescale
// calls 32-unit tiles (fp32 only, K = 6).  Each holds the 768 stored rows of
// GPT-2's attention and MLP-input weights.  A taller matrix (GPT-2's
// 3,072-row MLP projection) runs the two-pass tile in the same launch: tiles
// narrower than a line to fit its rows lost more to partial-line traffic
// than the second read costs.  Host and kernel share this rule.
#ifndef DSR_COL1_K_FWD
#define DSR_COL1_K_FWD 12
#endif
#ifndef DSR_COL1_K_BWD
#define DSR_COL1_K_BWD 12
#endif
#ifndef DSR_COL1_LANES_BWD
#define DSR_COL1_LANES_BWD 16
#endif
constexpr int kCol1KFwd = DSR_COL1_K_FWD, kCol1LanesFwd = 16;
constexpr int kCol1KBwd = DSR_COL1_K_BWD, kCol1LanesBwd = DSR_COL1_LANES_BWD;
constexpr int kCol1KRescale = 6, kCol1LanesRescale = 8;
// Whether a matrix of A stored rows, ld elements apart, takes the single-pass
// tile: A within the capacity, and 32-bit buffer offsets over every stored
// row a tile addresses.
__host__ __device__ constexpr inline bool col1_single(int64_t A, int64_t ld, int K, int lanes) {
  return A <= (int64_t)1024 * K / lanes && (int64_t)1024 * K / lanes * ld * 4 + 256 <= 0x7fffffff;
}

// Shape policy, measured on MI355X (the gradients use the same rules as
// their forward ops).  A row is spread over the smallest wave
// group G in {1, 2, 4, 8, 16} whose V = ceil(vectors / (64 G)) fits a limit:
//   bf16 rows (l2_rows, slerp_rows): V <= 2 up to 512 vectors (4,096
//     columns), V <= 4 beyond -- more, lighter waves stream best at these
//     widths, and slerp's per-row work favours V = 4 once rows are wider;
//   activation rows (gate, SwiGLU): V <= 2, so the fp32 column scales stay
//     in VGPRs; these kernels are ALU-bound and gain from more, lighter waves;
//   fp32 weight rows: V <= 6;
//   fp32 weight rows of single elements (a width that is not a multiple of
//     4, rare: a convolution's first layer): one wave with V the next power
//     of two >= ceil(cols / 64), else the smallest G with V = 16 (rows up to
//     kMaxElemCols); the buffer range check zeroes the unused vectors;
//   G = 16 may take V up to 16 (rows up to DS_MAX_COLS).
// The shape is a function of the width alone.  gen_instances.py evaluates
// these same rules over every width to list the kernels to instantiate.
constexpr int kBf16SmallVectors = 512;
constexpr int kVmaxBf16Small = 2;
constexpr int kVmaxBf16Large = 4;
constexpr int kVmaxAct = 2;
constexpr int kVmaxRownorm = 6;
constexpr int kVmaxWide = 16;
constexpr int kVmaxElem = 16;
constexpr int kMaxElemCols = 16 * 64 * kVmaxElem;   // 16,384

inline Shape pick_shape(int64_t vectors, int vmax) {
  for (int G = 1; G <= 16; G *= 2) {
    int64_t V = (vectors + 64 * G - 1) / (64 * G);
    if (V <= vmax || (G == 16 && V <= kVmaxWide)) return Shape{G, (int)V};
  }
  return Shape{};
}

// bf16 rows of `vectors` 16-byte vectors (8 columns each)
inline Shape pick_bf16_shape(int64_t vectors) {
  return pick_shape(vectors, vectors <= kBf16SmallVectors ? kVmaxBf16Small : kVmaxBf16Large);
}

// activation rows of `vectors` 16-byte vectors (8 columns each)
inline Shape pick_act_shape(int64_t vectors) { return pick_shape(vectors, kVmaxAct); }

// fp32 weight rows of `vectors` 16-byte vectors (4 columns each)
inline Shape pick_rownorm_shape(int64_t vectors) { return pick_shape(vectors, kVmaxRownorm); }

// fp32 weight rows of `cols` single elements
inline Shape pick_elem_shape(int64_t cols) {
  Shape s{};
  s.NE = 1;
  if (cols < 1 || cols > kMaxElemCols) return s;
  const int64_t v = (cols + 63) / 64;
  if (v <= kVmaxElem) {
    s.G = 1;
    for (s.V = 1; s.V < v; s.V *= 2) {}
  } else {
    for (s.G = 2; (int64_t)64 * s.G * kVmaxElem < cols; s.G *= 2) {}
    s.V = kVmaxElem;
  }
  return s;
}

// The shape of an fp32 weight row of `cols` values: 16-byte vectors when cols
// is a multiple of 4, single elements otherwise.
inline Shape pick_weight_shape(int64_t cols) {
  return cols % 4 == 0 ? pick_rownorm_shape(cols / 4) : pick_elem_shape(cols);
}

hipError_t launch_l2_rows(Shape s, const void* x, const void* r, void* y, int64_t rows,
                          int nvec, float eps, int grid, hipStream_t stream);
hipError_t launch_rms_rows(Shape s, const void* x, const void* r, void* y, int64_t rows,
                           int nvec, float eps, int grid, hipStream_t stream);
hipError_t launch_rms_rows_backward(Shape s, const void* x, const void* r, const void* dy,
                                    void* dx, int64_t rows, int nvec, float eps, int grid,
                                    hipStream_t stream);
hipError_t launch_slerp_rows(Shape s, const void* res, const void* out, const float* alpha,
                             void* h, int64_t rows, int nvec, float eps, int grid,
                             hipStream_t stream);
hipError_t launch_rownorm(Shape s, const TaskArgs<RownormTask>& args, int grid,
                          hipStream_t stream);
hipError_t launch_gate_l2_rows(Shape s, const void* o, const void* g, const float* sg, void* y,
                               int64_t rows, int nvec, float eps, int grid, hipStream_t stream);
hipError_t launch_swiglu_l2_rows(Shape s, const void* g, const void* u, const float* sug,
                                 const float* suu, void* y, int64_t rows, int nvec, float eps,
                                 int grid, int cus, hipStream_t stream);
hipError_t launch_rescale_project(Shape s, const TaskArgs<RescaleTask>& args, int grid,
                                  hipStream_t stream);
hipError_t launch_rescale_after_step(Shape s, const TaskArgs<RescaleTask>& args, int grid,
                                     hipStream_t stream);
hipError_t launch_qk_rows_l2(int head_dim, const QkArgs& args, int grid, hipStream_t stream);
hipError_t launch_l2_rows_backward(Shape s, const void* x, const void* r, const void* dy,
                                   void* dx, int64_t rows, int nvec, float eps, int grid,
                                   hipStream_t stream);
hipError_t launch_rownorm_backward(Shape s, const TaskArgs<RownormGradTask>& args, int grid,
                                   hipStream_t stream);
hipError_t launch_colblock_rownorm(const TaskArgs<RownormTask>& args, int grid,
                                   hipStream_t stream);
hipError_t launch_colblock_rownorm_backward(const TaskArgs<RownormGradTask>& args, int grid,
                                            hipStream_t stream);
hipError_t launch_colblock_rescale(bool after_step, const TaskArgs<RescaleTask>& args, int grid,
                                   hipStream_t stream);
hipError_t launch_colblock1_rownorm(const TaskArgs<RownormTask>& args, int grid,
                                    hipStream_t stream);
hipError_t launch_colblock1_rownorm_backward(const TaskArgs<RownormGradTask>& args, int grid,
                                             hipStream_t stream);
hipError_t launch_colblock1_rescale(bool after_step, const TaskArgs<RescaleTask>& args, int grid,
                                    hipStream_t stream);

}  // namespace dsr
