// Weight rows stored as column blocks: the fp32 weight ops on layers whose
// output unit is not a stored row.
//
// DragonScale README, "Supported layers": GPT-2's Conv1D stores its weight
// as [in, out] and a ConvTranspose as [in, out / groups, k...], so the
// values feeding output unit u (the unit row the method normalises) are
// spread over the stored rows: seg contiguous values at u * seg in each of
// the A = cols / seg stored rows, ld elements apart (Conv1D: seg = 1,
// ld = out; ConvTranspose, one group: seg = prod(k), ld = (out / groups)
// * prod(k)).  The arithmetic per unit is the row kernels' (sums of squares
// and products in fp32, the same rescue for sums out of range); only the
// order of the sums differs, fixed by the layout alone.
//
// One workgroup of 1024 threads (16 waves) takes a tile of TU = 64 / seg
// adjacent units: 64 / seg * seg <= 64 adjacent columns, lane c holding
// column c of every stored row.  Wave w reads stored rows w, w + 16, ...,
// eight of them in flight, accumulating into eight chains (stored row
// w + 16 (8 i + j) into chain j); sixteen waves keep each wave's walk down a
// tall matrix (GPT-2's 3072-row MLP projection) short.  A column's total is
// then a fixed tree: the eight chains pairwise, the sixteen waves pairwise,
// and a unit's seg columns pairwise (through LDS).  A second pass over the
// tile applies each unit's coefficients and writes the outputs.  The tile is
// read twice: the first pass with the default cache policy, so its lines stay
// in L2, and the second pass (its last use) with non-temporal loads and
// stores, so neither its re-reads nor its outputs push other tiles'
// first-pass lines out of L2 before their own second pass (GPT-2's Conv1D
// set: 139.6 -> 127.2 us forward, 229.5 -> 195.0 us gradient).
#pragma once

#include <type_traits>

#include "row_kernels.hpp"

namespace dsr {

enum class ColOp { kFwd, kBwd, kProject, kAfterStep };

constexpr int kColChains = 8;
#ifndef DSR_COL_WAVES
#define DSR_COL_WAVES 16      // waves per tile (tuning knob: 4, 8 or 16)
#endif
constexpr int kColWaves = DSR_COL_WAVES;
constexpr int kColThreads = 64 * kColWaves;

template <ColOp OP>
struct ColTaskOf { using T = RescaleTask; };
template <>
struct ColTaskOf<ColOp::kFwd> { using T = RownormTask; };
template <>
struct ColTaskOf<ColOp::kBwd> { using T = RownormGradTask; };

// Global-memory view of a task pointer: plain loads through it compile to
// global (not flat) accesses, counted only against the vector-memory counter.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem_out(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// The second input of a unit's sums: dL/dW_eff (bf16), the gradient or
// momentum v (fp32, may be absent after a step), or none (forward).  It is
// loaded as raw bits and converted once every load of a batch is in flight;
// LAST marks the second pass's loads (non-temporal).
template <ColOp OP>
__device__ __forceinline__ bool has_second(const typename ColTaskOf<OP>::T& t) {
  if constexpr (OP == ColOp::kBwd) {
    return true;
  } else if constexpr (OP == ColOp::kFwd) {
    return false;
  } else {
    return t.v != nullptr;
  }
}

template <ColOp OP, bool LAST = false>
__device__ __forceinline__ uint32_t second_bits(const typename ColTaskOf<OP>::T& t, int64_t off) {
  if constexpr (OP == ColOp::kBwd) {
    return LAST ? (uint32_t)__builtin_nontemporal_load(&gmem(t.dw_eff)[off])
                : (uint32_t)gmem(t.dw_eff)[off];
  } else if constexpr (OP == ColOp::kFwd) {
    return 0u;
  } else {
    return LAST ? __float_as_uint(__builtin_nontemporal_load(&gmem((const float*)t.v)[off]))
                : __float_as_uint(gmem((const float*)t.v)[off]);
  }
}

template <ColOp OP>
__device__ __forceinline__ float second_value(uint32_t bits) {
  if constexpr (OP == ColOp::kBwd) {
    return bf_lo(bits);
  } else {
    return __uint_as_float(bits);
  }
}

// Pairwise sum of the chains: ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7)).
__device__ __forceinline__ float chain_total(const float (&c)[kColChains]) {
  return ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
}

// Pairwise sum of the waves' values of one column.
__device__ __forceinline__ float waves_total(const float (&p)[kColWaves][64], int lane) {
  float q[kColWaves];
#pragma unroll
  for (int i = 0; i < kColWaves; ++i) q[i] = p[i][lane];
#pragma unroll
  for (int n = kColWaves; n > 1; n /= 2)
#pragma unroll
    for (int i = 0; i < n / 2; ++i) q[i] = q[2 * i] + q[2 * i + 1];
  return q[0];
}

// Per unit, after its first pass: whether the sums are out of fp32's range
// and can be rescued, with the power-of-two exponents for x and y.
template <ColOp OP>
__device__ __forceinline__ bool unit_rescue(float T, float P, float m0, float m1, int& sa,
                                            int& sb) {
  constexpr bool kTwo = OP != ColOp::kFwd;
  if constexpr (!kTwo) {
    P = 0.f;
    m1 = 0.f;
  }
  const bool out = !(T >= kTiny && T < __builtin_inff() && fabsf(P) < __builtin_inff());
  const bool fix = out && m0 > 0.f && m0 < __builtin_inff() && m1 < __builtin_inff();
  sa = fix ? rescue_shift(m0, 0.f) : 0;
  sb = (fix && m1 > 0.f) ? rescue_shift(m1, 0.f) : 0;
  return fix;
}

// Per unit: the output coefficients c[0], c[1] and the flag c[2] (a zero unit,
// which the gradient zeroes and the rescale calls leave as it is); writes the
// unit's length (forward) or gain gradient (gradient).
template <ColOp OP, class Task>
__device__ __forceinline__ void unit_coefficients(const Task& t, int64_t u, float T, float P,
                                                  bool scaled, int sa, int sb, float (&c)[3]) {
  c[0] = c[1] = c[2] = 0.f;
  if constexpr (OP == ColOp::kFwd) {
    const float rn = sqrtf(T);
    if (t.norm_out != nullptr) t.norm_out[u] = scaled ? ldexpf(rn, -sa) : rn;
    const float gr = row_gain(t, u) * t.radius;
    c[0] = (rn == 0.f) ? 0.f : gr / rn;
  } else if constexpr (OP == ColOp::kBwd) {
    const bool zero = T == 0.f;
    const float inv = inv_sqrt(T);
    float dg = (t.radius * P) * inv;
    if (scaled) dg = ldexpf(dg, -sb);
    if (t.dgain != nullptr) t.dgain[u] = zero ? 0.f : dg;
    c[0] = zero ? 0.f : row_gain(t, u) * t.radius * inv;   // c
    c[1] = zero ? 0.f : (P * inv) * inv;                    // k
    c[2] = zero ? 1.f : 0.f;
  } else {
    const float inv = inv_sqrt(T);
    c[0] = t.radius * inv;                                  // c
    c[1] = (P * inv) * inv;                                 // k
    c[2] = T == 0.f ? 1.f : 0.f;                           // untouched
  }
}

// One value's outputs from its unit's coefficients: o0 is the forward's
// W_eff value (before its bf16 rounding), the gradient's dW, or the rescale
// calls' new v; o1 is the new w after a step.
template <ColOp OP>
__device__ __forceinline__ void col_values(float xr, float yv, bool scaled, int sa, int sb,
                                           float c0, float c1, bool skip, float& o0, float& o1) {
  const float x = scaled ? ldexpf(xr, sa) : xr;
  o1 = 0.f;
  if constexpr (OP == ColOp::kFwd) {
    o0 = x * c0;
  } else if constexpr (OP == ColOp::kBwd) {
    const float y = scaled ? ldexpf(yv, sb) : yv;
    float o = c0 * __builtin_fmaf(-x, c1, y);
    if (scaled) o = ldexpf(o, sa - sb);
    o0 = skip ? 0.f : o;
  } else {
    const float y = scaled ? ldexpf(yv, sb) : yv;
    const float r = __builtin_fmaf(-x, c1, y);
    o0 = scaled ? ldexpf(r, -sb) : r;
    o1 = x * c0;
  }
}

struct ColScratch {
  float part[2][kColWaves][64];   // per wave: the lane's S and P totals
  float pmax[2][kColWaves][64];   // per wave: the lane's max |x| and max |y|
  float col[2][64];         // per column: S, P (then unit trees in place)
  float mx[2][64];          // per column: max |x|, max |y| (rescue)
  float coef[4][64];        // per unit: the output coefficients
  int shift[2][64];         // per unit: rescue exponents for x and y
  int any_rescue;
};

template <ColOp OP>
__global__ void __launch_bounds__(kColThreads) colblock_kernel(const TaskArgs<typename ColTaskOf<OP>::T> args) {
  using Task = typename ColTaskOf<OP>::T;
  constexpr bool kTwo = OP != ColOp::kFwd;          // a second input, and P
  __shared__ ColScratch sc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nitems = args.nitems;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int lo = __builtin_amdgcn_readfirstlane(owning_task(args, item, lane));
    const Task t = args.tasks != nullptr ? args.tasks[lo] : args.inline_tasks[lo];
    const int seg = t.seg;
    const int TU = 64 / seg;
    const int64_t u0 = (int64_t)(item - t.item_begin) * TU;
    const int tu = (int)min<int64_t>(TU, t.rows - u0);
    const int tw = tu * seg;
    const int A = t.cols / seg;
    const bool active = lane < tw;
    const int uo = lane / seg;                        // this column's unit in the tile
    const int64_t base = u0 * seg + lane;             // column offset in a stored row
    const int64_t first = u0 * seg;                   // the tile's first value
    const bool two = kTwo && has_second<OP>(t);        // uniform over the workgroup

    // ---- pass 1: column sums (scaled by the unit's shifts on a rescue)
    auto column_sums = [&](bool scaled) {
      const int sa = scaled && active ? sc.shift[0][uo] : 0;
      const int sb = scaled && active ? sc.shift[1][uo] : 0;
      float cs[kColChains], cp[kColChains];
      float mx = 0.f, my = 0.f;
#pragma unroll
      for (int j = 0; j < kColChains; ++j) cs[j] = cp[j] = 0.f;
      for (int a0 = wave; a0 < A; a0 += kColWaves * kColChains) {
        // every load of the batch is issued before any is used.  With a
        // second input a lane past the tile, or a stored row past the matrix,
        // reads the tile's first value (always present) and drops it: a
        // predicated load whose value is converted inside its branch would
        // wait there for every load in flight.  The forward's single input
        // needs no conversion, and its predicated loads measured as fast.
        float xr[kColChains];
        uint32_t yr[kColChains];
#pragma unroll
        for (int j = 0; j < kColChains; ++j) {
          const int a = a0 + kColWaves * j;
          const bool in = active && a < A;
          if constexpr (OP == ColOp::kFwd) {
            xr[j] = in ? gmem(t.w)[(int64_t)a * t.ld + base] : 0.f;
          } else {
            const int64_t off = in ? (int64_t)a * t.ld + base : first;
            xr[j] = gmem(t.w)[off];
            yr[j] = two ? second_bits<OP>(t, off) : 0u;
          }
        }
#pragma unroll
        for (int j = 0; j < kColChains; ++j) {
          const bool in = active && a0 + kColWaves * j < A;
          const float x = in ? xr[j] : 0.f;
          const float y = (two && in) ? second_value<OP>(yr[j]) : 0.f;
          if (!scaled) {
            mx = fmaxf(mx, fabsf(x));
            if constexpr (kTwo) my = fmaxf(my, fabsf(y));
          }
          const float xs = scaled ? ldexpf(x, sa) : x;
          cs[j] = __builtin_fmaf(xs, xs, cs[j]);
          if constexpr (kTwo) cp[j] = __builtin_fmaf(xs, scaled ? ldexpf(y, sb) : y, cp[j]);
        }
      }
      sc.part[0][wave][lane] = chain_total(cs);
      if constexpr (kTwo) sc.part[1][wave][lane] = chain_total(cp);
      sc.pmax[0][wave][lane] = mx;
      sc.pmax[1][wave][lane] = my;
      __syncthreads();
      if (wave == 0) {
        sc.col[0][lane] = waves_total(sc.part[0], lane);
        if constexpr (kTwo) sc.col[1][lane] = waves_total(sc.part[1], lane);
        if (!scaled) {
          float m0 = 0.f, m1 = 0.f;
#pragma unroll
          for (int i = 0; i < kColWaves; ++i) {
            m0 = fmaxf(m0, sc.pmax[0][i][lane]);
            m1 = fmaxf(m1, sc.pmax[1][i][lane]);
          }
          sc.mx[0][lane] = m0;
          sc.mx[1][lane] = m1;
        }
      }
      __syncthreads();
      // a unit's seg columns, pairwise: column c adds column c + s when c's
      // offset in its unit is a multiple of 2s and the partner is in the unit
      for (int s = 1; s < seg; s *= 2) {
        if (wave == 0 && active) {
          const int b = lane - uo * seg;
          if ((b % (2 * s)) == 0 && b + s < seg) {
            sc.col[0][lane] += sc.col[0][lane + s];
            if constexpr (kTwo) sc.col[1][lane] += sc.col[1][lane + s];
            if (!scaled) {
              sc.mx[0][lane] = fmaxf(sc.mx[0][lane], sc.mx[0][lane + s]);
              if constexpr (kTwo) sc.mx[1][lane] = fmaxf(sc.mx[1][lane], sc.mx[1][lane + s]);
            }
          }
        }
        __syncthreads();
      }
    };

    if (threadIdx.x == 0) sc.any_rescue = 0;
    column_sums(false);
    // ---- per unit: decide on a rescue (uniform over the tile)
    if (wave == 0 && lane < tu) {
      int sa, sb;
      const bool fix = unit_rescue<OP>(sc.col[0][lane * seg], sc.col[1][lane * seg],
                                       sc.mx[0][lane * seg], sc.mx[1][lane * seg], sa, sb);
      sc.shift[0][lane] = sa;
      sc.shift[1][lane] = sb;
      sc.coef[3][lane] = fix ? 1.f : 0.f;            // the unit was rescued
      if (fix) sc.any_rescue = 1;
    }
    __syncthreads();
    if (sc.any_rescue) column_sums(true);           // uniform: LDS read after a barrier

    // ---- per unit: the output coefficients
    if (wave == 0 && lane < tu) {
      const bool scaled = sc.coef[3][lane] != 0.f;
      const float P = kTwo ? sc.col[1][lane * seg] : 0.f;
      float c[3];
      unit_coefficients<OP>(t, u0 + lane, sc.col[0][lane * seg], P, scaled, sc.shift[0][lane],
                            sc.shift[1][lane], c);
      sc.coef[0][lane] = c[0];
      sc.coef[1][lane] = c[1];
      sc.coef[2][lane] = c[2];
    }
    __syncthreads();

    // ---- pass 2: outputs, eight stored rows in flight per wave.  A tile
    // with no rescued unit (the common case) takes a copy of the loop with
    // the rescue's scaling compiled out, not a select on every value.
    auto pass2 = [&](auto rescued) {
      constexpr bool kResc = decltype(rescued)::value;
      const bool scaled = kResc && sc.coef[3][uo] != 0.f;
      const int sa = sc.shift[0][uo], sb = sc.shift[1][uo];
      const float c0 = sc.coef[0][uo], c1 = sc.coef[1][uo];
      const bool skip = OP != ColOp::kFwd && sc.coef[2][uo] != 0.f;
      // a zero unit of the rescale calls is left as it is
      const bool work = !(skip && (OP == ColOp::kProject || OP == ColOp::kAfterStep));
      for (int a0 = wave; work && a0 < A; a0 += kColWaves * kColChains) {
        float xr[kColChains];
        uint32_t yr[kColChains];
#pragma unroll
        for (int j = 0; j < kColChains; ++j) {
          const int a = a0 + kColWaves * j;
          if constexpr (OP == ColOp::kFwd) {
            xr[j] = a < A ? __builtin_nontemporal_load(&gmem(t.w)[(int64_t)a * t.ld + base]) : 0.f;
          } else {
            const int64_t off = a < A ? (int64_t)a * t.ld + base : base;
            xr[j] = __builtin_nontemporal_load(&gmem(t.w)[off]);
            yr[j] = two ? second_bits<OP, true>(t, off) : 0u;
          }
        }
#pragma unroll
        for (int j = 0; j < kColChains; ++j) {
          const int a = a0 + kColWaves * j;
          if (a >= A) break;
          const int64_t off = (int64_t)a * t.ld + base;
          float o0, o1;
          col_values<OP>(xr[j], OP == ColOp::kFwd ? 0.f : second_value<OP>(yr[j]), scaled, sa,
                         sb, c0, c1, skip, o0, o1);
          if constexpr (OP == ColOp::kFwd) {
            __builtin_nontemporal_store((uint16_t)pack_bf16(o0, 0.f), &gmem_out(t.w_eff)[off]);
          } else if constexpr (OP == ColOp::kBwd) {
            __builtin_nontemporal_store(o0, &gmem_out(t.dw)[off]);
          } else {
            if (two) __builtin_nontemporal_store(o0, &gmem_out(t.v)[off]);
            if constexpr (OP == ColOp::kAfterStep) __builtin_nontemporal_store(o1, &gmem_out(t.w)[off]);
          }
        }
      }
    };
    if (active) {
      if (sc.any_rescue) {                          // uniform: LDS read after a barrier
        asm volatile("" ::: "memory");
        pass2(std::true_type{});
      } else {
        pass2(std::false_type{});
      }
    }
    __syncthreads();                                // LDS is reused by the next tile
  }
}

}  // namespace dsr
