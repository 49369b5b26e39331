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

#include "launch.hpp"
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
    if (t.norm_out != nullptr) gmem_out(t.norm_out)[u] = scaled ? ldexpf(rn, -sa) : rn;
    const float gr = row_gain(t, u) * t.radius;
    c[0] = (rn == 0.f) ? 0.f : gr / rn;
  } else if constexpr (OP == ColOp::kBwd) {
    const bool zero = T == 0.f;
    const float inv = inv_sqrt(T);
    float dg = (t.radius * P) * inv;
    if (scaled) dg = ldexpf(dg, -sb);
    if (t.dgain != nullptr) gmem_out(t.dgain)[u] = zero ? 0.f : dg;
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

// One tile of the two-pass kernel: units u0 = (item - t.item_begin) TU ..
// of task t.  Ends with a barrier: the LDS is free for the next tile.
template <ColOp OP, class Task>
__device__ __forceinline__ void col2_tile(const Task& t, int item, ColScratch& sc, int lane,
                                          int wave) {
  constexpr bool kTwo = OP != ColOp::kFwd;          // a second input, and P
  {
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

template <ColOp OP>
__global__ void __launch_bounds__(kColThreads) colblock_kernel(const TaskArgs<typename ColTaskOf<OP>::T> args) {
  __shared__ ColScratch sc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x)
    col2_tile<OP>(task_of(args, item, lane), item, sc, lane, wave);
}

// ------------------------------------------ single pass, 16-byte lanes (seg 1)
//
// GPT-2's Conv1D layout (seg = 1) with a unit count and ld that are
// multiples of 4 and 16-byte-aligned buffers: the tile is read from HBM once
// and held in registers until its outputs are written.  The two-pass kernel
// above reads every value twice, and a tile is far larger than its share of
// L2 (a 768 x 64 fp32 tile is 192 KiB; an XCD's 4 MiB L2 serves 64 resident
// workgroups), so most second-pass reads go back to memory.
//
// A tile is TW = 4 LPR adjacent units (LPR lanes per stored row, fixed per
// op: 64 units for the forward and the gradient, 32 for the fp32-only
// rescale calls, so every stream moves whole 128-byte lines).  Lane (cg, rs)
// = (lane % LPR, lane / LPR) holds columns 4 cg .. 4 cg + 3 of the stored
// rows a = (16 k + wave) RS + rs, k < K (RS = 64 / LPR stored rows per wave
// instruction), so the workgroup holds up to 1024 K / LPR stored rows (768
// for every op: GPT-2's attention and MLP-input weights).  Buffer resources
// bound each access by the tile's span: a stored row past A loads zeros and
// its stores are dropped.  A column's total is a fixed tree: the lane's K
// values pairwise (squares in the leaves, the second of a pair by fma), the
// RS row slots (DPP row rotations, then the permlane swaps), and the sixteen
// waves pairwise (DPP over a row of 16 lanes, each lane reading one wave's
// partial from LDS).  The LDS scratch is double buffered, so a tile takes two
// barriers and none stands between tiles.  A taller matrix runs col2_tile,
// in the same launch.
//
// Measured on MI355X against the two-pass kernel alone, GPT-2's Conv1D set:
// 126.8 -> 104.6 us forward, 195.3 -> 178.9 us gradient.  Narrower tiles (16
// or 8 units, to hold the 3,072-row projection) lost: their 32- and 64-byte
// pieces of each line cost more than the second read they save.

// sum over i < N of a[i] b[i]: pairwise, the leaves a product and an fma
template <int N>
__device__ __forceinline__ float dot_tree(const float* a, const float* b) {
  if constexpr (N == 1) {
    return a[0] * b[0];
  } else if constexpr (N == 2) {
    return __builtin_fmaf(a[1], b[1], a[0] * b[0]);
  } else {
    return dot_tree<N / 2>(a, b) + dot_tree<N - N / 2>(a + N / 2, b + N / 2);
  }
}

// Sum (or max) over the 64 / lpr row slots of a wave, lanes lpr apart
// (lpr in {2, 4, 8, 16}, uniform): complete in the lanes of row slot 0
// (lanes < lpr), which are the ones read.
__device__ __forceinline__ float slot_sum(float v, int lpr) {
  if (lpr <= 2) v = v + dpp_f<0x122>(v);    // row_ror:2
  if (lpr <= 4) v = v + dpp_f<0x124>(v);    // row_ror:4
  if (lpr <= 8) v = v + dpp_f<0x128>(v);    // row_ror:8
  f32x2_t p = swap16(v);
  v = p.x + p.y;
  p = swap32(v);
  return p.x + p.y;
}
__device__ __forceinline__ float slot_max(float v, int lpr) {
  if (lpr <= 2) v = fmaxf(v, dpp_f<0x122>(v));
  if (lpr <= 4) v = fmaxf(v, dpp_f<0x124>(v));
  if (lpr <= 8) v = fmaxf(v, dpp_f<0x128>(v));
  f32x2_t p = swap16(v);
  v = fmaxf(p.x, p.y);
  p = swap32(v);
  return fmaxf(p.x, p.y);
}

// Sum (or max) over a row of 16 lanes, in every lane of the row with the same
// bits: the pairwise tree ((v0 + v1) + (v2 + v3)) + ... over the lanes in
// order (each step adds two partner lanes' equal-bit values).
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v = v + dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v = v + dpp_f<0x141>(v);   // row_half_mirror
  return v + dpp_f<0x140>(v);  // row_mirror
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}

// The second input held per lane: four bf16 of dW_eff (gradient) or four
// fp32 of v (rescale calls); none for the forward.
template <ColOp OP>
struct Col1Second {
  using T = f32x4_t;
  static constexpr uint32_t kBytes = 4;
  __device__ static float get(const T& v, int j) { return v[j]; }
  __device__ static T load(const RowBuf& b, int e, int se) { return b.ld16f(e * 4, se * 4); }
};
template <>
struct Col1Second<ColOp::kBwd> {
  using T = u32x2_t;
  static constexpr uint32_t kBytes = 2;
  __device__ static float get(const T& v, int j) {
    return (j & 1) ? bf_hi(v[j >> 1]) : bf_lo(v[j >> 1]);
  }
  __device__ static T load(const RowBuf& b, int e, int se) { return b.ld8(e * 2, se * 2); }
};

struct Col1Scratch {
  float part[2][kColWaves][64];   // per wave: column totals S and P
  float pmax[2][kColWaves][64];   // per wave: column max |x| and max |y|
  float coef[4][64];              // per unit: c0, c1, a zero unit, a rescued unit
  int shift[2][64];               // per unit: rescue exponents for x and y
  int any_rescue;
};

// One tile: units u0 .. u0 + TW - 1 of task t.
//
// Addressing: lane element offset e = (wave RS + rs) ld + 4 cg from the
// tile's first value, and stored-row step k adds k * 16 RS ld.  The step
// goes into the buffer resource (its base, and its range cut to what is
// left of the tile's span), not the scalar offset field, which the range
// check does not cover: a stored row past A is out of range whatever k.  A
// lane past the tile's units gets an offset beyond any range, so its loads
// read zeros and its stores are dropped, with no branch.
//
// common() runs every tile: it writes the outputs, or reports a sum out of
// fp32's range (rare), and then rescue() runs the tile again.  The two run
// one after the other, not as two branches, so the compiler cannot merge
// their shared code (the coefficients) into a block both reach, which
// would keep the common path's tile registers live through the rescue.
template <ColOp OP, int K, class Task, int CPOL>
struct Col1Tile {
  using Sec = Col1Second<OP>;
  using Y = typename Sec::T;
  static constexpr bool kTwo = OP != ColOp::kFwd;

  const Task& t;
  const int64_t u0;
  Col1Scratch& sc;
  const int lane, wave, lpr;
  int tu, lane_off, nel, kstep, vo4, vo2, pc, pi;
  bool active, two, unit_lane;
  const float* xb;
  const void* yb;
  const void* ob;
  f32x4_t xv[K];                            // the lane's tile: W
  Y yv[K];                                  // and the second input

  __device__ __forceinline__ Col1Tile(const Task& t_, int64_t u0_, Col1Scratch& sc_, int lane_,
                                      int wave_, int lpr_)
      : t(t_), u0(u0_), sc(sc_), lane(lane_), wave(wave_), lpr(lpr_) {
    const int lg = __builtin_ctz(lpr);
    const int RS = 64 >> lg;
    const int cg = lane & (lpr - 1), rs = lane >> lg;
    tu = (int)min<int64_t>(4 * lpr, t.rows - u0);          // a multiple of 4
    lane_off = 4 * cg;
    active = lane_off < tu;
    two = kTwo && has_second<OP>(t);                       // uniform
    // the tile's span from its first value: (A - 1) ld + (rows - u0) elements
    nel = (int)((int64_t)(t.cols - 1) * t.ld + (t.rows - u0));
    kstep = 16 * RS * (int)t.ld;
    const int e = (wave * RS + rs) * (int)t.ld + lane_off;
    constexpr uint32_t kFar = 0x80000000u;                 // beyond every range
    vo4 = active ? e * 4 : (int)kFar;                      // fp32 buffers
    vo2 = active ? e * 2 : (int)kFar;                      // bf16 buffers
    // the sixteen waves' partials of a column: lane l of wave w reduces
    // column pc = 4 w + l / 16 over the partials of waves l % 16 (every lane
    // of the row gets the total); the row's first lane acts for the unit
    pc = 4 * wave + (lane >> 4);
    pi = lane & 15;
    unit_lane = pi == 0 && pc < tu;
    xb = t.w + u0;
    yb = xb;
    if constexpr (OP == ColOp::kBwd) {
      yb = t.dw_eff + u0;
    } else if constexpr (kTwo) {
      if (two) yb = t.v + u0;
    }
    if constexpr (OP == ColOp::kFwd) {
      ob = t.w_eff + u0;
    } else if constexpr (OP == ColOp::kBwd) {
      ob = t.dw + u0;
    } else {
      ob = two ? (const void*)(t.v + u0) : (const void*)(t.w + u0);
    }
  }

  __device__ __forceinline__ RowBuf step(const void* base, int esz, int k) const {
    const int left = nel - k * kstep;
    return RowBuf((const char*)base + (int64_t)k * kstep * esz,
                  left > 0 ? (uint32_t)(left * esz) : 0u);
  }
  // reads with cache policy CPOL (0: default; kCpolLd: non-temporal)
  __device__ __forceinline__ f32x4_t load_x(int k) const {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(step(xb, 4, k).r, vo4,
                                                                             0, CPOL));
  }
  __device__ __forceinline__ Y load_y(int k) const {
    if constexpr (OP == ColOp::kBwd) {
      return __builtin_amdgcn_raw_buffer_load_b64(step(yb, 2, k).r, vo2, 0, CPOL);
    } else {
      return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(step(yb, 4, k).r,
                                                                               vo4, 0, CPOL));
    }
  }
  __device__ __forceinline__ void load_tile(f32x4_t (&xv)[K], Y (&yv)[K]) const {
#pragma unroll
    for (int k = 0; k < K; ++k) xv[k] = load_x(k);
    if constexpr (kTwo) {
#pragma unroll
      for (int k = 0; k < K; ++k) yv[k] = two ? load_y(k) : Y{};
    }
  }

  // column sums (scaled by the unit's shifts on a rescue): wave w's column
  // totals into part[][w]
  template <bool kScaled>
  __device__ __forceinline__ void column_sums(const f32x4_t (&xv)[K], const Y (&yv)[K]) {
    float S[4], P[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int sa = 0, sb = 0;
      if constexpr (kScaled) {
        sa = sc.shift[0][lane_off + j];                    // lanes past the tile: unused
        sb = sc.shift[1][lane_off + j];
      }
      float xs[K], ys[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float x = xv[k][j];
        const float y = kTwo ? Sec::get(yv[k], j) : 0.f;
        xs[k] = kScaled ? ldexpf(x, sa) : x;
        ys[k] = kScaled ? ldexpf(y, sb) : y;
      }
      S[j] = slot_sum(dot_tree<K>(xs, xs), lpr);
      P[j] = kTwo ? slot_sum(dot_tree<K>(xs, ys), lpr) : 0.f;
    }
    if (lane < lpr) {
      *(f32x4_t*)&sc.part[0][wave][lane_off] = f32x4_t{S[0], S[1], S[2], S[3]};
      if constexpr (kTwo) *(f32x4_t*)&sc.part[1][wave][lane_off] = f32x4_t{P[0], P[1], P[2], P[3]};
    }
  }
  // column max |x| and max |y| into pmax[][w]
  __device__ __forceinline__ void column_max(const f32x4_t (&xv)[K], const Y (&yv)[K]) {
    float M0[4], M1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float m0 = 0.f, m1 = 0.f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        m0 = fmaxf(m0, fabsf(xv[k][j]));
        if constexpr (kTwo) m1 = fmaxf(m1, fabsf(Sec::get(yv[k], j)));
      }
      M0[j] = slot_max(m0, lpr);
      M1[j] = kTwo ? slot_max(m1, lpr) : 0.f;
    }
    if (lane < lpr) {
      *(f32x4_t*)&sc.pmax[0][wave][lane_off] = f32x4_t{M0[0], M0[1], M0[2], M0[3]};
      *(f32x4_t*)&sc.pmax[1][wave][lane_off] = f32x4_t{M1[0], M1[1], M1[2], M1[3]};
    }
  }
  __device__ __forceinline__ void totals(float& T, float& P) const {
    T = row16_sum(sc.part[0][pi][pc]);
    P = kTwo ? row16_sum(sc.part[1][pi][pc]) : 0.f;
  }
  // the unit lane's coefficients (and its length or gain gradient)
  __device__ __forceinline__ void coefficients(float T, float P, bool scaled, int sa, int sb) {
    if (!unit_lane) return;
    float c[3];
    unit_coefficients<OP>(t, u0 + pc, T, P, scaled, sa, sb, c);
    sc.coef[0][pc] = c[0];
    sc.coef[1][pc] = c[1];
    sc.coef[2][pc] = c[2];
  }
  __device__ __forceinline__ void coefs(f32x4_t& c0, f32x4_t& c1, f32x4_t& zu) const {
    const int lo = active ? lane_off : 0;   // lanes past the tile: unit 0's (stores dropped)
    c0 = *(const f32x4_t*)&sc.coef[0][lo];
    c1 = *(const f32x4_t*)&sc.coef[1][lo];
    zu = *(const f32x4_t*)&sc.coef[2][lo];
  }

  // one stored row's outputs (the lane's four columns) from x, y
  template <bool kResc>
  __device__ __forceinline__ void write_row(const f32x4_t& xk, const Y& yk, int k, const f32x4_t& c0,
                                            const f32x4_t& c1, const f32x4_t& zu) const {
    float o0[4], o1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = xk[j];
      const float y = kTwo ? Sec::get(yk, j) : 0.f;
      const bool skip = OP != ColOp::kFwd && zu[j] != 0.f;
      bool scaled = false;
      int sa = 0, sb = 0;
      if constexpr (kResc) {
        const int lo = active ? lane_off : 0;
        scaled = sc.coef[3][lo + j] != 0.f;
        sa = sc.shift[0][lo + j];
        sb = sc.shift[1][lo + j];
      }
      col_values<OP>(x, y, scaled, sa, sb, c0[j], c1[j], skip, o0[j], o1[j]);
      if constexpr (OP == ColOp::kProject || OP == ColOp::kAfterStep) {
        if (skip) {                         // a zero unit is left as it is: its own bits back
          o0[j] = y;
          o1[j] = x;
        }
      }
    }
    if constexpr (OP == ColOp::kFwd) {
      step(ob, 2, k).st8(u32x2_t{pack_bf16(o0[0], o0[1]), pack_bf16(o0[2], o0[3])}, vo2);
    } else if constexpr (OP == ColOp::kBwd) {
      step(ob, 4, k).st16(__builtin_bit_cast(u32x4_t, f32x4_t{o0[0], o0[1], o0[2], o0[3]}), vo4);
    } else {
      if (two)
        step(ob, 4, k).st16(__builtin_bit_cast(u32x4_t, f32x4_t{o0[0], o0[1], o0[2], o0[3]}), vo4);
      if constexpr (OP == ColOp::kAfterStep)
        step(xb, 4, k).st16(__builtin_bit_cast(u32x4_t, f32x4_t{o1[0], o1[1], o1[2], o1[3]}), vo4);
    }
  }

  // Returns true (uniform) when the tile needs rescue(); its outputs are
  // then not written.
  __device__ __forceinline__ bool common() {
    load_tile(xv, yv);
    if (threadIdx.x == 0) sc.any_rescue = 0;  // last read before the previous tile's first barrier
    column_sums<false>(xv, yv);
    if constexpr (kTwo) {
      // the second input's conversions are not kept from the sums for the
      // outputs: the packed values take half the registers
#pragma unroll
      for (int k = 0; k < K; ++k) asm volatile("" : "+v"(yv[k]));
    }
    __syncthreads();
    // each unit: its coefficients; a sum out of fp32's range sends the
    // whole tile to rescue(), which writes them again
    if (4 * wave < tu) {                                    // uniform
      float T, P;
      totals(T, P);
      const bool out = unit_lane && !(T >= kTiny && T < __builtin_inff() && fabsf(P) < __builtin_inff());
      if (__ballot(out) != 0 && lane == 0) sc.any_rescue = 1;
      coefficients(T, P, false, 0, 0);
    }
    __syncthreads();
    // uniform (LDS after a barrier); readfirstlane tells the compiler so
    const bool rescue = __builtin_amdgcn_readfirstlane(sc.any_rescue) != 0;
    if (!rescue) {
      f32x4_t c0, c1, zu;
      coefs(c0, c1, zu);
#pragma unroll
      for (int k = 0; k < K; ++k) write_row<false>(xv[k], yv[k], k, c0, c1, zu);
    }
    return rescue;
  }

  // A sum out of range: the rescue as in the row kernels, per unit.  The
  // column maxima decide which units are rescued and their shifts, the
  // scaled sums give their coefficients (a unit not rescued has shift 0 and
  // the same sums as in common()), and the outputs are written a stored row
  // at a time, reading the tile again.  A zero unit (T = 0) comes this way
  // too.
  __device__ __forceinline__ void rescue() {
    column_max(xv, yv);
    __syncthreads();
    if (4 * wave < tu) {
      float T, P;
      totals(T, P);
      const float m0 = row16_max(sc.pmax[0][pi][pc]);
      const float m1 = row16_max(sc.pmax[1][pi][pc]);
      if (unit_lane) {
        int sa = 0, sb = 0;
        const bool fix = unit_rescue<OP>(T, P, m0, m1, sa, sb);
        sc.shift[0][pc] = sa;
        sc.shift[1][pc] = sb;
        sc.coef[3][pc] = fix ? 1.f : 0.f;
      }
    }
    __syncthreads();
    column_sums<true>(xv, yv);
    __syncthreads();
    if (4 * wave < tu) {
      float T, P;
      totals(T, P);
      if (unit_lane) coefficients(T, P, sc.coef[3][pc] != 0.f, sc.shift[0][pc], sc.shift[1][pc]);
    }
    __syncthreads();
    f32x4_t c0, c1, zu;
    coefs(c0, c1, zu);
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
      const f32x4_t xk = load_x(k);
      const Y yk = two ? load_y(k) : Y{};
      write_row<true>(xk, yk, k, c0, c1, zu);
    }
  }
};


// The seg-1 column-block kernel: single-pass tiles of 4 LPR units for the
// matrices col1_single admits, two-pass tiles (col2_tile) for the others, in
// one launch (tasks tallest first, so the long two-pass tiles start early).
// The occupancy hint is a tuning knob: 4 waves per SIMD (one workgroup per
// compute unit) lets the single-pass tile keep its registers unspilled.
#ifndef DSR_COL1_WAVES_PER_EU
#define DSR_COL1_WAVES_PER_EU 4
#endif
template <ColOp OP, int K, int LPR>
__global__ void __launch_bounds__(kColThreads)
__attribute__((amdgpu_waves_per_eu(DSR_COL1_WAVES_PER_EU, DSR_COL1_WAVES_PER_EU)))
colblock1_kernel(const TaskArgs<typename ColTaskOf<OP>::T> args) {
  using Task = typename ColTaskOf<OP>::T;
  __shared__ Col1Scratch scr[2];
  __shared__ ColScratch sc2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nitems = args.nitems;
  // Workgroup b runs on XCD b % 8: the items running together on one XCD are
  // adjacent tiles, so a line two tiles share is fetched into one L2.
  const int G = gridDim.x;
  const int b = blockIdx.x;
#ifndef DSR_COL1_XCD
#define DSR_COL1_XCD 0            // tuning knob: 1 groups adjacent tiles per XCD
#endif
  const int first = (DSR_COL1_XCD && G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  // The tile's reads: the default cache policy measured faster for these
  // 256-byte pieces of the stored rows (GPT-2's 768-row attention weights:
  // 27.4 -> 22.3 us forward), but in a launch that also holds two-pass tiles
  // (tasks run tallest first, so task 0 tells) they would push the two-pass
  // tiles' first-pass lines out of L2 before their second pass: there the
  // reads are non-temporal.
  const Task t0 = task_of(args, 0, lane);
  const bool cached = col1_single(t0.cols, t0.ld, K, LPR);
  int buf = 0;
  for (int item = first; item < nitems; item += G) {
    const Task t = scalarize(task_of(args, item, lane));
    if (col1_single(t.cols, t.ld, K, LPR)) {              // uniform
      const int64_t u0 = (int64_t)(item - t.item_begin) * 4 * LPR;
      if (cached) {
        Col1Tile<OP, K, Task, 0> tile(t, u0, scr[buf], lane, wave, LPR);
        if (tile.common()) tile.rescue();
      } else {
        Col1Tile<OP, K, Task, kCpolLd> tile(t, u0, scr[buf], lane, wave, LPR);
        if (tile.common()) tile.rescue();
      }
      buf ^= 1;
    } else {
      col2_tile<OP>(t, item, sc2, lane, wave);
    }
  }
}

}  // namespace dsr
