// Row-L2 kernels for gfx950 (CDNA4, wave64).
//
// One wave group of G waves owns one row at a time; each lane holds V
// 16-byte vectors of the row in VGPRs, so every input byte is read from HBM
// once and every output byte written once.  Vector v of wave g in a row is
// the row's 16-byte vector number (v * G + g) * 64 + lane: at every v the
// group reads one contiguous stretch of 1 KiB per wave.
//
// Sums of squares accumulate in fp32 with fused multiply-adds in two chains
// per lane (even and odd elements), then a fixed wave64 tree (DPP quad
// swaps and mirrors inside each 16-lane row, then gfx950's permlane16/32
// swaps across rows), then, for G > 1, a fixed sequential sum of the G wave
// totals through LDS.  The tree depends on cols alone (cols picks G and V),
// so a row's bits never depend on the row count, the grid or the batch.
//
// The ops (TensorFold PR #1260's two unit-sphere row kernels, the DragonScale
// README's unit-row weight op):
//   l2_rows     y = bf16(s * inv_sqrt(S + eps)), s = x or bf16(x + r)
//   slerp_rows  a = bf16(l2(res)), b = bf16(l2(out)),
//               u = a + |alpha| * (b - a) in three rounded fp32 steps,
//               h = bf16(l2(u))
//   rownorm     n = sqrt(S), c = (g * rho) / n, W_eff = bf16(w * c)
// and their gradients (the gradient of the unrounded function at the
// forward's inputs; a bf16 rounding passes the gradient through):
//   l2_rows     ds = bf16((dy - s k) inv), inv = 1/sqrt(S + eps),
//               k = <s, dy> inv^2 -- the Jacobian of s * inv is
//               (I - y y^T) inv, and x and r share ds
//   rownorm     dW = (g rho inv) (dWe - w k), k = <w, dWe> inv^2,
//               dg = rho <w, dWe> inv, inv = 1/||w|| -- the DragonScale
//               README's gradient tangent to the rows ("What DragonScale
//               changes"), and the chain rule through g
//
// Range.  When S + eps overflows fp32 or falls below 2^-96 (where squares
// may have lost bits to underflow), the row is summed again scaled by 2^k,
// k chosen from max(max|s|, sqrt(eps)) so the scaled maximum lies in [1, 2):
// a power-of-two scaling is exact, so the result is the unscaled one.  That
// branch depends only on the row's own sum and is uniform over the group.
// Afterwards the sum handed to inv_sqrt is >= 2^-96, or 0 (a zero row with
// eps = 0), infinite or NaN.
//
// This file is compiled with -ffp-contract=off: only the explicit fmaf calls
// fuse, so the lerp's three steps stay three roundings.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsr {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

constexpr float kTiny = 0x1p-96f;   // below this, S + eps is recomputed scaled

// ------------------------------------------------------- buffer resources
//
// Each row is read and written through its own buffer resource (base = the
// row's first byte, size = the row's bytes).  Offsets are per-lane VGPRs, so
// the hardware range check covers them: loads past the row return 0 and
// stores past it are dropped, which handles a ragged last vector group with
// no predicate.  Streaming accesses carry the non-temporal hint.
#ifndef DSR_CPOL_LD
#define DSR_CPOL_LD 2         // aux bits of streaming loads: 2 = nt
#endif
#ifndef DSR_CPOL_ST
#define DSR_CPOL_ST 2         // aux bits of streaming stores: 2 = nt
#endif
constexpr int kCpolLd = DSR_CPOL_LD;
constexpr int kCpolSt = DSR_CPOL_ST;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

struct RowBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ RowBuf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3)) {}
  __device__ __forceinline__ u32x4_t ld16(int off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolLd);
  }
  __device__ __forceinline__ f32x4_t ld16f(int off) const {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolLd));
  }
  __device__ __forceinline__ f32x4_t ld16f_cached(int off) const {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  __device__ __forceinline__ u32x2_t ld8(int off) const {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolLd);
  }
  // with a wave-uniform byte offset `soff` added in the scalar offset field
  __device__ __forceinline__ f32x4_t ld16f(int off, int soff) const {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kCpolLd));
  }
  __device__ __forceinline__ u32x2_t ld8(int off, int soff) const {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, kCpolLd);
  }
  __device__ __forceinline__ void st16(u32x4_t v, int off, int soff) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, soff, kCpolSt);
  }
  __device__ __forceinline__ void st8(u32x2_t v, int off, int soff) const {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, soff, kCpolSt);
  }
  __device__ __forceinline__ void st16(u32x4_t v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolSt);
  }
  __device__ __forceinline__ void st8(u32x2_t v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpolSt);
  }
  // single elements (rows whose width is not a multiple of the vector)
  __device__ __forceinline__ float ld4f(int off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCpolLd));
  }
  __device__ __forceinline__ uint32_t ld2(int off) const {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kCpolLd);
  }
  __device__ __forceinline__ void st4(float v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kCpolSt);
  }
  __device__ __forceinline__ void st2(uint32_t v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, r, off, 0, kCpolSt);
  }
};

// ---------------------------------------------------------------- bf16 pack

__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// Two fp32 values -> two bf16 (round to nearest even), low half first.
// gfx950 does this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Pairs each lane with the lane 16 (permlane16_swap) or 32 (permlane32_swap)
// away and returns (low partner, high partner): identical in both lanes.
__device__ __forceinline__ f32x2_t swap16(float v) {
  uint32_t u = __float_as_uint(v);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return f32x2_t{__uint_as_float(p[0]), __uint_as_float(p[1])};
}
__device__ __forceinline__ f32x2_t swap32(float v) {
  uint32_t u = __float_as_uint(v);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return f32x2_t{__uint_as_float(p[0]), __uint_as_float(p[1])};
}

// Sum over the 64 lanes; every lane gets the same bits (each step adds two
// equal-bit partial sums, and fp32 addition is commutative).
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v = v + dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v = v + dpp_f<0x141>(v);   // row_half_mirror
  v = v + dpp_f<0x140>(v);   // row_mirror
  f32x2_t p = swap16(v);
  v = p.x + p.y;
  p = swap32(v);
  return p.x + p.y;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  f32x2_t p = swap16(v);
  v = fmaxf(p.x, p.y);
  p = swap32(v);
  return fmaxf(p.x, p.y);
}

// Combine the G wave totals of a row through LDS (G > 1): every wave sums
// them in the order 0..G-1.  `slot` is G floats of LDS used by this call
// only; the caller alternates two slots so one barrier per combine suffices.
template <int G, int N>
__device__ __forceinline__ void group_sum(float (&v)[N], float* slot, int g, int lane) {
  if constexpr (G > 1) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) slot[i * G + g] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float t = slot[i * G];
#pragma unroll
      for (int k = 1; k < G; ++k) t = t + slot[i * G + k];
      v[i] = t;
    }
  }
}

template <int G>
__device__ __forceinline__ float group_max(float v, float* slot, int g, int lane) {
  if constexpr (G > 1) {
    if (lane == 0) slot[g] = v;
    __syncthreads();
    float t = slot[0];
#pragma unroll
    for (int k = 1; k < G; ++k) t = fmaxf(t, slot[k]);
    return t;
  }
  return v;
}

// Two maxima combined at once (slot: 2 G floats).
template <int G>
__device__ __forceinline__ void group_max2(float (&v)[2], float* slot, int g, int lane) {
  if constexpr (G > 1) {
    if (lane == 0) {
      slot[g] = v[0];
      slot[G + g] = v[1];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float t = slot[i * G];
#pragma unroll
      for (int k = 1; k < G; ++k) t = fmaxf(t, slot[i * G + k]);
      v[i] = t;
    }
  }
}

// Round-robin LDS slots for the group combines (two buffers of 2*G floats).
template <int G>
struct GroupScratch {
  float buf[2][2 * G];
  __device__ __forceinline__ float* next(int& k) { float* p = buf[k]; k ^= 1; return p; }
};
// One wave per row combines nothing, and leaves the slot index alone: a
// mixed-shape kernel interleaves such rows with its multi-wave rows, whose
// consecutive combines must still alternate slots.
template <>
struct GroupScratch<1> {
  __device__ __forceinline__ float* next(int&) { return nullptr; }
};

// Geometry of one launch: which row this wave works on, and its lane/wave.
template <int G>
struct Geo {
  static constexpr int R = (G == 1) ? 4 : 1;        // rows per workgroup pass
  static constexpr int THREADS = 64 * G * R;
  int lane, g, rr;
  __device__ __forceinline__ Geo() {
    lane = threadIdx.x & 63;
    // the wave index is uniform within a wave; saying so keeps row addresses
    // and buffer resources in SGPRs
    int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    g = (G == 1) ? 0 : wave;
    rr = (G == 1) ? wave : 0;
  }
  // A Geo made inside a loop whose lane index the compiler cannot compute
  // once, ahead of the loop.  The mixed-shape kernels make one per item: with
  // the lane hoisted, every shape's lane offsets were computed before the
  // item loop and stayed live across it (the 256-thread fp32 rownorm kernel
  // rose to 96 VGPRs, five waves per SIMD, against 60 for its largest shape
  // alone); per item, only the running shape's offsets exist.
  static __device__ __forceinline__ Geo per_item() {
    Geo q;
    asm volatile("" : "+v"(q.lane));
    return q;
  }
  __device__ __forceinline__ int vec_index(int v) const { return (v * G + g) * 64 + lane; }
  template <int V>
  __device__ __forceinline__ void offsets(int (&off)[V], int vbytes) const {
#pragma unroll
    for (int v = 0; v < V; ++v) off[v] = vec_index(v) * vbytes;
  }
};

// 1 / sqrt(T) for the row ops: the hardware estimate (v_rsq_f32, measured
// under 0.81 ulp on gfx950) refined by one Newton step in fused
// multiply-adds.  With y = (1 + d)/sqrt(T), the step returns
// (1 - 1.5 d^2 - e1/2 + e2)/sqrt(T) with e1, e2 single roundings: relative
// error at most 1.5 units of fp32 rounding, less than a correctly rounded
// sqrt followed by a correctly rounded division (2 units), in ~6 instructions
// instead of ~30.  T = 0, +inf and NaN take the estimate (+inf, 0, NaN).
// Callers pass T >= 2^-96 otherwise (smaller sums are rescaled first).
__device__ __forceinline__ float inv_sqrt(float T) {
  const float y = __builtin_amdgcn_rsqf(T);
  const float p = T * y;
  const float e = __builtin_fmaf(-p, y, 1.0f);       // 1 - T y^2
  const float r = __builtin_fmaf(0.5f * y, e, y);    // y (1 + e/2)
  return (T > 0.f && T < __builtin_inff()) ? r : y;
}

// floor(log2(x)) for finite x > 0, normal or subnormal, from the bits.
__device__ __forceinline__ int floor_log2(float x) {
  const uint32_t b = __float_as_uint(x) & 0x7fffffffu;
  const int e = (int)(b >> 23);
  return e != 0 ? e - 127 : -118 - __builtin_clz(b);
}

// Scale exponent for a rescued row: k = -floor(log2(max(m, sqrt(eps)))), so
// that max(m, sqrt(eps)) * 2^k lies in [1, 2); floor(log2(sqrt(eps))) is
// floor(floor(log2(eps)) / 2).  Needs m > 0 or eps > 0, both finite.
__device__ __forceinline__ int rescue_shift(float m, float eps) {
  int E = -1000;
  if (m > 0.f) E = floor_log2(m);
  if (eps > 0.f) {
    const int le = floor_log2(eps);
    E = max(E, le >= 0 ? le / 2 : -((1 - le) / 2));
  }
  return -E;
}

// ------------------------------------------------- packed-bf16 row in VGPRs

// V 16-byte vectors per lane = 8 bf16 each, held as 4 packed uint32.
template <int V>
struct Bf16Row {
  uint32_t p[V][4];

  __device__ __forceinline__ void load(const RowBuf& b, const int (&off)[V]) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      u32x4_t t = b.ld16(off[v]);
      p[v][0] = t.x; p[v][1] = t.y; p[v][2] = t.z; p[v][3] = t.w;
    }
  }

  // Sum of squares in two fma chains (even, odd elements); the squares of
  // bf16 values are exact in fp32, so each step rounds once.
  __device__ __forceinline__ float sumsq() const {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float lo = bf_lo(p[v][k]), hi = bf_hi(p[v][k]);
        a0 = __builtin_fmaf(lo, lo, a0);
        a1 = __builtin_fmaf(hi, hi, a1);
      }
    return a0 + a1;
  }

  __device__ __forceinline__ float sumsq_scaled(int sh) const {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float lo = ldexpf(bf_lo(p[v][k]), sh), hi = ldexpf(bf_hi(p[v][k]), sh);
        a0 = __builtin_fmaf(lo, lo, a0);
        a1 = __builtin_fmaf(hi, hi, a1);
      }
    return a0 + a1;
  }

  // <p, d> in two fma chains; products of two bf16 values are exact in fp32.
  __device__ __forceinline__ float dot(const Bf16Row& d) const {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a0 = __builtin_fmaf(bf_lo(p[v][k]), bf_lo(d.p[v][k]), a0);
        a1 = __builtin_fmaf(bf_hi(p[v][k]), bf_hi(d.p[v][k]), a1);
      }
    return a0 + a1;
  }

  __device__ __forceinline__ float dot_scaled(const Bf16Row& d, int sa, int sb) const {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a0 = __builtin_fmaf(ldexpf(bf_lo(p[v][k]), sa), ldexpf(bf_lo(d.p[v][k]), sb), a0);
        a1 = __builtin_fmaf(ldexpf(bf_hi(p[v][k]), sa), ldexpf(bf_hi(d.p[v][k]), sb), a1);
      }
    return a0 + a1;
  }

  // Forget every value derived from p so far.  Without this the compiler keeps
  // the 8V unpacked fp32 values of the sum alive until the epilogue instead of
  // unpacking again (two ALU ops), which doubles the VGPRs and halves the
  // waves that keep loads in flight.  Emits no instruction.
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(p[v][k]));
  }

  // Largest |value| of the row, on the packed bits: with the sign cleared, a
  // bf16 pattern orders like its magnitude (infinity above every finite
  // value), so a packed unsigned 16-bit max needs no unpacking.  Only used
  // when the sum is finite, i.e. the row holds no NaN.
  __device__ __forceinline__ float maxabs() const {
    u16x2_t mx = {0, 0};
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, p[v][k] & 0x7fff7fffu));
    const uint32_t top = mx.x > mx.y ? mx.x : mx.y;
    return __uint_as_float(top << 16);
  }

  // p <- bf16(p * inv), or bf16((p * 2^sh) * inv) when scaled.
  __device__ __forceinline__ void scale(float inv, bool scaled, int sh) {
    if (!scaled) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          p[v][k] = pack_bf16(bf_lo(p[v][k]) * inv, bf_hi(p[v][k]) * inv);
    } else {
      fence();    // keeps the two branches from sharing (and hoisting) their unpacking
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          p[v][k] = pack_bf16(ldexpf(bf_lo(p[v][k]), sh) * inv, ldexpf(bf_hi(p[v][k]), sh) * inv);
    }
  }

  __device__ __forceinline__ void store(const RowBuf& b, const int (&off)[V]) const {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      u32x4_t t = {p[v][0], p[v][1], p[v][2], p[v][3]};
      b.st16(t, off[v]);
    }
  }
};

// Normalise a packed-bf16 row in place: p <- bf16(p / sqrt(S + eps)), where
// S is the row's (group-combined) fp32 sum of squares.  With MEAN the sum is
// first divided by the row's length n (IEEE division): the RMS norm
// p <- bf16(p / sqrt(S / n + eps)).
template <int G, int V, bool MEAN = false>
__device__ __forceinline__ void l2_in_place(Bf16Row<V>& s, float S, float eps,
                                            GroupScratch<G>& gs, int& slot,
                                            const Geo<G>& geo, float n = 1.f) {
  float T = (MEAN ? S / n : S) + eps;
  bool scaled = false;
  int sh = 0;
  if (T == __builtin_inff() || T < kTiny) {       // uniform over the group
    float m = group_max<G>(wave_max(s.maxabs()), gs.next(slot), geo.g, geo.lane);
    s.fence();
    if ((m > 0.f || eps > 0.f) && m < __builtin_inff()) {
      sh = rescue_shift(m, eps);
      float t[1] = {wave_sum(s.sumsq_scaled(sh))};
      group_sum<G, 1>(t, gs.next(slot), geo.g, geo.lane);
      T = (MEAN ? t[0] / n : t[0]) + ldexpf(eps, 2 * sh);
      scaled = true;
    }
  }
  float inv = inv_sqrt(T);
  s.fence();      // the epilogue unpacks again rather than share the rare branch's values
  s.scale(inv, scaled, sh);
}

// ------------------------------------------------------------------ l2_rows

// MEAN: rms_rows, the same row divided by sqrt(S / n + eps) (n = 8 nvec).
template <int G, int V, bool RES, bool MEAN = false>
__global__ void __launch_bounds__(Geo<G>::THREADS)
l2_rows_kernel(const u32x4_t* x, const u32x4_t* r, u32x4_t* y, int64_t rows, int nvec, float eps) {
  constexpr int R = Geo<G>::R;
  const Geo<G> geo;
  __shared__ GroupScratch<G> gs;
  int slot = 0;
  int off[V];
  geo.offsets(off, 16);
  const uint32_t row_bytes = (uint32_t)nvec * 16u;

  {
    const int64_t row = (int64_t)blockIdx.x * R + geo.rr;   // one row group per workgroup
    if (G == 1 && row >= rows) return;            // waves of a G == 1 group are independent
    Bf16Row<V> s;
    s.load(RowBuf(x + row * nvec, row_bytes), off);
    if constexpr (RES) {
      Bf16Row<V> rv;
      rv.load(RowBuf(r + row * nvec, row_bytes), off);
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          s.p[v][k] = pack_bf16(bf_lo(s.p[v][k]) + bf_lo(rv.p[v][k]),
                                bf_hi(s.p[v][k]) + bf_hi(rv.p[v][k]));
    }
    float S[1] = {wave_sum(s.sumsq())};
    s.fence();
    group_sum<G, 1>(S, gs.next(slot), geo.g, geo.lane);
    l2_in_place<G, V, MEAN>(s, S[0], eps, gs, slot, geo, (float)(8 * nvec));
    s.store(RowBuf(y + row * nvec, row_bytes), off);
  }
}

// --------------------------------------------------------- l2_rows gradient
//
// Holds the row s (x, or bf16(x + r)) and dy packed in VGPRs; one reduction
// pass gives S = sum s^2 and P = <s, dy>.  When S + eps or P is out of fp32's
// comfortable range (S + eps overflowing or below 2^-96, P overflowing), both
// are summed again with s scaled by 2^sa and dy by 2^sb (sa from
// max(max|s|, sqrt(eps)), sb from max|dy|, bringing each maximum to [1, 2)):
// the scaled row gives ds * 2^(sb - sa) exactly, undone by one ldexp.
// MEAN: the rms_rows gradient, with S and P each divided by n = 8 nvec (IEEE
// division) before inv and k are formed.

template <int G, int V, bool RES, bool MEAN = false>
__global__ void __launch_bounds__(Geo<G>::THREADS)
l2_rows_backward_kernel(const u32x4_t* x, const u32x4_t* r, const u32x4_t* dy, u32x4_t* dx,
                        int64_t rows, int nvec, float eps) {
  constexpr int R = Geo<G>::R;
  const Geo<G> geo;
  __shared__ GroupScratch<G> gs;
  int slot = 0;
  int off[V];
  geo.offsets(off, 16);
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  const float n = (float)(8 * nvec);

  {
    const int64_t row = (int64_t)blockIdx.x * R + geo.rr;   // one row group per workgroup
    if (G == 1 && row >= rows) return;
    Bf16Row<V> s, d;
    s.load(RowBuf(x + row * nvec, row_bytes), off);
    if constexpr (RES) {
      Bf16Row<V> rv;
      rv.load(RowBuf(r + row * nvec, row_bytes), off);
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          s.p[v][k] = pack_bf16(bf_lo(s.p[v][k]) + bf_lo(rv.p[v][k]),
                                bf_hi(s.p[v][k]) + bf_hi(rv.p[v][k]));
    }
    d.load(RowBuf(dy + row * nvec, row_bytes), off);
    float acc[2] = {wave_sum(s.sumsq()), wave_sum(s.dot(d))};
    s.fence();
    d.fence();
    group_sum<G, 2>(acc, gs.next(slot), geo.g, geo.lane);
    float T = (MEAN ? acc[0] / n : acc[0]) + eps;
    float P = MEAN ? acc[1] / n : acc[1];
    bool scaled = false;
    int sa = 0, sb = 0;
    // uniform over the group; NaN sums enter too, and leave with no rescue
    if (!(T >= kTiny && T < __builtin_inff() && fabsf(P) < __builtin_inff())) {
      float m[2] = {wave_max(s.maxabs()), wave_max(d.maxabs())};
      group_max2<G>(m, gs.next(slot), geo.g, geo.lane);
      s.fence();
      d.fence();
      if ((m[0] > 0.f || eps > 0.f) && m[0] < __builtin_inff() && m[1] < __builtin_inff()) {
        sa = rescue_shift(m[0], eps);
        sb = (m[1] > 0.f) ? rescue_shift(m[1], 0.f) : 0;
        float t[2] = {wave_sum(s.sumsq_scaled(sa)), wave_sum(s.dot_scaled(d, sa, sb))};
        group_sum<G, 2>(t, gs.next(slot), geo.g, geo.lane);
        T = (MEAN ? t[0] / n : t[0]) + ldexpf(eps, 2 * sa);
        P = MEAN ? t[1] / n : t[1];
        scaled = true;
      }
    }
    const float inv = inv_sqrt(T);
    const float kk = (P * inv) * inv;
    s.fence();
    d.fence();
    if (!scaled) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = __builtin_fmaf(-bf_lo(s.p[v][k]), kk, bf_lo(d.p[v][k])) * inv;
          const float hi = __builtin_fmaf(-bf_hi(s.p[v][k]), kk, bf_hi(d.p[v][k])) * inv;
          d.p[v][k] = pack_bf16(lo, hi);
        }
    } else {
      const int sh = sa - sb;
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float slo = ldexpf(bf_lo(s.p[v][k]), sa), shi = ldexpf(bf_hi(s.p[v][k]), sa);
          const float dlo = ldexpf(bf_lo(d.p[v][k]), sb), dhi = ldexpf(bf_hi(d.p[v][k]), sb);
          const float lo = ldexpf(__builtin_fmaf(-slo, kk, dlo) * inv, sh);
          const float hi = ldexpf(__builtin_fmaf(-shi, kk, dhi) * inv, sh);
          d.p[v][k] = pack_bf16(lo, hi);
        }
    }
    d.store(RowBuf(dx + row * nvec, row_bytes), off);
  }
}

// --------------------------------------------------------------- slerp_rows

// |alpha| for this lane's columns: loaded once, before any row, when it fits
// in registers (V <= 4); wider shapes load it next to each row's lerp.
template <int V>
struct AbsAlpha {
  static constexpr bool kHeld = V <= 4;
  float a[kHeld ? V : 1][8];
  static __device__ __forceinline__ void load_into(float (&dst)[8], const RowBuf& b, int off) {
    const f32x4_t a0 = b.ld16f_cached(2 * off);
    const f32x4_t a1 = b.ld16f_cached(2 * off + 16);
    dst[0] = fabsf(a0.x); dst[1] = fabsf(a0.y); dst[2] = fabsf(a0.z); dst[3] = fabsf(a0.w);
    dst[4] = fabsf(a1.x); dst[5] = fabsf(a1.y); dst[6] = fabsf(a1.z); dst[7] = fabsf(a1.w);
  }
  __device__ __forceinline__ void init(const RowBuf& b, const int (&off)[V]) {
    if constexpr (kHeld) {
#pragma unroll
      for (int v = 0; v < V; ++v) load_into(a[v], b, off[v]);
    }
  }
};

// One row with the rescues inline, the row and its u held in registers
// (u recomputed for V > 4): the kernel's path for wide shapes.
template <int G, int V>
__device__ __forceinline__ void slerp_row_full(const u32x4_t* res, const u32x4_t* out,
                                               const RowBuf& abuf, const AbsAlpha<V>& al,
                                               u32x4_t* h, int64_t row, int nvec, float eps,
                                               GroupScratch<G>& gs, int& slot, const Geo<G>& geo,
                                               const int (&off)[V]) {
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  Bf16Row<V> a, b;
  a.load(RowBuf(res + row * nvec, row_bytes), off);
  b.load(RowBuf(out + row * nvec, row_bytes), off);
  float S[2] = {wave_sum(a.sumsq()), wave_sum(b.sumsq())};
  a.fence();
  b.fence();
  group_sum<G, 2>(S, gs.next(slot), geo.g, geo.lane);
  l2_in_place<G, V>(a, S[0], eps, gs, slot, geo);   // a = bf16(l2(res))
  l2_in_place<G, V>(b, S[1], eps, gs, slot, geo);   // b = bf16(l2(out))

  // u = a + |alpha| * (b - a), three rounded fp32 steps.  Narrow shapes keep
  // u in VGPRs; wide ones (V > 4) recompute it, bit for bit, when storing.
  constexpr bool kKeepU = V <= 4;
  float u[kKeepU ? V : 1][8];
  // Wide shapes unpack a and b and re-load alpha (an L2 hit) in each pass:
  // the fences and the empty asm with a memory clobber stop the compiler
  // from keeping the first pass's unpacked values and alpha alive instead,
  // which would spill.  None of them emits an instruction.
  auto reload_point = [&]() {
    if constexpr (!kKeepU) {
      a.fence();
      b.fence();
      asm volatile("" ::: "memory");
    }
  };
  auto lerp = [&](int v, float (&uv)[8]) {
    float tmp[8];
    if constexpr (!kKeepU) asm volatile("" ::: "memory");   // one vector's alpha at a time
    if constexpr (!AbsAlpha<V>::kHeld) al.load_into(tmp, abuf, off[v]);
    const float* alv = AbsAlpha<V>::kHeld ? al.a[AbsAlpha<V>::kHeld ? v : 0] : tmp;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float alo = bf_lo(a.p[v][k]), ahi = bf_hi(a.p[v][k]);
      const float blo = bf_lo(b.p[v][k]), bhi = bf_hi(b.p[v][k]);
      const float dlo = blo - alo, dhi = bhi - ahi;
      const float tlo = alv[2 * k] * dlo, thi = alv[2 * k + 1] * dhi;
      uv[2 * k] = alo + tlo;
      uv[2 * k + 1] = ahi + thi;
    }
  };
  float a0 = 0.f, a1 = 0.f;
  float m = 0.f;
  reload_point();
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float t[8];
    lerp(v, t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a0 = __builtin_fmaf(t[2 * k], t[2 * k], a0);
      a1 = __builtin_fmaf(t[2 * k + 1], t[2 * k + 1], a1);
    }
    if constexpr (kKeepU) {
#pragma unroll
      for (int k = 0; k < 8; ++k) u[v][k] = t[k];
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(t[k]));
    }
  }
  float Su[1] = {wave_sum(a0 + a1)};
  group_sum<G, 1>(Su, gs.next(slot), geo.g, geo.lane);

  float T = Su[0] + eps;
  bool scaled = false;
  int sh = 0;
  if (T == __builtin_inff() || T < kTiny) {          // uniform over the group
    if constexpr (kKeepU) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(u[v][k]));
    }
    m = group_max<G>(wave_max(m), gs.next(slot), geo.g, geo.lane);
    if ((m > 0.f || eps > 0.f) && m < __builtin_inff()) {
      sh = rescue_shift(m, eps);
      float c0 = 0.f, c1 = 0.f;
      reload_point();
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float t[8];
        if constexpr (kKeepU) {
#pragma unroll
          for (int k = 0; k < 8; ++k) t[k] = u[v][k];
        } else {
          lerp(v, t);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = ldexpf(t[2 * k], sh), hi = ldexpf(t[2 * k + 1], sh);
          c0 = __builtin_fmaf(lo, lo, c0);
          c1 = __builtin_fmaf(hi, hi, c1);
        }
      }
      float tt[1] = {wave_sum(c0 + c1)};
      group_sum<G, 1>(tt, gs.next(slot), geo.g, geo.lane);
      T = tt[0] + ldexpf(eps, 2 * sh);
      scaled = true;
    }
  }
  const float inv = inv_sqrt(T);
  const RowBuf hb(h + row * nvec, row_bytes);
  reload_point();
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float t[8];
    if constexpr (kKeepU) {
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = u[v][k];
    } else {
      lerp(v, t);
    }
    uint32_t q[4];
    if (scaled) {
      // a branch of its own (the empty asm keeps the compiler from turning
      // it into an ldexp and a select on every element of the common path)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = ldexpf(t[k], sh);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = pack_bf16(t[2 * k] * inv, t[2 * k + 1] * inv);
    u32x4_t w = {q[0], q[1], q[2], q[3]};
    hb.st16(w, off[v]);
  }
}

// Whether a sum handed to inv_sqrt needs no rescue (the row kernels' range).
__device__ __forceinline__ bool plain_sum(float T) {
  return !(T == __builtin_inff() || T < kTiny);
}

// One row with a sum out of range, from memory: the same arithmetic as
// slerp_row_full, in the same order, one 16-byte vector at a time (each pass
// reads the row again), so it needs few registers beside the common path.
// S: the row's sums of squares of res and out, already combined.
template <int G, int V>
__device__ __forceinline__ void slerp_row_rescue(const u32x4_t* res, const u32x4_t* out,
                                                 const RowBuf& abuf, u32x4_t* h, int64_t row,
                                                 int nvec, float eps, const float (&S)[2],
                                                 GroupScratch<G>& gs, int& slot,
                                                 const Geo<G>& geo, const int (&off)[V]) {
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  const RowBuf rb[2] = {RowBuf(res + row * nvec, row_bytes), RowBuf(out + row * nvec, row_bytes)};
  // l2_in_place's scaling of each input: p <- bf16(p inv) or bf16((p 2^sh) inv)
  float inv[2];
  bool sc[2];
  int sh[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float T = S[i] + eps;
    sc[i] = false;
    sh[i] = 0;
    if (!plain_sum(T)) {
      u16x2_t mx = {0, 0};
#pragma unroll 1
      for (int v = 0; v < V; ++v) {
        const u32x4_t p = rb[i].ld16(off[v]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, p[k] & 0x7fff7fffu));
      }
      const float m = group_max<G>(wave_max(__uint_as_float((uint32_t)(mx.x > mx.y ? mx.x : mx.y) << 16)),
                                   gs.next(slot), geo.g, geo.lane);
      if ((m > 0.f || eps > 0.f) && m < __builtin_inff()) {
        sh[i] = rescue_shift(m, eps);
        float a0 = 0.f, a1 = 0.f;
#pragma unroll 1
        for (int v = 0; v < V; ++v) {
          const u32x4_t p = rb[i].ld16(off[v]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float lo = ldexpf(bf_lo(p[k]), sh[i]), hi = ldexpf(bf_hi(p[k]), sh[i]);
            a0 = __builtin_fmaf(lo, lo, a0);
            a1 = __builtin_fmaf(hi, hi, a1);
          }
        }
        float t[1] = {wave_sum(a0 + a1)};
        group_sum<G, 1>(t, gs.next(slot), geo.g, geo.lane);
        T = t[0] + ldexpf(eps, 2 * sh[i]);
        sc[i] = true;
      }
    }
    inv[i] = inv_sqrt(T);
  }
  // u for vector v: a and b rounded as above, then the lerp's three steps
  auto u_of = [&](int v, float (&uv)[8]) {
    float al[8];
    AbsAlpha<V>::load_into(al, abuf, off[v]);
    uint32_t q[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4_t p = rb[i].ld16(off[v]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = sc[i] ? ldexpf(bf_lo(p[k]), sh[i]) : bf_lo(p[k]);
        const float hi = sc[i] ? ldexpf(bf_hi(p[k]), sh[i]) : bf_hi(p[k]);
        q[i][k] = pack_bf16(lo * inv[i], hi * inv[i]);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float alo = bf_lo(q[0][k]), ahi = bf_hi(q[0][k]);
      const float blo = bf_lo(q[1][k]), bhi = bf_hi(q[1][k]);
      const float dlo = blo - alo, dhi = bhi - ahi;
      const float tlo = al[2 * k] * dlo, thi = al[2 * k + 1] * dhi;
      uv[2 * k] = alo + tlo;
      uv[2 * k + 1] = ahi + thi;
    }
  };
  float a0 = 0.f, a1 = 0.f, m = 0.f;
#pragma unroll 1
  for (int v = 0; v < V; ++v) {
    float t[8];
    u_of(v, t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a0 = __builtin_fmaf(t[2 * k], t[2 * k], a0);
      a1 = __builtin_fmaf(t[2 * k + 1], t[2 * k + 1], a1);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(t[k]));
  }
  float Su[1] = {wave_sum(a0 + a1)};
  group_sum<G, 1>(Su, gs.next(slot), geo.g, geo.lane);
  float T = Su[0] + eps;
  bool scaled = false;
  int shu = 0;
  if (!plain_sum(T)) {                                 // uniform over the group
    m = group_max<G>(wave_max(m), gs.next(slot), geo.g, geo.lane);
    if ((m > 0.f || eps > 0.f) && m < __builtin_inff()) {
      shu = rescue_shift(m, eps);
      float c0 = 0.f, c1 = 0.f;
#pragma unroll 1
      for (int v = 0; v < V; ++v) {
        float t[8];
        u_of(v, t);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = ldexpf(t[2 * k], shu), hi = ldexpf(t[2 * k + 1], shu);
          c0 = __builtin_fmaf(lo, lo, c0);
          c1 = __builtin_fmaf(hi, hi, c1);
        }
      }
      float tt[1] = {wave_sum(c0 + c1)};
      group_sum<G, 1>(tt, gs.next(slot), geo.g, geo.lane);
      T = tt[0] + ldexpf(eps, 2 * shu);
      scaled = true;
    }
  }
  const float invu = inv_sqrt(T);
  const RowBuf hb(h + row * nvec, row_bytes);
  // every wave has read all of its vectors before the first barrier above,
  // so writing h over res or out (in place) reads nothing it wrote
#pragma unroll 1
  for (int v = 0; v < V; ++v) {
    float t[8];
    u_of(v, t);
    if (scaled) {
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = ldexpf(t[k], shu);
    }
    u32x4_t w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16(t[2 * k] * invu, t[2 * k + 1] * invu);
    hb.st16(w, off[v]);
  }
}

// The kernel.  The launcher gives every row group its own workgroup (a call
// with more row groups than one launch should hold runs as several
// launches).  Shapes up to V = 4 run a row straight through, with no rescue
// branch in the way of the schedule: a and b are loaded, then |alpha|; only a
// row whose sum falls outside the range (S + eps overflowing or below 2^-96,
// rare) is done again by slerp_row_rescue, from memory, before anything of it
// is stored.  Wider shapes take slerp_row_full.  V < 4 runs its one row with
// no loop; V >= 4 keeps a grid-stride loop (which runs once).  Measured on
// MI355X against the previous kernel (slerp_row_full in a grid-stride loop):
//   8,192 x 4,096 (4, 2): 34.4 -> 33.9 us; with the loop, 34.6;
//   8,192 x 7,168 (4, 4): 58.4-59.0 -> 59.2 us; without the loop, 59.6-59.8;
//   4,096 x 16,384 (8, 4): 69.9 -> 68.3 us; without the loop, 69.0.
template <int G, int V>
__global__ void __launch_bounds__(Geo<G>::THREADS)
slerp_rows_kernel(const u32x4_t* res, const u32x4_t* out, const f32x4_t* alpha, u32x4_t* h,
                  int64_t rows, int nvec, float eps) {
  constexpr int R = Geo<G>::R;
  const Geo<G> geo;
  __shared__ GroupScratch<G> gs;
  int slot = 0;
  int off[V];
  geo.offsets(off, 16);
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  const RowBuf abuf(alpha, row_bytes * 2u);        // alpha: cols fp32 = 2 x row_bytes
  AbsAlpha<V> al;
  if constexpr (V > 4) al.init(abuf, off);

  auto do_row = [&](int64_t row) {
    if constexpr (V > 4) {
      slerp_row_full<G, V>(res, out, abuf, al, h, row, nvec, eps, gs, slot, geo, off);
    } else {
      Bf16Row<V> a, b;
      a.load(RowBuf(res + row * nvec, row_bytes), off);
      b.load(RowBuf(out + row * nvec, row_bytes), off);
      al.init(abuf, off);
      float S[2] = {wave_sum(a.sumsq()), wave_sum(b.sumsq())};
      a.fence();
      b.fence();
      group_sum<G, 2>(S, gs.next(slot), geo.g, geo.lane);
      bool done = false;
      if (plain_sum(S[0] + eps) && plain_sum(S[1] + eps)) {    // uniform over the group
        a.scale(inv_sqrt(S[0] + eps), false, 0);                 // a = bf16(l2(res))
        b.scale(inv_sqrt(S[1] + eps), false, 0);                 // b = bf16(l2(out))
        // u = a + |alpha| (b - a), three rounded fp32 steps
        float u[V][8];
        float c0 = 0.f, c1 = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float alo = bf_lo(a.p[v][k]), ahi = bf_hi(a.p[v][k]);
            const float blo = bf_lo(b.p[v][k]), bhi = bf_hi(b.p[v][k]);
            const float dlo = blo - alo, dhi = bhi - ahi;
            const float tlo = al.a[v][2 * k] * dlo, thi = al.a[v][2 * k + 1] * dhi;
            u[v][2 * k] = alo + tlo;
            u[v][2 * k + 1] = ahi + thi;
            c0 = __builtin_fmaf(u[v][2 * k], u[v][2 * k], c0);
            c1 = __builtin_fmaf(u[v][2 * k + 1], u[v][2 * k + 1], c1);
          }
        float Su[1] = {wave_sum(c0 + c1)};
        group_sum<G, 1>(Su, gs.next(slot), geo.g, geo.lane);
        if (plain_sum(Su[0] + eps)) {                            // uniform over the group
          const float inv = inv_sqrt(Su[0] + eps);
          const RowBuf hb(h + row * nvec, row_bytes);
#pragma unroll
          for (int v = 0; v < V; ++v) {
            u32x4_t w;
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = pack_bf16(u[v][2 * k] * inv, u[v][2 * k + 1] * inv);
            hb.st16(w, off[v]);
          }
          done = true;
        }
      }
      if (__builtin_expect(!done, 0))
        slerp_row_rescue<G, V>(res, out, abuf, h, row, nvec, eps, S, gs, slot, geo, off);
    }
  };
  if constexpr (V >= 4) {
    for (int64_t base = (int64_t)blockIdx.x * R; base < rows; base += (int64_t)gridDim.x * R) {
      const int64_t row = base + geo.rr;
      if (G == 1 && row >= rows) break;
      do_row(row);
    }
  } else {
    const int64_t row = (int64_t)blockIdx.x * R + geo.rr;
    if (G == 1 && row >= rows) return;            // waves of a G == 1 group are independent
    do_row(row);
  }
}

// ---------------------------------------------------------- activation rows
//
// TensorFold PR #1260's two activation rows for Dory, each an elementwise
// prologue in front of l2_rows' normalisation over the whole row:
//   gate    t = bf16(o * sigmoid(g * sg)),                       y = bf16(l2(t))
//   swiglu  a = bf16(g * sug), b = bf16(u * suu),
//           p = bf16(silu(a) * b),                               y = bf16(l2(p))
// sigmoid(x) = 1 / (1 + exp(-x)) and silu(x) = x / (1 + exp(-x)) in fp32
// with IEEE division (torch's fp32 forms).  The scale vectors are fp32, one
// value per column, shared by every row.
//
// exp(x) = 2^(x log2 e) on gfx950's v_exp_f32, with log2 e split into two
// fp32 parts (Cody and Waite's splitting) so that the product's rounding
// error is carried into a first-order correction: t = fl(x L), d = x L - t
// + x L_lo (two fmas), exp(x) = 2^t (1 + d ln 2).  Measured against float64
// over 23M arguments spanning exp's range: within 1.22 ulp wherever the
// result is a normal fp32 number; results below 2^-126 lie in [0, 2^-126]
// (the hardware flushes), where they only ever feed 1 + e = 1.  8 VALU
// instructions against 13 for the device library's expf.

enum class Act { kGate, kSwiglu };

__device__ __forceinline__ float exp_split(float x) {
  const float kL = 0x1.715476p+0f;        // log2(e) rounded to fp32
  const float kLlo = 0x1.4ae0cp-26f;      // log2(e) - kL, rounded to fp32
  const float kLn2 = 0x1.62e430p-1f;      // ln(2) rounded to fp32
  const float t = x * kL;
  float d = __builtin_fmaf(x, kL, -t);    // exactly x kL - t
  d = __builtin_fmaf(x, kLlo, d);         // + x (log2(e) - kL)
  const float e0 = __builtin_amdgcn_exp2f(t);
  const float r = __builtin_fmaf(e0, d * kLn2, e0);   // 2^t (1 + d ln 2)
  // 2^t overflowed (inf + inf * d is NaN for d < 0), or x is not finite:
  // 2^t alone is the limit
  return __builtin_isfinite(r) ? r : e0;
}

// 1 / b for b in [1, 2^126): gfx950's v_rcp_f32 estimate y and one fma
// correction, y + y (1 - b y).  Over every fp32 b in [1, 2^126) this equals
// the IEEE quotient (checked exhaustively on the GPU by the tests); from
// 2^126 up the quotient is subnormal, which v_rcp_f32 flushes, so callers
// take the IEEE division there.
__device__ __forceinline__ float recip_fast(float b) {
  const float y = __builtin_amdgcn_rcpf(b);
  return __builtin_fmaf(__builtin_fmaf(-b, y, 1.0f), y, y);
}

// silu(a) = a / (1 + exp(-a)) in fp32 with IEEE division.
__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + exp_split(-a)); }

// The SwiGLU silu table.  SwiGLU's silu input a = bf16(g * sug) is a bf16
// value, so silu(a) can come from a table instead of the exp, the add and
// the division.  A workgroup that loops over many rows fills one table in
// LDS and reuses it: silu(a) for the 8,192 bf16 values whose exponent field
// lies in [kSiluE0, kSiluE0 + 31] (magnitudes 2^-25 up to 2^7, both signs),
// entry (sign << 12) | ((bits & 0x7fff) - (kSiluE0 << 7)).  Each entry is
// computed by silu_f32, the code of the formula path, so a lookup returns
// the bits the formula does.  Any other a (zero, tiny, huge, infinite, NaN)
// takes the formula.
constexpr uint32_t kSiluE0 = 102;
constexpr uint32_t kSiluBase = kSiluE0 << 7;
constexpr int kSiluEntries = 8192;
// rows a resident workgroup must have to fill a table (measured)
constexpr int kSiluTableRows = 2;

// The fp32 column scales of this lane's columns: NV vectors of 8 values per
// 16-byte row vector; held in VGPRs when the shape is narrow, else re-read
// (from L2) next to each row.
template <int V, int NS>
struct ColScales {
  static constexpr bool kHeld = V * NS <= 4;
  float c[kHeld ? V : 1][NS][8];
  __device__ __forceinline__ static void load_into(float (&dst)[8], const RowBuf& b, int off) {
    const f32x4_t a0 = b.ld16f_cached(2 * off);
    const f32x4_t a1 = b.ld16f_cached(2 * off + 16);
    dst[0] = a0.x; dst[1] = a0.y; dst[2] = a0.z; dst[3] = a0.w;
    dst[4] = a1.x; dst[5] = a1.y; dst[6] = a1.z; dst[7] = a1.w;
  }
  __device__ __forceinline__ void init(const RowBuf& b0, const RowBuf& b1, const int (&off)[V]) {
    if constexpr (kHeld) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        load_into(c[v][0], b0, off[v]);
        if constexpr (NS == 2) load_into(c[v][NS - 1], b1, off[v]);
      }
    }
  }
};

// One row vector's 8 outputs of the prologue, packed: x0 and x1 hold the two
// input rows' packed values (o, g for the gate; g, u for SwiGLU).
template <Act A, bool TABLE = false>
__device__ __forceinline__ void act_prologue(uint32_t (&out)[4], const uint32_t (&x0)[4],
                                             const uint32_t (&x1)[4], const float* s0,
                                             const float* s1, const float* tab = nullptr) {
  float sig[8];
  if constexpr (A == Act::kGate) {
    // sigmoid(g * sg) = 1 / b, b = 1 + exp(-g sg) in [1, +inf] or NaN: the
    // reciprocal and one fma correction, which equals the IEEE quotient for
    // every fp32 b in [1, 2^126) (checked exhaustively on gfx950); past that
    // the quotient is subnormal (v_rcp_f32 flushes it), +0 or NaN, so a
    // vector holding such a b in any lane takes the IEEE division for all
    // its values (a wave-uniform branch).
    float b[8];
    bool slow = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = ((j & 1) ? bf_hi(x1[j / 2]) : bf_lo(x1[j / 2])) * s0[j];   // g * sg
      b[j] = 1.0f + exp_split(-x);
      sig[j] = recip_fast(b[j]);
      slow |= !(b[j] < 0x1p126f);
    }
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
      asm volatile("" ::: "memory");     // a branch of its own, not a select per value
#pragma unroll
      for (int j = 0; j < 8; ++j) sig[j] = 1.0f / b[j];
    }
  }
  if constexpr (A == Act::kGate) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        r[h] = (h ? bf_hi(x0[k]) : bf_lo(x0[k])) * sig[2 * k + h];   // o * sigmoid, rounded below
      out[k] = pack_bf16(r[0], r[1]);
    }
  } else {
    // a = bf16(g * sug) and b = bf16(u * suu), both elements of a pair at once
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t ap = pack_bf16(bf_lo(x0[k]) * s0[2 * k], bf_hi(x0[k]) * s0[2 * k + 1]);
      const uint32_t bp = pack_bf16(bf_lo(x1[k]) * s1[2 * k], bf_hi(x1[k]) * s1[2 * k + 1]);
      float sl, sh;
      const uint32_t ilo = (ap & 0x7fffu) - kSiluBase, ihi = ((ap >> 16) & 0x7fffu) - kSiluBase;
      // a value outside the table sends the wave's pair to the formula (a
      // wave-uniform branch)
      if (!TABLE || __builtin_amdgcn_ballot_w64((ilo >= 4096u) | (ihi >= 4096u)) != 0) {
        sl = silu_f32(bf_lo(ap));
        sh = silu_f32(bf_hi(ap));
      } else {
        sl = tab[ilo | ((ap >> 3) & 0x1000u)];
        sh = tab[ihi | ((ap >> 19) & 0x1000u)];
      }
      out[k] = pack_bf16(sl * bf_lo(bp), sh * bf_hi(bp));   // silu(a) b, rounded
    }
  }
}

// TABLE (SwiGLU only): fill the silu table first; the launcher then runs a
// grid of resident workgroups, each looping over several rows.
template <int G, int V, Act A, bool TABLE>
__device__ __forceinline__ void act_rows(const u32x4_t* in0, const u32x4_t* in1,
                                         const f32x4_t* sc0, const f32x4_t* sc1, u32x4_t* y,
                                         int64_t rows, int nvec, float eps) {
  static_assert(!TABLE || A == Act::kSwiglu, "the table holds silu");
  constexpr int R = Geo<G>::R;
  constexpr int NS = (A == Act::kGate) ? 1 : 2;
  const Geo<G> geo;
  __shared__ GroupScratch<G> gs;
  __shared__ float tab[TABLE ? kSiluEntries : 1];
  int off[V];
  geo.offsets(off, 16);
  const uint32_t row_bytes = (uint32_t)nvec * 16u;
  Bf16Row<V> t, q;
  bool loaded = false;
  int64_t base = (int64_t)blockIdx.x * R;
  if constexpr (TABLE) {
    // the first row's loads go out before the table is filled, so the fill
    // runs while they are in flight
    const int64_t row = base + geo.rr;
    if (row < rows) {
      t.load(RowBuf(in0 + row * nvec, row_bytes), off);
      q.load(RowBuf(in1 + row * nvec, row_bytes), off);
      loaded = true;
    }
    for (int i = (int)threadIdx.x; i < kSiluEntries; i += Geo<G>::THREADS) {
      const uint32_t bits = ((uint32_t)(i >> 12) << 15) | (kSiluBase + (uint32_t)(i & 4095));
      tab[i] = silu_f32(__uint_as_float(bits << 16));
    }
    __syncthreads();
  }
  int slot = 0;
  const RowBuf sb0(sc0, row_bytes * 2u);                        // cols fp32 = 2 x row bytes
  const RowBuf sb1(NS == 2 ? sc1 : sc0, row_bytes * 2u);
  ColScales<V, NS> cs;
  cs.init(sb0, sb1, off);

  for (; base < rows; base += (int64_t)gridDim.x * R) {
    const int64_t row = base + geo.rr;
    if (G == 1 && row >= rows) break;
    if (!loaded) {
      t.load(RowBuf(in0 + row * nvec, row_bytes), off);
      q.load(RowBuf(in1 + row * nvec, row_bytes), off);
    }
    loaded = false;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float tmp[NS][8];
      if constexpr (!ColScales<V, NS>::kHeld) {
        asm volatile("" ::: "memory");          // one vector's scales at a time
        ColScales<V, NS>::load_into(tmp[0], sb0, off[v]);
        if constexpr (NS == 2) ColScales<V, NS>::load_into(tmp[NS - 1], sb1, off[v]);
      }
      const float* s0 = ColScales<V, NS>::kHeld ? cs.c[ColScales<V, NS>::kHeld ? v : 0][0] : tmp[0];
      const float* s1 = ColScales<V, NS>::kHeld ? cs.c[ColScales<V, NS>::kHeld ? v : 0][NS - 1]
                                                : tmp[NS - 1];
      act_prologue<A, TABLE>(t.p[v], t.p[v], q.p[v], s0, s1, tab);
    }
    float S[1] = {wave_sum(t.sumsq())};
    t.fence();
    group_sum<G, 1>(S, gs.next(slot), geo.g, geo.lane);
    l2_in_place<G, V>(t, S[0], eps, gs, slot, geo);
    t.store(RowBuf(y + row * nvec, row_bytes), off);
  }
}

template <int G, int V, Act A>
__global__ void __launch_bounds__(Geo<G>::THREADS)
act_l2_rows_kernel(const u32x4_t* in0, const u32x4_t* in1, const f32x4_t* sc0,
                   const f32x4_t* sc1, u32x4_t* y, int64_t rows, int nvec, float eps) {
  act_rows<G, V, A, false>(in0, in1, sc0, sc1, y, rows, nvec, eps);
}

// SwiGLU through the silu table (the launcher runs the resident workgroups).
template <int G, int V>
__global__ void __launch_bounds__(Geo<G>::THREADS)
swiglu_table_l2_rows_kernel(const u32x4_t* in0, const u32x4_t* in1, const f32x4_t* sc0,
                            const f32x4_t* sc1, u32x4_t* y, int64_t rows, int nvec, float eps) {
  act_rows<G, V, Act::kSwiglu, true>(in0, in1, sc0, sc1, y, rows, nvec, eps);
}

// ----------------------------------------------------------------- q/k rows
//
// TensorFold PR #1260's q/k row kernel, in dory.py's order: rotate-half RoPE
// on the projection's bf16 heads with the fp32 angle fp32(pos) * inv_i,
// rounded to bf16 (r); each head's L2 norm with eps, rounded (n); q's heads
// times an fp32 scale vector, rounded; k's heads are n.
//   r_i        = bf16(x_i cos t_i - x_{i+HD/2} sin t_i)        i < HD/2
//   r_{i+HD/2} = bf16(x_{i+HD/2} cos t_i + x_i sin t_i)
// each product and the sum rounded once in fp32 (no contraction).
//
// Two waves per token row, two rows per workgroup.  A head spreads over 32
// lanes: NV = HD/32 values each (16 bytes for HD = 256, 8 for HD = 128).
// Lane l of a head holds elements NV (l mod 16) .. +NV-1 of half l / 16, so
// its rotate-half partner is 16 lanes away -- one v_permlane16_swap per
// packed dword gives every lane both halves -- and two heads go through the
// wave at a time (a wave step).  The row's q steps followed by its k steps
// are split into two contiguous halves, one per wave; each head's arithmetic
// is the same whichever wave runs it.  A row has HD/2 distinct angles, the
// same for every head: the row's two waves evaluate them once between them,
// one per lane (the device library's sincosf, with its full-range argument
// reduction, of the fp32 product pos * inv), and put them in LDS; after a
// barrier every lane reads its NV cosines and sines (a lane would otherwise
// evaluate NV of them itself, and every angle is needed by 8 lanes of the
// row).  Heads are loaded CH wave steps at a time to keep several loads in
// flight.  For 8,192 rows of 16 + 4 heads of 256, the second wave per row
// took it from 40.4 to 37.5 us, and 16-byte lanes (half the wave steps and
// per-head sums) from there to 34.8 us.

struct QkArgs {
  const uint16_t* q;
  const uint16_t* k;            // may be null when nk == 0
  const int32_t* pos;
  const float* inv_freq;        // [HD/2]
  const float* q_scale;         // [nq * HD]
  uint16_t* qo;
  uint16_t* ko;
  int64_t ldq, ldk, ldqo, ldko; // row strides in elements
  int64_t rows;
  int32_t nq, nk;
  float eps;
};

// Sum and maximum over each 32-lane half of the wave (one head each).
__device__ __forceinline__ float head_sum(float v) {
  v = v + dpp_f<0xB1>(v);
  v = v + dpp_f<0x4E>(v);
  v = v + dpp_f<0x141>(v);
  v = v + dpp_f<0x140>(v);
  const f32x2_t p = swap16(v);
  return p.x + p.y;
}

__device__ __forceinline__ float head_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const f32x2_t p = swap16(v);
  return fmaxf(p.x, p.y);
}

// (low-half value, high-half value) of a packed dword between rotate-half
// partners, 16 lanes apart
__device__ __forceinline__ void partner_pair(uint32_t u, uint32_t& lo, uint32_t& hi) {
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  lo = p[0];
  hi = p[1];
}

// Rows per 256-thread workgroup: two waves each.
constexpr int kQkRowsPerBlock = 2;

template <int HD>
__global__ void __launch_bounds__(256) qk_rows_l2_kernel(const QkArgs a) {
  constexpr int NV = HD / 32;            // values per lane
  constexpr int L = 32;                  // lanes per head
  constexpr int HPW = 64 / L;            // heads per wave step
  // wave steps loaded at once (measured with two waves per row): at HD = 256
  // 3 (34.4 us for 16 + 4 heads, against 35.3 at 4 and 35.7 at 5); at
  // HD = 128, 5 (3 and 4 were slower)
  constexpr int CH = HD == 256 ? 3 : 5;
  static_assert(HD == 256 || HD == 128, "head_dim 128 or 256");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave & 1;             // which half of the row's wave steps
  const int rsub = wave >> 1;            // which row of the workgroup
  const int ll = lane % L;               // lane within its head
  const int hsub = lane / L;             // head within the wave step
  const bool upper = ll >= L / 2;        // holds the second half of the head
  const int e0 = (upper ? HD / 2 : 0) + NV * (ll % (L / 2));   // first element of the lane
  const int f0 = NV * (ll % (L / 2));                          // first frequency of the lane
  // the angle this lane evaluates for its row: frequency part * NF/2 + lane
  constexpr int NF = HD / 2;
  const int fi = part * (NF / 2) + lane;
  const bool evaluates = lane < NF / 2;
  const float invf = evaluates ? a.inv_freq[fi] : 0.f;
  // per row of the workgroup: cos then sin of its NF angles; two buffers,
  // alternated per row, so one barrier per row orders the writes and reads
  __shared__ __attribute__((aligned(16))) float trig[2][kQkRowsPerBlock][2][NF];
  int buf = 0;
  const RowBuf sb(a.q_scale, (uint32_t)a.nq * (uint32_t)HD * 4u);
  const int nsteps[2] = {(a.nq + HPW - 1) / HPW, (a.nk + HPW - 1) / HPW};
  // this wave's steps: [first, last) of q's then k's, as a range in each
  const int total = nsteps[0] + nsteps[1];
  const int first = part * ((total + 1) / 2), last = min(total, first + (total + 1) / 2);
  const int lo[2] = {min(first, nsteps[0]), max(0, min(first - nsteps[0], nsteps[1]))};
  const int hi[2] = {min(last, nsteps[0]), max(0, min(last - nsteps[0], nsteps[1]))};

  // one row group per workgroup (no loop); every wave takes part in the
  // barrier (it is workgroup-wide), and a wave whose row is past the end
  // leaves after it
  {
    const int64_t base = (int64_t)blockIdx.x * kQkRowsPerBlock;
    const int64_t row = base + rsub;
    const bool valid = row < a.rows;
    float(&cs)[2][NF] = trig[buf][rsub];
    buf ^= 1;
    if (valid && evaluates) {
      float sv, cv;
      sincosf((float)a.pos[row] * invf, &sv, &cv);
      cs[0][fi] = cv;
      cs[1][fi] = sv;
    }
    __syncthreads();
    if (!valid) return;
    float c[NV], s[NV];
#pragma unroll
    for (int q4 = 0; q4 < NV / 4; ++q4) {
      const f32x4_t cv = *reinterpret_cast<const f32x4_t*>(&cs[0][f0 + 4 * q4]);
      const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(&cs[1][f0 + 4 * q4]);
      c[4 * q4] = cv.x; c[4 * q4 + 1] = cv.y; c[4 * q4 + 2] = cv.z; c[4 * q4 + 3] = cv.w;
      s[4 * q4] = sv.x; s[4 * q4 + 1] = sv.y; s[4 * q4 + 2] = sv.z; s[4 * q4 + 3] = sv.w;
    }
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const int nh = which == 0 ? a.nq : a.nk;
      if (lo[which] >= hi[which]) continue;           // q's heads, then k's
      const uint16_t* src = which == 0 ? a.q + row * a.ldq : a.k + row * a.ldk;
      uint16_t* dst = which == 0 ? a.qo + row * a.ldqo : a.ko + row * a.ldko;
      const uint32_t bytes = (uint32_t)nh * (uint32_t)HD * 2u;
      const RowBuf ib(src, bytes), ob(dst, bytes);
      for (int st0 = lo[which]; st0 < hi[which]; st0 += CH) {
        uint32_t x[CH][NV / 2];
#pragma unroll
        for (int c4 = 0; c4 < CH; ++c4) {
          // only this wave's steps (the other wave loads the rest); a head
          // index past the last head reads 0 through the range check
          const int h = (st0 + c4) * HPW + hsub;
          if constexpr (NV == 8) {
            const u32x4_t t = st0 + c4 < hi[which] ? ib.ld16((h * HD + e0) * 2) : u32x4_t{0u, 0u, 0u, 0u};
            x[c4][0] = t.x; x[c4][1] = t.y; x[c4][2] = t.z; x[c4][3] = t.w;
          } else {
            const u32x2_t t = st0 + c4 < hi[which] ? ib.ld8((h * HD + e0) * 2) : u32x2_t{0u, 0u};
            x[c4][0] = t.x; x[c4][1] = t.y;
          }
        }
#pragma unroll
        for (int c4 = 0; c4 < CH; ++c4) {
          if (st0 + c4 >= hi[which]) break;            // uniform
          const int h = (st0 + c4) * HPW + hsub;
          float own[NV], par[NV];
#pragma unroll
          for (int d = 0; d < NV / 2; ++d) {
            uint32_t plo, phi;
            partner_pair(x[c4][d], plo, phi);
            const uint32_t pq = upper ? plo : phi;
            own[2 * d] = bf_lo(x[c4][d]); own[2 * d + 1] = bf_hi(x[c4][d]);
            par[2 * d] = bf_lo(pq); par[2 * d + 1] = bf_hi(pq);
          }
          // own value times cos plus the partner's times +-sin: the lower half
          // is x1 c + x2 (-s), the upper x2 c + x1 s; fl(a + fl(-b s)) is
          // fl(a - fl(b s)), so negating first changes no rounding
          float rot[NV];
#pragma unroll
          for (int j = 0; j < NV; ++j) rot[j] = own[j] * c[j] + par[j] * (upper ? s[j] : -s[j]);
          uint32_t r[NV / 2];
#pragma unroll
          for (int d = 0; d < NV / 2; ++d) r[d] = pack_bf16(rot[2 * d], rot[2 * d + 1]);
          float rv[NV];
#pragma unroll
          for (int d = 0; d < NV / 2; ++d) { rv[2 * d] = bf_lo(r[d]); rv[2 * d + 1] = bf_hi(r[d]); }
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < NV; ++j) acc = __builtin_fmaf(rv[j], rv[j], acc);
          float T = head_sum(acc) + a.eps;
          int sh = 0;
          const bool need = T == __builtin_inff() || T < kTiny;
          if (__builtin_amdgcn_ballot_w64(need) != 0) {  // any head of this wave step
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) m = fmaxf(m, fabsf(rv[j]));
            m = head_max(m);
            if (need && (m > 0.f || a.eps > 0.f) && m < __builtin_inff()) sh = rescue_shift(m, a.eps);
            float acc2 = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
              const float v = ldexpf(rv[j], sh);
              acc2 = __builtin_fmaf(v, v, acc2);
            }
            const float T2 = head_sum(acc2) + ldexpf(a.eps, 2 * sh);
            if (sh != 0) T = T2;
#pragma unroll
            for (int j = 0; j < NV; ++j) rv[j] = ldexpf(rv[j], sh);
          }
          const float inv = inv_sqrt(T);
          uint32_t n[NV / 2];
#pragma unroll
          for (int d = 0; d < NV / 2; ++d) n[d] = pack_bf16(rv[2 * d] * inv, rv[2 * d + 1] * inv);
          if (which == 0) {
#pragma unroll
            for (int q4 = 0; q4 < NV / 4; ++q4) {
              const f32x4_t sc = sb.ld16f_cached((h * HD + e0 + 4 * q4) * 4);
              n[2 * q4] = pack_bf16(bf_lo(n[2 * q4]) * sc.x, bf_hi(n[2 * q4]) * sc.y);
              n[2 * q4 + 1] = pack_bf16(bf_lo(n[2 * q4 + 1]) * sc.z, bf_hi(n[2 * q4 + 1]) * sc.w);
            }
          }
          if constexpr (NV == 8) {
            const u32x4_t o = {n[0], n[1], n[2], n[3]};
            ob.st16(o, (h * HD + e0) * 2);
          } else {
            const u32x2_t o = {n[0], n[1]};
            ob.st8(o, (h * HD + e0) * 2);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------- weight rownorm+gain
//
// The fp32 weight kernels take NE values per lane-vector: NE = 4 (16-byte
// accesses) for rows whose width is a multiple of 4, NE = 1 (single
// elements) for the others, such as a convolution's 3 x 7 x 7 = 147.  A
// lane's values at vector v are elements NE * vec_index(v) + k of the row.

template <int NE>
struct F32Vec {
  static_assert(NE == 4 || NE == 1, "4 or 1 values per lane-vector");
  __device__ __forceinline__ static void load(const RowBuf& b, int off, float (&d)[NE]) {
    if constexpr (NE == 4) {
      const f32x4_t q = b.ld16f(off);
      d[0] = q.x; d[1] = q.y; d[2] = q.z; d[3] = q.w;
    } else {
      d[0] = b.ld4f(off);
    }
  }
  __device__ __forceinline__ static void store(const RowBuf& b, int off, const float (&v)[NE]) {
    if constexpr (NE == 4) {
      const f32x4_t o = {v[0], v[1], v[2], v[3]};
      b.st16(__builtin_bit_cast(u32x4_t, o), off);
    } else {
      b.st4(v[0], off);
    }
  }
};

// NE bf16 values, packed two to a register (one, in the low half, for NE = 1).
template <int NE>
struct Bf16Vec {
  static constexpr int P = (NE + 1) / 2;
  uint32_t p[P];
  __device__ __forceinline__ void load(const RowBuf& b, int off) {
    if constexpr (NE == 4) {
      const u32x2_t q = b.ld8(off);
      p[0] = q.x; p[1] = q.y;
    } else {
      p[0] = b.ld2(off);
    }
  }
  __device__ __forceinline__ float get(int k) const { return (k & 1) ? bf_hi(p[k / 2]) : bf_lo(p[k / 2]); }
  // |max| over the packed values, on the bits (a bf16 pattern with the sign
  // cleared orders like its magnitude)
  __device__ __forceinline__ u16x2_t absmax(u16x2_t mx) const {
#pragma unroll
    for (int i = 0; i < P; ++i)
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, p[i] & 0x7fff7fffu));
    return mx;
  }
};

// Store NE values as bf16 (round to nearest even).
template <int NE>
__device__ __forceinline__ void store_bf16(const RowBuf& b, int off, const float (&v)[NE]) {
  if constexpr (NE == 4) {
    const u32x2_t o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    b.st8(o, off);
  } else {
    b.st2(pack_bf16(v[0], 0.f), off);
  }
}

// One matrix of a ragged call, as the kernel reads it.  Items are groups of
// R rows; matrix m owns items [item_begin, item_begin + ceil(rows / R)).
struct RownormTask {
  const float* w;
  const float* gain;    // null: no gain (g = 1)
  float* norm_out;      // may be null
  uint16_t* w_eff;
  int64_t rows;
  int32_t cols;
  float radius;
  int32_t item_begin;
  int32_t gain_stride;  // 1: a gain per row; 0: one gain for the matrix
  int32_t seg;          // column-block layouts: values per stored row (0: rows)
  int32_t shape;        // row kernel shape key, NE * 10000 + G * 100 + V
  int64_t ld;           // column-block layouts: elements between stored rows
};

// One matrix of a ragged gradient call.
struct RownormGradTask {
  const float* w;
  const float* gain;    // null: no gain (g = 1)
  const uint16_t* dw_eff;
  float* dw;
  float* dgain;         // may be null; each row's share rho <w, dWe> / ||w||
  int64_t rows;
  int32_t cols;
  float radius;
  int32_t item_begin;
  int32_t gain_stride;  // 1: a gain per row; 0: one gain for the matrix
  int32_t seg;          // column-block layouts (as in RownormTask)
  int32_t shape;        // as in RownormTask
  int64_t ld;
};

// Global-memory view of a task pointer: plain loads and stores through it
// compile to global (not flat) accesses, counted only against the
// vector-memory counter.  A flat access also counts against the counter the
// scalar loads wait on, so a row's last flat store would hold up the next
// item's task load.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem_out(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// The gain of a row: its own, the matrix's one value, or 1 with no gain.
template <class Task>
__device__ __forceinline__ float row_gain(const Task& t, int64_t row) {
  return t.gain != nullptr ? gmem(t.gain)[row * t.gain_stride] : 1.f;
}

// The tasks of one launch.  Up to kInlineTasks of them travel inside the
// kernel arguments (no copy, no device allocation, safe to capture in a
// graph); larger batches point at a table staged in device memory.
constexpr int kInlineTasks = 48;
template <class Task>
struct TaskArgs {
  const Task* tasks;             // staged table, or null: use the inline arrays
  const int32_t* begins;         // staged item_begin array (with `tasks`)
  int32_t ntasks;
  int32_t nitems;
  int32_t inline_begins[kInlineTasks];
  Task inline_tasks[kInlineTasks];
};
using RownormArgs = TaskArgs<RownormTask>;
using RownormGradArgs = TaskArgs<RownormGradTask>;
static_assert(sizeof(RownormArgs) <= 4096, "kernel arguments are limited to 4 KiB");
static_assert(sizeof(RownormGradArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Index of the task owning `item`: the number of tasks whose first item is
// <= item, minus one.  Tasks are in ascending item_begin order; each lane
// tests one task and a ballot counts them, 64 per pass.
template <class Task>
__device__ __forceinline__ int owning_task(const TaskArgs<Task>& a, int item, int lane) {
  const int32_t* begins = a.tasks != nullptr ? a.begins : a.inline_begins;
  int count = 0;
  for (int base = 0; base < a.ntasks; base += 64) {
    const int k = base + lane;
    const int b = (k < a.ntasks) ? begins[k] : 0x7fffffff;
    const int c = __popcll(__ballot(b <= item));
    count += c;
    if (c < 64) break;                        // uniform: the ballot is the same in every lane
  }
  return count - 1;
}

// A value known to be uniform, moved word by word into scalar registers.
template <class T>
__device__ __forceinline__ T scalarize(const T& v) {
  static_assert(sizeof(T) % 4 == 0, "whole words");
  struct Words {
    uint32_t w[sizeof(T) / 4];
  };
  Words a = __builtin_bit_cast(Words, v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) a.w[i] = __builtin_amdgcn_readfirstlane(a.w[i]);
  return __builtin_bit_cast(T, a);
}

// The task owning `item`, in scalar registers.  The owner comes from the
// ballot search (none for a launch of one task); a task in the kernel
// arguments is then read with scalar loads, one in a staged table with a
// vector load whose words are moved to scalar registers.  Either way every
// address the row's buffer resources are made from is uniform and in scalar
// registers: a task left in VGPRs makes the compiler wrap each buffer load
// and store of the row in a readfirstlane loop.  (A scan of the kernel
// arguments' item starts on the scalar unit instead of the ballot was
// measured slower: the compiler kept all 47 starts in SGPRs across the item
// loop, spilling, and a 768-wide item's rows are short.)
template <class Task>
__device__ __forceinline__ Task task_of(const TaskArgs<Task>& a, int item, int lane) {
  if (a.tasks == nullptr) {
    const int lo = a.ntasks == 1 ? 0 : __builtin_amdgcn_readfirstlane(owning_task(a, item, lane));
    return a.inline_tasks[lo];
  }
  const int lo = __builtin_amdgcn_readfirstlane(owning_task(a, item, lane));
  return scalarize(a.tasks[lo]);
}

// One item (R rows) of a task.  Shared by the one-shape kernel below and the
// mixed-shape kernels of a ragged call (one launch per workgroup size).
template <int G, int V, int NE>
__device__ __forceinline__ void rownorm_item(const RownormTask& t, int item, const Geo<G>& geo,
                                             GroupScratch<G>& gs, int& slot) {
  constexpr int R = Geo<G>::R;
  int off[V];
  geo.offsets(off, 4 * NE);
  {
    const int64_t row = (int64_t)(item - t.item_begin) * R + geo.rr;
    if (G == 1 && row >= t.rows) return;            // independent waves only
    // the gain is read with the row, ahead of any store (a later read could
    // not move above the norm store, and would add a memory round trip)
    const float gr = row_gain(t, row) * t.radius;
    const RowBuf wb(t.w + row * t.cols, (uint32_t)t.cols * 4u);
    float w[V][NE];
#pragma unroll
    for (int v = 0; v < V; ++v) F32Vec<NE>::load(wb, off[v], w[v]);
    // two fma chains, alternating over the row's elements
    float a[2] = {0.f, 0.f};
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < NE; ++k) a[(v * NE + k) & 1] = __builtin_fmaf(w[v][k], w[v][k], a[(v * NE + k) & 1]);
    float S[1] = {wave_sum(a[0] + a[1])};
    group_sum<G, 1>(S, gs.next(slot), geo.g, geo.lane);
    float T = S[0];
    bool scaled = false;
    int sh = 0;
    if (T == __builtin_inff() || T < kTiny) {
      float m = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < NE; ++k) m = fmaxf(m, fabsf(w[v][k]));
      m = group_max<G>(wave_max(m), gs.next(slot), geo.g, geo.lane);
      if (m > 0.f && m < __builtin_inff()) {
        sh = rescue_shift(m, 0.f);
        float c[2] = {0.f, 0.f};
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < NE; ++k) {
            const float q = ldexpf(w[v][k], sh);
            c[(v * NE + k) & 1] = __builtin_fmaf(q, q, c[(v * NE + k) & 1]);
          }
        float tt[1] = {wave_sum(c[0] + c[1])};
        group_sum<G, 1>(tt, gs.next(slot), geo.g, geo.lane);
        T = tt[0];
        scaled = true;
      }
    }
    const float rn = sqrtf(T);                       // length (of the scaled row)
    if (t.norm_out != nullptr && geo.g == 0 && geo.lane == 0)
      gmem_out(t.norm_out)[row] = scaled ? ldexpf(rn, -sh) : rn;
    const float c = (rn == 0.f) ? 0.f : gr / rn;
    const RowBuf eb(t.w_eff + row * t.cols, (uint32_t)t.cols * 2u);
    if (scaled) {
      // a rescued row's values, scaled in a branch of its own: the empty asm
      // keeps the compiler from turning it into an ldexp and a select on
      // every element of the common path
      asm volatile("" ::: "memory");
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < NE; ++k) w[v][k] = ldexpf(w[v][k], sh);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float q[NE];
#pragma unroll
      for (int k = 0; k < NE; ++k) q[k] = w[v][k] * c;
      store_bf16<NE>(eb, off[v] / 2, q);
    }
  }
}

template <int G, int V, int NE>
__global__ void __launch_bounds__(Geo<G>::THREADS)
rownorm_kernel(const RownormArgs args) {
  const Geo<G> geo;
  __shared__ GroupScratch<G> gs;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x)
    rownorm_item<G, V, NE>(task_of(args, item, geo.lane), item, geo, gs, slot);
}

// ------------------------------------------------ weight rownorm gradient
//
// Per row: S = sum w^2 and P = <w, dWe> in one pass (w fp32, dWe bf16), then
// dg = (rho P) inv, k = (P inv) inv, c = (g rho) inv and
// dW_j = c (dWe_j - w_j k).  Out-of-range sums are recomputed with w scaled
// by 2^sa and dWe by 2^sb (as for l2_rows' gradient; no eps here).  A zero
// row gets exact zeros: the forward scales it by the constant 0.

template <int G, int V, int NE>
__device__ __forceinline__ void rownorm_backward_item(const RownormGradTask& t, int item,
                                                      const Geo<G>& geo, GroupScratch<G>& gs,
                                                      int& slot) {
  constexpr int R = Geo<G>::R;
  int off[V];
  geo.offsets(off, 4 * NE);
  {
    const int64_t row = (int64_t)(item - t.item_begin) * R + geo.rr;
    if (G == 1 && row >= t.rows) return;
    const float gr = row_gain(t, row) * t.radius;
    const RowBuf wb(t.w + row * t.cols, (uint32_t)t.cols * 4u);
    const RowBuf eb(t.dw_eff + row * t.cols, (uint32_t)t.cols * 2u);
    float w[V][NE];
    Bf16Vec<NE> e[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      F32Vec<NE>::load(wb, off[v], w[v]);
      e[v].load(eb, off[v] / 2);
    }
    float a[2] = {0.f, 0.f}, p[2] = {0.f, 0.f};
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int ch = (v * NE + k) & 1;
        a[ch] = __builtin_fmaf(w[v][k], w[v][k], a[ch]);
        p[ch] = __builtin_fmaf(w[v][k], e[v].get(k), p[ch]);
      }
    float acc[2] = {wave_sum(a[0] + a[1]), wave_sum(p[0] + p[1])};
    group_sum<G, 2>(acc, gs.next(slot), geo.g, geo.lane);
    float T = acc[0];
    float P = acc[1];
    bool scaled = false;
    int sa = 0, sb = 0;
    if (!(T >= kTiny && T < __builtin_inff() && fabsf(P) < __builtin_inff())) {
      float m[2] = {0.f, 0.f};
      u16x2_t mx = {0, 0};
#pragma unroll
      for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int k = 0; k < NE; ++k) m[0] = fmaxf(m[0], fabsf(w[v][k]));
        mx = e[v].absmax(mx);
      }
      m[1] = __uint_as_float((uint32_t)(mx.x > mx.y ? mx.x : mx.y) << 16);
      m[0] = wave_max(m[0]);
      m[1] = wave_max(m[1]);
      group_max2<G>(m, gs.next(slot), geo.g, geo.lane);
      if (m[0] > 0.f && m[0] < __builtin_inff() && m[1] < __builtin_inff()) {
        sa = rescue_shift(m[0], 0.f);
        sb = (m[1] > 0.f) ? rescue_shift(m[1], 0.f) : 0;
        float c[2] = {0.f, 0.f}, q[2] = {0.f, 0.f};
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < NE; ++k) {
            const int ch = (v * NE + k) & 1;
            const float x = ldexpf(w[v][k], sa);
            c[ch] = __builtin_fmaf(x, x, c[ch]);
            q[ch] = __builtin_fmaf(x, ldexpf(e[v].get(k), sb), q[ch]);
          }
        float tt[2] = {wave_sum(c[0] + c[1]), wave_sum(q[0] + q[1])};
        group_sum<G, 2>(tt, gs.next(slot), geo.g, geo.lane);
        T = tt[0];
        P = tt[1];
        scaled = true;
      }
    }
    const bool zero = T == 0.f;                     // after any rescue: every w is 0
    const float inv = inv_sqrt(T);
    float dg = (t.radius * P) * inv;
    if (scaled) dg = ldexpf(dg, -sb);
    const float kk = zero ? 0.f : (P * inv) * inv;
    const float c = zero ? 0.f : gr * inv;
    if (t.dgain != nullptr && geo.g == 0 && geo.lane == 0) gmem_out(t.dgain)[row] = zero ? 0.f : dg;
    const RowBuf ob(t.dw + row * t.cols, (uint32_t)t.cols * 4u);
    const int sh = sa - sb;
    // three uniform cases, each a branch of its own (the empty asm keeps the
    // compiler from merging them into selects on every element)
    if (!scaled && !zero) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float o[NE];
#pragma unroll
        for (int k = 0; k < NE; ++k) o[k] = c * __builtin_fmaf(-w[v][k], kk, e[v].get(k));
        F32Vec<NE>::store(ob, off[v], o);
      }
    } else if (zero) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float o[NE];
#pragma unroll
        for (int k = 0; k < NE; ++k) o[k] = 0.f;
        F32Vec<NE>::store(ob, off[v], o);
      }
    } else {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float o[NE];
#pragma unroll
        for (int k = 0; k < NE; ++k) {
          const float wv = ldexpf(w[v][k], sa), ev = ldexpf(e[v].get(k), sb);
          o[k] = ldexpf(c * __builtin_fmaf(-wv, kk, ev), sh);
        }
        F32Vec<NE>::store(ob, off[v], o);
      }
    }
  }
}

template <int G, int V, int NE>
__global__ void __launch_bounds__(Geo<G>::THREADS)
rownorm_backward_kernel(const RownormGradArgs args) {
  const Geo<G> geo;
  __shared__ GroupScratch<G> gs;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x)
    rownorm_backward_item<G, V, NE>(task_of(args, item, geo.lane), item, geo, gs, slot);
}

// ------------------------------------------------------------ rescale method
//
// DragonScale README, "Optimizer": with raw rows (method "rescale"), the
// part of the gradient that would change a row's length is removed before
// each step; after it the same part is removed from the momentum and the
// row is rescaled to its radius.  Per row of fp32 w and v (a gradient or a
// momentum), S = sum w^2 and P = <w, v> in one pass:
//   v <- v - w k,  k = (P inv) inv,  inv = 1/sqrt(S)      (v may be absent)
//   w <- w (rho inv)                                      (after a step only)
// Sums out of fp32's range are recomputed with w scaled by 2^sa and v by
// 2^sb, as for the weight gradient.  A zero row is left as it is.

struct RescaleTask {
  float* w;
  float* v;             // may be null (after a step without momentum)
  int64_t rows;
  int32_t cols;
  float radius;
  int32_t item_begin;
  int32_t seg;          // column-block layouts (as in RownormTask)
  int32_t shape;        // as in RownormTask
  int64_t ld;
};
using RescaleArgs = TaskArgs<RescaleTask>;
static_assert(sizeof(RescaleArgs) <= 4096, "kernel arguments are limited to 4 KiB");

template <int G, int V, int NE, bool RESCALE>
__device__ __forceinline__ void rescale_item(const RescaleTask& t, int item, const Geo<G>& geo,
                                             GroupScratch<G>& gs, int& slot) {
  constexpr int R = Geo<G>::R;
  int off[V];
  geo.offsets(off, 4 * NE);
  {
    const int64_t row = (int64_t)(item - t.item_begin) * R + geo.rr;
    if (G == 1 && row >= t.rows) return;
    const bool has_v = t.v != nullptr;             // uniform
    const uint32_t bytes = (uint32_t)t.cols * 4u;
    const RowBuf wb(t.w + row * t.cols, bytes);
    const RowBuf vb(has_v ? t.v + row * t.cols : t.w, has_v ? bytes : 0u);
    float w[V][NE], v[V][NE];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      F32Vec<NE>::load(wb, off[k], w[k]);
      F32Vec<NE>::load(vb, off[k], v[k]);          // zeros when there is no v
    }
    float a[2] = {0.f, 0.f}, p[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int ch = (k * NE + j) & 1;
        a[ch] = __builtin_fmaf(w[k][j], w[k][j], a[ch]);
        p[ch] = __builtin_fmaf(w[k][j], v[k][j], p[ch]);
      }
    float acc[2] = {wave_sum(a[0] + a[1]), wave_sum(p[0] + p[1])};
    group_sum<G, 2>(acc, gs.next(slot), geo.g, geo.lane);
    float T = acc[0];
    float P = acc[1];
    bool scaled = false;
    int sa = 0, sb = 0;
    if (!(T >= kTiny && T < __builtin_inff() && fabsf(P) < __builtin_inff())) {
      float m[2] = {0.f, 0.f};
#pragma unroll
      for (int k = 0; k < V; ++k)
#pragma unroll
        for (int j = 0; j < NE; ++j) {
          m[0] = fmaxf(m[0], fabsf(w[k][j]));
          m[1] = fmaxf(m[1], fabsf(v[k][j]));
        }
      m[0] = wave_max(m[0]);
      m[1] = wave_max(m[1]);
      group_max2<G>(m, gs.next(slot), geo.g, geo.lane);
      if (m[0] > 0.f && m[0] < __builtin_inff() && m[1] < __builtin_inff()) {
        sa = rescue_shift(m[0], 0.f);
        sb = (m[1] > 0.f) ? rescue_shift(m[1], 0.f) : 0;
        float c[2] = {0.f, 0.f}, q[2] = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
          for (int j = 0; j < NE; ++j) {
            const int ch = (k * NE + j) & 1;
            const float x = ldexpf(w[k][j], sa);
            c[ch] = __builtin_fmaf(x, x, c[ch]);
            q[ch] = __builtin_fmaf(x, ldexpf(v[k][j], sb), q[ch]);
          }
        float tt[2] = {wave_sum(c[0] + c[1]), wave_sum(q[0] + q[1])};
        group_sum<G, 2>(tt, gs.next(slot), geo.g, geo.lane);
        T = tt[0];
        P = tt[1];
        scaled = true;
      }
    }
    if (T == 0.f) return;                          // a zero row: nothing to do (uniform)
    const float inv = inv_sqrt(T);
    const float kk = (P * inv) * inv;
    const float c = t.radius * inv;
    // the rescued case is a branch of its own (the empty asm keeps the
    // compiler from merging the two into selects on every element)
    if (!scaled) {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float ov[NE], ow[NE];
#pragma unroll
        for (int j = 0; j < NE; ++j) {
          ov[j] = __builtin_fmaf(-w[k][j], kk, v[k][j]);
          ow[j] = w[k][j] * c;
        }
        if (has_v) F32Vec<NE>::store(vb, off[k], ov);
        if constexpr (RESCALE) F32Vec<NE>::store(wb, off[k], ow);
      }
    } else {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float ov[NE], ow[NE];
#pragma unroll
        for (int j = 0; j < NE; ++j) {
          const float wj = ldexpf(w[k][j], sa);
          const float vj = ldexpf(v[k][j], sb);
          ov[j] = ldexpf(__builtin_fmaf(-wj, kk, vj), -sb);
          ow[j] = wj * c;
        }
        if (has_v) F32Vec<NE>::store(vb, off[k], ov);
        if constexpr (RESCALE) F32Vec<NE>::store(wb, off[k], ow);
      }
    }
  }
}

template <int G, int V, int NE, bool RESCALE>
__global__ void __launch_bounds__(Geo<G>::THREADS)
rescale_kernel(const RescaleArgs args) {
  const Geo<G> geo;
  __shared__ GroupScratch<G> gs;
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x)
    rescale_item<G, V, NE, RESCALE>(task_of(args, item, geo.lane), item, geo, gs, slot);
}

}  // namespace dsr
