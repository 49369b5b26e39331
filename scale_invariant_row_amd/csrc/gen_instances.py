"""Writes inst_l2.hip, inst_slerp.hip and inst_rownorm.hip: one launcher per op
with a case for every kernel shape (G waves per row, V vectors per lane) that
launch.hpp's pick_shape() can return for that op's V limit.  Run it after a
change of kVmaxL2 / kVmaxSlerp / kVmaxRownorm / kVmaxWide."""
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))


def limits():
    text = open(os.path.join(HERE, "launch.hpp")).read()
    get = lambda name: int(re.search(rf"{name}\s*=\s*(\d+)", text).group(1))
    return get("kVmaxL2"), get("kVmaxSlerp"), get("kVmaxRownorm"), get("kVmaxWide")


def shapes(vmax, wide):
    """(G, V) pairs reachable for rows of up to DS_MAX_COLS columns."""
    out = []
    for G in (1, 2, 4, 8, 16):
        lo = 1 if G == 1 else vmax // 2 + 1
        hi = vmax if G < 16 else max(vmax, wide)
        out += [(G, V) for V in range(lo, hi + 1)]
    return out


HEAD = '''// {what}: one launcher over every kernel shape pick_shape() can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {{
'''


def cases(lst, call):
    return "\n".join(f"    case {G * 100 + V}: {call.format(G=G, V=V)}" for G, V in lst)


def main():
    vl2, vsl, vrn, vwide = limits()
    # widest rows: 65536 bf16 = 8192 vectors (l2, slerp); 65536 fp32 = 16384 (rownorm)
    l2_wide = -(-8192 // (64 * 16))
    rn_wide = -(-16384 // (64 * 16))
    l2 = HEAD.format(what="l2_rows") + '''
template <int G, int V>
static hipError_t run(const void* x, const void* r, void* y, int64_t rows, int nvec, float eps,
                      int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  if (r != nullptr)
    l2_rows_kernel<G, V, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, (const u32x4_t*)r, (u32x4_t*)y, rows, nvec, eps);
  else
    l2_rows_kernel<G, V, false><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, nullptr, (u32x4_t*)y, rows, nvec, eps);
  return hipGetLastError();
}

hipError_t launch_l2_rows(Shape s, const void* x, const void* r, void* y, int64_t rows,
                          int nvec, float eps, int grid, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
''' + cases(shapes(vl2, min(vwide, l2_wide)),
            "return run<{G}, {V}>(x, r, y, rows, nvec, eps, grid, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    sl = HEAD.format(what="slerp_rows") + '''
template <int G, int V>
static hipError_t run(const void* res, const void* out, const float* alpha, void* h,
                      int64_t rows, int nvec, float eps, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  slerp_rows_kernel<G, V><<<grid, T, 0, stream>>>(
      (const u32x4_t*)res, (const u32x4_t*)out, (const f32x4_t*)alpha, (u32x4_t*)h, rows, nvec,
      eps);
  return hipGetLastError();
}

hipError_t launch_slerp_rows(Shape s, const void* res, const void* out, const float* alpha,
                             void* h, int64_t rows, int nvec, float eps, int grid,
                             hipStream_t stream) {
  switch (s.G * 100 + s.V) {
''' + cases(shapes(vsl, min(vwide, l2_wide)),
            "return run<{G}, {V}>(res, out, alpha, h, rows, nvec, eps, grid, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    rn = HEAD.format(what="weight rownorm+gain") + '''
template <int G, int V>
static hipError_t run(const RownormArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rownorm_kernel<G, V><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_rownorm(Shape s, const RownormArgs& args, int grid, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
''' + cases(shapes(vrn, min(vwide, rn_wide)),
            "return run<{G}, {V}>(args, grid, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    for name, text in (("inst_l2.hip", l2), ("inst_slerp.hip", sl), ("inst_rownorm.hip", rn)):
        with open(os.path.join(HERE, name), "w") as f:
            f.write(text)


if __name__ == "__main__":
    main()
