"""Writes inst_l2.hip, inst_slerp.hip, inst_rownorm.hip, inst_l2_bwd.hip,
inst_rownorm_bwd.hip, inst_act.hip, inst_rescale.hip, inst_rms.hip and
inst_rms_bwd.hip: one launcher per op
with a case for every kernel shape (G waves per row, V vectors per lane) that
launch.hpp's shape policy returns for some width up to DS_MAX_COLS, found by
evaluating the policy (reproduced below from launch.hpp's constants) at every
width.  The fp32 weight ops also get mixed-shape kernels, one per workgroup
size, that switch on each task's shape key.  Run it after a change of the
policy."""
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
MAX_COLS = 65536


def limits():
    text = open(os.path.join(HERE, "launch.hpp")).read()
    get = lambda name: int(re.search(rf"{name}\s*=\s*(\d+)", text).group(1))
    return {k: get(k) for k in ("kBf16SmallVectors", "kVmaxBf16Small", "kVmaxBf16Large",
                                "kVmaxAct", "kVmaxRownorm", "kVmaxWide", "kVmaxElem")}


def pick_shape(vectors, vmax, wide):
    """launch.hpp's pick_shape, in Python."""
    for G in (1, 2, 4, 8, 16):
        V = -(-vectors // (64 * G))
        if V <= vmax or (G == 16 and V <= wide):
            return G, V
    return None


def bf16_shape(vectors, lim):
    vmax = lim["kVmaxBf16Small"] if vectors <= lim["kBf16SmallVectors"] else lim["kVmaxBf16Large"]
    return pick_shape(vectors, vmax, lim["kVmaxWide"])


def act_shape(vectors, lim):
    return pick_shape(vectors, lim["kVmaxAct"], lim["kVmaxWide"])


def act_shapes(lim):
    """Every shape the activation-row policy returns for rows up to MAX_COLS columns."""
    return sorted({act_shape(n, lim) for n in range(1, MAX_COLS // 8 + 1)})


def rownorm_shape(vectors, lim):
    return pick_shape(vectors, lim["kVmaxRownorm"], lim["kVmaxWide"])


def bf16_shapes(lim):
    """Every shape the bf16 policy returns for rows up to MAX_COLS columns."""
    return sorted({bf16_shape(n, lim) for n in range(1, MAX_COLS // 8 + 1)})


def rownorm_shapes(lim):
    """Every shape the fp32 weight policy returns for rows up to MAX_COLS columns."""
    return sorted({rownorm_shape(n, lim) for n in range(1, MAX_COLS // 4 + 1)})


MAX_ELEM_COLS = 16 * 64 * 16


def elem_shape(cols, lim):
    """launch.hpp's pick_elem_shape, in Python."""
    vmax = lim["kVmaxElem"]
    v = -(-cols // 64)
    if v <= vmax:
        V = 1
        while V < v:
            V *= 2
        return 1, V
    G = 2
    while 64 * G * vmax < cols:
        G *= 2
    return G, vmax


def elem_shapes(lim):
    """Every shape the single-element fp32 policy returns (rows up to 16,384)."""
    return sorted({elem_shape(n, lim) for n in range(1, MAX_ELEM_COLS + 1)})


HEAD = '''// {what}: one launcher over every kernel shape the shape policy can return.
// Written by gen_instances.py.
#include "row_kernels.hpp"
#include "launch.hpp"

namespace dsr {{
'''


def cases(lst, call, ne=None):
    """Switch cases over shapes; with ne, keys are NE * 10000 + G * 100 + V."""
    key = (lambda G, V: G * 100 + V) if ne is None else (lambda G, V: ne * 10000 + G * 100 + V)
    return "\n".join(f"    case {key(G, V)}: {call.format(G=G, V=V, NE=ne)}" for G, V in lst)


def threads_of(G):
    """Workgroup size of a row shape: four one-wave rows, or one row of G waves."""
    return 256 if G == 1 else 64 * G


# Workgroup sizes with a mixed-shape kernel (launch.hpp's kMaxMixedThreads):
# at 1,024 threads the union of the bodies no longer fits the registers.
# Each item builds its geometry with Geo::per_item, so a mixed kernel needs
# the registers of its largest shape, not of all its shapes' lane offsets
# at once.
MIXED_THREADS = (128, 256, 512)


def mixed(name, item, args, task, lists, rescale=False):
    """Mixed-shape kernels: one per workgroup size in MIXED_THREADS, each
    switching on its task's shape key to the matching item body, and their
    launcher run_mixed(threads, ...).  With rescale, both are templates on
    RESCALE."""
    by_threads = {}
    for ne, lst in lists:
        for G, V in lst:
            if threads_of(G) in MIXED_THREADS:
                by_threads.setdefault(threads_of(G), []).append((ne, G, V))
    tmpl = "template <bool RESCALE>\n" if rescale else ""
    extra = ", RESCALE" if rescale else ""
    inst = "<RESCALE>" if rescale else ""
    out = []
    for T in sorted(by_threads):
        shapes = by_threads[T]
        decl = "\n".join(f"  __shared__ GroupScratch<{G}> gs{G};"
                         for G in sorted({G for _, G, _ in shapes}))
        body = "\n".join(
            f"      case {ne * 10000 + G * 100 + V}: "
            f"{item}<{G}, {V}, {ne}{extra}>(t, item, Geo<{G}>::per_item(), gs{G}, slot); break;"
            for ne, G, V in shapes)
        out.append(f"""
{tmpl}__global__ void __launch_bounds__({T}) {name}_mixed_{T}(const {args} args) {{
{decl}
  int slot = 0;
  for (int item = blockIdx.x; item < args.nitems; item += gridDim.x) {{
    const {task} t = task_of(args, item, (int)(threadIdx.x & 63));
    switch (t.shape) {{
{body}
      default: break;
    }}
  }}
}}
""")
    launch = "\n".join(f"    case {T}: {name}_mixed_{T}{inst}<<<grid, {T}, 0, stream>>>(args); break;"
                        for T in sorted(by_threads))
    out.append(f"""
// The classes of a ragged call that share a workgroup size, in one launch.
{tmpl}static hipError_t run_mixed(int threads, const {args}& args, int grid, hipStream_t stream) {{
  switch (threads) {{
{launch}
    default: return hipErrorInvalidValue;
  }}
  return hipGetLastError();
}}
""")
    return "".join(out)


def main():
    lim = limits()
    bf16 = bf16_shapes(lim)
    rown = rownorm_shapes(lim)
    elem = elem_shapes(lim)
    actsh = act_shapes(lim)
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
''' + cases(bf16, "return run<{G}, {V}>(x, r, y, rows, nvec, eps, grid, stream);") + '''
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
''' + cases(bf16, "return run<{G}, {V}>(res, out, alpha, h, rows, nvec, eps, grid, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    rn = HEAD.format(what="weight rownorm+gain") + '''
template <int G, int V, int NE>
static hipError_t run(const RownormArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rownorm_kernel<G, V, NE><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}

''' + mixed("rownorm", "rownorm_item", "RownormArgs", "RownormTask", ((4, rown), (1, elem))) + '''
hipError_t launch_rownorm(Shape s, const RownormArgs& args, int grid, hipStream_t stream) {
  if (s.mixed > 0) return run_mixed(s.mixed, args, grid, stream);
  switch (s.key()) {
''' + cases(rown, "return run<{G}, {V}, {NE}>(args, grid, stream);", 4) + "\n" + cases(elem, "return run<{G}, {V}, {NE}>(args, grid, stream);", 1) + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    l2b = HEAD.format(what="l2_rows gradient") + '''
template <int G, int V>
static hipError_t run(const void* x, const void* r, const void* dy, void* dx, int64_t rows,
                      int nvec, float eps, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  if (r != nullptr)
    l2_rows_backward_kernel<G, V, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, (const u32x4_t*)r, (const u32x4_t*)dy, (u32x4_t*)dx, rows, nvec, eps);
  else
    l2_rows_backward_kernel<G, V, false><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, nullptr, (const u32x4_t*)dy, (u32x4_t*)dx, rows, nvec, eps);
  return hipGetLastError();
}

hipError_t launch_l2_rows_backward(Shape s, const void* x, const void* r, const void* dy,
                                   void* dx, int64_t rows, int nvec, float eps, int grid,
                                   hipStream_t stream) {
  switch (s.G * 100 + s.V) {
''' + cases(bf16, "return run<{G}, {V}>(x, r, dy, dx, rows, nvec, eps, grid, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    rnb = HEAD.format(what="weight rownorm+gain gradient") + '''
template <int G, int V, int NE>
static hipError_t run(const RownormGradArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rownorm_backward_kernel<G, V, NE><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}

''' + mixed("rownorm_backward", "rownorm_backward_item", "RownormGradArgs", "RownormGradTask",
             ((4, rown), (1, elem))) + '''
hipError_t launch_rownorm_backward(Shape s, const RownormGradArgs& args, int grid,
                                   hipStream_t stream) {
  if (s.mixed > 0) return run_mixed(s.mixed, args, grid, stream);
  switch (s.key()) {
''' + cases(rown, "return run<{G}, {V}, {NE}>(args, grid, stream);", 4) + "\n" + cases(elem, "return run<{G}, {V}, {NE}>(args, grid, stream);", 1) + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    act = HEAD.format(what="gate and SwiGLU activation rows") + '''
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
''' + cases(actsh, "return run<{G}, {V}, Act::kGate>(o, g, sg, nullptr, y, rows, nvec, eps, grid, stream);") + '''
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
''' + cases(actsh, "return run_swiglu<{G}, {V}>(g, u, sug, suu, y, rows, nvec, eps, grid, cus, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    rsc = HEAD.format(what="rescale method (projection; rescale after a step)") + '''
template <int G, int V, int NE, bool RESCALE>
static hipError_t run(const RescaleArgs& args, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  rescale_kernel<G, V, NE, RESCALE><<<grid, T, 0, stream>>>(args);
  return hipGetLastError();
}

''' + mixed("rescale", "rescale_item", "RescaleArgs", "RescaleTask", ((4, rown), (1, elem)), True) + '''
hipError_t launch_rescale_project(Shape s, const RescaleArgs& args, int grid, hipStream_t stream) {
  if (s.mixed > 0) return run_mixed<false>(s.mixed, args, grid, stream);
  switch (s.key()) {
''' + cases(rown, "return run<{G}, {V}, {NE}, false>(args, grid, stream);", 4) + "\n" + cases(elem, "return run<{G}, {V}, {NE}, false>(args, grid, stream);", 1) + '''
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rescale_after_step(Shape s, const RescaleArgs& args, int grid,
                                     hipStream_t stream) {
  if (s.mixed > 0) return run_mixed<true>(s.mixed, args, grid, stream);
  switch (s.key()) {
''' + cases(rown, "return run<{G}, {V}, {NE}, true>(args, grid, stream);", 4) + "\n" + cases(elem, "return run<{G}, {V}, {NE}, true>(args, grid, stream);", 1) + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    rms = HEAD.format(what="rms_rows (l2_rows' kernel with the mean)") + '''
template <int G, int V>
static hipError_t run(const void* x, const void* r, void* y, int64_t rows, int nvec, float eps,
                      int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  if (r != nullptr)
    l2_rows_kernel<G, V, true, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, (const u32x4_t*)r, (u32x4_t*)y, rows, nvec, eps);
  else
    l2_rows_kernel<G, V, false, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, nullptr, (u32x4_t*)y, rows, nvec, eps);
  return hipGetLastError();
}

hipError_t launch_rms_rows(Shape s, const void* x, const void* r, void* y, int64_t rows,
                           int nvec, float eps, int grid, hipStream_t stream) {
  switch (s.G * 100 + s.V) {
''' + cases(bf16, "return run<{G}, {V}>(x, r, y, rows, nvec, eps, grid, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    rmsb = HEAD.format(what="rms_rows gradient (l2_rows' gradient kernel with the mean)") + '''
template <int G, int V>
static hipError_t run(const void* x, const void* r, const void* dy, void* dx, int64_t rows,
                      int nvec, float eps, int grid, hipStream_t stream) {
  constexpr int T = Geo<G>::THREADS;
  if (r != nullptr)
    l2_rows_backward_kernel<G, V, true, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, (const u32x4_t*)r, (const u32x4_t*)dy, (u32x4_t*)dx, rows, nvec, eps);
  else
    l2_rows_backward_kernel<G, V, false, true><<<grid, T, 0, stream>>>(
        (const u32x4_t*)x, nullptr, (const u32x4_t*)dy, (u32x4_t*)dx, rows, nvec, eps);
  return hipGetLastError();
}

hipError_t launch_rms_rows_backward(Shape s, const void* x, const void* r, const void* dy,
                                    void* dx, int64_t rows, int nvec, float eps, int grid,
                                    hipStream_t stream) {
  switch (s.G * 100 + s.V) {
''' + cases(bf16, "return run<{G}, {V}>(x, r, dy, dx, rows, nvec, eps, grid, stream);") + '''
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsr
'''
    for name, text in (("inst_l2.hip", l2), ("inst_rms.hip", rms), ("inst_rms_bwd.hip", rmsb), ("inst_slerp.hip", sl), ("inst_rownorm.hip", rn),
                       ("inst_l2_bwd.hip", l2b), ("inst_rownorm_bwd.hip", rnb),
                       ("inst_act.hip", act), ("inst_rescale.hip", rsc)):
        with open(os.path.join(HERE, name), "w") as f:
            f.write(text)


if __name__ == "__main__":
    main()
