"""The generated kernel launchers cover every shape the policy can return.

The shape (G waves per row, V vectors per lane) is chosen from the row width
alone, so each row's reduction tree -- and its bits -- never depends on the
row count.  A width whose shape had no kernel would fail at launch; this
checks the generated launch switches against the policy at every width.
"""
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "scale_invariant_row_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_instances as gen  # noqa: E402


def cases(name):
    """(G, V) of each case; (NE, G, V) where keys carry NE * 10000."""
    text = open(os.path.join(CSRC, name)).read()
    out = set()
    for c in map(int, re.findall(r"case (\d+):", text)):
        out.add((c // 10000, c // 100 % 100, c % 100) if c >= 10000 else (c // 100, c % 100))
    return out


def test_bf16_launchers_cover_policy():
    lim = gen.limits()
    need = {gen.bf16_shape(n, lim) for n in range(1, 65536 // 8 + 1)}
    assert None not in need
    assert need <= cases("inst_l2.hip")
    assert need <= cases("inst_slerp.hip")
    assert need <= cases("inst_rms.hip")
    assert need <= cases("inst_rms_bwd.hip")


def test_rownorm_launcher_covers_policy():
    lim = gen.limits()
    need = {(4,) + gen.rownorm_shape(n, lim) for n in range(1, 65536 // 4 + 1)}
    need |= {(1,) + gen.elem_shape(n, lim) for n in range(1, gen.MAX_ELEM_COLS + 1)}
    assert None not in need
    assert need <= cases("inst_rownorm.hip")
    assert need <= cases("inst_rownorm_bwd.hip")
    assert need <= cases("inst_rescale.hip")


def test_gradient_and_activation_launchers_cover_policy():
    lim = gen.limits()
    need = {gen.bf16_shape(n, lim) for n in range(1, 65536 // 8 + 1)}
    assert need <= cases("inst_l2_bwd.hip")
    need = {gen.act_shape(n, lim) for n in range(1, 65536 // 8 + 1)}
    assert None not in need
    assert need <= cases("inst_act.hip")


def test_policy_is_measured_choice():
    """The widths of the workloads map to the shapes measured fastest."""
    lim = gen.limits()
    assert gen.bf16_shape(1024 // 8, lim) == (1, 2)
    assert gen.bf16_shape(4096 // 8, lim) == (4, 2)
    assert gen.bf16_shape(7168 // 8, lim) == (4, 4)
    assert gen.bf16_shape(8192 // 8, lim) == (4, 4)
    assert gen.rownorm_shape(768 // 4, lim) == (1, 3)
    assert gen.rownorm_shape(3072 // 4, lim) == (2, 6)
    assert gen.act_shape(4096 // 8, lim) == (4, 2)
    assert gen.act_shape(7168 // 8, lim) == (8, 2)


def test_reduction_depth_bound():
    """Deepest sum path (two fma chains, wave tree, group sum) stays <= 64."""
    lim = gen.limits()
    for G, V in gen.bf16_shapes(lim):
        assert 4 * V + 1 + 6 + (G - 1) <= 64
    for G, V in gen.rownorm_shapes(lim):
        assert 2 * V + 1 + 6 + (G - 1) <= 64
    for G, V in gen.act_shapes(lim):
        assert 4 * V + 1 + 6 + (G - 1) <= 64


def mixed_cases(name):
    """{workgroup size: {(NE, G, V)}} of the mixed-shape kernels' switches."""
    text = open(os.path.join(CSRC, name)).read()
    out = {}
    for m in re.finditer(r"__global__ void __launch_bounds__\((\d+)[^)]*\) \w+_mixed_(\d+)\(", text):
        assert m.group(1) == m.group(2)
        body = text[m.end():text.find("\n}\n", m.end())]
        keys = set()
        for c in map(int, re.findall(r"case (\d+):", body)):
            keys.add((c // 10000, c // 100 % 100, c % 100))
        out.setdefault(int(m.group(1)), set()).update(keys)
    return out


def test_mixed_kernels_cover_policy():
    """Each mixed-shape kernel holds every weight shape of its workgroup size
    (one row of G waves, or four one-wave rows), for the sizes launch.hpp
    allows to mix."""
    lim = gen.limits()
    need = {(4,) + gen.rownorm_shape(n, lim) for n in range(1, 65536 // 4 + 1)}
    need |= {(1,) + gen.elem_shape(n, lim) for n in range(1, gen.MAX_ELEM_COLS + 1)}
    text = open(os.path.join(CSRC, "launch.hpp")).read()
    max_mixed = int(re.search(r"kMaxMixedThreads\s*=\s*(\d+)", text).group(1))
    sizes = {gen.threads_of(G) for _, G, _ in need if gen.threads_of(G) <= max_mixed}
    assert sizes == set(gen.MIXED_THREADS)
    for name in ("inst_rownorm.hip", "inst_rownorm_bwd.hip", "inst_rescale.hip"):
        got = mixed_cases(name)
        assert set(got) == sizes, name
        for T in sizes:
            assert got[T] == {s for s in need if gen.threads_of(s[1]) == T}, (name, T)
