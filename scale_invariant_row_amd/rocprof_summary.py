"""Summaries of rocprofv3 runs of bench.py, as committed under profiles/.

    python -m scale_invariant_row_amd.rocprof_summary trace <trace dir> [-o out] [--cmd C]...
    python -m scale_invariant_row_amd.rocprof_summary traffic <fetch dir> <write dir>
        [--req <request-size dir>] [--bubble <TCC_BUBBLE dir>] [-o out] [--cmd C]...
    python -m scale_invariant_row_amd.rocprof_summary sq <pass A dir> <pass B dir> [-o out] [--cmd C]...

Each reads the CSV files rocprofv3 wrote under a ``-d`` directory
(``--output-format csv``) and prints a text table per (kernel, grid):

* ``trace``: dispatches and their average/min/max duration, and for the
  library's kernels the algorithmic bytes of one launch (each input read
  once, each output written once, from the workload bench.py runs) and the
  GB/s and fraction of MI355X's 8 TB/s they make at the average duration;
* ``traffic``: HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE, each
  scaled by what it reads for bench.py's torch device copy of known size,
  against the algorithmic bytes; with ``--req``, also the bytes read counted
  from the L2's read requests by size (TCC_EA0_RDREQ_32B, _64B, _128B), which
  needs no calibration;
* ``sq``: SQ counters per dispatch (median), per wave, and per output element.

``--cmd`` lines (the rocprofv3 commands that made the input) are copied into
the summary's header.

Nothing here runs on the GPU.  bench.py reads the ``traffic`` lines of the
traffic summary for its roofline.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import math
import os
import re
import statistics
import sys
from collections import defaultdict
from typing import Dict, List, Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HBM_PEAK_GBPS = 8000.0
CUS = 256                        # MI355X compute units
MAX_LAUNCH_GROUPS = 64 * CUS     # workgroups per launch, at most (the library's grid cap)
XCDS = 8                         # accelerator complex dies: GRBM counters are summed over them
COPY_BYTES = 8192 * 4096 * 3     # bench.py's torch copy: one 100,663,296-byte buffer
COPY_KERNEL = "__amd_rocclr_copyBuffer"

# ------------------------------------------------------------------ names


def short_name(name: str) -> str:
    """'void dsr::l2_rows_kernel<4, 2, true, false>(uint4 const*, ...)' ->
    'l2_rows_kernel<4, 2, true, false>' (the template arguments kept)."""
    n = name.strip().replace("(anonymous namespace)::", "")
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):            # the argument list: the first '(' outside <>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    n = re.sub(r"^(void|int|float)\s+", "", n)
    n = re.sub(r"^(\w+::)+", "", n)
    n = re.sub(r"\bdsr::", "", n)
    return n.strip()


# ------------------------------------------------- the launches bench.py makes

def _policy():
    sys.path.insert(0, CSRC)
    try:
        import gen_instances as gi
    finally:
        sys.path.pop(0)
    return gi, gi.limits()


def _weight_shape(cols: int, gi, lim) -> Tuple[int, int, int]:
    """(G, V, NE) of an fp32 weight row: launch.hpp's pick_weight_shape."""
    if cols % 4 == 0:
        G, V = gi.rownorm_shape(cols // 4, lim)
        return G, V, 4
    G, V = gi.elem_shape(cols, lim)
    return G, V, 1


def _ragged(mats, op: str, gi, lim) -> List[Tuple[str, int, int, int, int]]:
    """The launches of one ragged weight call, grouped as launch_ragged
    groups them: [(kernel, grid threads, read bytes, write bytes, elements)].
    ``mats``: (rows, cols, bytes read per element, bytes written per element,
    bytes read per row, bytes written per row) per matrix."""
    classes: Dict[Tuple[int, int, int], List] = defaultdict(list)
    for m in mats:
        classes[_weight_shape(m[1], gi, lim)].append(m)
    groups: Dict[object, Dict] = {}
    for shape, ms in classes.items():
        G, V, NE = shape
        R = 4 if G == 1 else 1
        threads = 64 * G * R
        items = sum(-(-m[0] // R) for m in ms)
        mixable = threads <= 512 and items < 32 * CUS
        key = -threads if mixable else shape
        groups.setdefault(key, {})[shape] = (ms, items, threads)
    out = []
    base = {"fwd": "rownorm", "bwd": "rownorm_backward", "project": "rescale",
            "after": "rescale"}[op]
    for key, cls in groups.items():
        items = sum(v[1] for v in cls.values())
        threads = next(iter(cls.values()))[2]
        if len(cls) > 1:
            kname = f"{base}_mixed_{threads}"
            if op in ("project", "after"):
                kname += "<true>" if op == "after" else "<false>"
        else:
            G, V, NE = next(iter(cls))
            extra = {"fwd": "", "bwd": "", "project": ", false", "after": ", true"}[op]
            kname = f"{base}_kernel<{G}, {V}, {NE}{extra}>"
        grid = min(items, MAX_LAUNCH_GROUPS) * threads
        rd = wr = el = 0
        for ms, _, _ in cls.values():
            for rows, cols, re_, we, rr, wr_ in ms:
                rd += rows * cols * re_ + rows * rr
                wr += rows * cols * we + rows * wr_
                el += rows * cols
        out.append((kname, grid, rd, wr, el))
    return out


def bench_launches() -> Dict[Tuple[str, Optional[int]], Tuple[str, int, int, int]]:
    """(kernel, grid threads or None for any) -> (workload, read bytes, write
    bytes, output elements) for the launches bench.py times."""
    gi, lim = _policy()
    t: Dict[Tuple[str, Optional[int]], Tuple[str, int, int, int]] = {}

    def rows_launch(kernel, rows, cols, per_block, threads, rd_per_elt, wr_per_elt, extra_rd,
                    label):
        # one row group per workgroup, a call split into launches of at most
        # MAX_LAUNCH_GROUPS row groups (equal pieces for these workloads)
        units = -(-rows // per_block)
        pieces = -(-units // MAX_LAUNCH_GROUPS)
        grid = min(units, MAX_LAUNCH_GROUPS) * threads
        n = rows * cols // pieces
        t[(kernel, grid)] = (label if pieces == 1 else f"{label} (one of {pieces} launches)",
                             n * rd_per_elt + extra_rd, n * wr_per_elt, n)

    rows_launch("l2_rows_kernel<4, 2, true, false>", 8192, 4096, 1, 256, 4, 2, 0,
                "l2_rows + residual 8192x4096")
    rows_launch("stream_rows_kernel<4, 2>", 8192, 4096, 1, 256, 4, 2, 0,
                "stream reference (y = x ^ r) 8192x4096")
    rows_launch("slerp_rows_kernel<4, 2>", 8192, 4096, 1, 256, 4, 2, 4096 * 4,
                "slerp_rows 8192x4096")
    rows_launch("slerp_rows_kernel<4, 4>", 8192, 7168, 1, 256, 4, 2, 7168 * 4,
                "slerp_rows 8192x7168")
    rows_launch("l2_rows_kernel<4, 4, true, false>", 32768, 8192, 1, 256, 4, 2, 0,
                "l2_rows + residual 32768x8192")
    rows_launch("l2_rows_kernel<1, 2, false, false>", 64, 1024, 4, 256, 2, 2, 0,
                "l2_rows 64x1024")
    rows_launch("l2_rows_backward_kernel<4, 2, true, false>", 8192, 4096, 1, 256, 6, 2, 0,
                "l2_rows gradient 8192x4096")
    rows_launch("l2_rows_kernel<1, 2, false, true>", 16384, 768, 4, 256, 2, 2, 0,
                "rms_rows 16384x768")
    rows_launch("l2_rows_backward_kernel<1, 2, false, true>", 16384, 768, 4, 256, 4, 2, 0,
                "rms_rows gradient 16384x768")
    rows_launch("l2_rows_kernel<4, 2, true, true>", 8192, 4096, 1, 256, 4, 2, 0,
                "rms_rows + residual 8192x4096")
    rows_launch("act_l2_rows_kernel<4, 2, (Act)0>", 8192, 4096, 1, 256, 4, 2, 4096 * 4,
                "gate_l2_rows 8192x4096")
    n = 8192 * 7168
    t[("swiglu_table_l2_rows_kernel<8, 2>", None)] = (
        "swiglu_l2_rows 8192x7168", n * 4 + 7168 * 8, n * 2, n)
    t[("act_l2_rows_kernel<8, 2, (Act)1>", None)] = t[("swiglu_table_l2_rows_kernel<8, 2>", None)]
    n = 8192 * 20 * 256
    t[("qk_rows_l2_kernel<256>", None)] = (
        "qk_rows_l2 8192 rows, 16+4 heads of 256", n * 2 + 8192 * 4 + 128 * 4 + 16 * 256 * 4,
        n * 2, n)

    from . import inputs
    lin = inputs.transformer_linears()
    res = inputs.resnet50_convs()
    emb = [(50304, 768)]
    big = [(11008, 4096)]
    # per matrix: rows, cols, read/elt, write/elt, read/row, write/row
    fwd = lambda shapes: [(r, c, 4, 2, 4, 4) for r, c in shapes]
    bwd = lambda shapes: [(r, c, 6, 4, 4, 4) for r, c in shapes]
    for label, shapes in (("48 linears", lin), ("ResNet-50", res), ("embedding 50304x768", emb),
                          ("11008x4096", big)):
        for op, mats, what in (("fwd", fwd(shapes), "W rownorm"), ("bwd", bwd(shapes), "W gradient")):
            for kname, grid, rd, wr, el in _ragged(mats, op, gi, lim):
                t[(kname, grid)] = (f"{what}, {label}", rd, wr, el)
    for op, per, what in (("project", (8, 4), "rescale project"),
                          ("after", (8, 8), "rescale after step")):
        mats = [(r, c, per[0], per[1], 0, 0) for r, c in lin]
        for kname, grid, rd, wr, el in _ragged(mats, op, gi, lim):
            t[(kname, grid)] = (f"{what}, 48 linears", rd, wr, el)
    # GPT-2's Conv1D weights as column blocks: units are stored columns
    conv = inputs.gpt2_conv1d()
    el = sum(a * b for a, b in conv)
    units = sum(b for _, b in conv)
    # (the seg-1 kernel: single-pass tiles for the 768-row weights, two-pass
    # tiles for the 3,072-row MLP projections, one launch per op)
    fwd_w = ("W rownorm, GPT-2 Conv1D (column blocks)", el * 4 + units * 4, el * 2 + units * 4, el)
    bwd_w = ("W gradient, GPT-2 Conv1D (column blocks)", el * 6 + units * 4, el * 4 + units * 4,
             el)
    t[("colblock1_kernel<(ColOp)0, 12, 16>", None)] = fwd_w
    t[("colblock1_kernel<(ColOp)1, 12, 16>", None)] = bwd_w
    t[("colblock_kernel<(ColOp)0>", None)] = fwd_w
    t[("colblock_kernel<(ColOp)1>", None)] = bwd_w
    return t


def lookup(table, kernel: str, grid: int):
    return table.get((kernel, grid)) or table.get((kernel, None))


# ------------------------------------------------------------------ CSVs


def _csvs(d: str, suffix: str) -> List[str]:
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return files


def _col(row: dict, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names)


def read_trace(d: str) -> Dict[Tuple[str, int], List[float]]:
    """(kernel, grid threads) -> durations in microseconds."""
    out: Dict[Tuple[str, int], List[float]] = defaultdict(list)
    for f in _csvs(d, "kernel_trace.csv"):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                k = short_name(_col(row, "Kernel_Name"))
                g = int(_col(row, "Grid_Size_X", "Grid_Size")) * int(row.get("Grid_Size_Y") or 1) \
                    * int(row.get("Grid_Size_Z") or 1)
                dt = (int(_col(row, "End_Timestamp")) - int(_col(row, "Start_Timestamp"))) / 1e3
                out[(k, g)].append(dt)
    return out


def read_counters(d: str) -> Dict[Tuple[str, int], Dict[str, List[float]]]:
    """(kernel, grid threads) -> counter -> values per dispatch."""
    per_dispatch: Dict[Tuple[str, int, str], Dict[str, float]] = defaultdict(dict)
    for f in _csvs(d, "counter_collection.csv"):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                k = short_name(_col(row, "Kernel_Name"))
                g = int(_col(row, "Grid_Size"))
                disp = f + ":" + _col(row, "Dispatch_Id", "Correlation_Id")
                c = _col(row, "Counter_Name")
                per_dispatch[(k, g, disp)][c] = per_dispatch[(k, g, disp)].get(c, 0.0) + \
                    float(_col(row, "Counter_Value"))
    out: Dict[Tuple[str, int], Dict[str, List[float]]] = defaultdict(lambda: defaultdict(list))
    for (k, g, _), cs in per_dispatch.items():
        for c, v in cs.items():
            out[(k, g)][c].append(v)
    return out


def kernel_sources_hash(files=("row_kernels.hpp", "launch.hpp", "colblock_kernels.hpp",
                               "ds_rows.hip", "bench_stream.hip")) -> str:
    """The hash bench.py compares with the traffic summary's: the sources every
    kernel's code comes from, and the launchers."""
    h = hashlib.sha256()
    names = list(files) + sorted(os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "inst_*.hip")))
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ reports


def _fmt_int(v) -> str:
    return f"{int(round(v)):,}"


def trace_report(d: str) -> str:
    table = bench_launches()
    tr = read_trace(d)
    lines = ["# rocprofv3 kernel-trace summary of bench.py on MI355X (gfx950); durations in us",
             f"# from: {d}", "",
             f"{'kernel':<46}{'grid':>10}{'calls':>7}{'avg_us':>10}{'min_us':>9}{'max_us':>9}"]
    rows = sorted(tr.items(), key=lambda kv: -statistics.fmean(kv[1]) * len(kv[1]))
    for (k, g), ds in rows:
        lines.append(f"{k[:46]:<46}{g:>10}{len(ds):>7}{statistics.fmean(ds):>10.2f}"
                     f"{min(ds):>9.2f}{max(ds):>9.2f}")
    lines += ["", "Algorithmic bytes per launch (each input read once, each output written once) "
              "and GB/s = bytes / average duration:", ""]
    for (k, g), ds in rows:
        w = lookup(table, k, g)
        if w is None:
            continue
        label, rd, wr, _ = w
        avg = statistics.fmean(ds)
        gbps = (rd + wr) / (avg * 1e-6) / 1e9
        lines.append(f"  {k[:44]:<44} {label[:42]:<42} {_fmt_int(rd + wr):>15} B  {avg:8.2f} us  "
                     f"{gbps:7.1f} GB/s = {gbps / HBM_PEAK_GBPS:.3f}")
    return "\n".join(lines) + "\n"


def _median(vs):
    return statistics.median(vs) if vs else float("nan")


def traffic_report(fetch_dir: str, write_dir: str, req_dir: Optional[str] = None,
                   bubble_dir: Optional[str] = None) -> str:
    table = bench_launches()
    fc, wc = read_counters(fetch_dir), read_counters(write_dir)
    rq = read_counters(req_dir) if req_dir else {}
    bb = read_counters(bubble_dir) if bubble_dir else {}

    def req_bytes(key):
        c = rq.get(key)
        if not c:
            return float("nan")
        n32, n64, n128 = (_median(c.get(f"TCC_EA0_RDREQ_{b}B", [])) for b in (32, 64, 128))
        return 32 * n32 + 64 * n64 + 128 * n128

    def copy_scale(cs, name):
        keys = [k for k in cs if k[0].startswith(COPY_KERNEL)]
        best = max(keys, key=lambda k: _median(cs[k][name])) if keys else None
        if best is None:
            raise SystemExit(f"no {COPY_KERNEL} dispatch for {name} calibration")
        kib = _median(cs[best][name])
        return COPY_BYTES / (kib * 1024.0), best

    fs, fkey = copy_scale(fc, "FETCH_SIZE")
    ws, wkey = copy_scale(wc, "WRITE_SIZE")
    lines = ["# HBM traffic per dispatch from rocprofv3 counters, bench.py on MI355X (gfx950)",
             f"# FETCH_SIZE from: {fetch_dir}", f"# WRITE_SIZE from: {write_dir}",
             "# Counters are KiB per dispatch (median over dispatches), each scaled by what it",
             f"# reads for bench.py's device copy of {COPY_BYTES:,} bytes ({fkey[0]}, grid {fkey[1]}):",
             f"#   FETCH_SIZE scale = {fs:.4f}   WRITE_SIZE scale = {ws:.4f}"]
    if rq:
        cp = rq.get(fkey, {})
        n = {b: _median(cp.get(f"TCC_EA0_RDREQ_{b}B", [])) for b in (32, 64, 128)}
        tot = _median(cp.get("TCC_EA0_RDREQ", []))
        lines += ["# read_req_B: bytes read counted from the L2's read requests by size,",
                  "#   32 x TCC_EA0_RDREQ_32B + 64 x TCC_EA0_RDREQ_64B + 128 x TCC_EA0_RDREQ_128B (no calibration).",
                  f"#   The copy: {_fmt_int(tot)} read requests = {_fmt_int(n[32])} of 32 B + {_fmt_int(n[64])} of 64 B"
                  f" + {_fmt_int(n[128])} of 128 B = {_fmt_int(req_bytes(fkey))} bytes."]
    if bb:
        cb = bb.get(fkey, {})
        lines += [f"#   TCC_BUBBLE (the 128-byte request count in FETCH_SIZE's expression) for the copy: "
                  f"{_fmt_int(_median(cb.get('TCC_BUBBLE', [])))}"]
    lines += ["", f"{'kernel':<46}{'grid':>10}{'n':>5}{'read_B':>15}{'written_B':>15}{'algo_read_B':>15}"
              f"{'algo_write_B':>15}{'ratio':>8}" + (f"{'read_req_B':>15}{'ratio_req':>10}" if rq else "")]
    traffic = []
    for key in sorted(set(fc) & set(wc)):
        k, g = key
        w = lookup(table, k, g)
        if w is None:
            continue
        label, ard, awr, _ = w
        rd = _median(fc[key]["FETCH_SIZE"]) * 1024.0 * fs
        wr = _median(wc[key]["WRITE_SIZE"]) * 1024.0 * ws
        n = len(fc[key]["FETCH_SIZE"])
        line = (f"{k[:46]:<46}{g:>10}{n:>5}{_fmt_int(rd):>15}{_fmt_int(wr):>15}"
                f"{_fmt_int(ard):>15}{_fmt_int(awr):>15}{(rd + wr) / (ard + awr):>8.4f}")
        if rq:
            rb = req_bytes(key)
            line += (f"{_fmt_int(rb):>15}{(rb + wr) / (ard + awr):>10.4f}" if not math.isnan(rb)
                     else f"{'-':>15}{'-':>10}")
        lines.append(line)
        traffic.append((k, g, rd + wr))
    lines += ["", "ratio = measured (read + written) / algorithmic bytes; 1.0 means no re-reads.", "",
              "# read by bench.py (roofline.traffic): kernel sources hash, then bytes per dispatch",
              f"kernel_hash {kernel_sources_hash()}"]
    for name, grid in (("l2_rows_kernel<4, 2, true, false>", 2097152),
                       ("slerp_rows_kernel<4, 2>", 2097152),
                       ("stream_rows_kernel<4, 2>", 2097152)):
        for k, g, b in traffic:
            if k == name and g == grid:
                lines.append(f"traffic {name.split('<')[0]} {int(round(b))}")
    return "\n".join(lines) + "\n"


PASS_A = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR",
          "SQ_INSTS_LDS", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"]
PASS_B = ["SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY", "SQ_LDS_BANK_CONFLICT",
          "SQ_INST_CYCLES_VMEM_RD", "SQ_INST_CYCLES_VMEM_WR", "GRBM_GUI_ACTIVE"]


def sq_report(a_dir: str, b_dir: str) -> str:
    table = bench_launches()
    ca, cb = read_counters(a_dir), read_counters(b_dir)
    lines = ["# rocprofv3 SQ counters per dispatch (median over dispatches), bench.py on MI355X (gfx950)",
             f"# pass A ({' '.join(PASS_A)}) from: {a_dir}",
             f"# pass B ({' '.join(PASS_B)}) from: {b_dir}",
             "# per wave: instructions each wave issued (VALU, SALU, vector memory reads/writes, LDS);",
             "# VALU/elt: VALU instructions per output element (SQ_INSTS_VALU x 64 / elements);",
             "# valu%: SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES and wait%: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES,",
             "#   the share of an average wave's lifetime spent issuing VALU work and waiting to issue",
             "#   (on a dependency: a load, an LDS access, a barrier);",
             "# VALU busy: SQ_INSTS_VALU x 4 cycles / (GRBM_GUI_ACTIVE / 8 x 1,024 SIMDs), the share of the",
             "#   chip's VALU issue slots the dispatch used (a wave64 instruction occupies a SIMD for 4 cycles;",
             "#   GRBM_GUI_ACTIVE is summed over the 8 XCDs: divided by 8 it is the dispatch's duration in cycles);",
             "# LDS_conf: SQ_LDS_BANK_CONFLICT summed over the dispatch.", "",
             f"{'kernel':<44}{'grid':>9}{'waves':>8}{'VALU/w':>9}{'SALU/w':>8}{'VMRD/w':>8}{'VMWR/w':>8}"
             f"{'LDS/w':>7}{'VALU/elt':>9}{'valu%':>7}{'wait%':>7}{'VALUbusy':>9}{'LDS_conf':>9}  workload"]
    for key in sorted(ca):
        k, g = key
        m = {c: _median(ca[key].get(c, [])) for c in PASS_A}
        mb = {c: _median(cb.get(key, {}).get(c, [])) for c in PASS_B}
        waves = m["SQ_WAVES"]
        if not waves or math.isnan(waves) or waves == 0:
            continue
        w = lookup(table, k, g)
        per = lambda c: m[c] / waves
        velt = (m["SQ_INSTS_VALU"] * 64 / w[3]) if w else float("nan")
        wc = m["SQ_WAVE_CYCLES"]
        valu_pct = 100 * mb["SQ_ACTIVE_INST_VALU"] / wc if wc else float("nan")
        wait_pct = 100 * mb["SQ_WAIT_INST_ANY"] / wc if wc else float("nan")
        busy = 100 * m["SQ_INSTS_VALU"] * 4 / (mb["GRBM_GUI_ACTIVE"] / XCDS * 4 * CUS) \
            if mb["GRBM_GUI_ACTIVE"] else float("nan")
        lines.append(f"{k[:44]:<44}{g:>9}{int(waves):>8}{per('SQ_INSTS_VALU'):>9.1f}"
                     f"{per('SQ_INSTS_SALU'):>8.1f}{per('SQ_INSTS_VMEM_RD'):>8.1f}"
                     f"{per('SQ_INSTS_VMEM_WR'):>8.1f}{per('SQ_INSTS_LDS'):>7.1f}{velt:>9.1f}"
                     f"{valu_pct:>7.1f}{wait_pct:>7.1f}{busy:>8.1f}%{_fmt_int(mb['SQ_LDS_BANK_CONFLICT'] if not math.isnan(mb['SQ_LDS_BANK_CONFLICT']) else 0):>9}"
                     f"  {w[0] if w else ''}")
    return "\n".join(lines) + "\n"


def main(argv=None) -> None:
    import argparse
    ap = argparse.ArgumentParser(prog="python -m scale_invariant_row_amd.rocprof_summary",
                                 description="Summaries of rocprofv3 runs of bench.py")
    ap.add_argument("what", choices=["trace", "traffic", "sq"])
    ap.add_argument("dirs", nargs="+", help="rocprofv3 -d directories (see the module docstring)")
    ap.add_argument("--req", help="traffic: a run of TCC_EA0_RDREQ and its 32B/64B/128B counts")
    ap.add_argument("--bubble", help="traffic: a run of TCC_BUBBLE")
    ap.add_argument("-o", "--out", help="write the summary here (default: stdout)")
    ap.add_argument("--cmd", action="append", default=[], help="a command that made the input")
    a = ap.parse_args(argv)
    need = {"trace": 1, "traffic": 2, "sq": 2}[a.what]
    if len(a.dirs) != need:
        ap.error(f"{a.what} takes {need} directories")
    if a.what == "trace":
        text = trace_report(*a.dirs)
    elif a.what == "traffic":
        text = traffic_report(*a.dirs, req_dir=a.req, bubble_dir=a.bubble)
    else:
        text = sq_report(*a.dirs)
    head = "".join(f"# command: {c}\n" for c in a.cmd)
    if head:
        first, rest = text.split("\n", 1)
        text = first + "\n" + head + rest
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
