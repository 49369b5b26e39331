"""Throughput of the row-L2 hot path on one MI355X.

A step is one pass of the path over one batch at the workload the headline
metric is quoted on: ds_l2_rows with the fused residual on 8192 x 4096 bf16
rows, then ds_slerp_rows on 8192 x 4096 bf16 rows (synthetic, seeded inputs).
The other shapes, the weight op and the gradients are timed after the
headline steps and reported in ``ops``.
Inputs are resident in HBM before timing starts; the steps rotate over
several buffer sets whose total is well above the 256 MB last-level cache, so
every launch streams from HBM.  The weight op (ds_weight_rownorm_gain over a
12-layer transformer's 48 linears) is timed after the headline steps and
reported beside them.  Two plain stream kernels (libdsbench.so, built beside
the library) give the reference rates: y = x ^ r over bf16 rows with l2_rows'
launch (the ``stream_ceiling`` of the roofline), and y = bf16(x) over fp32
rows with the weight op's launch for the width (the ``stream_f32_ceiling``
lines).

Prints one JSON line.  ``value`` is the step's algorithmic bytes (each input
read once, each output written once) over its time, in GB/s.  The K steps are
timed with events at the two ends of the region only; each kernel's average
duration (``ops``, ``roofline``) comes from max(K, 200) back-to-back launches
of that kernel between two events on the launch stream.  The two step
kernels are timed alone first, then come the W warmup steps and the K timed
steps, then the other lines.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S] [--no-cpu]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
ROWS, COLS = 8192, 4096
EPS = 1e-6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_all_row_kernels.txt")
def traffic_for(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each calibrated on a copy of known size; written
    by scale_invariant_row_amd.rocprof_summary), or None when it is missing or
    was taken from different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    found, khash = None, None
    for line in lines:
        parts = line.split()
        if len(parts) == 2 and parts[0] == "kernel_hash":
            khash = parts[1]
        if len(parts) == 3 and parts[0] == "traffic" and parts[1] == kernel:
            found = int(parts[2])
    from scale_invariant_row_amd.rocprof_summary import kernel_sources_hash
    return found if khash == kernel_sources_hash() else None


def cpu_baseline(l2c, slc, rows: int):
    """The CPU oracle as it stands, timed on the first `rows` rows of each op."""
    from oracle.rows import l2_rows, slerp_rows
    t0 = time.perf_counter()
    l2_rows(l2c.x[:rows], l2c.r[:rows], EPS)
    t1 = time.perf_counter()
    slerp_rows(slc.res[:rows], slc.out[:rows], slc.alpha, EPS)
    t2 = time.perf_counter()
    nbytes = rows * COLS * 6 * 2 + COLS * 4
    return {
        "value": round(nbytes / (t2 - t0) / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"first {rows} of {ROWS} rows of each op (l2_rows {t1 - t0:.1f} s, "
                   f"slerp_rows {t2 - t1:.1f} s), float64 numpy/math.fsum, one thread; "
                   f"host reports {os.cpu_count()} cpus"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=6, help="rotating buffer sets")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=ROWS)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the row ops shard by rows with no exchange, "
              "and this build has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from scale_invariant_row_amd import binding as B
    from scale_invariant_row_amd import inputs

    L = B.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating inputs {ROWS}x{COLS}", file=sys.stderr, flush=True)
    l2c = inputs.make("l2_rows_res_8192x4096")
    slc = inputs.make("slerp_rows_8192x4096")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    x0, r0, res0, out0 = to_dev(l2c.x), to_dev(l2c.r), to_dev(slc.res), to_dev(slc.out)
    alpha = torch.from_numpy(slc.alpha).to(dev)
    sets = []
    for _ in range(args.sets):
        sets.append(dict(x=x0.clone(), r=r0.clone(), y=torch.empty_like(x0),
                         res=res0.clone(), out=out0.clone(), h=torch.empty_like(res0)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    eps = ctypes.c_float(EPS)

    def l2(s):
        return L.ds_l2_rows(s["x"].data_ptr(), s["r"].data_ptr(), s["y"].data_ptr(), ROWS, COLS, eps, sp)

    def slerp(s):
        return L.ds_slerp_rows(s["res"].data_ptr(), s["out"].data_ptr(), alpha.data_ptr(),
                               s["h"].data_ptr(), ROWS, COLS, eps, sp)

    K = args.steps

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # per-kernel duration: NK back-to-back launches of one kernel between two
    # events on the launch stream (an event between every pair of launches
    # would add its own ~2 us to each).  At least 200 launches whatever K is,
    # so that a short run's per-kernel averages are not a handful of launches.
    NK = max(K, 200)

    def batch_us(fn):
        for i in range(3):             # untimed: the first launch of a kernel loads its code
            if fn(sets[i % len(sets)]):
                raise RuntimeError("launch failed")
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(NK):
            if fn(sets[i % len(sets)]):
                raise RuntimeError("launch failed")
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / NK

    # the two kernels alone first, then the W warmup steps and the K timed steps
    l2_us = batch_us(l2)
    sl_us = batch_us(slerp)

    for i in range(args.warmup):
        s = sets[i % len(sets)]
        assert l2(s) == 0 and slerp(s) == 0
    torch.cuda.synchronize()

    # timed region: exactly K steps, events at its two ends only
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        s = sets[i % len(sets)]
        st1 = l2(s)
        st2 = slerp(s)
        if st1 or st2:
            raise RuntimeError(f"launch failed: {B.ds_status_string(st1 or st2)}")
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K

    # the achievable-bandwidth reference: a plain read-2-write-1 stream with
    # l2_rows' launch (shape, grid, buffer resources, cache hints), y = x ^ r,
    # over the same rotating buffers (libdsbench.so, built beside the library)
    BL = ctypes.CDLL(B.LIB_PATH.replace("libdsrows.so", "libdsbench.so"))
    BL.dsb_stream_rows.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
    BL.dsb_stream_rows.restype = ctypes.c_int

    def stream_ref(s):
        return BL.dsb_stream_rows(s["x"].data_ptr(), s["r"].data_ptr(), s["y"].data_ptr(),
                                  ROWS, COLS, sp)

    st_us = batch_us(stream_ref)

    l2_bytes = ROWS * COLS * 2 * 3                      # x, r read; y written
    sl_bytes = ROWS * COLS * 2 * 3 + COLS * 4           # res, out read; h written; alpha once
    step_bytes = l2_bytes + sl_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    def op(us, nbytes, rows):
        gbps = nbytes / (us * 1e-6) / 1e9
        return {"us": round(us, 2), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "rows_per_s": round(rows / (us * 1e-6), 1), "bytes": nbytes}

    ops = {"l2_rows_res_8192x4096": op(l2_us, l2_bytes, ROWS),
           "slerp_rows_8192x4096": op(sl_us, sl_bytes, ROWS),
           "stream_ceiling_8192x4096": op(st_us, l2_bytes, ROWS)}
    ops["stream_ceiling_8192x4096"]["note"] = (
        "stream_rows_kernel: y = x ^ r with l2_rows' launch shape, grid and cache hints "
        "(reads 2, writes 1): the rate a kernel of this shape reaches with no arithmetic")

    # ---- the weight op, rotating 3 copies of the 48 matrices (3 x 510 MB)
    rn = inputs.make("rownorm_gain_12x4_d768")
    rn_sets = []
    for _ in range(3):
        ws = [torch.from_numpy(w).to(dev) for w in rn.w]
        gs = [torch.from_numpy(g).to(dev) for g in rn.gain]
        ns = [torch.empty(w.shape[0], dtype=torch.float32, device=dev) for w in rn.w]
        es = [torch.empty(w.shape, dtype=torch.int16, device=dev) for w in rn.w]
        descs = (B.RownormDesc * len(ws))()
        for i in range(len(ws)):
            descs[i] = B.RownormDesc(ws[i].data_ptr(), gs[i].data_ptr(), 1.0, ns[i].data_ptr(),
                                     es[i].data_ptr(), ws[i].shape[0], ws[i].shape[1])
        rn_sets.append((descs, ws, gs, ns, es))
    n_rn = len(rn.w)
    for i in range(10):
        assert L.ds_weight_rownorm_gain(rn_sets[i % 3][0], n_rn, sp) == 0
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(stream)
    for i in range(60):
        assert L.ds_weight_rownorm_gain(rn_sets[i % 3][0], n_rn, sp) == 0
    b.record(stream)
    torch.cuda.synchronize()
    rn_us = a.elapsed_time(b) * 1e3 / 60
    rn_bytes = rn.total_elems * 6 + rn.total_rows * 8
    ops["weight_rownorm_gain_12x4_d768"] = op(rn_us, rn_bytes, rn.total_rows)
    ops["weight_rownorm_gain_12x4_d768"]["note"] = ("one call: one launch per large shape class, "
                                                    "descriptor tables in the kernel arguments")

    # ---- a plain device copy of the same bytes as l2_rows moves (reference ceiling)
    src = torch.empty(l2_bytes // 2, dtype=torch.uint8, device=dev)   # read + write = l2_bytes
    dsts = [torch.empty_like(src) for _ in range(4)]
    srcs = [torch.empty_like(src) for _ in range(4)]
    for i in range(5):
        dsts[i % 4].copy_(srcs[i % 4])
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(stream)
    for i in range(40):
        dsts[i % 4].copy_(srcs[i % 4])
    b.record(stream)
    torch.cuda.synchronize()
    cp_us = a.elapsed_time(b) * 1e3 / 40
    ops["torch_copy_same_bytes"] = op(cp_us, 2 * src.numel(), ROWS)
    del srcs, dsts, src

    # ---- the other workloads' shapes, beside the headline (random bf16 rows of
    # the same shapes; one buffer set rotation each): reported, not in `value`
    def shaped_us(rows, cols, fn, nsets, n=40, ntens=3):
        bufs = [[torch.randn(rows, cols, device=dev).to(torch.bfloat16) for _ in range(ntens)]
                for _ in range(nsets)]
        torch.cuda.synchronize()
        for i in range(4):
            assert fn(bufs[i % nsets], rows, cols) == 0
        a, b = ev(), ev()
        a.record(stream)
        for i in range(n):
            fn(bufs[i % nsets], rows, cols)
        b.record(stream)
        torch.cuda.synchronize()
        del bufs
        torch.cuda.empty_cache()
        return a.elapsed_time(b) * 1e3 / n

    alpha7 = (torch.rand(7168, device=dev) - 0.5) * 0.4
    c1_us = shaped_us(64, 1024, lambda t, r, c: L.ds_l2_rows(
        t[0].data_ptr(), None, t[2].data_ptr(), r, c, eps, sp), 4, n=200)
    c3_us = shaped_us(8192, 7168, lambda t, r, c: L.ds_slerp_rows(
        t[0].data_ptr(), t[1].data_ptr(), alpha7.data_ptr(), t[2].data_ptr(), r, c, eps, sp), 4)
    c5_us = shaped_us(32768, 8192, lambda t, r, c: L.ds_l2_rows(
        t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), r, c, eps, sp), 2, n=20)
    # the l2_rows gradient at the headline shape: x, r, dy read, dx written
    c2b_us = shaped_us(ROWS, COLS, lambda t, r, c: L.ds_l2_rows_backward(
        t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), t[3].data_ptr(), r, c, eps, sp),
        4, n=100, ntens=4)
    ops["l2_rows_res_bwd_8192x4096"] = op(c2b_us, ROWS * COLS * 8, ROWS)

    # ---- RMSNorm rows: the GPT page's d_model 768 over 8 x 2048 tokens (x read,
    # y written; the gradient reads x and dy, writes dx), and the headline shape
    # with a residual for comparison with l2_rows
    rms_f_us = shaped_us(16384, 768, lambda t, r, c: L.ds_rms_rows(
        t[0].data_ptr(), None, t[1].data_ptr(), r, c, eps, sp), 8, n=100, ntens=2)
    rms_b_us = shaped_us(16384, 768, lambda t, r, c: L.ds_rms_rows_backward(
        t[0].data_ptr(), None, t[1].data_ptr(), t[2].data_ptr(), r, c, eps, sp), 8, n=100)
    rms_h_us = shaped_us(ROWS, COLS, lambda t, r, c: L.ds_rms_rows(
        t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), r, c, eps, sp), 4, n=100)
    ops["rms_rows_16384x768"] = op(rms_f_us, 16384 * 768 * 4, 16384)
    ops["rms_rows_bwd_16384x768"] = op(rms_b_us, 16384 * 768 * 6, 16384)
    ops["rms_rows_res_8192x4096"] = op(rms_h_us, ROWS * COLS * 6, ROWS)

    # ---- weight gradients: the 48 linears, and the one 11008 x 4096 matrix the
    # DragonScale README times forward + backward (device-random fp32 weights
    # N(0, 0.02), gains U(0.5, 2), bf16 upstream gradients N(0, 1))
    gen = torch.Generator(device=dev).manual_seed(4242)

    def weight_sets(shapes, nsets, seg=0, rho=1.0):
        """Descriptor sets over stored fp32 weights; seg > 0: column blocks
        (units = stored columns / seg)."""
        out = []
        for _ in range(nsets):
            ws = [0.02 * torch.randn(sh, device=dev, generator=gen) for sh in shapes]
            lay = [(sh[0], sh[1], 0, 0) if not seg else (sh[1] // seg, sh[0] * seg, seg, sh[1])
                   for sh in shapes]
            gs = [0.5 + 1.5 * torch.rand(ly[0], device=dev, generator=gen) for ly in lay]
            de = [torch.randn(sh, device=dev, generator=gen).to(torch.bfloat16) for sh in shapes]
            fw = (B.RownormDesc * len(ws))()
            bw = (B.RownormGradDesc * len(ws))()
            keep = [ws, gs, de]
            for i, w in enumerate(ws):
                units, cols, sg, ld = lay[i]
                n_out = torch.empty(units, device=dev)
                e_out = torch.empty(w.shape, dtype=torch.int16, device=dev)
                dw = torch.empty_like(w)
                dg = torch.empty(units, device=dev)
                keep += [n_out, e_out, dw, dg]
                fw[i] = B.RownormDesc(w.data_ptr(), gs[i].data_ptr(), rho, n_out.data_ptr(),
                                      e_out.data_ptr(), units, cols, 0, sg, ld)
                bw[i] = B.RownormGradDesc(w.data_ptr(), gs[i].data_ptr(), rho, de[i].data_ptr(),
                                          dw.data_ptr(), dg.data_ptr(), units, cols, 0, None,
                                          sg, ld)
            out.append((fw, bw, len(ws), keep))
        torch.cuda.synchronize()
        return out

    def ragged_us(wsets, which, n):
        call = L.ds_weight_rownorm_gain if which == 0 else L.ds_weight_rownorm_gain_backward
        for i in range(4):
            assert call(wsets[i % len(wsets)][which], wsets[i % len(wsets)][2], sp) == 0
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for i in range(n):
            call(wsets[i % len(wsets)][which], wsets[i % len(wsets)][2], sp)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    lin = inputs.transformer_linears()
    n_el = sum(r * c for r, c in lin)
    n_rows = sum(r for r, _ in lin)
    wsets = weight_sets(lin, 3)
    rnb_us = ragged_us(wsets, 1, 60)
    ops["weight_rownorm_gain_bwd_12x4_d768"] = op(rnb_us, n_el * 10 + n_rows * 8, n_rows)
    del wsets

    # ---- other layers' weights, forward and backward: ResNet-50's convolutions
    # (rows = output channels; the stem's 147-wide rows on single elements),
    # GPT-2 small's 48 Conv1D weights (column blocks: each output unit a column
    # of the stored [in, out]), and a 50304 x 768 embedding at radius sqrt(768)
    for name, shapes, seg, rho in (
            ("resnet50", inputs.resnet50_convs(), 0, 1.0),
            ("gpt2_conv1d", inputs.gpt2_conv1d(), 1, 1.0),
            ("embedding_50304x768", [(50304, 768)], 0, float(np.sqrt(np.float32(768))))):
        sets = weight_sets(shapes, 3, seg, rho)
        el = sum(a * b for a, b in shapes)
        units = sum((b // seg) if seg else a for a, b in shapes)
        ops[f"weight_rownorm_gain_{name}"] = op(ragged_us(sets, 0, 40), el * 6 + units * 8, units)
        ops[f"weight_rownorm_gain_bwd_{name}"] = op(ragged_us(sets, 1, 40), el * 10 + units * 8,
                                                    units)
        del sets
        torch.cuda.empty_cache()
    # ---- the rescale method on the 48 linears: project (W, G read; G written) and
    # after a step (W, M read and written)
    rs_sets = []
    for _ in range(3):
        ws = [0.02 * torch.randn(sh, device=dev, generator=gen) for sh in lin]
        vs = [1e-3 * torch.randn(sh, device=dev, generator=gen) for sh in lin]
        ms = [1e-3 * torch.randn(sh, device=dev, generator=gen) for sh in lin]
        pd = (B.RescaleDesc * len(lin))()
        ad = (B.RescaleDesc * len(lin))()
        for i, (r, c) in enumerate(lin):
            pd[i] = B.RescaleDesc(ws[i].data_ptr(), vs[i].data_ptr(), 1.0, r, c)
            ad[i] = B.RescaleDesc(ws[i].data_ptr(), ms[i].data_ptr(), 1.0, r, c)
        rs_sets.append((pd, ad, ws, vs, ms))
    torch.cuda.synchronize()

    def rescale_us(which, n=60):
        call = L.ds_rescale_project if which == 0 else L.ds_rescale_after_step
        for i in range(4):
            assert call(rs_sets[i % 3][which], len(lin), sp) == 0
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for i in range(n):
            call(rs_sets[i % 3][which], len(lin), sp)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    ops["rescale_project_12x4_d768"] = op(rescale_us(0), n_el * 12, n_rows)
    ops["rescale_after_step_12x4_d768"] = op(rescale_us(1), n_el * 16, n_rows)
    del rs_sets
    torch.cuda.empty_cache()

    # the weight op's own stream reference: fp32 rows read, bf16 written, with
    # the launch the weight op gives rows of that width (libdsbench.so), over
    # each set's matrix in turn
    BL.dsb_stream_f32_rows.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
    BL.dsb_stream_f32_rows.restype = ctypes.c_int

    def f32_stream_us(sets, n):
        def one(s):
            w, e = s[3][0][0], s[3][4]           # the set's weight and its bf16 output
            return BL.dsb_stream_f32_rows(w.data_ptr(), e.data_ptr(), w.shape[0], w.shape[1], sp)
        for i in range(4):
            assert one(sets[i % len(sets)]) == 0
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for i in range(n):
            one(sets[i % len(sets)])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    big = [(11008, 4096)]
    wsets = weight_sets(big, 4)
    f_us = ragged_us(wsets, 0, 40)
    b_us = ragged_us(wsets, 1, 40)
    fs_us = f32_stream_us(wsets, 40)
    del wsets
    torch.cuda.empty_cache()
    # the 48 linears' 768-wide rows (qkv, o, up: 73,728 of them) as one matrix
    tall = [(73728, 768)]
    wsets = weight_sets(tall, 3)
    t_us = ragged_us(wsets, 0, 40)
    ts_us = f32_stream_us(wsets, 40)
    del wsets
    torch.cuda.empty_cache()
    n_tall = 73728 * 768
    f32_note = ("stream_f32_rows_kernel: fp32 rows read, bf16 written, with the weight op's launch "
                "for the width (shape, grid, buffer resources, cache hints): the weight op's "
                "traffic with no arithmetic")
    ops["weight_rownorm_gain_73728x768"] = op(t_us, n_tall * 6 + 73728 * 8, 73728)
    ops["stream_f32_ceiling_73728x768"] = op(ts_us, n_tall * 6, 73728)
    ops["stream_f32_ceiling_73728x768"]["note"] = f32_note
    ops["stream_f32_ceiling_11008x4096"] = op(fs_us, 11008 * 4096 * 6, 11008)
    ops["stream_f32_ceiling_11008x4096"]["note"] = f32_note
    n_big = 11008 * 4096
    ops["weight_rownorm_gain_11008x4096"] = op(f_us, n_big * 6 + 11008 * 8, 11008)
    ops["weight_rownorm_gain_bwd_11008x4096"] = op(b_us, n_big * 10 + 11008 * 8, 11008)
    ops["weight_rownorm_gain_fwd_bwd_11008x4096"] = op(
        f_us + b_us, n_big * 16 + 11008 * 16, 11008)
    ops["weight_rownorm_gain_fwd_bwd_11008x4096"]["note"] = (
        "forward (fp32 W read, bf16 W_eff and fp32 norms written) plus backward (W and bf16 "
        "dW_eff read, fp32 dW and dg written): the op the DragonScale README reports at 85-96% "
        "of the card's bandwidth on V100/2080 Ti/3090/4090, where its W_eff is fp32")

    # ---- activation rows at the Dory widths (o, g or g, u read; y written;
    # fp32 column scales once per launch)
    sg4 = 0.5 + 1.5 * torch.rand(4096, device=dev)
    sug7 = 0.5 + 1.5 * torch.rand(7168, device=dev)
    suu7 = 0.5 + 1.5 * torch.rand(7168, device=dev)
    gate_us = shaped_us(ROWS, 4096, lambda t, r, c: L.ds_gate_l2_rows(
        t[0].data_ptr(), t[1].data_ptr(), sg4.data_ptr(), t[2].data_ptr(), r, c, eps, sp), 5)
    swiglu_us = shaped_us(ROWS, 7168, lambda t, r, c: L.ds_swiglu_l2_rows(
        t[0].data_ptr(), t[1].data_ptr(), sug7.data_ptr(), suu7.data_ptr(), t[2].data_ptr(),
        r, c, eps, sp), 4)
    ops["gate_l2_rows_8192x4096"] = op(gate_us, ROWS * 4096 * 6 + 4096 * 4, ROWS)

    # ---- q/k rows: 16 q heads over 4 kv heads of 256, a third of the rows far
    # along (positions 199,800..); q and k read and written, positions once per row
    nq, nk, hd = 16, 4, 256
    posv = torch.cat([torch.arange(ROWS - ROWS // 3), 199_800 + torch.arange(ROWS // 3)]).to(
        device=dev, dtype=torch.int32)
    invf = torch.from_numpy(inputs.rope_inv_freq(hd)).to(dev)
    qsc = 0.5 + 1.5 * torch.rand(nq * hd, device=dev)
    qk_sets = [(torch.randn(ROWS, nq * hd, device=dev).to(torch.bfloat16),
                torch.randn(ROWS, nk * hd, device=dev).to(torch.bfloat16),
                torch.empty(ROWS, nq * hd, dtype=torch.bfloat16, device=dev),
                torch.empty(ROWS, nk * hd, dtype=torch.bfloat16, device=dev)) for _ in range(6)]

    def qk(t):
        return L.ds_qk_rows_l2(t[0].data_ptr(), nq * hd, t[1].data_ptr(), nk * hd,
                               posv.data_ptr(), invf.data_ptr(), qsc.data_ptr(),
                               t[2].data_ptr(), nq * hd, t[3].data_ptr(), nk * hd,
                               ROWS, nq, nk, hd, eps, sp)
    for i in range(4):
        assert qk(qk_sets[i % 6]) == 0
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(stream)
    for i in range(60):
        qk(qk_sets[i % 6])
    b.record(stream)
    torch.cuda.synchronize()
    qk_us = a.elapsed_time(b) * 1e3 / 60
    del qk_sets
    torch.cuda.empty_cache()
    qk_bytes = ROWS * (nq + nk) * hd * 2 * 2 + ROWS * 4 + hd // 2 * 4 + nq * hd * 4
    ops["qk_rows_l2_8192_h16x4_d256"] = op(qk_us, qk_bytes, ROWS)
    ops["swiglu_l2_rows_8192x7168"] = op(swiglu_us, ROWS * 7168 * 6 + 7168 * 8, ROWS)

    ops["l2_rows_64x1024"] = op(c1_us, 64 * 1024 * 4, 64)
    ops["l2_rows_64x1024"]["note"] = "latency-bound: one small launch"
    ops["slerp_rows_8192x7168"] = op(c3_us, 8192 * 7168 * 6 + 7168 * 4, 8192)
    ops["l2_rows_res_32768x8192"] = op(c5_us, 32768 * 8192 * 6, 32768)

    dominant = "slerp_rows_8192x4096" if sl_us >= l2_us else "l2_rows_res_8192x4096"
    kname = {"slerp_rows_8192x4096": "slerp_rows_kernel",
             "l2_rows_res_8192x4096": "l2_rows_kernel"}[dominant]
    d = ops[dominant]
    roofline = {"bound": "hbm", "kernel": kname, "achieved": d["GBps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": d["frac"],
                "traffic": traffic_for(kname),
                "algorithmic_bytes_per_launch": d["bytes"],
                "stream_ceiling": {"kernel": "stream_rows_kernel",
                                   "GBps": ops["stream_ceiling_8192x4096"]["GBps"],
                                   "frac": ops["stream_ceiling_8192x4096"]["frac"]}}

    result = {
        "metric": "achieved HBM GB/s (% of peak) for bf16 l2_rows/slerp_rows at 8192x4096",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "l2_rows with fused residual + slerp_rows, 8192 x 4096 rows",
                   "rows": ROWS, "cols": COLS, "io": "bf16", "eps": EPS,
                   "buffer_sets": args.sets,
                   "bytes_per_step": step_bytes,
                   "frac_of_peak": round(value / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "ops": ops,
    }
    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(l2c, slc, args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
