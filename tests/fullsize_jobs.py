"""Every element of a full-size workload against the oracle, in row chunks.

TEST HELPER.  The GPU test process hands each chunk of rows (the GPU's bits
and the chunk's inputs) to a pool of CPU worker processes; each worker runs
the float64 oracle and the two checks of oracle/check.py on its chunk and
returns counts.  The workers import numpy and oracle/ only: they never touch
the GPU (the pool uses the "spawn" start method, so a worker is a fresh
interpreter, not a copy of the process that holds the device).

A chunk's result is a dict of counts:

  n          elements compared
  beyond     elements beyond the 1-bf16-ulp (2e-6 for fp32) contract among
             those where the contract applies
  differ     elements whose bits differ from the oracle's rounding
  max_steps  the largest distance from the oracle, in bf16 steps
  outside    elements outside the strict admissible set (plus sets the
             bound cannot make sharp, which also fail the check)
  two        elements whose admissible set holds two values (near-ties)
  first_bad  flat indices (within the whole workload) of the first failures

and, for slerp, ``nonunique`` (elements where a or b may round either way,
so the contract is waived and only the strict set applies),
``nonunique_beyond`` and ``nonunique_max_steps``.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time
from concurrent.futures import ProcessPoolExecutor
from typing import Callable, Iterable, List

import numpy as np

CHUNK_ROWS = 1024


def workers() -> int:
    """Worker processes for the oracle: at most 8, fewer on a small host."""
    return max(1, min(8, os.cpu_count() or 1))


def run_pool(fn: Callable, jobs: Iterable[tuple], deadline_s: float = 600.0) -> List[dict]:
    """fn(*job) for every job, in worker processes, results in job order.

    Fails (rather than waiting on) a pool whose workers die or stall: each
    result is awaited until a common deadline, and on any error the workers
    are terminated before the error propagates.
    """
    jobs = list(jobs)
    ctx = mp.get_context("spawn")
    ex = ProcessPoolExecutor(max_workers=min(workers(), max(1, len(jobs))), mp_context=ctx)
    end = time.monotonic() + deadline_s
    try:
        futs = [ex.submit(fn, *j) for j in jobs]
        out = [f.result(timeout=max(1.0, end - time.monotonic())) for f in futs]
    except BaseException:
        for p in list(getattr(ex, "_processes", {}).values()):
            p.terminate()
        ex.shutdown(wait=False, cancel_futures=True)
        raise
    ex.shutdown(wait=True)
    return out


def merge(results: List[dict]) -> dict:
    out: dict = {}
    for r in results:
        for k, v in r.items():
            if k == "first_bad":
                out[k] = (out.get(k, []) + v)[:20]
            elif k.endswith("max_steps"):
                out[k] = max(out.get(k, 0), v)
            else:
                out[k] = out.get(k, 0) + v
    return out


def _steps(got, want) -> np.ndarray:
    """Distance in bf16 steps (NaN-vs-NaN and equal bits count 0)."""
    from oracle.check import ordered
    g = np.asarray(got, np.uint16)
    w = np.asarray(want, np.uint16)
    gn = (g & 0x7FFF) > 0x7F80
    wn = (w & 0x7FFF) > 0x7F80
    d = np.abs(ordered(g) - ordered(w))
    return np.where(gn & wn, 0, d)


def _counts(got, want, ok, rep, base, cols) -> dict:
    bad = np.flatnonzero(~ok)
    st = _steps(got, want)
    return {
        "n": int(np.size(got)),
        "beyond": int(bad.size),
        "differ": int(np.count_nonzero(np.asarray(got) != np.asarray(want))),
        "max_steps": int(st.max()) if st.size else 0,
        "outside": int(rep.outside + rep.loose),
        "two": int(rep.two),
        "first_bad": [int(base * cols + b) for b in bad[:10]] + list(rep.first_bad[:10]),
    }


# ------------------------------------------------------------------ jobs

def l2_job(got, x, r, eps, depth, base, mean=False):
    """l2_rows (or rms_rows with mean=True) over rows base.. of a workload."""
    from oracle.check import admissible_l2_rows, contract_bf16
    from oracle.rows import l2_rows, rms_rows
    want = (rms_rows if mean else l2_rows)(x, r, eps)
    ok = contract_bf16(got, want)
    ids = np.arange(base, base + x.shape[0])
    rep = admissible_l2_rows(got, x, r, eps, depth=depth, row_ids=ids, mean=mean)
    return _counts(got, want, ok, rep, base, x.shape[1])


def slerp_job(got, res, out, alpha, eps, depth, base):
    from oracle.check import admissible_slerp_rows, contract_bf16, slerp_unique_mask
    from oracle.rows import slerp_rows
    want = slerp_rows(res, out, alpha, eps)
    ok = contract_bf16(got, want)
    uniq = slerp_unique_mask(res, out, eps, depth)
    ids = np.arange(base, base + res.shape[0])
    rep = admissible_slerp_rows(got, res, out, alpha, eps, depth, row_ids=ids)
    c = _counts(got, want, ok | ~uniq, rep, base, res.shape[1])
    st = _steps(got, want)
    nu = ~uniq
    c["nonunique"] = int(np.count_nonzero(nu))
    c["nonunique_beyond"] = int(np.count_nonzero(~ok & nu))
    c["nonunique_max_steps"] = int(st[nu].max()) if nu.any() else 0
    return c


def rownorm_job(got_n, got_w, w, g, rho, depth, base):
    """One matrix's rows base..: fp32 norms (2e-6) and bf16 W_eff (1 ulp)."""
    from oracle.check import admissible_rownorm, contract_bf16, contract_rel
    from oracle.rows import weight_rownorm_gain
    n_ref, w_ref = weight_rownorm_gain([w], [g], [rho])
    okn = contract_rel(got_n, n_ref[0])
    okw = contract_bf16(got_w, w_ref[0], zero_sign=False)
    rn, rw = admissible_rownorm(got_n, got_w, w, g, rho, depth=depth)
    c = _counts(got_w, w_ref[0], okw, rw, base, w.shape[1])
    c["norms"] = int(got_n.size)
    c["norms_beyond"] = int(np.count_nonzero(~okn))
    c["outside"] += int(rn.outside + rn.loose)
    return c


def qk_job(got_q, got_k, q, k, pos, inv_freq, q_scale, head_dim, eps, depth, base):
    """q/k rows: the strict set everywhere, the contract where the set has
    one value (a near-tie of the rotated head may move the result)."""
    from oracle.check import admissible_qk_rows, contract_bf16
    from oracle.rows import qk_rows_l2
    rq, rk, uq, uk = admissible_qk_rows(got_q, got_k, q, k, pos, inv_freq, q_scale, head_dim,
                                        eps, depth=depth)
    wq, wk = qk_rows_l2(q, k, pos, inv_freq, q_scale, head_dim, eps)
    out = []
    for got, want, u, rep in ((got_q, wq, uq, rq), (got_k, wk, uk, rk)):
        if got is None:
            continue
        ok = contract_bf16(got, want, zero_sign=False) | ~u
        c = _counts(got, want, ok, rep, base, got.shape[1])
        c["nonunique"] = int(np.count_nonzero(~u))
        c["wide"] = int(rep.wide)
        out.append(c)
    return merge(out)


def act_job(kind, got, a, b, s0, s1, eps, depth, base):
    """gate (kind "gate": o, g, sg) or SwiGLU (kind "swiglu": g, u, sug, suu)."""
    from oracle.check import (act_unique_mask, admissible_act_rows, contract_bf16,
                              gate_candidates, swiglu_candidates)
    from oracle.rows import gate_l2_rows, swiglu_l2_rows
    if kind == "gate":
        want = gate_l2_rows(a, b, s0, eps)
        lo, hi = gate_candidates(a, b, s0)
    else:
        want = swiglu_l2_rows(a, b, s0, s1, eps)
        lo, hi = swiglu_candidates(a, b, s0, s1)
    uniq = act_unique_mask(lo, hi)
    ok = contract_bf16(got, want) | ~uniq
    finite = np.isfinite(lo).all(axis=1) & np.isfinite(hi).all(axis=1)
    rep = admissible_act_rows(got, lo, hi, want, finite, eps, depth)
    c = _counts(got, want, ok, rep, base, a.shape[1])
    c["nonunique"] = int(np.count_nonzero(~uniq))
    return c


def l2_backward_job(got, x, r, dy, eps, depth, base, mean=False):
    from oracle.bf16 import bf16_rne, bf16_value
    from oracle.check import admissible_l2_backward, contract_grad, l2_grad_terms
    from oracle.rows import eps_as_passed, l2_rows_backward, rms_rows_backward
    want = (rms_rows_backward if mean else l2_rows_backward)(x, r, dy, eps)
    xv = bf16_value(x)
    with np.errstate(all="ignore"):
        s = xv if r is None else bf16_value(bf16_rne(xv + bf16_value(r)))
    terms = l2_grad_terms(s, bf16_value(dy), eps_as_passed(eps), mean=mean)
    ok = contract_grad(got, want, terms)
    ids = np.arange(base, base + x.shape[0])
    rep = admissible_l2_backward(got, x, r, dy, eps, depth=depth, row_ids=ids, mean=mean)
    c = _counts(got, want, ok, rep, base, x.shape[1])
    c["wide"] = int(rep.wide)
    return c


def rownorm_backward_job(got_dw, got_dg, w, g, rho, dwe, depth, base):
    from oracle.bf16 import bf16_value
    from oracle.check import admissible_rownorm_backward, contract_grad, rownorm_grad_terms
    from oracle.rows import weight_rownorm_gain_backward
    dw_ref, dg_ref = weight_rownorm_gain_backward([w], [g], [rho], [dwe])
    terms_w, terms_g = rownorm_grad_terms(w.astype(np.float64), g.astype(np.float64),
                                          float(np.float32(rho)), bf16_value(dwe))
    okw = contract_grad(got_dw, dw_ref[0], terms_w, fmt="f32")
    okg = contract_grad(got_dg, dg_ref[0], terms_g, fmt="f32")
    rw, rg = admissible_rownorm_backward(got_dw, got_dg, w, g, rho, dwe, depth=depth)
    return {
        "n": int(got_dw.size),
        "beyond": int(np.count_nonzero(~okw)),
        "differ": int(np.count_nonzero(got_dw != dw_ref[0].astype(np.float32))),
        "outside": int(rw.outside + rw.loose + rg.outside + rg.loose),
        "two": 0,
        "wide": int(rw.wide + rg.wide),
        "dg": int(got_dg.size),
        "dg_beyond": int(np.count_nonzero(~okg)),
        "first_bad": [int(base * w.shape[1] + b) for b in np.flatnonzero(~okw)[:10]]
                     + list(rw.first_bad[:5]) + list(rg.first_bad[:5]),
    }


def chunks(rows: int, chunk: int = CHUNK_ROWS):
    """(start, stop) row ranges covering [0, rows)."""
    return [(a, min(rows, a + chunk)) for a in range(0, rows, chunk)]


def rescale_job(got_w, got_v, w, v, rho, after_step, depth, base):
    """The rescale method's rows base..: v (the projected gradient or momentum)
    against the gradient contract, w (after a step) within 2e-6, and both
    inside the strict set."""
    from oracle.check import admissible_rescale, contract_grad, contract_rel, rescale_terms
    from oracle.rows import rescale_after_step, rescale_project
    if after_step:
        ws, ms = rescale_after_step([w], [v], [rho])
        okw = contract_rel(got_w, ws[0])
    else:
        ms = rescale_project([w], [v])
        okw = got_w == w
    terms = rescale_terms(w.astype(np.float64), v.astype(np.float64))
    okv = contract_grad(got_v, ms[0], terms, "f32")
    rw, rv = admissible_rescale(got_w, got_v, w, v, rho, after_step, depth=depth)
    bad = np.flatnonzero(~(okv & okw))
    return {
        "n": int(got_v.size),
        "beyond": int(bad.size),
        "outside": int(rv.outside + rv.loose + (rw.outside + rw.loose if after_step else 0)),
        "two": 0,
        "wide": int(rv.wide),
        "first_bad": [int(base * w.shape[1] + b) for b in bad[:10]] + list(rv.first_bad[:10]),
    }
