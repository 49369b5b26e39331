"""The full-size checking harness finds what it is there to find (CPU only).

The oracle's own outputs pass every count; the same outputs with one
element moved by two bf16 steps fail both the contract and the strict set,
and the failure is reported at its flat index in the whole workload.
"""
import numpy as np

import fullsize_jobs as J
from oracle.rows import l2_rows, slerp_rows
from scale_invariant_row_amd import inputs


def test_l2_job_clean_and_planted():
    c = inputs.l2_case(40, 1024, 31)
    got = l2_rows(c.x, c.r, c.eps)
    base = 5000                       # the chunk's first row within its workload
    clean = J.l2_job(got, c.x, c.r, c.eps, 48, base)
    assert clean["n"] == got.size and clean["beyond"] == 0 and clean["outside"] == 0
    assert clean["differ"] == 0 and clean["max_steps"] == 0
    bad = got.copy()
    bad[7, 100] += 2                  # two steps up (a normal value)
    planted = J.l2_job(bad, c.x, c.r, c.eps, 48, base)
    flat = (base + 7) * 1024 + 100
    assert planted["beyond"] == 1 and planted["outside"] == 1
    assert planted["differ"] == 1 and planted["max_steps"] == 2
    assert flat in planted["first_bad"]


def test_slerp_job_counts_nonunique():
    c = inputs.slerp_case(30, 4096, 32)
    got = slerp_rows(c.res, c.out, c.alpha, c.eps)
    counts = J.slerp_job(got, c.res, c.out, c.alpha, c.eps, 96, 0)
    assert counts["beyond"] == 0 and counts["outside"] == 0
    assert 0 < counts["nonunique"] < 0.03 * counts["n"]
    bad = got.copy()
    bad[0, 0] ^= 0x8000               # a sign flip is outside every set
    assert J.slerp_job(bad, c.res, c.out, c.alpha, c.eps, 96, 0)["outside"] >= 1


def test_pool_runs_jobs_in_order_and_merges():
    c = inputs.l2_case(64, 512, 33)
    got = l2_rows(c.x, c.r, c.eps)
    got[50, 3] += 3
    jobs = [(got[a:b], c.x[a:b], c.r[a:b], c.eps, 40, a) for a, b in J.chunks(64, 16)]
    res = J.run_pool(J.l2_job, jobs)
    assert [r["n"] for r in res] == [16 * 512] * 4
    m = J.merge(res)
    assert m["n"] == 64 * 512 and m["beyond"] == 1 and m["max_steps"] == 3
    assert 50 * 512 + 3 in m["first_bad"]
    assert J.chunks(10, 4) == [(0, 4), (4, 8), (8, 10)]
