"""The binding refuses bad arguments with ValueError before any launch.

CPU tensors throughout: every shape, dtype, stride and row-count check runs
before the device check, so each bad argument is named on its own, and a
call whose arguments are all well formed still stops at the device check
(CPU tensors are not on a HIP device) without reaching the library.
"""
import pytest
import torch

from scale_invariant_row_amd import binding as B

ROWS, HD, NQ, NK = 6, 64, 3, 1


def qk_args(**over):
    a = dict(q=torch.zeros(ROWS, NQ * HD, dtype=torch.bfloat16),
             k=torch.zeros(ROWS, NK * HD, dtype=torch.bfloat16),
             positions=torch.zeros(ROWS, dtype=torch.int32),
             inv_freq=torch.ones(HD // 2, dtype=torch.float32),
             q_scale=torch.ones(NQ * HD, dtype=torch.float32),
             head_dim=HD)
    a.update(over)
    return a


def refused(match, **over):
    with pytest.raises(ValueError, match=match):
        B.ds_qk_rows_l2(**qk_args(**over))


def test_qk_well_formed_stops_at_device():
    refused("HIP device")


@pytest.mark.parametrize("over,match", [
    (dict(k=torch.zeros(ROWS - 1, NK * HD, dtype=torch.bfloat16)), "^k: expected 6 rows"),
    (dict(k=torch.zeros(ROWS, NK * HD + 3, dtype=torch.bfloat16)), "^k: its width"),
    (dict(k=torch.zeros(ROWS, NK * HD, dtype=torch.float32)), "^k: expected a bf16"),
    (dict(k=torch.zeros(NK * HD, ROWS, dtype=torch.bfloat16).t()), "^k: expected a bf16"),
    (dict(q=torch.zeros(ROWS, NQ * HD - 8, dtype=torch.bfloat16)), "^q: must hold"),
    (dict(q_out=torch.zeros(ROWS - 2, NQ * HD, dtype=torch.bfloat16)), "^q_out: expected"),
    (dict(q_out=torch.zeros(ROWS, NQ * HD, dtype=torch.float32)), "^q_out: expected a bf16"),
    (dict(k_out=torch.zeros(ROWS, NK * HD - 8, dtype=torch.bfloat16)), "^k_out: expected"),
    (dict(k=None, k_out=torch.zeros(ROWS, HD, dtype=torch.bfloat16)), "^k_out: given without k"),
    (dict(positions=torch.zeros(ROWS + 1, dtype=torch.int32)), "^positions"),
    (dict(positions=torch.zeros(ROWS, dtype=torch.int64)), "^positions"),
    (dict(positions=torch.zeros(2 * ROWS, dtype=torch.int32)[::2]), "^positions"),
    (dict(inv_freq=torch.ones(HD, dtype=torch.float32)), "^inv_freq"),
    (dict(inv_freq=torch.ones(HD, dtype=torch.float32)[::2]), "^inv_freq"),
    (dict(q_scale=torch.ones(NQ * HD + 5, dtype=torch.float32)), "^q_scale: its length"),
    (dict(q_scale=torch.ones(2 * NQ * HD, dtype=torch.float32)[::2]), "^q_scale"),
    (dict(q_scale=torch.ones(NQ * HD, dtype=torch.float64)), "^q_scale"),
    (dict(head_dim=0), "^head_dim"),
])
def test_qk_bad_argument_named(over, match):
    refused(match, **over)


def test_rownorm_norm_out_must_be_contiguous():
    w = torch.zeros(4, 8)
    g = torch.ones(4)
    with pytest.raises(ValueError, match=r"^norm_out\[0\]"):
        B.ds_weight_rownorm_gain([w], [g], norm_out=[torch.zeros(8)[::2]])


def test_rownorm_backward_dgain_must_be_contiguous():
    w = torch.zeros(4, 8)
    g = torch.ones(4)
    de = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"^dgain\[0\]"):
        B.ds_weight_rownorm_gain_backward([w], [g], [de], dgain=[torch.zeros(8)[::2]])


def test_rownorm_backward_cpu_tensors_refused_before_allocating():
    """A scalar gain's temporary is allocated only after every check passed."""
    w = torch.zeros(4, 8)
    de = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        B.ds_weight_rownorm_gain_backward([w], [torch.ones(())], [de])
