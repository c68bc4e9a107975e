"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from oracle_pins import ALL_PINS, golden
from channel_gated_delta_amd import workloads


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle.default())


def test_generator_respects_gate_bound():
    """Workloads draw g in [lb, 0]; with lb = -5 every 16-token window sums into
    the bounded range the walkthrough's 彩蛋 section states."""
    gd = golden("k3_sizes.json")
    spec = workloads.PrefillSpec("t", [300], heads=2, dk=8, dv=8, conv=False, seed=3)
    inp = workloads.make_prefill(spec)
    g = inp["g"].double().numpy()
    assert g.max() <= 0.0 and g.min() >= spec.gate_lb
    win = np.lib.stride_tricks.sliding_window_view(g, gd["subchunk_tokens"], axis=0).sum(-1)
    lo, hi = gd["subchunk_cumulative_log_decay_range"]
    assert win.min() >= lo and win.max() <= hi


def test_generator_is_seeded():
    spec = workloads.standard_specs()["tiny_fp32"]
    a = workloads.make_prefill(spec)
    b = workloads.make_prefill(spec)
    for key in ("q", "k", "v", "g", "beta"):
        assert torch.equal(a[key], b[key])
    assert torch.allclose(a["q"].double().norm(dim=-1), torch.ones(64, 1, dtype=torch.float64),
                          atol=1e-6)
