"""The oracle's anti-diagonal schedule against a hand-written fixture and the
closed forms of the (layer, segment) grid."""
import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc

import pins


def test_golden_L4_S6():
    pins.pin_schedule_golden()


@pytest.mark.parametrize("L", range(1, 13))
@pytest.mark.parametrize("S", range(1, 13))
def test_invariants_small(L, S):
    pins.pin_schedule_invariants(L, S)


@pytest.mark.parametrize("cfg", [ri.TINY_LINEAR_GELU, ri.NORM_SWIGLU_1B, ri.LLAMA_1B, ri.LLAMA_8B],
                         ids=lambda c: c.name)
def test_invariants_workload_grids(cfg):
    pins.pin_schedule_invariants(cfg.L, cfg.S)


@pytest.mark.parametrize("L,S,ramp", [(16, 128, 240), (32, 64, 992), (16, 32, 240), (4, 6, 12)])
def test_ramp_cells(L, S, ramp):
    # cells on diagonals with fewer than min(L, S) active cells: two triangles
    # of 1 + 2 + ... + (min(L, S) - 1) cells each
    k = min(L, S) - 1
    assert ramp == k * (k + 1)
    diags = orc.schedule(L, S)
    assert sum(len(dg) for dg in diags if len(dg) < min(L, S)) == ramp


def test_table_csr():
    diag_ptr, cells = orc.schedule_table(4, 6)
    golden = pins.load_golden_schedule()
    assert diag_ptr.tolist() == np.cumsum([0] + [len(dg) for dg in golden]).tolist()
    flat = [(l, s, slot) for dg in golden for slot, (l, s) in enumerate(dg)]
    assert [tuple(r) for r in cells.tolist()] == flat
