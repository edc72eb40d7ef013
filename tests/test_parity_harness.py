"""CPU checks of the parity harness's near-tie rule (tests/_parity.py): the
GPU may list a selected set in another order only where consecutive selected
scores are near-tied, and may select another set only at a near-tied top-k
boundary.  Fixture: a DeepSeek-V3-style token (sigmoid + selection bias,
top-8 of 256) whose 6th and 7th keys are 4e-8 apart."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import make_workload
from tests import _parity as P


@pytest.fixture(scope="module")
def case():
    wl = make_workload(4, T=256, d=8448, h=256)
    ref = O.layer(wl, with_ffn=False)["route"]
    order_gap = P.order_gap_of(wl, ref)
    t = int(np.argmin(order_gap))
    assert order_gap[t] < P.NEAR_TIE <= ref["gap"][t]
    return wl, ref, t


def _with(ref, t, ids_row):
    ids = ref["ids"].copy()
    ids[t] = ids_row
    return {"ids": ids}


def test_reordered_near_tie_is_accepted(case):
    wl, ref, t = case
    keys = P.selection_keys(wl, ref)
    chosen = keys[t, ref["ids"][t]]
    j = int(np.argmin(chosen[:-1] - chosen[1:]))
    row = ref["ids"][t].copy()
    row[[j, j + 1]] = row[[j + 1, j]]
    exempt = P.check_route(wl, _with(ref, t, row), ref)
    assert exempt[t]


def test_reordering_a_clear_gap_is_rejected(case):
    wl, ref, t = case
    keys = P.selection_keys(wl, ref)
    chosen = keys[t, ref["ids"][t]]
    gaps = chosen[:-1] - chosen[1:]
    j = int(np.argmax(gaps))
    assert gaps[j] > 1e-3
    row = ref["ids"][t].copy()
    row[[j, j + 1]] = row[[j + 1, j]]
    with pytest.raises(AssertionError):
        P.check_route(wl, _with(ref, t, row), ref)


def test_swapping_in_the_next_expert_is_rejected(case):
    wl, ref, t = case
    keys = P.selection_keys(wl, ref)
    order = np.argsort(-keys[t], kind="stable")
    row = ref["ids"][t].copy()
    row[-1] = order[wl.k]  # the (k+1)-th expert, 1.2e-4 below the k-th
    with pytest.raises(AssertionError):
        P.check_route(wl, _with(ref, t, row), ref)
