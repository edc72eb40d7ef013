"""GPU parity of the matrix-core router (bf16 activations, E <= 32,
d a multiple of 1024, more than 1024 tokens): softmax and sigmoid scores,
with and without renormalisation, the selection-only bias, and token counts
that leave a ragged last tile of 32.

Besides the whole layer against the fp64 oracle, the selection is checked
bit for bit against the oracle's selection on the logits the kernel itself
wrote (same fp32 keys, ties to the lower expert index).
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import make_workload
from tests.test_gpu_parity import _say, full_parity

pytestmark = pytest.mark.gpu

CASES = [
    (2, dict(T=2085, d=1024, h=256)),                                   # E=8 top-2 softmax
    (2, dict(T=4128, d=2048, h=256, E=16, k=4, R=8)),                   # E=16
    (2, dict(T=2085, d=1024, h=256, E=32, k=8, R=8, renorm=False)),     # E=32, no renorm
    (4, dict(T=2085, d=1024, h=256, E=32, k=8, R=8)),                   # sigmoid + bias
    (4, dict(T=3001, d=1024, h=256, E=16, k=4, R=8, renorm=False)),     # sigmoid, raw scores
    (2, dict(T=1057, d=1024, h=256, E=3, k=2, R=1)),                    # odd E, T just past 1024
    (4, dict(T=1100, d=1024, h=256, E=5, k=3, R=1)),                    # odd E, sigmoid + bias
    (2, dict(T=1025, d=1024, h=256, E=1, k=1, R=1)),                    # one expert, one token past a tile
]


@pytest.mark.parametrize("cfg,over", CASES)
def test_mfma_router(cfg, over):
    wl = make_workload(cfg, **over)
    assert wl.act_dtype == "bf16" and wl.E <= 32 and wl.d % 1024 == 0 and wl.T > 1024
    g, _ = full_parity(wl, label=f"mfma router {wl.score} E={wl.E} k={wl.k} renorm={wl.renorm}")
    key = O.selection_keys32(np.asarray(g["logits"], np.float32), wl.score, wl.b_select)
    _say(f"[mfma router] selection on the kernel's own logits, T={wl.T}")
    np.testing.assert_array_equal(g["ids"], O.topk_select(key, wl.k))
