"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (tiled expert weights), plus routing variants.

* Identical-logits mode at full T for the prefill, Switch and DeepSeek-V3
  workloads: the oracle's fp32 logits are fed to the GPU route, and ids,
  counts, offsets, slots and src must match bit for bit.
* DeepSeek-V3 share (T=8192): every float output element by element.
* Prefill layer (T=16384): every float output element by element.
* Switch layer under the two other readings of its Zipf offset (the
  logarithm of the Zipf weights, about 91% of assignments dropped; the
  normalised probabilities, about 2% dropped): full parity at full size.
* Sigmoid scores with a selection-only bias at E = 8, 16 and 64 (the small
  and row-wise top-k kernels), and weights without renormalisation for
  softmax and sigmoid scoring.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import make_workload
from tests.test_gpu_parity import _identical_logits, full_parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import expert_token_routing_gemm_amd as M  # noqa: F401  (fails loudly without libmoe.so)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_identical_logits_full_size(cfg):
    wl = make_workload(cfg)
    _say(f"[identical-logits] cfg{cfg} T={wl.T} E={wl.E} k={wl.k} full size")
    r = O.layer(wl, with_ffn=False)
    g = _identical_logits(wl, r["route"]["logits32"])
    assert int(g["counts"].sum()) == wl.T * wl.k


@pytest.mark.slow
def test_c4_full_size_every_element():
    """DeepSeek-V3 share at full size, tiled fp8 weights (the bench's
    configuration): logits, weights, every integer stage, the packed send
    buffer, the executed experts' outputs, the shared expert and y."""
    full_parity(make_workload(4), label="c4 deepseek share, every element", w_layout=1)


@pytest.mark.slow
def test_c2_full_size_every_element():
    """Prefill layer at full size on tiled weights (the bench's
    configuration): every integer stage, the pack, all 32768 expert output
    rows and the whole layer output, element by element."""
    full_parity(make_workload(2), label="c2 prefill, every element", w_layout=1)


@pytest.mark.parametrize("reading", ["zipf_log", "zipf_pmf"])
def test_c3_other_zipf_readings_full_size(reading):
    wl = make_workload(3, offset=(reading, 1.1))
    g, _ = full_parity(wl, label=f"c3 switch, offset {reading}", w_layout=1)
    frac = float((g["slot"] < 0).mean())
    if reading == "zipf_log":
        assert frac > 0.8  # most assignments exceed their expert's capacity
    else:
        assert 0 < frac < 0.1


@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (64, 8)])
def test_sigmoid_selection_bias_small_expert_counts(E, k):
    """Sigmoid + selection-only bias on the route kernels for E <= 64:
    bit-exact under identical logits, and the full layer."""
    wl = make_workload(4, T=700, d=256, h=256, E=E, k=k, R=E // 2 if E > 8 else 8)
    assert wl.b_select is not None and wl.score == "sigmoid"
    r = O.layer(wl, with_ffn=False)
    _say(f"[sigmoid-bias] E={E} k={k}: identical logits")
    _identical_logits(wl, r["route"]["logits32"])
    full_parity(wl, label=f"sigmoid + selection bias, E={E}, k={k}")


@pytest.mark.parametrize("cfg,over", [(2, dict(T=1000, d=512, h=640)),
                                      (4, dict(T=256, d=512, h=256)),
                                      (4, dict(T=300, d=256, h=256, E=16, k=4, R=8))])
def test_weights_without_renormalisation(cfg, over):
    wl = make_workload(cfg, renorm=False, **over)
    g, ref = full_parity(wl, label=f"cfg{cfg} renorm=False {wl.score} E={wl.E}")
    # without renormalisation the weights are the raw scores of the chosen experts
    s = ref["route"]["scores"]
    np.testing.assert_allclose(g["weights"], np.take_along_axis(s, g["ids"].astype(np.int64), 1),
                               rtol=0, atol=5e-5)
