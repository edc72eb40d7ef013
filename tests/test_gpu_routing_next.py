"""GPU parity for the two routing extensions: group-limited top-k and the
bias-balancing update, both against the fp64 oracle through the C ABI.

Group-limited selection and the bias update are integer decisions on fp32
keys, so in the identical-logits mode (both sides given the same fp32 logits)
ids, dispatch arrays and bias vectors must match bit for bit.  With computed
logits, tokens whose group or expert score gap is below the near-tie bound
may differ and are checked for validity instead.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import make_workload
from tests import _parity as P

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


def _grouped_identical(wl, L, ng, tg):
    from expert_token_routing_gemm_amd import MoELayer
    _say(f"[grouped] cfg{wl.cfg} T={wl.T} E={wl.E} k={wl.k} score={wl.score} ng={ng} tg={tg}")
    C = O.capacity(wl.T, wl.k, wl.E, wl.cf)
    layer = MoELayer(wl, capacity=C, logits_input=L, n_groups=ng, topk_groups=tg)
    layer.route()
    layer.dispatch()
    g = layer.results()
    key = O.group_limit_keys(O.selection_keys32(L, wl.score, wl.b_select), ng, tg)
    ids = O.topk_select(key, wl.k)
    np.testing.assert_array_equal(g["ids"], ids)
    # every token's experts come from at most tg groups
    assert max(len(set((row // (wl.E // ng)).tolist())) for row in g["ids"]) <= tg
    P.check_dispatch(wl, g, ids, C)
    return g


# (cfg, overrides, n_groups, topk_groups): group sizes 4 and 32 (inside a
# wave), 64 and 128 (whole wave slots); softmax and sigmoid scoring
GROUPED = [
    (4, dict(T=512, d=256, h=256), 8, 4),
    (4, dict(T=512, d=256, h=256), 4, 2),
    (4, dict(T=300, d=256, h=256), 2, 1),
    (4, dict(T=257, d=256, h=256), 64, 3),
    (2, dict(T=1024, d=256, h=256), 4, 2),
    (0, dict(), 2, 1),
    (3, dict(T=2048, d=256, h=256), 8, 1),
]


@pytest.mark.parametrize("cfg,over,ng,tg", GROUPED)
def test_grouped_identical_logits_bit_exact(cfg, over, ng, tg):
    wl = make_workload(cfg, **over)
    if wl.k > tg * (wl.E // ng):
        pytest.skip("k exceeds the experts of the kept groups")
    r = O.layer(wl, with_ffn=False)
    _grouped_identical(wl, r["route"]["logits32"], ng, tg)


def test_grouped_exact_ties():
    """Exact ties between group scores go to the lower group index; within
    the kept groups exact key ties go to the lower expert index."""
    wl = make_workload(4, T=256, d=256, h=256)
    rng = np.random.default_rng(7)
    L = np.round(rng.standard_normal((wl.T, wl.E)) * 2).astype(np.float32) / 2
    _grouped_identical(wl, L, 8, 4)
    # every group and every expert tied: zero selection bias, constant logits
    wl0 = dataclasses.replace(wl, b_select=np.zeros_like(wl.b_select))
    L[:, :] = np.float32(0.5)
    g = _grouped_identical(wl0, L, 8, 4)
    np.testing.assert_array_equal(g["ids"], np.tile(np.arange(wl.k, dtype=np.int32), (wl.T, 1)))


def test_grouped_all_groups_kept_is_plain_topk():
    wl = make_workload(4, T=128, d=256, h=256)
    r = O.layer(wl, with_ffn=False)
    L = r["route"]["logits32"]
    g = _grouped_identical(wl, L, 8, 8)
    np.testing.assert_array_equal(g["ids"], O.topk_select(O.selection_keys32(L, wl.score,
                                                                             wl.b_select), wl.k))


@pytest.mark.parametrize("ng,tg", [(8, 4), (4, 1)])
def test_grouped_full_layer(ng, tg):
    """Computed logits through the whole layer with group-limited routing."""
    from expert_token_routing_gemm_amd import MoELayer, to_host
    wl = make_workload(4, T=384, d=256, h=256)
    _say(f"[grouped layer] T={wl.T} E={wl.E} ng={ng} tg={tg}")
    C = O.capacity(wl.T, wl.k, wl.E, wl.cf)
    layer = MoELayer(wl, capacity=C, n_groups=ng, topk_groups=tg)
    layer.forward()
    g = layer.results()
    ref = O.layer(wl, n_groups=ng, topk_groups=tg)
    exempt = np.minimum(ref["route"]["gap"], P.order_gap_of(wl, ref["route"])) < P.NEAR_TIE
    diff = np.any(g["ids"] != ref["route"]["ids"], axis=1)
    assert not (diff & ~exempt).any()
    assert max(len(set((row // (wl.E // ng)).tolist())) for row in g["ids"]) <= tg
    if diff.any():
        ref = O.layer(wl, ids_override=g["ids"], n_groups=ng, topk_groups=tg)
    P.check_dispatch(wl, g, g["ids"], C)
    np.testing.assert_allclose(g["weights"], ref["route"]["weights"], rtol=0, atol=5e-5)
    y = to_host(layer.y)
    e_y = P.check_close("y", P.act_to_f64(y, wl.act_dtype), ref["y"], P.tol_of(wl))
    _say(f"[grouped layer] ok: y err {e_y:.2e}, near-tie tokens {int(diff.sum())}")


def test_grouped_full_layer_valu_router():
    """Group-limited routing on an 8-expert layer: the logits come from the
    VALU router kernel, then the grouped top-k."""
    from expert_token_routing_gemm_amd import MoELayer, to_host
    wl = make_workload(2, T=300, d=256, h=256)
    ng, tg = 4, 2
    _say(f"[grouped layer valu] T={wl.T} E={wl.E} ng={ng} tg={tg}")
    C = O.capacity(wl.T, wl.k, wl.E, wl.cf)
    layer = MoELayer(wl, capacity=C, n_groups=ng, topk_groups=tg)
    layer.forward()
    g = layer.results()
    ref = O.layer(wl, n_groups=ng, topk_groups=tg)
    exempt = np.minimum(ref["route"]["gap"], P.order_gap_of(wl, ref["route"])) < P.NEAR_TIE
    diff = np.any(g["ids"] != ref["route"]["ids"], axis=1)
    assert not (diff & ~exempt).any()
    assert max(len(set((row // (wl.E // ng)).tolist())) for row in g["ids"]) <= tg
    if diff.any():
        ref = O.layer(wl, ids_override=g["ids"], n_groups=ng, topk_groups=tg)
    P.check_dispatch(wl, g, g["ids"], C)
    np.testing.assert_allclose(g["weights"], ref["route"]["weights"], rtol=0, atol=5e-5)
    y = to_host(layer.y)
    e_y = P.check_close("y", P.act_to_f64(y, wl.act_dtype), ref["y"], P.tol_of(wl))
    _say(f"[grouped layer valu] ok: y err {e_y:.2e}")


def test_grouped_rejects_bad_arguments():
    from expert_token_routing_gemm_amd import MoELayer
    wl = make_workload(4, T=64, d=256, h=256)
    for ng, tg in [(3, 1), (128, 4), (8, 0), (64, 1)]:  # 256/3, >64 groups, no group, k > 4
        layer = MoELayer(wl, n_groups=ng, topk_groups=tg)
        with pytest.raises(RuntimeError):
            layer.route()


# ------------------------------------------------------------------ bias update


def test_bias_update_single_step_exact():
    from expert_token_routing_gemm_amd import moe_bias_update, to_device, to_host
    rng = np.random.default_rng(3)
    for E, T, k in [(256, 4096, 8), (8, 100, 2), (64, 0, 1), (16, 7, 3)]:
        counts = rng.integers(0, max(1, 3 * T * k // E) + 1, E).astype(np.int32)
        counts[0] = T * k // E if (T * k) % E == 0 else counts[0]  # an exactly-even expert
        b = rng.standard_normal(E).astype(np.float32)
        db, dc = to_device(b, "cuda"), to_device(counts, "cuda")
        moe_bias_update(dc, db, T, k, 1e-3)
        np.testing.assert_array_equal(to_host(db), O.bias_update(b, counts, T, k, 1e-3))


def test_bias_balancing_loop_bit_exact():
    """Route -> dispatch -> bias update, repeated on fixed skewed logits: every
    step's ids and the bias vector follow the oracle bit for bit, and the
    load imbalance falls."""
    from expert_token_routing_gemm_amd import MoELayer, to_host
    wl = make_workload(4, T=1024, d=256, h=256)
    rng = np.random.default_rng(11)
    L = (rng.standard_normal((wl.T, wl.E)) + np.linspace(-1.5, 1.5, wl.E)).astype(np.float32)
    C = O.capacity(wl.T, wl.k, wl.E, 0)
    layer = MoELayer(wl, capacity=C, logits_input=L)
    b = np.asarray(wl.b_select, np.float32).copy()
    gamma = 1e-2
    imb = []
    for step in range(40):
        layer.route()
        layer.dispatch()
        layer.update_bias(gamma)
        ids = O.topk_select(O.selection_keys32(L, wl.score, b), wl.k)
        counts = np.bincount(ids.ravel(), minlength=wl.E)
        g_ids = to_host(layer.ids)
        assert np.array_equal(g_ids, ids), f"step {step}: ids differ"
        b = O.bias_update(b, counts, wl.T, wl.k, gamma)
        np.testing.assert_array_equal(to_host(layer.b_select), b, err_msg=f"step {step}")
        imb.append(counts.max() / (wl.T * wl.k / wl.E))
    _say(f"[bias] max/mean load {imb[0]:.2f} -> {imb[-1]:.2f}")
    assert imb[-1] < 0.25 * imb[0]


# ------------------------------------------------------------------ auxiliary loss


@pytest.mark.parametrize("cfg,over", [(4, dict(T=512, d=256, h=256)), (2, dict(T=2048, d=256, h=256)),
                                      (3, dict(T=37, d=256, h=256)), (4, dict(T=8192, d=256, h=256))])
def test_aux_loss_matches_oracle(cfg, over):
    """The loss value and the mean probabilities from the GPU's own fp32
    logits and counts, against the fp64 oracle on the same inputs."""
    from expert_token_routing_gemm_amd import MoELayer, to_host
    wl = make_workload(cfg, **over)
    _say(f"[aux] cfg{cfg} T={wl.T} E={wl.E} score={wl.score}")
    layer = MoELayer(wl)
    layer.route()
    layer.dispatch()
    pm, loss = layer.aux_loss(0.01)
    L32 = to_host(layer.logits)
    counts = to_host(layer.counts)
    P, ref = O.aux_balance_loss(L32.astype(np.float64), counts, wl.k, wl.score, 0.01)
    np.testing.assert_allclose(to_host(pm), P, rtol=2e-5, atol=1e-8)
    np.testing.assert_allclose(to_host(loss)[0], ref, rtol=2e-5)
    pm2, loss2 = layer.aux_loss(0.01)  # deterministic
    np.testing.assert_array_equal(to_host(pm2), to_host(pm))
    np.testing.assert_array_equal(to_host(loss2), to_host(loss))


def test_aux_loss_empty_batch():
    from expert_token_routing_gemm_amd import moe_aux_loss, to_host
    logits = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    counts = torch.zeros((8,), dtype=torch.int32, device="cuda")
    pm, loss = moe_aux_loss(logits, counts, 2, 0, 0.01)
    assert (to_host(pm) == 0).all() and to_host(loss)[0] == 0
