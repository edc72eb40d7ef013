"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: the figures
the pages print, closed forms, brute force on tiny inputs, library routines
(torch, scipy) and invariants.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy.special import softmax as sp_softmax

from oracle import oracle as O
from synth import make_workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- P1 / P2


@pytest.fixture(scope="module")
def c0():
    return make_workload(0)


@pytest.fixture(scope="module")
def c0_route(c0):
    return O.layer(c0, with_ffn=False)


def test_snippet_loads_match_printed_figures(c0, c0_route):
    """Ultralytics "How Tokens Move Between GPUs": the listing prints expert
    loads spanning 948..1087 (even share 1024) and rank loads 1968..2139 of
    8192 assignments."""
    g = _gold("ultralytics_snippet_loads.json")
    counts = c0_route["dispatch"]["counts"]
    ranks = counts.reshape(g["R"], -1).sum(axis=1)
    assert counts.sum() == g["total_assignments"] == g["T"] * g["k"]
    assert counts.min() == g["expert_load_min"]
    assert counts.max() == g["expert_load_max"]
    assert g["total_assignments"] // g["E"] == g["even_share"]
    assert ranks.min() == g["rank_load_min"]
    assert ranks.max() == g["rank_load_max"]
    # per-rank counts of the dispatch equal the per-rank sums
    np.testing.assert_array_equal(c0_route["dispatch"]["rank_counts"], ranks)


def test_snippet_loads_match_torch_listing(c0, c0_route):
    """The listing itself, re-run with torch's own top-k and bincount (not
    used by the oracle), gives the same per-expert and per-rank vectors."""
    x = torch.from_numpy(c0.x)
    w = torch.from_numpy(c0.w_router)
    b = torch.from_numpy(c0.b_router)
    _, experts = torch.nn.functional.linear(x, w, b).topk(2, dim=-1)
    ref_e = torch.bincount(experts.flatten(), minlength=8).numpy()
    ref_r = torch.bincount((experts // 2).flatten(), minlength=4).numpy()
    np.testing.assert_array_equal(c0_route["dispatch"]["counts"], ref_e)
    np.testing.assert_array_equal(c0_route["dispatch"]["rank_counts"], ref_r)
    # the selected sets agree too (no near-ties at this seed)
    ids = c0_route["route"]["ids"]
    assert c0_route["route"]["gap"].min() > 1e-6
    np.testing.assert_array_equal(np.sort(ids, axis=1), np.sort(experts.numpy(), axis=1))


# ---------------------------------------------------------------- P3 capacity


def test_capacity_closed_form():
    # 1.25 x even share (Ultralytics "Load Balancing and Capacity")
    assert O.capacity(4096, 2, 8, 1.25) == 1280
    assert O.capacity(32768, 1, 64, 1.25) == 640
    assert O.capacity(150, 1, 1, 100 / 150) == 100
    assert O.capacity(10, 3, 7, 1.0) == math.ceil(30 / 7)
    assert O.capacity(100, 2, 8, None) == O.INT32_MAX
    assert O.capacity(100, 2, 8, 0.0) == O.INT32_MAX
    # ceil of an exact integer stays put
    assert O.capacity(64, 2, 8, 1.0) == 16


def test_forced_drop_count_c0(c0, c0_route):
    """cf = 1.0 gives C = even share = 1024; with the printed max load 1087
    at least 63 assignments of the busiest expert are dropped, and the total
    dropped equals sum(max(count - C, 0))."""
    ids = c0_route["route"]["ids"]
    d = O.dispatch(ids, 8, 4, O.capacity(4096, 2, 8, 1.0))
    counts = d["counts"]
    assert (counts.max() - 1024) == 1087 - 1024
    dropped = int((d["slot"] < 0).sum())
    assert dropped == int(np.maximum(counts - 1024, 0).sum()) == 154
    assert int(d["kept"].sum()) + dropped == 4096 * 2


# ---------------------------------------------------------------- P4 drop example


def _workload_like(T, d, E, k, h, act="relu", R=1, score="softmax", renorm=True,
                   seed=0, cf=None, shared=False):
    rng = np.random.default_rng(seed)

    class W:
        pass

    w = W()
    w.T, w.d, w.E, w.k, w.R, w.h = T, d, E, k, R, h
    w.act, w.act_dtype, w.w_dtype = act, "f32", "f32"
    w.score, w.renorm, w.cf = score, renorm, cf
    w.e_begin, w.e_end = 0, E
    w.x = rng.standard_normal((T, d)).astype(np.float32)
    w.w_router = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    w.b_router = None
    w.b_select = None
    w.w1 = (rng.standard_normal((E, h, d)) / math.sqrt(d)).astype(np.float32)
    w.w3 = (rng.standard_normal((E, h, d)) / math.sqrt(d)).astype(np.float32) if act == "swiglu" else None
    w.w2 = (rng.standard_normal((E, d, h)) / math.sqrt(h)).astype(np.float32)
    w.s1 = w.s2 = w.s3 = None
    w.shared = None
    if shared:
        w.shared = dict(w1=(rng.standard_normal((h, d)) / math.sqrt(d)).astype(np.float32),
                        w3=(rng.standard_normal((h, d)) / math.sqrt(d)).astype(np.float32) if act == "swiglu" else None,
                        w2=(rng.standard_normal((d, h)) / math.sqrt(h)).astype(np.float32))
    return w


def test_capacity_example_150_to_100():
    """ai360xpert "Load Balancing and Dropped Tokens": 150 tokens routed to a
    100-slot expert; the extra 50 are dropped and pass on unchanged."""
    g = _gold("ai360xpert_capacity_example.json")
    w = _workload_like(T=g["routed"], d=16, E=2, k=1, h=8)
    w.w_router[:] = 0.0
    w.b_router = np.array([1.0, 0.0], np.float32)  # every token prefers expert 0
    res = O.layer(w, cf=g["capacity"] / g["routed"] * 2)  # C = ceil(cf*150/2) = 100
    assert res["capacity"] == g["capacity"]
    slot = res["dispatch"]["slot"][:, 0]
    np.testing.assert_array_equal(slot[:100], np.arange(100))
    assert (slot[100:] == -1).all() and int((slot < 0).sum()) == g["dropped"]
    x64 = w.x.astype(np.float64)
    # dropped tokens leave unchanged; kept tokens do not
    np.testing.assert_array_equal(res["y"][100:], x64[100:])
    assert not np.array_equal(res["y"][:100], x64[:100])
    np.testing.assert_array_equal(res["dispatch"]["src"], np.arange(100))


# ---------------------------------------------------------------- P5 invariants


def _check_dispatch_invariants(ids, d, E, R, C):
    T, k = ids.shape
    slot, src, off, kept, counts = d["slot"], d["src"], d["off"], d["kept"], d["counts"]
    assert counts.sum() == T * k
    np.testing.assert_array_equal(kept, np.minimum(counts, C))
    assert off[0] == 0 and off[-1] == kept.sum() == src.size
    np.testing.assert_array_equal(np.diff(off), kept)
    dropped = int((slot < 0).sum())
    assert kept.sum() + dropped == T * k
    # src is a bijection onto kept assignments, consistent with slot
    s = slot[slot >= 0]
    assert np.array_equal(np.sort(s), np.arange(src.size))
    tt = np.nonzero(slot >= 0)[0]
    np.testing.assert_array_equal(src[slot[slot >= 0]], tt)
    # each row lies in its expert's segment; token order within a segment
    for e in range(E):
        seg = src[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        rows = slot[ids == e]
        rows = rows[rows >= 0]
        assert np.all((rows >= off[e]) & (rows < off[e + 1]))
    per = E // R
    np.testing.assert_array_equal(d["rank_counts"], kept.reshape(R, per).sum(axis=1))
    np.testing.assert_array_equal(d["rank_off"], np.append(off[::per][:R], off[-1]))
    # dropped = the assignments beyond the first C of each expert, in token order
    for e in range(E):
        tj = np.argwhere(ids == e)  # row-major = token-major order
        keep = slot[tj[:, 0], tj[:, 1]] >= 0
        assert keep[:C].all() and not keep[C:].any()


@pytest.mark.parametrize("cf", [1.25, 1.0, 0.5])
def test_dispatch_invariants_c0(c0_route, cf):
    ids = c0_route["route"]["ids"]
    C = O.capacity(4096, 2, 8, cf)
    _check_dispatch_invariants(ids, O.dispatch(ids, 8, 4, C), 8, 4, C)


def test_dispatch_invariants_switch_small():
    wl = make_workload(3, T=2048)
    res = O.layer(wl, with_ffn=False)
    ids = res["route"]["ids"]
    d = res["dispatch"]
    _check_dispatch_invariants(ids, d, 64, 16, res["capacity"])
    # heavy skew: the Zipf offset makes expert 0 the busiest and forces drops
    assert d["counts"].argmax() == 0
    assert (d["slot"] < 0).sum() > 0


# ---------------------------------------------------------------- P6 bias


@pytest.fixture(scope="module")
def c4_small():
    return make_workload(4, T=96, d=256, h=256)


def test_bias_changes_selection_only(c4_small):
    wl = c4_small
    x64 = O.to_f64(wl.x, "bf16")
    wr64 = O.to_f64(wl.w_router, "bf16")
    base = O.route(x64, wr64, None, wl.b_select, wl.k, "sigmoid", True)
    # weights follow the unbiased sigmoid scores of the selected experts
    s = O.sigmoid(base["logits"])
    sel = np.take_along_axis(s, base["ids"].astype(np.int64), axis=1)
    np.testing.assert_allclose(base["weights"], sel / sel.sum(1, keepdims=True), rtol=1e-15)
    # the same ids under a different bias give the same weights
    other = O.route(x64, wr64, None, wl.b_select * -3.0, wl.k, "sigmoid", True,
                    ids_override=base["ids"])
    np.testing.assert_array_equal(other["weights"], base["weights"])
    # a constant shift of the bias keeps the selection (away from near-ties)
    shifted = O.route(x64, wr64, None, wl.b_select + np.float32(0.25), wl.k, "sigmoid", True)
    ok = base["gap"] > 1e-5
    np.testing.assert_array_equal(shifted["ids"][ok], base["ids"][ok])
    # a huge bias on one expert puts it in every token's set, first
    big = wl.b_select.copy()
    big[37] = 100.0
    forced = O.route(x64, wr64, None, big, wl.k, "sigmoid", True)
    assert (forced["ids"][:, 0] == 37).all()
    w37 = forced["weights"][:, 0]
    sel = np.take_along_axis(s, forced["ids"].astype(np.int64), axis=1)
    np.testing.assert_allclose(w37, sel[:, 0] / sel.sum(1), rtol=1e-15)
    # without the bias expert 37 is not always picked
    assert not (base["ids"] == 37).any(axis=1).all()


# ---------------------------------------------------------------- P7 brute force


def _brute_topk(key, k):
    """All k-subsets: the chosen set beats every outsider in (key desc, idx
    asc); its order is by how many members each member loses to."""
    T, E = key.shape
    out = np.zeros((T, k), np.int64)
    beats = lambda a, b, row: (row[a] > row[b]) or (row[a] == row[b] and a < b)
    for t in range(T):
        row = key[t]
        found = None
        for S in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in S]
            if all(beats(a, b, row) for a in S for b in rest):
                found = S
                break
        assert found is not None
        order = sorted(found, key=lambda a: sum(beats(b, a, row) for b in found))
        out[t] = order
    return out


def _brute_dispatch(ids, E, C):
    T, k = ids.shape
    lists = [[(t, j) for t in range(T) for j in range(k) if ids[t, j] == e] for e in range(E)]
    kept = [min(len(l), C) for l in lists]
    off = [0]
    for e in range(E):
        off.append(off[-1] + kept[e])
    slot = -np.ones((T, k), np.int64)
    for e in range(E):
        for p, (t, j) in enumerate(lists[e][:C]):
            slot[t, j] = off[e] + p
    return np.array([len(l) for l in lists]), np.array(off), slot


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 16), E=st.sampled_from([2, 4, 6, 8]), k=st.integers(1, 4),
       C=st.integers(1, 5), seed=st.integers(0, 10_000), ties=st.booleans())
def test_bruteforce_route_dispatch(T, E, k, C, seed, ties):
    k = min(k, E)
    rng = np.random.default_rng(seed)
    key = rng.standard_normal((T, E)).astype(np.float32)
    if ties:  # coarse values force exact ties
        key = np.round(key * 2).astype(np.float32)
    ids = O.topk_select(key, k)
    np.testing.assert_array_equal(ids, _brute_topk(key, k))
    d = O.dispatch(ids, E, 1 if E % 2 else 2, C)
    counts, off, slot = _brute_dispatch(ids, E, C)
    np.testing.assert_array_equal(d["counts"], counts)
    np.testing.assert_array_equal(d["off"], off)
    np.testing.assert_array_equal(d["slot"], slot)


def test_bruteforce_topk_e256_full_sort():
    rng = np.random.default_rng(7)
    key = rng.standard_normal((12, 256)).astype(np.float32)
    key[:, 200] = key[:, 5]  # exact ties across far-apart experts
    ids = O.topk_select(key, 8)
    for t in range(12):
        order = sorted(range(256), key=lambda e: (-float(key[t, e]), e))
        np.testing.assert_array_equal(ids[t], order[:8])


def test_tie_goes_to_lower_index():
    key = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], np.float32)
    np.testing.assert_array_equal(O.topk_select(key, 2), [[1, 2]])
    np.testing.assert_array_equal(O.topk_select(key, 4), [[1, 2, 4, 3]])


# ---------------------------------------------------------------- P8 reductions


def test_single_expert_is_dense_ffn():
    """E = 1, k = 1, no capacity limit, renormalised: y = x + FFN(x)."""
    for act in ("relu", "gelu", "swiglu"):
        w = _workload_like(T=20, d=32, E=1, k=1, h=24, act=act, seed=3)
        res = O.layer(w)
        x = torch.from_numpy(w.x).double()
        w1 = torch.from_numpy(w.w1[0]).double()
        w2 = torch.from_numpy(w.w2[0]).double()
        z1 = x @ w1.T
        if act == "relu":
            a = torch.relu(z1)
        elif act == "gelu":
            a = torch.nn.functional.gelu(z1)  # exact erf form
        else:
            a = torch.nn.functional.silu(z1) * (x @ torch.from_numpy(w.w3[0]).double().T)
        ref = (x + a @ w2.T).numpy()
        np.testing.assert_allclose(res["y"], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(res["route"]["weights"], np.ones((20, 1)))


def test_k_equals_E_weights_are_full_softmax():
    w = _workload_like(T=16, d=12, E=5, k=5, h=4, seed=9)
    res = O.layer(w, with_ffn=False)
    L = res["route"]["logits"]
    ids = res["route"]["ids"]
    full = sp_softmax(L, axis=1)
    np.testing.assert_allclose(res["route"]["weights"],
                               np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-13)
    np.testing.assert_allclose(res["route"]["scores"], full, rtol=1e-13)


def test_top1_without_renorm_uses_raw_probability():
    w = _workload_like(T=16, d=12, E=6, k=1, h=4, seed=11, renorm=False)
    res = O.layer(w, with_ffn=False)
    full = sp_softmax(res["route"]["logits"], axis=1)
    np.testing.assert_allclose(res["route"]["weights"][:, 0], full.max(axis=1), rtol=1e-13)
    assert res["route"]["weights"].max() < 1.0


@pytest.mark.parametrize("act,k,cf,shared", [("relu", 2, 0.6, False), ("gelu", 1, 1.0, False),
                                             ("swiglu", 3, None, True), ("swiglu", 2, 0.5, True)])
def test_permuted_layer_equals_per_token_formulation(act, k, cf, shared):
    w = _workload_like(T=40, d=16, E=6, k=k, h=12, act=act, R=3, seed=5, cf=cf, shared=shared)
    w.e_begin, w.e_end = 1, 5  # only part of the experts execute here
    res = O.layer(w)
    d = res["dispatch"]
    y2 = O.token_outputs(w, np.arange(40), res["route"]["ids"], res["route"]["weights"], d["slot"])
    np.testing.assert_allclose(res["y"], y2, rtol=1e-12, atol=1e-12)


def test_ffn_closed_form_permutation_weights():
    """Permutation / diagonal weights give a closed form; a transposed operand
    or swapped w1/w3 would fail it."""
    d, h = 6, 6
    perm = np.array([2, 0, 5, 1, 3, 4])
    P = np.eye(h)[perm]          # (P x)[i] = x[perm[i]]
    D = np.diag(np.arange(1.0, d + 1))
    x = np.random.default_rng(1).standard_normal((4, d))
    out = O.ffn(x, "relu", P, None, D)
    np.testing.assert_allclose(out, np.maximum(x[:, perm], 0) * np.arange(1.0, d + 1))
    out = O.ffn(x, "swiglu", P, np.eye(h), D)
    z = x[:, perm]
    np.testing.assert_allclose(out, (z / (1 + np.exp(-z))) * x * np.arange(1.0, d + 1))


def test_activations_against_torch():
    z = np.linspace(-8, 8, 1001)
    t = torch.from_numpy(z)
    np.testing.assert_allclose(O.activation(z, "gelu"), torch.nn.functional.gelu(t).numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(O.activation(z, "relu"), torch.relu(t).numpy())
    np.testing.assert_allclose(O.activation(z, "swiglu", np.ones_like(z)),
                               torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-16)


def test_combine_closed_form_identity_experts():
    """Identity experts (relu on positive inputs, W = I): y = x (1 + sum of
    kept weights), and a token with every assignment dropped is x exactly."""
    w = _workload_like(T=30, d=8, E=4, k=2, h=8, act="relu", R=2, seed=2, cf=0.5)
    w.x = np.abs(w.x) + np.float32(0.5)
    w.w1[:] = np.eye(8, dtype=np.float32)
    w.w2[:] = np.eye(8, dtype=np.float32)
    res = O.layer(w)
    slot = res["dispatch"]["slot"]
    kw = np.where(slot >= 0, res["route"]["weights"], 0.0).sum(1)
    x64 = w.x.astype(np.float64)
    np.testing.assert_allclose(res["y"], x64 * (1 + kw)[:, None], rtol=1e-14)
    gone = (slot < 0).all(axis=1)
    assert gone.any()
    np.testing.assert_array_equal(res["y"][gone], x64[gone])


def test_executed_experts_use_their_own_weights_closed_form():
    """A rank executes experts [e_begin, e_end) and holds only their weights,
    local index e - e_begin.  With W1 = I and W2 = (e + 1) I for expert e
    (its global index baked into the weights), positive x and relu:
    y = x (1 + sum over kept assignments to executed experts of w (e + 1)),
    the sampled-check helpers give (e + 1) x for expert e's rows and 7 x for
    a shared expert with W2 = 7 I.  Catches: weights looked up by global
    instead of local index, work done for experts of other ranks, a shared
    expert left out or counted twice."""
    d = 8
    w = _workload_like(T=40, d=d, E=6, k=2, h=d, act="relu", R=3, seed=6, cf=None, shared=True)
    w.e_begin, w.e_end = 2, 4
    w.x = np.abs(w.x) + np.float32(0.25)
    n = w.e_end - w.e_begin
    w.w1 = np.stack([np.eye(d, dtype=np.float32)] * n)
    w.w2 = np.stack([np.float32(e + 1) * np.eye(d, dtype=np.float32)
                     for e in range(w.e_begin, w.e_end)])
    w.shared = dict(w1=np.eye(d, dtype=np.float32), w3=None,
                    w2=np.float32(7.0) * np.eye(d, dtype=np.float32))
    res = O.layer(w)
    ids, wts = res["route"]["ids"], res["route"]["weights"]
    slot = res["dispatch"]["slot"]
    mine = (slot >= 0) & (ids >= w.e_begin) & (ids < w.e_end)
    gain = np.where(mine, wts * (ids + 1), 0.0).sum(1)
    x64 = w.x.astype(np.float64)
    assert mine.any() and (~mine).any()
    np.testing.assert_allclose(res["y"], x64 * (1 + 7 + gain)[:, None], rtol=1e-13)
    for e in range(w.e_begin, w.e_end):
        np.testing.assert_allclose(O.expert_rows(w, x64[:5], e), (e + 1) * x64[:5], rtol=1e-14)
    np.testing.assert_allclose(O.shared_rows(w, x64[:5]), 7 * x64[:5], rtol=1e-14)
    np.testing.assert_allclose(O.token_outputs(w, np.arange(40), ids, wts, slot), res["y"],
                               rtol=1e-13)


# ---------------------------------------------------------------- P9 formats


def test_e4m3fn_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 2 ** 16, 4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = O.decode_bf16(bits)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.isnan(ours), nan)


def test_block_dequant_layout():
    q = np.zeros((256, 384), np.uint8)
    q[:, :] = 0x38  # 1.0
    s = np.arange(2 * 3, dtype=np.float32).reshape(2, 3) + 1
    w = O.dequant_blocks(q, s)
    assert w[0, 0] == 1 and w[127, 127] == 1 and w[0, 128] == 2 and w[128, 0] == 4 and w[255, 383] == 6


def test_softmax_selection_on_fp32_logits_matches_fp64_order(c0_route):
    r = c0_route["route"]
    L = r["logits"]
    ids64 = np.argsort(-L, axis=1, kind="stable")[:, :2]
    ok = r["gap"] > 1e-6
    np.testing.assert_array_equal(r["ids"][ok], ids64[ok])
    np.testing.assert_allclose(r["weights"].sum(1), 1.0, rtol=1e-15)


# ---------------------------------------------------------------- group-limited routing


def _brute_group_topk(key, n_groups, M, k):
    """Enumerate every set of M groups; the chosen set contains the best
    group score, then the next best, ... (score desc, index asc); the experts
    are the k best keys inside the chosen groups."""
    T, E = key.shape
    gs = E // n_groups
    out = np.zeros((T, k), np.int64)
    for t in range(T):
        gscore = [max(key[t, g * gs:(g + 1) * gs]) for g in range(n_groups)]
        best = None
        for S in itertools.combinations(range(n_groups), M):
            rest = [g for g in range(n_groups) if g not in S]
            if all((gscore[a] > gscore[b]) or (gscore[a] == gscore[b] and a < b) for a in S for b in rest):
                best = S
                break
        allowed = [e for e in range(E) if e // gs in best]
        order = sorted(allowed, key=lambda e: (-float(key[t, e]), e))
        out[t] = order[:k]
    return out


@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 12), ng=st.sampled_from([2, 4, 8]), M=st.integers(1, 4), seed=st.integers(0, 9999),
       ties=st.booleans())
def test_group_limited_topk_bruteforce(T, ng, M, seed, ties):
    E = 16
    M = min(M, ng)
    gs = E // ng
    k = min(3, M * gs)
    rng = np.random.default_rng(seed)
    key = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        key = np.round(key * 2).astype(np.float32)
    ids = O.topk_select(O.group_limit_keys(key, ng, M), k)
    np.testing.assert_array_equal(ids, _brute_group_topk(key, ng, M, k))
    # the chosen experts span at most M groups
    assert all(len(set((ids[t] // gs).tolist())) <= M for t in range(T))


def test_group_limit_reduces_to_plain_topk():
    rng = np.random.default_rng(3)
    key = rng.standard_normal((50, 256)).astype(np.float32)
    np.testing.assert_array_equal(O.topk_select(O.group_limit_keys(key, 8, 8), 8), O.topk_select(key, 8))
    one = O.topk_select(O.group_limit_keys(key, 8, 1), 8)
    best_group = key.reshape(50, 8, 32).max(axis=2).argmax(axis=1)
    np.testing.assert_array_equal(one // 32, np.repeat(best_group[:, None], 8, axis=1))


def test_group_limited_route_weights_and_gap(c4_small):
    wl = c4_small
    x64 = O.to_f64(wl.x, "bf16")
    wr64 = O.to_f64(wl.w_router, "bf16")
    r = O.route(x64, wr64, None, wl.b_select, wl.k, "sigmoid", True, n_groups=8, topk_groups=4)
    assert all(len(set((r["ids"][t] // 32).tolist())) <= 4 for t in range(wl.T))
    np.testing.assert_allclose(r["weights"].sum(axis=1), 1.0, rtol=1e-14)
    # the near-tie gap never exceeds the group-score gap
    s64 = O.sigmoid(r["logits"]) + wl.b_select.astype(np.float64)
    assert np.all(r["gap"] <= O.group_gap(s64, 8, 4))


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def test_group_gap_hand_values():
    """group_gap = (topk_groups-th best group score) - (next one), a group's
    score being its largest expert score.  Catches: a group scored by its sum
    or mean instead of its max, the wrong pair of ranks, a sign error."""
    s = np.array([[0.10, 0.90, 0.50, 0.60],     # groups {0,1} {2,3}: maxes 0.90, 0.60
                  [0.20, 0.30, 0.35, 0.10]])    # maxes 0.30, 0.35 -> sorted 0.35, 0.30
    np.testing.assert_allclose(O.group_gap(s, 2, 1), [0.30, 0.05], rtol=0, atol=1e-15)
    s3 = np.array([[0.10, 0.70, 0.65, 0.20, 0.30, 0.40]])  # maxes 0.70, 0.65, 0.40
    np.testing.assert_allclose(O.group_gap(s3, 3, 2), [0.25], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.group_gap(s3, 3, 1), [0.05], rtol=0, atol=1e-15)
    # every group kept: no group boundary, infinite gap
    assert np.isinf(O.group_gap(s3, 3, 3)).all()


def test_group_limited_route_gap_hand_values():
    """route()'s near-tie gap with groups = min(group gap, gap between the
    k-th and (k+1)-th expert inside the kept groups), on sigmoid scores
    computed here with math.exp.  Row 0: the group gap decides; row 1: the
    expert gap inside the kept group decides.  Catches either term dropped."""
    L = np.array([[0.0, 2.0, 1.0, 1.5],
                  [1.0, 1.125, -3.0, -2.0]], np.float32)  # exact in fp32
    r = O.route(None, None, None, None, 1, "sigmoid", True, logits32=L, n_groups=2,
                topk_groups=1)
    g0 = _sig(2.0) - _sig(1.5)          # group maxes sigma(2) vs sigma(1.5)
    e0 = _sig(2.0) - _sig(0.0)          # inside group 0: sigma(2) vs sigma(0)
    g1 = _sig(1.125) - _sig(-2.0)
    e1 = _sig(1.125) - _sig(1.0)
    np.testing.assert_allclose(r["gap"], [min(g0, e0), min(g1, e1)], rtol=0, atol=1e-15)
    assert min(g0, e0) == g0 and min(g1, e1) == e1
    np.testing.assert_array_equal(r["ids"][:, 0], [1, 1])


def test_sigmoid_key_adds_bias_after_sigmoid():
    """The selection key is sigma(L) + b, not sigma(L + b) (the bias is added
    to the router scores: Ultralytics, "Load Balancing and Capacity",
    bias-based balancing bullet).  With L = [0, 3], b = [0.5, 0]:
    sigma(0) + 0.5 = 1.0 beats sigma(3) = 0.9526, so expert 0 is chosen,
    while sigma(L + b) = [0.622, 0.953] would choose expert 1.  The weight
    uses the unbiased score: sigma(0) = 0.5 without renormalisation."""
    L = np.array([[0.0, 3.0]], np.float32)
    b = np.array([0.5, 0.0], np.float32)
    key = O.selection_keys32(L, "sigmoid", b)
    np.testing.assert_array_equal(key, np.array([[np.float32(0.5) + np.float32(0.5),
                                                  np.float32(_sig(3.0))]], np.float32))
    r = O.route(None, None, None, b, 1, "sigmoid", False, logits32=L)
    assert r["ids"][0, 0] == 0
    np.testing.assert_allclose(r["weights"][0, 0], 0.5, rtol=0, atol=1e-15)
    # the fp64 near-tie gap is taken on sigma + b as well: 1.0 - 0.9526
    np.testing.assert_allclose(r["gap"][0], 1.0 - _sig(3.0), rtol=0, atol=1e-12)
    # the opposite composition would pick expert 1
    assert _sig(0.0 + 0.5) < _sig(3.0)


def test_rowmax_rel_err_hand_values():
    """The tolerance metric: max over rows of (max_i |got - ref|) / (max_i
    |ref|).  Hand values where the plausible variants differ: normalising by
    the global max gives 0.01, averaging over rows 0.055, normalising by
    |got| 0.0909; the stated metric gives 0.1."""
    ref = np.array([[1.0, 0.5], [100.0, 0.0]])
    got = np.array([[1.1, 0.5], [100.0, 1.0]])
    assert O.rowmax_rel_err(got, ref) == pytest.approx(0.1, abs=1e-15)
    # sign of the error does not matter
    assert O.rowmax_rel_err(2 * ref - got, ref) == pytest.approx(0.1, abs=1e-15)
    # a negative reference entry sets the row's scale through its magnitude
    assert O.rowmax_rel_err(np.array([[-3.0, 0.3]]), np.array([[-4.0, 0.0]])) == \
        pytest.approx(0.25, abs=1e-15)
    # an all-zero reference row falls back to the absolute error
    assert O.rowmax_rel_err(np.array([[0.5, 0.0]]), np.zeros((1, 2))) == 0.5
    # identical arrays and empty arrays give zero
    assert O.rowmax_rel_err(ref, ref) == 0.0
    assert O.rowmax_rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


# ---------------------------------------------------------------- bias balancing


def test_bias_update_rule_hand_example():
    b = np.array([0.5, 0.0, -0.25], np.float32)
    # T*k = 8 over E = 3: mean 8/3; loads 5 (over), 1 (under), 2 (under)
    out = O.bias_update(b, [5, 1, 2], T=4, k=2, gamma=0.125)
    np.testing.assert_array_equal(out, np.array([0.375, 0.125, -0.125], np.float32))
    # an exactly average load keeps its bias (compared in integers, not floats)
    np.testing.assert_array_equal(O.bias_update(b, [2, 2, 2], T=3, k=2, gamma=0.5), b)


def test_bias_update_balances_skewed_routing():
    """Iterating route -> histogram -> update on skewed synthetic logits
    shrinks the busiest expert's load (the rule's purpose)."""
    rng = np.random.default_rng(0)
    T, E, k = 2048, 32, 4
    L = (rng.standard_normal((T, E)) * 0.3 + np.linspace(1.0, -1.0, E)[None, :]).astype(np.float32)
    b = np.zeros(E, np.float32)
    first = None
    for step in range(60):
        ids = O.topk_select(O.selection_keys32(L, "sigmoid", b), k)
        counts = np.bincount(ids.ravel(), minlength=E)
        if first is None:
            first = counts.max() / (T * k / E)
        b = O.bias_update(b, counts, T, k, gamma=0.01)
    last = counts.max() / (T * k / E)
    assert first > 2.0 and last < 0.6 * first


# ---------------------------------------------------------------- auxiliary loss
# Pins of the auxiliary balancing loss (closed forms and invariants, not the
# formula retyped): perfectly even routing with uniform probabilities gives
# exactly alpha; everything on one expert with probability -> 1 gives alpha*E;
# the mean probabilities sum to 1; relabelling experts permutes P and leaves
# the loss unchanged; the loss is linear in alpha.


def test_aux_loss_even_routing_is_alpha():
    T, E, k = 64, 8, 2
    L = np.zeros((T, E))
    counts = np.full(E, T * k // E)
    for score in ("softmax", "sigmoid"):
        P, loss = O.aux_balance_loss(L, counts, k, score, 0.01)
        np.testing.assert_allclose(P, 1.0 / E, rtol=0, atol=1e-15)
        assert abs(loss - 0.01) < 1e-15


def test_aux_loss_collapse_is_alpha_times_E():
    T, E, k = 32, 16, 1
    L = np.full((T, E), -60.0)
    L[:, 3] = 60.0
    counts = np.zeros(E, np.int64)
    counts[3] = T
    P, loss = O.aux_balance_loss(L, counts, k, "softmax", 0.5)
    assert abs(loss - 0.5 * E) < 1e-9
    assert abs(P[3] - 1.0) < 1e-12


def test_aux_loss_invariants():
    rng = np.random.default_rng(4)
    T, E, k = 50, 12, 3
    L = rng.standard_normal((T, E)) * 2
    ids = O.topk_select(L.astype(np.float32), k)
    counts = np.bincount(ids.ravel(), minlength=E)
    perm = rng.permutation(E)
    for score in ("softmax", "sigmoid"):
        P, loss = O.aux_balance_loss(L, counts, k, score, 0.1)
        assert abs(P.sum() - 1.0) < 1e-12
        P2, loss2 = O.aux_balance_loss(L[:, perm], counts[perm], k, score, 0.1)
        np.testing.assert_allclose(P2, P[perm], rtol=1e-13)
        assert abs(loss2 - loss) < 1e-13
        _, loss3 = O.aux_balance_loss(L, counts, k, score, 0.3)
        assert abs(loss3 - 3 * loss) < 1e-13
