"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the fp64 oracle.

Tolerances (max-abs error normalised by the row max, on the expert outputs
before combine and on the layer output): fp32 1e-4, bf16 2e-2, fp8 weights
6e-2.  Integer outputs must match bit for bit.  Route ids may differ only on
near-ties: the selected set where the oracle's k-th and (k+1)-th scores are
within 1e-6, the order inside it where two consecutive selected scores are;
integer stages are then compared with the oracle replayed on the GPU's ids.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
NEAR_TIE = 1e-6


def tol_of(wl) -> float:
    return TOL["fp8"] if wl.w_dtype == "fp8" else TOL[wl.act_dtype]


def act_to_f64(arr: np.ndarray, act_dtype: str) -> np.ndarray:
    return O.to_f64(arr, act_dtype)


def selection_keys(wl, ref_route: dict) -> np.ndarray:
    """fp64 keys the top-k orders by: the scores, plus the selection bias."""
    p = ref_route["scores"]
    return p if wl.score == "softmax" or wl.b_select is None else p + wl.b_select.astype(np.float64)


def order_gap_of(wl, ref_route: dict) -> np.ndarray:
    """Smallest fp64 gap between consecutive keys of the oracle's selected
    experts (ids are listed by key, so a near-tie there only reorders them)."""
    ids_o = ref_route["ids"]
    if wl.k < 2:
        return np.full(len(ids_o), np.inf)
    chosen = np.take_along_axis(selection_keys(wl, ref_route), ids_o.astype(np.int64), axis=1)
    return np.min(chosen[:, :-1] - chosen[:, 1:], axis=1)


def check_route(wl, gpu: dict, ref_route: dict) -> np.ndarray:
    """ids equal except on near-ties; near-tie ids must still be a valid top-k
    within the tie tolerance.  The selected set may differ only where the
    k-th and (k+1)-th scores are within NEAR_TIE; the order inside the set
    (ids are listed by score) only where two consecutive selected scores
    are.  Returns the mask of exempt tokens."""
    ids_g, ids_o = gpu["ids"], ref_route["ids"]
    gap = ref_route["gap"]
    s = selection_keys(wl, ref_route)
    order_gap = order_gap_of(wl, ref_route)
    set_diff = np.any(np.sort(ids_g, axis=1) != np.sort(ids_o, axis=1), axis=1)
    diff = np.any(ids_g != ids_o, axis=1)
    exempt = np.minimum(gap, order_gap) < NEAR_TIE
    bad = (set_diff & ~(gap < NEAR_TIE)) | (diff & ~exempt)
    assert not bad.any(), (f"{int(bad.sum())} tokens route differently with gap >= {NEAR_TIE}: "
                           f"first {np.nonzero(bad)[0][:8].tolist()}, gaps {gap[bad][:8].tolist()}, "
                           f"order gaps {order_gap[bad][:8].tolist()}")
    # exempt tokens: every chosen expert's score is within the tolerance of
    # the k-th best, and consecutive choices are ordered within it
    for t in np.nonzero(diff)[0]:
        kth = np.sort(s[t])[::-1][wl.k - 1]
        chosen = s[t, ids_g[t]]
        assert np.all(chosen >= kth - NEAR_TIE), f"token {t}: invalid near-tie choice"
        assert np.all(chosen[:-1] >= chosen[1:] - NEAR_TIE), f"token {t}: ids out of order"
        assert len(set(ids_g[t].tolist())) == wl.k
    return exempt


def check_dispatch(wl, gpu: dict, ids: np.ndarray, C: int) -> dict:
    """Integer stages bit-exact against the oracle replayed on ``ids``."""
    ref = O.dispatch(ids, wl.E, wl.R, C)
    for key in ("counts", "kept", "off", "rank_counts", "rank_off", "slot", "src"):
        g = np.asarray(gpu[key])
        r = np.asarray(ref[key])
        assert g.shape == r.shape, (key, g.shape, r.shape)
        if not np.array_equal(g, r):
            idx = np.argwhere(g != r)[:5]
            raise AssertionError(f"dispatch {key} differs at {idx.tolist()}: "
                                 f"gpu {g[tuple(idx.T)].tolist()} oracle {r[tuple(idx.T)].tolist()}")
    return ref


def check_pack(wl, x_send_host: np.ndarray, src: np.ndarray) -> None:
    """Send rows are byte copies of the source tokens' rows."""
    n = src.size
    np.testing.assert_array_equal(x_send_host[:n], wl.x[src.astype(np.int64)])


def check_close(name: str, got: np.ndarray, ref: np.ndarray, tol: float) -> float:
    err = O.rowmax_rel_err(got, ref)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert err <= tol, f"{name}: normalised error {err:.3e} > {tol:.1e}"
    return err


def check_residual_passthrough(wl, y_host: np.ndarray, ids: np.ndarray, slot: np.ndarray) -> int:
    """Tokens with no kept assignment to an executed expert (and no shared
    expert) leave bit-identical to x."""
    if wl.shared is not None:
        return 0
    use = (slot >= 0) & (ids >= wl.e_begin) & (ids < wl.e_end)
    none = ~use.any(axis=1)
    if none.any():
        np.testing.assert_array_equal(y_host[none], wl.x[none])
    return int(none.sum())
