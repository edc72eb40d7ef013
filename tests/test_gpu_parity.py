"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes: every workload once at shapes the oracle finishes in seconds that
still span several tiles and ragged row tails, with full element-by-element
comparison; the decode, Switch and tiny workloads also at their full sizes
with full comparison; the prefill and DeepSeek-V3-share workloads at full
size with every integer output compared and sampled float outputs.
"""
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


def run_layer(wl, capacity=None, logits_input=None, w_layout=0):
    from expert_token_routing_gemm_amd import MoELayer, to_host
    layer = MoELayer(wl, capacity=capacity, logits_input=logits_input, w_layout=w_layout)
    layer.forward()
    g = layer.results()
    g["x_send"] = to_host(layer.x_send)
    g["y_send"] = to_host(layer.y_send)
    g["y"] = to_host(layer.y)
    if layer.y_dense is not None:
        g["y_dense"] = to_host(layer.y_dense)
    g["capacity"] = layer.capacity
    return layer, g


def full_parity(wl, cf=None, label="", w_layout=0):
    """Everything element by element."""
    _say(f"[parity] {label} cfg{wl.cfg} T={wl.T} d={wl.d} h={wl.h} E={wl.E} k={wl.k} "
         f"w_layout={w_layout}")
    C = O.capacity(wl.T, wl.k, wl.E, wl.cf if cf is None else cf)
    layer, g = run_layer(wl, capacity=C, w_layout=w_layout)
    assert g["capacity"] == C
    ref = O.layer(wl, cf=cf)
    P.check_route(wl, g, ref["route"])
    if not np.array_equal(g["ids"], ref["route"]["ids"]):
        ref = O.layer(wl, cf=cf, ids_override=g["ids"])
    np.testing.assert_allclose(g["logits"], ref["route"]["logits"], rtol=0, atol=2e-4)
    np.testing.assert_allclose(g["weights"], ref["route"]["weights"], rtol=0, atol=5e-5)
    P.check_dispatch(wl, g, g["ids"], C)
    P.check_pack(wl, g["x_send"], g["src"])
    tol = P.tol_of(wl)
    off = g["off"]
    a, b = int(off[wl.e_begin]), int(off[wl.e_end])
    e_ys = 0.0
    if b > a:
        e_ys = P.check_close("Ys", P.act_to_f64(g["y_send"][a:b], wl.act_dtype), ref["ys"][a:b], tol)
    if wl.shared is not None:
        P.check_close("shared", P.act_to_f64(g["y_dense"], wl.act_dtype), ref["shared"], tol)
    e_y = P.check_close("y", P.act_to_f64(g["y"], wl.act_dtype), ref["y"], tol)
    n_pass = P.check_residual_passthrough(wl, g["y"], g["ids"], g["slot"])
    _say(f"[parity] ok: err Ys {e_ys:.2e} y {e_y:.2e}, dropped {int((g['slot'] < 0).sum())}, "
         f"pass-through tokens {n_pass}")
    return g, ref


def sampled_parity(wl, n_tok=192, rows_per_expert=24, seed=0, label="", w_layout=0):
    """Integer stages and the pack in full; floats on sampled rows/tokens."""
    _say(f"[parity-sampled] {label} cfg{wl.cfg} T={wl.T} d={wl.d} h={wl.h} E={wl.E} k={wl.k} "
         f"w_layout={w_layout}")
    C = O.capacity(wl.T, wl.k, wl.E, wl.cf)
    layer, g = run_layer(wl, capacity=C, w_layout=w_layout)
    x64 = O.to_f64(wl.x, wl.act_dtype)
    wr64 = O.to_f64(wl.w_router, wl.act_dtype)
    r = O.route(x64, wr64, wl.b_router, wl.b_select, wl.k, wl.score, wl.renorm)
    P.check_route(wl, g, r)
    np.testing.assert_allclose(g["logits"], r["logits"], rtol=0, atol=2e-4)
    r_g = O.route(x64, wr64, wl.b_router, wl.b_select, wl.k, wl.score, wl.renorm,
                  ids_override=g["ids"])
    np.testing.assert_allclose(g["weights"], r_g["weights"], rtol=0, atol=5e-5)
    P.check_dispatch(wl, g, g["ids"], C)
    P.check_pack(wl, g["x_send"], g["src"])
    tol = P.tol_of(wl)
    rng = np.random.default_rng(seed)
    off, src = g["off"], g["src"]
    cache = {}
    worst = 0.0
    for e in range(wl.e_begin, wl.e_end):
        a, b = int(off[e]), int(off[e + 1])
        if b <= a:
            continue
        pick = np.unique(np.concatenate([[a, b - 1], rng.integers(a, b, rows_per_expert)]))
        ref = O.expert_rows(wl, x64[src[pick]], e, cache)
        worst = max(worst, P.check_close(f"Ys expert {e}", P.act_to_f64(g["y_send"][pick], wl.act_dtype),
                                         ref, tol))
    toks = np.unique(np.concatenate([[0, wl.T - 1], rng.integers(0, wl.T, n_tok)]))
    if wl.shared is not None:
        ref = O.shared_rows(wl, x64[toks], cache)
        P.check_close("shared", P.act_to_f64(g["y_dense"][toks], wl.act_dtype), ref, tol)
    ref_y = O.token_outputs(wl, toks, g["ids"], r_g["weights"], g["slot"], cache=cache)
    e_y = P.check_close("y", P.act_to_f64(g["y"][toks], wl.act_dtype), ref_y, tol)
    _say(f"[parity-sampled] ok: worst Ys {worst:.2e}, y {e_y:.2e}")
    return g


# ---------------------------------------------------------------- small shapes


SMALL = {
    "c0-ragged": (0, dict(T=1000, d=256, h=384)),
    "c1-small": (1, dict(T=40, d=512, h=768)),
    # h a multiple of 7 * 128: the SwiGLU streaming GEMM takes 7-wave workgroups
    "c1-seven-wave": (1, dict(T=40, d=512, h=896)),
    # d = h = 384 (six 64-element chunks): both streaming GEMMs split K into
    # exactly two slices; the skewed case has experts past 64 rows
    "c1-k-split-2": (1, dict(T=40, d=384, h=384)),
    "c2-decode-skewed-k-split-2": (2, dict(T=256, d=384, h=384)),
    "c2-small": (2, dict(T=1000, d=512, h=640)),
    # E = 16: above the small-router limit and not a multiple of 64, so the
    # logits come from the VALU kernel (bf16 and fp32) before the top-k kernel
    "c3-valu-router": (3, dict(T=1000, d=256, h=512, E=16)),
    "c0-valu-router": (0, dict(T=600, d=256, h=256, E=16)),
    "c3-small": (3, dict(T=4096, d=256, h=512)),
    "c4-small": (4, dict(T=256, d=512, h=256)),
    # just above the single-workgroup dispatch limit (T*k > 4096): multi-block path
    "c2-multiblock-dispatch": (2, dict(T=2100, d=256, h=384)),
    "c4-multiblock-dispatch": (4, dict(T=600, d=256, h=256)),
    # decode-sized batch on the streaming path with skewed routing: experts
    # of 191 and 72 rows take several 64-row passes over the same weights
    "c2-decode-skewed": (2, dict(T=256, d=256, h=384)),
    # GELU at the fp32 tolerance (the kernels' erf is a rational approximation)
    # and GELU on the decode streaming path
    "c0-gelu-fp32": (0, dict(T=600, d=256, h=256, act="gelu")),
    "c3-decode-gelu-stream": (3, dict(T=64, d=256, h=256)),
    # row-major fp8 weights with h above the LDS-DMA kernel's fp8 K limit
    # (16384): the register-staged grouped kernel runs both expert GEMMs
    "c4-fp8-long-h-grouped": (4, dict(T=256, d=256, h=16640)),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    cfg, over = SMALL[name]
    full_parity(make_workload(cfg, **over), label=name)


def test_c0_full_size():
    g, ref = full_parity(make_workload(0), label="c0")
    # the page's printed loads (Ultralytics listing) on the GPU's histogram
    assert g["counts"].min() == 948 and g["counts"].max() == 1087
    assert g["rank_counts"].min() == 1968 and g["rank_counts"].max() == 2139


@pytest.mark.parametrize("cf", [1.0, 0.5])
def test_c0_forced_drops(cf):
    g, ref = full_parity(make_workload(0), cf=cf, label=f"c0 cf={cf}")
    assert (g["slot"] < 0).sum() > 0
    if cf == 1.0:
        assert int((g["slot"] < 0).sum()) == 154


def test_capacity_example_150_to_100():
    """150 tokens routed to one expert of capacity 100: the last 50 pass
    through unchanged (ai360xpert, "Load Balancing and Dropped Tokens")."""
    wl = make_workload(0, T=150, d=128, h=128, E=2, k=1, R=1, cf=100 / 150 * 2)
    wl.w_router[:] = 0.0
    wl.b_router = np.array([1.0, 0.0], np.float32)
    g, ref = full_parity(wl, label="150->100")
    assert g["capacity"] == 100
    np.testing.assert_array_equal(g["slot"][:, 0], np.r_[np.arange(100), -np.ones(50, int)])
    np.testing.assert_array_equal(g["y"][100:], wl.x[100:])


def test_tiny_edge_shapes():
    # one token; k = E; single expert; minimal dims
    full_parity(make_workload(0, T=1, d=128, h=128), label="T=1")
    full_parity(make_workload(0, T=37, d=128, h=128, E=4, k=4, R=2), label="k=E")
    full_parity(make_workload(1, T=9, d=128, h=128, E=1, k=1), label="E=1")
    full_parity(make_workload(3, T=300, d=128, h=256, E=64, k=1, R=16, cf=0.25), label="heavy drop")


@pytest.mark.parametrize("T", [64, 2304])
def test_all_256_experts_and_shared(T):
    """The most FFN groups there can be: all 256 experts of the DeepSeek-V3
    shape executed (fp8 weights) plus the shared expert, 257 groups; T = 64
    takes the weight-streaming kernels, T = 2304 (18432 rows) the LDS-DMA
    ones."""
    full_parity(make_workload(4, T=T, d=256, h=256, e_begin=0, e_end=256),
                label=f"E=256 all executed + shared, T={T}")


def test_zero_capacity_drops_everything():
    """C = 0: every assignment skips its expert and every token leaves as x."""
    wl = make_workload(0, T=300, d=128, h=128)
    layer, g = run_layer(wl, capacity=0)
    ref = O.dispatch(O.layer(wl, with_ffn=False)["route"]["ids"], wl.E, wl.R, 0)
    np.testing.assert_array_equal(g["counts"], ref["counts"])
    assert (g["slot"] == -1).all() and (g["kept"] == 0).all() and int(g["off"][-1]) == 0
    np.testing.assert_array_equal(g["y"], wl.x)


@pytest.mark.parametrize("cfg,over", [(2, dict(T=256, d=256, h=256, e_begin=3, e_end=3)),
                                      (4, dict(T=128, d=256, h=256, e_begin=0, e_end=0))])
def test_rank_executing_no_experts(cfg, over):
    """A rank whose share holds no executed expert (e_begin == e_end) still
    routes and dispatches the full send layout; the layer output is the
    residual bit for bit (plus the shared expert where there is one)."""
    wl = make_workload(cfg, **over)
    C = O.capacity(wl.T, wl.k, wl.E, wl.cf)
    layer, g = run_layer(wl, capacity=C)
    ref = O.layer(wl)
    P.check_route(wl, g, ref["route"])
    P.check_dispatch(wl, g, ref["route"]["ids"], C)
    if wl.shared is None:
        np.testing.assert_array_equal(g["y"], wl.x)
    else:
        P.check_close("y", P.act_to_f64(g["y"], wl.act_dtype), ref["y"], P.tol_of(wl))


def test_empty_batch():
    from expert_token_routing_gemm_amd import MoELayer
    wl = make_workload(0, T=1, d=128, h=128)
    layer = MoELayer(wl)
    for obj in (layer.args.route, layer.args.dispatch, layer.args.combine):
        obj.T = 0
    layer.args.ffn.max_rows = 0
    layer.forward()
    torch.cuda.synchronize()
    assert layer.counts.sum().item() == 0 and layer.expert_off[-1].item() == 0


def test_deterministic_rerun():
    wl = make_workload(3, T=4096, d=256, h=512)
    from expert_token_routing_gemm_amd import MoELayer, to_host
    layer = MoELayer(wl)
    layer.forward()
    first = {k: to_host(getattr(layer, k)).copy() for k in ("ids", "slot", "src", "x_send", "y_send", "y")}
    layer.forward()
    for k, v in first.items():
        np.testing.assert_array_equal(to_host(getattr(layer, k)), v, err_msg=k)


# ---------------------------------------------------------------- tiled weights


def test_weight_tile_layout():
    """moe_weight_tile is the stated byte permutation (bit-exact)."""
    from expert_token_routing_gemm_amd import moe_weight_tile, to_host
    rng = np.random.default_rng(5)
    for n, rows, rb in [(3, 48, 192), (1, 16, 64), (2, 128, 1024)]:
        w = rng.integers(0, 256, (n, rows, rb), dtype=np.uint8)
        got = to_host(moe_weight_tile(torch.from_numpy(w).cuda(), n, rows)).reshape(-1)
        # tile t, piece j, lane 16q + r, 16 bytes  <-  row 16t + r, bytes 64j + 16q
        want = w.reshape(n * rows // 16, 16, rb // 64, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
        np.testing.assert_array_equal(got, want)


def test_helpers_on_a_side_stream():
    """moe_weight_tile (from a non-contiguous view: a temporary copy) and
    moe_aux_loss (a temporary workspace) launched on another stream give the
    current stream's results, with the temporaries kept alive for it."""
    from expert_token_routing_gemm_amd import moe_aux_loss, moe_weight_tile, to_host
    g = torch.Generator().manual_seed(9)
    w = torch.randint(0, 256, (2, 64, 512), dtype=torch.uint8, generator=g).cuda()
    view = w.transpose(1, 2)  # [2, 512, 64]: non-contiguous
    logits = torch.randn((300, 64), generator=g).cuda()
    counts = torch.randint(0, 10, (64,), dtype=torch.int32, generator=g).cuda()
    ref_tile = to_host(moe_weight_tile(view, 2, 512))
    ref_pm, ref_loss = (to_host(t) for t in moe_aux_loss(logits, counts, 2, 0, 0.01))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        tiled = moe_weight_tile(view, 2, 512, stream=side)
        pm, loss = moe_aux_loss(logits, counts, 2, 0, 0.01, stream=side)
        junk = torch.full((1 << 20,), 7, dtype=torch.uint8, device="cuda")  # reuses freed blocks
        del junk
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(tiled), ref_tile)
    np.testing.assert_array_equal(to_host(pm), ref_pm)
    np.testing.assert_array_equal(to_host(loss), ref_loss)


TILED = {
    # streaming path
    "c1-small": (1, dict(T=40, d=512, h=768)),
    "c1-tiny-ragged": (1, dict(T=5, d=256, h=384)),
    "c1-seven-wave": (1, dict(T=40, d=512, h=896)),
    "c1-k-split-2": (1, dict(T=40, d=384, h=384)),
    "c4-decode": (4, dict(T=48, d=512, h=256)),
    # LDS-DMA path: bf16 and fp8 weights, 128- and 256-row tiles
    "c2-small": (2, dict(T=1000, d=512, h=640)),
    "c2-256-row-tiles": (2, dict(T=4096, d=512, h=512)),
    "c3-small": (3, dict(T=4096, d=256, h=512)),
    "c4-small": (4, dict(T=256, d=512, h=256)),
    # fp8 with more than 64 scale blocks along K (the second scale register)
    "c4-long-k-gemm1": (4, dict(T=256, d=8448, h=256)),
    "c4-long-k-gemm2": (4, dict(T=256, d=512, h=8448)),
}


@pytest.mark.parametrize("name", list(TILED))
def test_tiled_weights_parity(name):
    """Streaming path on tiled weights: oracle parity, and bit-identical to
    the same call on row-major weights (same arithmetic order)."""
    cfg, over = TILED[name]
    wl = make_workload(cfg, **over)
    g, _ = full_parity(wl, label=name, w_layout=1)
    _, g_row = run_layer(wl, capacity=g["capacity"])
    np.testing.assert_array_equal(g["y"], g_row["y"])
    a, b = int(g["off"][wl.e_begin]), int(g["off"][wl.e_end])  # rows the FFN wrote
    assert b > a
    np.testing.assert_array_equal(g["y_send"][a:b], g_row["y_send"][a:b])


def test_tiled_weights_full_decode(c1):
    """The decode workload at full size: tiled == row-major, bit for bit."""
    _say("[tiled] c1 full size")
    _, g_t = run_layer(c1, w_layout=1)
    _, g_r = run_layer(c1)
    np.testing.assert_array_equal(g_t["y"], g_r["y"])


def test_tiled_weights_rejected_where_unsupported():
    """fp32 activations have no tiled-weight kernel: a clear error, no launch."""
    from expert_token_routing_gemm_amd import MoEError
    wl = make_workload(0, T=512, d=256, h=256)
    with pytest.raises(MoEError, match="tiled"):
        run_layer(wl, w_layout=1)


# ---------------------------------------------------------------- identical logits


def _identical_logits(wl, logits32):
    from expert_token_routing_gemm_amd import MoELayer
    C = O.capacity(wl.T, wl.k, wl.E, wl.cf)
    layer = MoELayer(wl, capacity=C, logits_input=logits32)
    layer.route()
    layer.dispatch()
    g = layer.results()
    key = O.selection_keys32(logits32, wl.score, wl.b_select)
    ids = O.topk_select(key, wl.k)
    np.testing.assert_array_equal(g["ids"], ids)
    P.check_dispatch(wl, g, ids, C)
    return g


@pytest.mark.parametrize("cfg,over", [(0, {}), (2, dict(T=2048, d=256, h=256)),
                                      (3, dict(T=4096, d=256, h=256)),
                                      (4, dict(T=512, d=256, h=256))])
def test_identical_logits_bit_exact(cfg, over):
    wl = make_workload(cfg, **over)
    r = O.layer(wl, with_ffn=False)
    _identical_logits(wl, r["route"]["logits32"])


def test_identical_logits_exact_ties():
    """Exact fp32 ties in the selection key go to the lower expert index."""
    wl = make_workload(4, T=256, d=256, h=256)
    rng = np.random.default_rng(1)
    L = np.round(rng.standard_normal((wl.T, wl.E)) * 4).astype(np.float32) / 4  # many exact ties
    _identical_logits(wl, L)
    wl2 = make_workload(3, T=1024, d=256, h=256)
    L2 = np.round(rng.standard_normal((wl2.T, wl2.E))).astype(np.float32)
    _identical_logits(wl2, L2)


# ---------------------------------------------------------------- full sizes


@pytest.fixture(scope="module")
def c1():
    return make_workload(1)


# Full sizes, in the launch configuration bench.py times (tiled weights for
# the bf16-activation workloads) and on row-major weights.


@pytest.mark.parametrize("w_layout", [0, 1])
def test_c1_full_size(c1, w_layout):
    full_parity(c1, label="c1 decode", w_layout=w_layout)


@pytest.mark.parametrize("w_layout", [0, 1])
def test_c3_full_size(w_layout):
    g, _ = full_parity(make_workload(3), label="c3 switch", w_layout=w_layout)
    assert (g["slot"] < 0).sum() > 0  # the Zipf skew forces drops


@pytest.mark.slow
@pytest.mark.parametrize("w_layout", [0, 1])
def test_c2_full_size_sampled(w_layout):
    sampled_parity(make_workload(2), label="c2 prefill", w_layout=w_layout)


@pytest.mark.slow
@pytest.mark.parametrize("w_layout", [0, 1])
def test_c4_full_size_sampled(w_layout):
    sampled_parity(make_workload(4), label="c4 deepseek share", w_layout=w_layout)


# ---------------------------------------------------------------- HIP graphs


@pytest.mark.parametrize("cfg,over,w_layout", [(1, dict(T=64, d=512, h=768), 1),
                                               (2, dict(T=1000, d=512, h=640), 1),
                                               (4, dict(T=256, d=512, h=256), 0)])
def test_layer_forward_in_hip_graph(cfg, over, w_layout):
    """moe_layer_forward allocates, fills and synchronises nothing, so it can
    be captured in a HIP graph; every replay (with eager work on the buffers
    in between) reproduces the eager forward bit for bit."""
    from expert_token_routing_gemm_amd import MoELayer, to_host
    wl = make_workload(cfg, **over)
    _say(f"[graph] cfg{cfg} T={wl.T} w_layout={w_layout}")
    layer = MoELayer(wl, w_layout=w_layout)
    layer.forward()
    ref = {k: to_host(getattr(layer, k)) for k in ("y", "ids", "slot", "counts")}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward()  # warm-up on the capture-side stream
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward()
    torch.cuda.synchronize()
    for _ in range(3):
        for k in ("y", "ids", "slot", "counts"):
            getattr(layer, k).zero_()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            np.testing.assert_array_equal(to_host(getattr(layer, k)), v, err_msg=k)


def _hip_runtime():
    """The HIP runtime torch already loaded (for raw hipEvent_t handles)."""
    import ctypes
    path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), None)
    h = ctypes.CDLL(path or "libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def test_layer_forward_partial_events():
    """NULL entries of the event array are skipped: recording only the two
    events around the first expert GEMM times it and changes no result."""
    import ctypes

    from expert_token_routing_gemm_amd import MOE_LAYER_EVENTS, MoELayer, to_host
    wl = make_workload(1, T=64, d=512, h=768)
    _say("[events] cfg1 T=64, events at the first GEMM only")
    layer = MoELayer(wl, w_layout=1)
    layer.forward()
    ref = {k: to_host(getattr(layer, k)) for k in ("y", "ids", "slot", "counts")}
    hip = _hip_runtime()
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    try:
        arr = [None] * MOE_LAYER_EVENTS
        arr[2], arr[3] = evs
        for k in ("y", "ids", "slot", "counts"):
            getattr(layer, k).zero_()
        layer.forward(events=arr)
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0
        assert ms.value > 0
        for k, v in ref.items():
            np.testing.assert_array_equal(to_host(getattr(layer, k)), v, err_msg=k)
    finally:
        for e in evs:
            hip.hipEventDestroy(e)
