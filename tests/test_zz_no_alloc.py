"""The no-allocation layer entry point (moe_layer_forward_noalloc): it runs
the same kernels as moe_layer_forward on the library's static scratch, so its
outputs must equal that entry point's bit for bit, also on consecutive calls
that reuse the scratch with a smaller input.  Layers needing more workspace
than the scratch holds are refused before any launch."""
import numpy as np
import pytest
import torch

from synth import make_workload

pytestmark = pytest.mark.gpu

OUTS = ("ids", "weights", "counts", "kept", "expert_off", "slot", "x_send", "y_send", "y")


def _say(*a):
    print(*a, flush=True)


def _snapshot(layer):
    from expert_token_routing_gemm_amd import to_host
    torch.cuda.synchronize()
    n = int(layer.expert_off[-1].item())
    out = {k: to_host(getattr(layer, k)).copy() for k in OUTS}
    out["src"] = to_host(layer.src[:n]).copy()
    out["x_send"] = out["x_send"][:n]
    # the expert FFN writes only the executed experts' send rows
    wl = layer.wl
    a, b = int(out["expert_off"][wl.e_begin]), int(out["expert_off"][wl.e_end])
    out["y_send"] = out["y_send"][a:b]
    return out


def _clear(layer):
    for k in OUTS:
        t = getattr(layer, k)
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


@pytest.mark.parametrize("big,small", [
    # decode-sized streaming path, then a smaller batch
    ((1, dict(T=96, d=1024, h=2048)), (1, dict(T=40, d=512, h=768))),
    # many-row LDS-DMA path (bf16), then a smaller batch on the same path
    ((2, dict(T=1000, d=512, h=640)), (2, dict(T=600, d=256, h=512))),
    # fp8 weights, sigmoid + selection bias, shared expert
    ((4, dict(T=256, d=512, h=256)), (4, dict(T=100, d=256, h=256))),
])
def test_noalloc_matches_workspace_entry_point(big, small):
    from expert_token_routing_gemm_amd import MoELayer
    from expert_token_routing_gemm_amd._abi import MOE_STATIC_SCRATCH_BYTES
    layers = []
    for cfg, over in (big, small):
        wl = make_workload(cfg, **over)
        layer = MoELayer(wl)
        assert layer.workspace.numel() <= MOE_STATIC_SCRATCH_BYTES
        _say(f"[noalloc] cfg{cfg} T={wl.T} d={wl.d} h={wl.h}: workspace entry point")
        layer.forward()
        layers.append((layer, _snapshot(layer)))
    # two no-allocation calls in a row, the second on the smaller input
    for layer, _ in layers:
        _clear(layer)
    for layer, _ in layers:
        _say(f"[noalloc] T={layer.T}: no-allocation entry point")
        layer.forward_noalloc()
    for layer, ref in layers:
        got = _snapshot(layer)
        for k, v in ref.items():
            np.testing.assert_array_equal(got[k], v, err_msg=k)
    # and again, now the smaller one first: the scratch keeps the last
    # call's contents, which no kernel relies on
    for layer, _ in reversed(layers):
        _clear(layer)
        layer.forward_noalloc()
        got = _snapshot(layer)
        ref = next(r for l, r in layers if l is layer)
        for k, v in ref.items():
            np.testing.assert_array_equal(got[k], v, err_msg=k)


def test_noalloc_refuses_layers_beyond_the_scratch():
    from expert_token_routing_gemm_amd import MoEError, MoELayer, to_host
    from expert_token_routing_gemm_amd._abi import MOE_ERR_WORKSPACE, MOE_STATIC_SCRATCH_BYTES
    wl = make_workload(2, T=4608, d=512, h=4096)  # 9216 rows x 4096 x 2 B of activations
    layer = MoELayer(wl)
    _say(f"[noalloc] workspace {layer.workspace.numel()} > {MOE_STATIC_SCRATCH_BYTES}: refused")
    assert layer.workspace.numel() > MOE_STATIC_SCRATCH_BYTES
    layer.y.fill_(3.0)
    torch.cuda.synchronize()
    with pytest.raises(MoEError, match="static scratch") as ei:
        layer.forward_noalloc()
    assert ei.value.status == MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (to_host(layer.y) == to_host(torch.full_like(layer.y, 3.0))).all()  # nothing launched


@pytest.mark.parametrize("cfg,over", [(1, dict(T=64, d=512, h=768)),
                                      (2, dict(T=1000, d=512, h=640)),
                                      (4, dict(T=256, d=512, h=256))])
def test_noalloc_in_hip_graph(cfg, over):
    """Code under HIP graph capture is among the callers the no-allocation
    entry point is for: after one eager call (which looks up the scratch's
    device address), the captured forward replays bit for bit equal to the
    workspace entry point's outputs, with eager work between the replays."""
    from expert_token_routing_gemm_amd import MoELayer
    wl = make_workload(cfg, **over)
    _say(f"[noalloc graph] cfg{cfg} T={wl.T} d={wl.d} h={wl.h}")
    layer = MoELayer(wl)
    layer.forward()
    ref = _snapshot(layer)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward_noalloc()  # eager call on the capture-side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward_noalloc()
    torch.cuda.synchronize()
    for _ in range(3):
        _clear(layer)  # eager work on the outputs between replays
        graph.replay()
        got = _snapshot(layer)
        for k, v in ref.items():
            np.testing.assert_array_equal(got[k], v, err_msg=k)
