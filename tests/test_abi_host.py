"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/moe.h declares, computes the capacity exactly like the
oracle's closed form, and rejects bad arguments before launching anything."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import expert_token_routing_gemm_amd as M
from expert_token_routing_gemm_amd import _abi
from oracle import oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "moe_layer_forward" in names and len(names) == len(_abi.PROTOTYPES)
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in _abi.PROTOTYPES, n


def test_struct_layouts_match_the_c_compiler(tmp_path):
    """Every field offset of the ctypes mirror equals what a C compiler gives
    for include/moe.h."""
    structs = {"moe_route_args": _abi.RouteArgs, "moe_dispatch_args": _abi.DispatchArgs,
               "moe_ffn_args": _abi.FfnArgs, "moe_combine_args": _abi.CombineArgs,
               "moe_layer_args": _abi.LayerArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for ln in out:
        if ln:
            c, f, v = ln.split()
            got[(c, f)] = int(v)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == C.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


@pytest.mark.parametrize("T,k,E,cf", [(4096, 2, 8, 1.25), (32768, 1, 64, 1.25), (150, 1, 2, 100 / 75),
                                      (10, 3, 7, 1.0), (64, 2, 8, 1.0), (1, 1, 1, 0.001),
                                      (12345, 8, 256, 1.1), (8192, 8, 256, 3.0000001),
                                      (100, 2, 8, 0.0), (100, 2, 8, -1.0)])
def test_capacity_matches_oracle(T, k, E, cf):
    assert M.moe_capacity(T, k, E, cf) == O.capacity(T, k, E, cf)


def test_capacity_random_exact():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        T = int(rng.integers(1, 1 << 20))
        k = int(rng.integers(1, 9))
        E = int(rng.integers(1, 257))
        cf = float(rng.uniform(0.01, 4.0))
        assert M.moe_capacity(T, k, E, cf) == O.capacity(T, k, E, cf), (T, k, E, cf)


def test_send_rows_max():
    assert M.moe_send_rows_max(4096, 2, 8, 1280) == 8192
    assert M.moe_send_rows_max(32768, 1, 64, 640) == 32768
    assert M.moe_send_rows_max(32768, 1, 64, 100) == 6400
    assert M.moe_send_rows_max(10, 2, 8, _abi.INT32_MAX) == 20


def test_route_rejects_bad_arguments_before_launch():
    a = _abi.RouteArgs(T=16, d=128, E=8, k=9, act_dtype=_abi.MOE_BF16, score=_abi.MOE_SOFTMAX)
    assert M.lib().moe_route(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID
    assert b"k out of range" in M.lib().moe_last_error()
    a.k, a.E = 2, 300
    assert M.lib().moe_route(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID
    a.E = 8
    a.score = 7
    assert M.lib().moe_route(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID


def test_dispatch_rejects_bad_arguments_before_launch():
    a = _abi.DispatchArgs(T=16, d=128, E=8, k=2, R=3, capacity=10, act_dtype=_abi.MOE_BF16)
    assert M.lib().moe_dispatch(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID
    assert b"multiple of R" in M.lib().moe_last_error()


def test_ffn_rejects_bad_arguments_before_launch():
    a = _abi.FfnArgs(d=100, h=256, E=8, e_begin=0, e_end=8, act=_abi.MOE_SWIGLU,
                     act_dtype=_abi.MOE_BF16, w_dtype=_abi.MOE_BF16)
    assert M.lib().moe_expert_ffn(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID
    a.d, a.e_end = 256, 9
    assert M.lib().moe_expert_ffn(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID
    a.e_end, a.act_dtype, a.w_dtype = 8, _abi.MOE_F32, _abi.MOE_BF16
    assert M.lib().moe_expert_ffn(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID


def test_combine_rejects_bad_arguments_before_launch():
    a = _abi.CombineArgs(T=4, d=100, k=2, e_begin=0, e_end=8, act_dtype=_abi.MOE_BF16)
    assert M.lib().moe_combine(C.byref(a), None) == _abi.MOE_ERR_INVALID


def test_ffn_rejects_unknown_weight_layout():
    a = _abi.FfnArgs(d=256, h=256, E=8, e_begin=0, e_end=8, act=_abi.MOE_SWIGLU,
                     act_dtype=_abi.MOE_BF16, w_dtype=_abi.MOE_BF16, w_layout=5)
    assert M.lib().moe_expert_ffn(C.byref(a), None, 0, None) == _abi.MOE_ERR_INVALID
    assert b"w_layout" in M.lib().moe_last_error()


def test_weight_tile_rejects_bad_arguments_before_launch():
    L = M.lib()
    assert L.moe_weight_tile(None, None, 1, 15, 64, None) == _abi.MOE_ERR_INVALID  # rows % 16
    assert L.moe_weight_tile(None, None, 1, 16, 96, None) == _abi.MOE_ERR_INVALID  # row_bytes % 64
    assert L.moe_weight_tile(None, None, 1, 16, 64, None) == _abi.MOE_ERR_INVALID  # null
    assert L.moe_weight_tile(4096, 4096 + 512, 1, 16, 64, None) == _abi.MOE_ERR_INVALID  # overlap
    assert b"overlaps" in L.moe_last_error()
    assert L.moe_weight_tile(None, None, 0, 16, 64, None) == _abi.MOE_OK  # nothing to do


def test_ffn_rejects_tiled_fp8_beyond_the_register_scales():
    """Tiled fp8 weights off the streaming path keep a tile's block scales in
    registers, which bounds d and h by 16384: beyond it, a clear error before
    any launch (pointers are never dereferenced on this path)."""
    fake = 1 << 20  # 16-byte aligned, never touched
    a = _abi.FfnArgs(d=256, h=16640, E=8, e_begin=0, e_end=8, act=_abi.MOE_SWIGLU,
                     act_dtype=_abi.MOE_BF16, w_dtype=_abi.MOE_FP8_E4M3,
                     w_layout=_abi.MOE_W_TILED16, max_rows=8 * 1024,
                     x_send=fake, expert_off=fake, w1=fake, w3=fake, w2=fake,
                     s1=fake, s3=fake, s2=fake, y_send=fake)
    need = M.lib().moe_ffn_workspace_bytes(C.byref(a))
    assert M.lib().moe_expert_ffn(C.byref(a), fake, need, None) == _abi.MOE_ERR_UNSUPPORTED
    assert b"tiled" in M.lib().moe_last_error()


def _layer_args():
    """A consistent decode-sized layer (T=4, d=h=256, E=8, top-2, SwiGLU, bf16)
    on fake 16-byte-aligned device addresses: only the checks ever see them."""
    fk = iter(range(1 << 24, 1 << 30, 1 << 20))
    T, d, E, k, h = 4, 256, 8, 2, 256
    x, wr, logits, ids, wts = (next(fk) for _ in range(5))
    counts, kept, off, rc, ro, slot, src, xs = (next(fk) for _ in range(8))
    w1, w3, w2, ys, y = (next(fk) for _ in range(5))
    a = _abi.LayerArgs()
    a.route = _abi.RouteArgs(T=T, d=d, E=E, k=k, act_dtype=_abi.MOE_BF16, score=_abi.MOE_SOFTMAX,
                             renorm=1, x=x, w_router=wr, logits=logits, ids=ids, weights=wts)
    a.dispatch = _abi.DispatchArgs(T=T, d=d, E=E, k=k, R=1, capacity=T * k,
                                   act_dtype=_abi.MOE_BF16, ids=ids, x=x, counts=counts, kept=kept,
                                   expert_off=off, rank_counts=rc, rank_off=ro, slot=slot, src=src,
                                   x_send=xs)
    a.ffn = _abi.FfnArgs(d=d, h=h, E=E, e_begin=0, e_end=E, act=_abi.MOE_SWIGLU,
                         act_dtype=_abi.MOE_BF16, w_dtype=_abi.MOE_BF16, max_rows=T * k,
                         x_send=xs, expert_off=off, w1=w1, w3=w3, w2=w2, y_send=ys)
    a.combine = _abi.CombineArgs(T=T, d=d, k=k, e_begin=0, e_end=E, act_dtype=_abi.MOE_BF16,
                                 x=x, y_send=ys, ids=ids, slot=slot, weights=wts, y=y)
    return a


@pytest.mark.parametrize("breaks,match", [
    (lambda a: setattr(a.combine, "d", 100), b"moe_combine"),          # a later stage's own check
    (lambda a: setattr(a.combine, "k", 1), b"same k"),
    (lambda a: setattr(a.dispatch, "T", 5), b"same T"),
    (lambda a: setattr(a.combine, "ids", a.combine.ids + 4096), b"ids, weights and slot"),
    (lambda a: setattr(a.ffn, "x_send", a.ffn.x_send + 4096), b"x_send, expert_off"),
    (lambda a: setattr(a.combine, "e_end", 4), b"executed experts"),
])
def test_layer_checks_every_stage_and_the_wiring_before_launch(breaks, match):
    """moe_layer_forward rejects a bad later stage or inconsistent wiring with
    MOE_ERR_INVALID before launching anything (a launch on this GPU-less host
    would have failed with MOE_ERR_HIP instead)."""
    a = _layer_args()
    breaks(a)
    L = M.lib()
    need = L.moe_workspace_bytes(C.byref(a))
    assert L.moe_layer_forward(C.byref(a), 1 << 30, need, None) == _abi.MOE_ERR_INVALID
    assert match in L.moe_last_error()
