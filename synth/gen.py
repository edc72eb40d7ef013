"""Seeded synthetic workloads for the five MoE-layer configurations.

Every array is drawn with torch's CPU generator and returned as numpy:
fp32 arrays as ``float32``, bf16 arrays as their raw ``uint16`` bit patterns,
fp8 e4m3 arrays as raw ``uint8`` bytes with ``float32`` block scales.

Draw order (fixed, so that a seed names one workload):
  hidden states X, router weight W_r (and the Linear bias for the tiny fp32
  layer), per-expert logit offsets or selection bias, then for each executed
  expert in index order w1, [w3 for SwiGLU], w2, then the shared expert.

The tiny fp32 layer reproduces the routing snippet on the Ultralytics
"Expert Parallelism" page (section "How Tokens Move Between GPUs"): the global
torch seed 0, ``randn(4096, 512)`` hidden states and an ``nn.Linear(512, 8)``
router, drawn in that order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# Shapes of the five workloads.  R = simulated expert-parallel ranks.
# e_begin/e_end = the experts this GPU executes (its rank's share).
CONFIGS = {
    0: dict(name="tiny-fp32", T=4096, d=512, E=8, k=2, R=4, h=512, act="relu",
            act_dtype="f32", w_dtype="f32", score="softmax", renorm=True,
            cf=1.25, e_begin=0, e_end=8, shared=False, seed=0,
            router_bias="linear", offset=None, select_bias=None,
            w_std=None),
    1: dict(name="decode-mixtral-bf16", T=128, d=4096, E=8, k=2, R=1, h=14336,
            act="swiglu", act_dtype="bf16", w_dtype="bf16", score="softmax",
            renorm=True, cf=None, e_begin=0, e_end=8, shared=False, seed=1,
            router_bias=None, offset=None, select_bias=None, w_std=0.02),
    2: dict(name="prefill-mixtral-bf16", T=16384, d=4096, E=8, k=2, R=8,
            h=14336, act="swiglu", act_dtype="bf16", w_dtype="bf16",
            score="softmax", renorm=True, cf=None, e_begin=0, e_end=8,
            shared=False, seed=2, router_bias=None, offset=("normal", 0.5),
            select_bias=None, w_std=0.02),
    3: dict(name="switch-top1-bf16", T=32768, d=1024, E=64, k=1, R=16, h=4096,
            act="gelu", act_dtype="bf16", w_dtype="bf16", score="softmax",
            renorm=False, cf=1.25, e_begin=0, e_end=64, shared=False, seed=3,
            router_bias=None, offset=("zipf", 1.1), select_bias=None,
            w_std=0.02),
    4: dict(name="deepseek-v3-share-fp8", T=8192, d=7168, E=256, k=8, R=32,
            h=2048, act="swiglu", act_dtype="bf16", w_dtype="fp8",
            score="sigmoid", renorm=True, cf=None, e_begin=0, e_end=8,
            shared=True, seed=4, router_bias=None, offset=None,
            select_bias=0.1, w_std=0.02),
}

FP8_MAX = 448.0  # largest finite OCP e4m3fn value
BLOCK = 128      # fp8 weight scale block (rows x cols)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the raw bits."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def fp8_block_quantise(w: torch.Tensor):
    """Encode an fp32 matrix [rows, cols] as e4m3fn bytes plus one fp32 scale
    per 128x128 block: scale = amax/448 (1 for an all-zero block), and
    q = round-to-nearest-even(w/scale) clamped to +-448."""
    rows, cols = w.shape
    assert rows % BLOCK == 0 and cols % BLOCK == 0
    wb = w.reshape(rows // BLOCK, BLOCK, cols // BLOCK, BLOCK)
    amax = wb.abs().amax(dim=(1, 3), keepdim=True)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (wb / scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    qbytes = q.reshape(rows, cols).view(torch.uint8).numpy().copy()
    return qbytes, scale.reshape(rows // BLOCK, cols // BLOCK).numpy().astype(np.float32).copy()


@dataclass
class Workload:
    """One seeded input set.  Dtype tags: 'f32', 'bf16' (uint16 bits), 'fp8'
    (uint8 e4m3fn bytes + float32 block scales)."""
    cfg: int
    name: str
    T: int
    d: int
    E: int
    k: int
    R: int
    h: int
    act: str
    act_dtype: str
    w_dtype: str
    score: str
    renorm: bool
    cf: Optional[float]
    e_begin: int
    e_end: int
    seed: int
    x: np.ndarray = None             # [T, d]
    w_router: np.ndarray = None      # [E, d]
    b_router: Optional[np.ndarray] = None   # [E] float32 logit offset / bias
    b_select: Optional[np.ndarray] = None   # [E] float32 selection-only bias
    w1: np.ndarray = None            # [E_x, h, d]
    w3: Optional[np.ndarray] = None  # [E_x, h, d] (SwiGLU only)
    w2: np.ndarray = None            # [E_x, d, h]
    s1: Optional[np.ndarray] = None  # fp8 scales [E_x, h/128, d/128]
    s3: Optional[np.ndarray] = None
    s2: Optional[np.ndarray] = None  # [E_x, d/128, h/128]
    shared: Optional[dict] = None    # keys w1, w3, w2 (+ s1, s3, s2) for one expert
    extra: dict = field(default_factory=dict)

    @property
    def n_exec(self) -> int:
        return self.e_end - self.e_begin


def _encode(t: torch.Tensor, dtype: str):
    if dtype == "f32":
        return t.numpy().astype(np.float32, copy=True), None
    if dtype == "bf16":
        return bf16_bits(t), None
    if dtype == "fp8":
        return fp8_block_quantise(t)
    raise ValueError(dtype)


def _draw_expert(gen, d, h, act, std, w_dtype):
    """Draw one expert: w1 [h,d], (w3 [h,d]), w2 [d,h], N(0, std)."""
    out = {}
    names = ["w1", "w3", "w2"] if act == "swiglu" else ["w1", "w2"]
    for nm in names:
        shape = (h, d) if nm != "w2" else (d, h)
        t = torch.randn(shape, generator=gen) * std
        q, s = _encode(t, w_dtype)
        out[nm] = q
        if s is not None:
            out["s" + nm[1]] = s
    return out


def make_workload(cfg: int, **over) -> Workload:
    """Build config ``cfg`` (0-4) with optional shape overrides (T, d, h, E,
    k, R, e_begin, e_end, cf, seed, offset, select_bias).  Overrides keep the
    value distributions and draw order of the named config."""
    c = dict(CONFIGS[cfg])
    if "E" in over and "e_end" not in over:
        c["e_end"] = min(c["e_end"], over["E"])
    c.update(over)
    T, d, E, k, h = c["T"], c["d"], c["E"], c["k"], c["h"]
    wl = Workload(cfg=cfg, name=c["name"], T=T, d=d, E=E, k=k, R=c["R"], h=h,
                  act=c["act"], act_dtype=c["act_dtype"], w_dtype=c["w_dtype"],
                  score=c["score"], renorm=c["renorm"], cf=c["cf"],
                  e_begin=c["e_begin"], e_end=c["e_end"], seed=c["seed"])
    nx = wl.n_exec
    if c["router_bias"] == "linear":
        # Exactly the page's snippet: global seed, randn tokens, nn.Linear router.
        torch.manual_seed(c["seed"])
        x = torch.randn(T, d)
        lin = torch.nn.Linear(d, E)
        wl.x = x.numpy().astype(np.float32, copy=True)
        wl.w_router = lin.weight.detach().numpy().astype(np.float32, copy=True)
        wl.b_router = lin.bias.detach().numpy().astype(np.float32, copy=True)
        # Experts continue on the global generator: N(0, variance 1/fan_in),
        # fan_in = d for w1 and h for w2.
        experts = []
        for _ in range(nx):
            w1 = torch.randn(h, d) * (1.0 / math.sqrt(d))
            w2 = torch.randn(d, h) * (1.0 / math.sqrt(h))
            experts.append({"w1": w1.numpy().astype(np.float32), "w2": w2.numpy().astype(np.float32)})
    else:
        gen = torch.Generator().manual_seed(c["seed"])
        x = torch.randn((T, d), generator=gen)
        wl.x, _ = _encode(x, wl.act_dtype)
        bound = 1.0 / math.sqrt(d)
        wr = (torch.rand((E, d), generator=gen) * 2.0 - 1.0) * bound
        wl.w_router, _ = _encode(wr, wl.act_dtype)
        off = c["offset"]
        if off is not None and off[0] == "normal":
            wl.b_router = (torch.randn((E,), generator=gen) * off[1]).numpy().astype(np.float32)
        elif off is not None and off[0] == "zipf":
            s = off[1]
            wl.b_router = np.array([(e + 1.0) ** (-s) for e in range(E)], dtype=np.float32)
        elif off is not None and off[0] == "zipf_log":
            # the logarithm of the Zipf weights (an alternative reading of
            # the Switch workload's offset; far heavier skew)
            s = off[1]
            wl.b_router = np.array([-s * math.log(e + 1.0) for e in range(E)], dtype=np.float32)
        elif off is not None and off[0] == "zipf_pmf":
            # the normalised Zipf probabilities (another alternative reading;
            # mild skew)
            s = off[1]
            w = np.array([(e + 1.0) ** (-s) for e in range(E)])
            wl.b_router = (w / w.sum()).astype(np.float32)
        if c["select_bias"] is not None:
            wl.b_select = (torch.randn((E,), generator=gen) * c["select_bias"]).numpy().astype(np.float32)
        experts = [_draw_expert(gen, d, h, wl.act, c["w_std"], wl.w_dtype) for _ in range(nx)]
        if c["shared"]:
            wl.shared = _draw_expert(gen, d, h, wl.act, c["w_std"], wl.w_dtype)
    wl.w1 = np.stack([e["w1"] for e in experts]) if nx else None
    wl.w2 = np.stack([e["w2"] for e in experts]) if nx else None
    if wl.act == "swiglu" and nx:
        wl.w3 = np.stack([e["w3"] for e in experts])
    if wl.w_dtype == "fp8" and nx:
        wl.s1 = np.stack([e["s1"] for e in experts])
        wl.s2 = np.stack([e["s2"] for e in experts])
        if wl.act == "swiglu":
            wl.s3 = np.stack([e["s3"] for e in experts])
    return wl
