"""fp64 CPU oracle for the expert-parallel MoE layer forward (one GPU's share).

TEST INFRASTRUCTURE ONLY.  This file is the slow, plain definition that the
HIP library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code, table or helper with the HIP library and imports nothing from
it.  Inputs are the raw arrays of a seeded workload (fp32 arrays, bf16 bit
patterns as uint16, fp8 e4m3fn bytes as uint8 with fp32 block scales).

Where it comes from (page titles and sections of the source pages):

* The layer runs four steps - route, dispatch, local expert compute, combine -
  as listed in Ultralytics "Expert Parallelism", section "How Tokens Move
  Between GPUs" (numbered list), and again in ai360xpert "Expert Parallelism",
  section "The All-to-All Bottleneck", and mbrenndoerfer "Expert Parallelism >
  Summary" (the pipeline paragraph).
* Route: the router is a linear layer scoring every token against every
  expert; the top-k experts are kept (Ultralytics, "How Tokens Move Between
  GPUs", step 1 and the code listing's ``router(tokens).topk``).
* Placement: experts sit on ranks in contiguous equal blocks,
  rank = expert // (E / R) (Ultralytics code listing; ai360xpert, "Enter Expert
  Parallelism" list).
* Histogram: per-expert and per-rank assignment counts (the listing's
  ``bincount`` lines).
* Capacity: each expert takes at most a fixed number of assignments, e.g. 1.25x
  the even share T*k/E, the rest skip that expert (Ultralytics, "Load Balancing
  and Capacity", capacity-factor bullet; ai360xpert, "Load Balancing and
  Dropped Tokens", capacity bullet: 150 routed to a 100-slot expert drops 50).
* Dropped assignments pass through the residual unchanged (Ultralytics, "Load
  Balancing and Capacity", paragraph after the bullets; ai360xpert, same
  bullet).
* Selection-only bias: a per-expert bias changes which experts are picked but
  not the weights (Ultralytics, "Load Balancing and Capacity", bias-based
  balancing bullet).
* Token order is preserved through dispatch, compute and combine
  (mbrenndoerfer "Summary", implementation bullet on variable-length buffers).
* Combine: at the token's origin each expert output is scaled by its router
  weight and the scaled outputs are added
  (Ultralytics, "How Tokens Move Between GPUs", step 4).

Readings where the pages are silent (score function, renormalisation, FFN
forms, tie order, drop order) follow the workload definitions and are listed
in the design notes; each function below states the reading it uses.

Precision: everything is fp64, except where a floating-point value decides an
integer (the top-k selection).  That decision is taken on fp32 keys, the
precision the GPU kernels use, so that both sides decide identically when
given identical fp32 logits.

Pins: every function here is checked by the CPU tests against values the
pages print (the listing's expert and rank loads), closed forms, brute force
on tiny inputs, library routines and invariants.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
from scipy.special import erf

F64 = np.float64
F32 = np.float32

# --------------------------------------------------------------------------
# Input decoding: straight from the number-format definitions.
# --------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper 16 bits of an IEEE binary32; widen and read."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen as NaN
        return b.view(np.float32).astype(F64)


def decode_e4m3fn(q: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ('fn' variant): 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6;
    S.1111.111 is NaN; there are no infinities."""
    q = np.asarray(q, dtype=np.uint8)
    sign = np.where(q & 0x80, -1.0, 1.0)
    e = ((q >> 3) & 0xF).astype(np.int64)
    m = (q & 0x7).astype(F64)
    normal = (1.0 + m / 8.0) * np.exp2((e - 7).astype(F64))
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((q & 7) == 7), np.nan, val)
    return val


def dequant_blocks(q: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """w[r, c] = decode(q[r, c]) * scales[r // block, c // block]."""
    w = decode_e4m3fn(q)
    s = np.repeat(np.repeat(np.asarray(scales, F64), block, axis=0), block, axis=1)
    return w * s


def to_f64(arr, dtype: str, scales=None) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(F64)
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "fp8":
        return dequant_blocks(arr, scales)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Route
# --------------------------------------------------------------------------


def router_logits(x64: np.ndarray, wr64: np.ndarray, b_router=None) -> np.ndarray:
    """L = X W_r^T (+ b).  The router is a linear layer scoring every token
    against every expert (Ultralytics, "How Tokens Move Between GPUs", step 1;
    the listing builds it as ``nn.Linear(d, E)``).  ``b_router`` is the
    Linear bias or a per-expert logit offset that shifts routing."""
    L = x64 @ wr64.T
    if b_router is not None:
        L = L + np.asarray(b_router, F64)[None, :]
    return L


def softmax(L: np.ndarray) -> np.ndarray:
    m = L.max(axis=1, keepdims=True)
    z = np.exp(L - m)
    return z / z.sum(axis=1, keepdims=True)


def sigmoid(L: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-L))


def route_scores(L: np.ndarray, score: str) -> np.ndarray:
    """Router scores: softmax over all E experts, or an independent sigmoid
    per expert (DeepSeek-V3 style).  The pages name no score function; the
    workload definitions fix it."""
    if score == "softmax":
        return softmax(L)
    if score == "sigmoid":
        return sigmoid(L)
    raise ValueError(score)


def selection_keys32(L32: np.ndarray, score: str, b_select=None) -> np.ndarray:
    """fp32 keys on which the top-k decision is taken.

    softmax: the logit itself (softmax is monotone in the logit, so the
    selected set and order are those of the scores).
    sigmoid: fp32(sigmoid evaluated in fp64 on the fp32 logit), then the
    selection-only bias added in fp32.  The bias only changes which experts are
    picked (Ultralytics, "Load Balancing and Capacity", bias-based balancing
    bullet)."""
    L32 = np.asarray(L32, dtype=F32)
    if score == "softmax":
        return L32.copy()
    s32 = sigmoid(L32.astype(F64)).astype(F32)
    if b_select is None:
        return s32
    return (s32 + np.asarray(b_select, F32)[None, :]).astype(F32)


def topk_select(key: np.ndarray, k: int) -> np.ndarray:
    """ids[t, :] = the k largest keys of row t, in order (key desc, expert
    index asc); an exact tie goes to the lower expert index.  A stable sort on
    -key keeps equal keys in index order."""
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def group_limit_keys(key32: np.ndarray, n_groups: int, topk_groups: int) -> np.ndarray:
    """Group-limited routing: each token may use experts of at most
    ``topk_groups`` of the ``n_groups`` contiguous expert groups (DeepSeek-V3
    lets one token use experts of no more than four nodes: Ultralytics, "Load
    Balancing and Capacity", communication paragraph).  How the groups are
    chosen is not on the pages; reading taken: a group's score is its largest
    selection key, the best ``topk_groups`` groups are kept (score desc, group
    index asc) and the keys of all other experts become -inf."""
    T, E = key32.shape
    gs = E // n_groups
    gmax = key32.reshape(T, n_groups, gs).max(axis=2)
    chosen = np.argsort(-gmax, axis=1, kind="stable")[:, :topk_groups]
    keep = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(keep, chosen, True, axis=1)
    return np.where(np.repeat(keep, gs, axis=1), key32, np.float32(-np.inf)).astype(F32)


def group_gap(score64: np.ndarray, n_groups: int, topk_groups: int) -> np.ndarray:
    """fp64 gap between the topk_groups-th and next group score (inf if all
    groups are kept)."""
    T, E = score64.shape
    if topk_groups >= n_groups:
        return np.full(T, np.inf)
    gmax = score64.reshape(T, n_groups, E // n_groups).max(axis=2)
    srt = -np.sort(-gmax, axis=1)
    return srt[:, topk_groups - 1] - srt[:, topk_groups]


def route_weights(p: np.ndarray, ids: np.ndarray, renorm: bool) -> np.ndarray:
    """Combine weights from the (unbiased) router scores of the selected
    experts: renormalised over the k selected ones, or the raw score."""
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


def selection_gap(p: np.ndarray, score: str, b_select, k: int) -> np.ndarray:
    """Score gap between the k-th and (k+1)-th best expert per token, in fp64,
    on the score the selection orders by (softmax probability, or sigmoid plus
    selection bias).  Inf when k = E."""
    s = p if (score == "softmax" or b_select is None) else p + np.asarray(b_select, F64)[None, :]
    E = s.shape[1]
    if k >= E:
        return np.full(s.shape[0], np.inf)
    srt = -np.sort(-s, axis=1)
    return srt[:, k - 1] - srt[:, k]


def route(x64, wr64, b_router, b_select, k: int, score: str, renorm: bool,
          logits32=None, ids_override=None, n_groups: int = 0, topk_groups: int = 0) -> dict:
    """Route step.  ``logits32`` (optional) replaces the logits by given fp32
    values (the identical-logits mode); ``ids_override`` replaces the
    selection by given ids (weights still follow the oracle's own scores).
    ``n_groups``/``topk_groups`` > 0 enable group-limited selection."""
    if logits32 is not None:
        L = np.asarray(logits32, F32).astype(F64)
    else:
        L = router_logits(x64, wr64, b_router)
    L32 = L.astype(F32)
    p = route_scores(L, score)
    key32 = selection_keys32(L32, score, b_select)
    grouped = n_groups > 0 and 0 < topk_groups < n_groups
    if grouped:
        key32 = group_limit_keys(key32, n_groups, topk_groups)
    ids = topk_select(key32, k) if ids_override is None else np.asarray(ids_override, np.int32)
    w = route_weights(p, ids, renorm)
    if grouped:
        s64 = p if (score == "softmax" or b_select is None) else p + np.asarray(b_select, F64)[None, :]
        ggap = group_gap(s64, n_groups, topk_groups)
        masked = np.where(np.isfinite(key32), s64, -np.inf)
        srt = -np.sort(-masked, axis=1)
        egap = srt[:, k - 1] - srt[:, k] if k < masked.shape[1] else np.full(len(srt), np.inf)
        gap = np.minimum(ggap, np.where(np.isfinite(egap), egap, np.inf))
    else:
        gap = selection_gap(p, score, b_select, k)
    return dict(logits=L, logits32=L32, scores=p, key32=key32, ids=ids, weights=w, gap=gap)


def bias_update(b_select32: np.ndarray, counts: np.ndarray, T: int, k: int, gamma: float) -> np.ndarray:
    """Bias-based balancing after a step (Ultralytics, "Load Balancing and
    Capacity", bias bullet): the bias of an expert loaded above the mean
    T*k/E goes down, below the mean up.  The pages give no step size; rule
    taken: b <- b - gamma * sign(count - T*k/E), the comparison made exactly in
    integers (count*E vs T*k), the update in fp32."""
    counts = np.asarray(counts, np.int64)
    E = counts.size
    sgn = np.sign(counts * E - np.int64(T) * k).astype(F32)
    return (np.asarray(b_select32, F32) - np.float32(gamma) * sgn).astype(F32)


def aux_balance_loss(L64: np.ndarray, counts: np.ndarray, k: int, score: str, alpha: float):
    """Auxiliary balancing loss value of one step (forward only).  The pages
    say only that an extra loss term rewards the router for spreading tokens
    evenly (Ultralytics, "Load Balancing and Capacity", auxiliary-loss bullet;
    ai360xpert, "Load Balancing and Dropped Tokens", auxiliary-loss bullet).
    Reading taken, the Switch-Transformer form:
        loss = alpha * E * sum_e f_e * P_e,
    f_e = counts_e / (T*k) the fraction of the step's assignments (before
    capacity) routed to e, P_e the mean over tokens of the router's
    probability for e: softmax over all E, or for sigmoid scoring the
    sigmoids normalised per token.  Returns (P [E], loss)."""
    L64 = np.asarray(L64, F64)
    T, E = L64.shape
    if score == "softmax":
        p = softmax(L64)
    else:
        sg = sigmoid(L64)
        p = sg / sg.sum(axis=1, keepdims=True)
    P = p.mean(axis=0) if T > 0 else np.zeros(E)
    f = np.asarray(counts, F64) / (T * k) if T > 0 else np.zeros(E)
    return P, float(alpha) * E * float(np.dot(f, P))


# --------------------------------------------------------------------------
# Dispatch
# --------------------------------------------------------------------------


INT32_MAX = 2 ** 31 - 1


def capacity(T: int, k: int, E: int, cf) -> int:
    """C = ceil(cf * T * k / E), the even share T*k/E scaled by the capacity
    factor (Ultralytics, "Load Balancing and Capacity", capacity bullet; the
    listing's printout gives T*k/E as the even share).  Exact rational
    arithmetic on the binary value of cf.  cf None or <= 0: no limit."""
    if cf is None or cf <= 0:
        return INT32_MAX
    c = math.ceil(Fraction(cf) * T * k / E)
    return min(c, INT32_MAX)


def dispatch(ids: np.ndarray, E: int, R: int, C: int) -> dict:
    """Histogram, capacity drop, offsets and the stable permutation.

    Assignments (t, j) are visited in token-major order.  Each expert keeps
    its first C assignments in that order; later ones are dropped (they skip
    the expert).  Kept rows are laid out expert-major, and since experts sit
    on ranks in contiguous blocks this is also rank-major: the send buffer an
    all-to-all would move, each segment in token order.

    Returns counts[E] (raw), kept[E], off[E+1], rank_counts[R], rank_off[R+1],
    slot[T,k] (row in the send buffer, -1 if dropped), src[N] (token of each
    row)."""
    T, k = ids.shape
    if E % R != 0:
        raise ValueError("E must be a multiple of R")
    fill = np.zeros(E, dtype=np.int64)
    pos = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            pos[t, j] = fill[e]
            fill[e] += 1
    counts = fill.copy()
    kept = np.minimum(counts, C)
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(kept)
    slot = np.full((T, k), -1, dtype=np.int64)
    src = np.zeros(int(off[E]), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if pos[t, j] < C:
                s = off[e] + pos[t, j]
                slot[t, j] = s
                src[s] = t
    per = E // R
    rank_counts = np.array([kept[r * per:(r + 1) * per].sum() for r in range(R)], dtype=np.int64)
    rank_off = np.array([off[r * per] for r in range(R)] + [off[E]], dtype=np.int64)
    i32 = lambda a: a.astype(np.int32)
    return dict(counts=i32(counts), kept=i32(kept), off=i32(off), rank_counts=i32(rank_counts),
                rank_off=i32(rank_off), slot=i32(slot), src=i32(src))


def pack(x64: np.ndarray, src: np.ndarray) -> np.ndarray:
    """Send buffer rows: Xs[s] = X[src[s]]."""
    return x64[np.asarray(src, np.int64)]


# --------------------------------------------------------------------------
# Expert FFN
# --------------------------------------------------------------------------


def activation(z1: np.ndarray, act: str, z3=None) -> np.ndarray:
    """ReLU max(z, 0); GELU with the exact erf form 0.5 z (1 + erf(z/sqrt 2));
    SwiGLU silu(z1) * z3 with silu(z) = z * sigmoid(z)."""
    if act == "relu":
        return np.maximum(z1, 0.0)
    if act == "gelu":
        return 0.5 * z1 * (1.0 + erf(z1 / math.sqrt(2.0)))
    if act == "swiglu":
        return z1 * sigmoid(z1) * z3
    raise ValueError(act)


def ffn(rows64: np.ndarray, act: str, w1, w3, w2) -> np.ndarray:
    """One expert: act(rows W1^T [, rows W3^T]) W2^T, weights in nn.Linear
    [out, in] layout, no biases.  Experts are independent and run on their
    own rows (Ultralytics, "How Tokens Move Between GPUs", step 3)."""
    z1 = rows64 @ w1.T
    z3 = rows64 @ w3.T if act == "swiglu" else None
    a = activation(z1, act, z3)
    return a @ w2.T


def expert_weights64(wl, local: int, cache: dict = None):
    """fp64 weights of executed expert ``local`` (0-based within the rank).
    ``cache`` (optional dict) keeps decoded experts for repeated use."""
    if cache is not None and local in cache:
        return cache[local]
    s = lambda nm: getattr(wl, nm)[local] if getattr(wl, nm) is not None else None
    w1 = to_f64(wl.w1[local], wl.w_dtype, s("s1"))
    w3 = to_f64(wl.w3[local], wl.w_dtype, s("s3")) if wl.act == "swiglu" else None
    w2 = to_f64(wl.w2[local], wl.w_dtype, s("s2"))
    if cache is not None:
        cache[local] = (w1, w3, w2)
    return w1, w3, w2


def shared_weights64(wl, cache: dict = None):
    if cache is not None and "shared" in cache:
        return cache["shared"]
    sh = wl.shared
    w1 = to_f64(sh["w1"], wl.w_dtype, sh.get("s1"))
    w3 = to_f64(sh["w3"], wl.w_dtype, sh.get("s3")) if wl.act == "swiglu" else None
    w2 = to_f64(sh["w2"], wl.w_dtype, sh.get("s2"))
    if cache is not None:
        cache["shared"] = (w1, w3, w2)
    return w1, w3, w2


def expert_ffn(wl, xs64: np.ndarray, off: np.ndarray) -> np.ndarray:
    """Ys for the executed experts [e_begin, e_end): row s of expert e's
    segment [off[e], off[e+1]) is FFN_e(Xs[s]).  Rows of other experts are
    left as NaN (not computed on this rank)."""
    ys = np.full(xs64.shape, np.nan)
    for e in range(wl.e_begin, wl.e_end):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            w1, w3, w2 = expert_weights64(wl, e - wl.e_begin)
            ys[a:b] = ffn(xs64[a:b], wl.act, w1, w3, w2)
    return ys


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------


def combine(x64, shared64, ys64, ids, slot, w, e_begin: int, e_end: int) -> np.ndarray:
    """y[t] = x[t] (+ shared[t]) + sum_j w[t,j] * Ys[slot[t,j]] over the kept
    assignments to executed experts.  A dropped assignment contributes
    nothing and the other weights are not renormalised; a token with no
    contribution leaves as its residual x[t] unchanged (Ultralytics, "Load
    Balancing and Capacity"; ai360xpert, "Load Balancing and Dropped
    Tokens")."""
    y = x64.copy()
    if shared64 is not None:
        y = y + shared64
    T, k = ids.shape
    for j in range(k):
        e = ids[:, j]
        use = (slot[:, j] >= 0) & (e >= e_begin) & (e < e_end)
        if np.any(use):
            rows = slot[use, j].astype(np.int64)
            y[use] += w[use, j][:, None] * ys64[rows]
    return y


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------


def layer(wl, cf=None, logits32=None, ids_override=None, with_ffn=True, n_groups=0,
          topk_groups=0) -> dict:
    """route -> dispatch -> pack -> expert FFN (+ shared) -> combine on a
    workload ``wl`` (attribute access only).  ``cf`` overrides the workload's
    capacity factor; ``logits32`` / ``ids_override`` / the group limit as in
    :func:`route`."""
    x64 = to_f64(wl.x, wl.act_dtype)
    wr64 = to_f64(wl.w_router, wl.act_dtype)
    r = route(x64, wr64, wl.b_router, wl.b_select, wl.k, wl.score, wl.renorm,
              logits32=logits32, ids_override=ids_override, n_groups=n_groups,
              topk_groups=topk_groups)
    C = capacity(wl.T, wl.k, wl.E, wl.cf if cf is None else cf)
    dsp = dispatch(r["ids"], wl.E, wl.R, C)
    out = dict(route=r, dispatch=dsp, capacity=C)
    if not with_ffn:
        return out
    xs = pack(x64, dsp["src"])
    ys = expert_ffn(wl, xs, dsp["off"])
    shared = None
    if wl.shared is not None:
        shared = ffn(x64, wl.act, *shared_weights64(wl))
    y = combine(x64, shared, ys, r["ids"], dsp["slot"], r["weights"], wl.e_begin, wl.e_end)
    out.update(xs=xs, ys=ys, shared=shared, y=y)
    return out


def token_outputs(wl, tokens, ids, weights, slot, with_shared=True, cache=None) -> np.ndarray:
    """Second formulation, no permutation: for each listed token,
    y[t] = x[t] (+ shared(x[t])) + sum_j w[t,j] FFN_{ids[t,j]}(x[t]) over the
    kept (slot >= 0) executed assignments.  Used for sampled checks at full
    size and to cross-check :func:`layer`."""
    tokens = np.asarray(tokens, np.int64)
    x64 = to_f64(wl.x[tokens], wl.act_dtype)
    y = x64.copy()
    if wl.shared is not None and with_shared:
        y += ffn(x64, wl.act, *shared_weights64(wl, cache))
    for e in range(wl.e_begin, wl.e_end):
        hit = [(i, j) for i, t in enumerate(tokens) for j in range(ids.shape[1])
               if ids[t, j] == e and slot[t, j] >= 0]
        if not hit:
            continue
        w1, w3, w2 = expert_weights64(wl, e - wl.e_begin, cache)
        ii = np.array([i for i, _ in hit])
        jj = np.array([j for _, j in hit])
        out = ffn(x64[ii], wl.act, w1, w3, w2)
        np.add.at(y, ii, weights[tokens[ii], jj][:, None] * out)
    return y


def expert_rows(wl, rows_x64: np.ndarray, e: int, cache=None) -> np.ndarray:
    """FFN of executed expert e on the given rows (for sampled Ys checks)."""
    w1, w3, w2 = expert_weights64(wl, e - wl.e_begin, cache)
    return ffn(rows_x64, wl.act, w1, w3, w2)


def rowmax_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over rows of max_i |got - ref| / max_i |ref| (rows with an all-zero
    reference use an absolute error)."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    if ref.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def shared_rows(wl, rows_x64: np.ndarray, cache=None) -> np.ndarray:
    """Shared-expert FFN on the given rows."""
    return ffn(rows_x64, wl.act, *shared_weights64(wl, cache))
