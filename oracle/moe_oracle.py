"""fp64 reference of the MoE layer forward: Gate -> Scatter -> Expert Compute -> Gather.

Test infrastructure only (see the package docstring). Everything is evaluated in
float64 on the exact stored input values (bf16 / fp32 upcast, int8 and int4 as
q * scale),
one expert at a time, with no blocking, fusion or reordering beyond the
definitions below.

Readings of the pages taken here where they are silent or disagree:
  * expert FFN is SwiGLU with three matrices and no biases:
    silu(x W_gate) * (x W_up) W_down, silu(z) = z / (1 + exp(-z));
  * the k experts are chosen on raw logits ordered by (logit desc, id asc),
    slot 0 holding the largest; -0.0 and +0.0 compare equal;
  * the routing weights are the softmax over the k chosen logits (identical to
    the full softmax renormalised over the chosen set); as an option, the
    chosen raw logits themselves (top-k on raw logits with no softmax);
  * the scatter orders assignments a = t*k + j stably by expert, and
    expert_offsets has E + 1 token-row entries;
  * the shared expert is one SwiGLU FFN applied to every token, scaled by
    sigmoid(x . w_s).
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- Gate
def router_logits(x, w_router, b_router=None) -> np.ndarray:
    """logits[T, E] = x[T, d] @ w_router[d, E] (+ b_router[E]).

    [hotelren §3.2]: the router is a linear projection of the token with a
    router weight and bias (a GEMV per token); [0539edu §2.1]: the gate output
    has one logit per expert.
    """
    logits = _f64(x) @ _f64(w_router)
    if b_router is not None:
        logits = logits + _f64(b_router)[None, :]
    return logits


def select_topk(logits, k: int):
    """Top-k experts per token and the k-th/(k+1)-th logit margin.

    [hotelren §2.1 step 2] take the top-k of the router logits; [mhpq §3.2] the
    routing kernel keeps the running maximum with a strict greater-than test, so
    of two equal logits the lower expert id wins and slot 0 holds the maximum.
    Returns idx[T, k] (int64) and margin[T] = l_(k) - l_(k+1) (inf when k == E).
    """
    L = _f64(logits)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("top_k must be in [1, n_experts]")
    ids = np.broadcast_to(np.arange(E), L.shape)
    # primary key: logit descending; secondary: expert id ascending
    order = np.lexsort((ids, -L), axis=-1)
    idx = order[:, :k].copy()
    if k == E:
        margin = np.full(T, np.inf)
    else:
        srt = np.take_along_axis(L, order, axis=-1)
        margin = srt[:, k - 1] - srt[:, k]
    return idx, margin


def topk_weights(logits, idx) -> np.ndarray:
    """w[t, j] = exp(l[t, idx[t, j]]) / sum_j' exp(l[t, idx[t, j']]).

    [0539edu §2.1] softmax is taken over the gate logits; [hotelren §2.1 step 6]
    and [hotelren §2.3 combine_kernel] weight the k expert outputs by these
    gating scores. Computed with the slot-0 logit subtracted (the maximum), which
    leaves the ratio unchanged.
    """
    L = _f64(logits)
    chosen = np.take_along_axis(L, np.asarray(idx), axis=-1)
    e = np.exp(chosen - chosen[:, :1])
    return e / e.sum(axis=-1, keepdims=True)


def topk_raw_weights(logits, idx) -> np.ndarray:
    """w[t, j] = l[t, idx[t, j]]: the chosen logits themselves, unnormalised.

    [hotelren §3.2] the router's two steps are the linear projection and the
    top-k taken directly on the raw logits, with no softmax; [hotelren §2.3]
    combine_kernel weights the k expert outputs by the router's gating score.
    Read together: with no softmax, a chosen expert's gating score is its raw
    logit (bias included, after the clamp when that option is on).
    """
    L = _f64(logits)
    return np.take_along_axis(L, np.asarray(idx), axis=-1).copy()


def shared_gate(x, w_shared_gate) -> np.ndarray:
    """g_s[t] = sigmoid(x[t] . w_s) = 1 / (1 + exp(-x[t] . w_s)).

    The shared-expert-augmented MoE variant ([0539edu §2.2], [trdm §8]) adds an
    always-on expert; its scalar gate is a sigmoid of a linear function of the
    token.
    """
    z = _f64(x) @ _f64(w_shared_gate)
    return 1.0 / (1.0 + np.exp(-z))


# ---------------------------------------------------------------- Scatter
def scatter_stable_sort(idx, n_experts: int):
    """Group the T*k assignments by expert ([0539edu §2.2] Scatter stage;
    [hotelren §2.3] dispatch_kernel; [mhpq §2.1] contiguous per-expert batches).

    Assignment a = t*k + j routes token t to expert idx[t, j]. Returns
    counts[E], offsets[E+1] (offsets[E] = T*k; an exclusive prefix sum as in
    [pptc §3.3]) and sorted_assign[T*k], the assignments stably sorted by expert.
    """
    flat = np.asarray(idx).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_assign = np.argsort(flat, kind="stable").astype(np.int64)
    return counts, offsets, sorted_assign


def scatter_counting(idx, n_experts: int):
    """The same grouping written as an explicit counting sort (an independent
    second formulation, used to cross-check scatter_stable_sort)."""
    flat = [int(v) for v in np.asarray(idx).reshape(-1)]
    counts = [0] * n_experts
    for e in flat:
        counts[e] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_assign = [0] * len(flat)
    for a, e in enumerate(flat):
        sorted_assign[cursor[e]] = a
        cursor[e] += 1
    return (np.array(counts, dtype=np.int64), np.array(offsets, dtype=np.int64),
            np.array(sorted_assign, dtype=np.int64))


# ---------------------------------------------------------------- Expert compute
def dequantize(q, scale) -> np.ndarray:
    """w[..., i, o] = q[..., i, o] * scale[..., o]: symmetric int8 with one scale
    per output channel ([0539edu §3.1] symmetric scale = max|w| / 127, range
    [-127, 127]; applied per output channel). Exact in fp64."""
    return _f64(q) * _f64(scale)[..., None, :]


def dequantize_groupwise(q, scale, group: int) -> np.ndarray:
    """w[..., i, o] = q[..., i, o] * scale[..., i // group, o]: int4 weights with one
    scale per `group` consecutive input rows of each output column ([mhpq §4.2]:
    group-wise int4 quantisation with group size 128; [trdm §6.1]: int4 halves the
    int8 footprint, two values per byte). Exact in fp64."""
    q = _f64(q)
    s = np.repeat(_f64(scale), group, axis=-2)
    assert s.shape == q.shape, "scale rows times the group size must equal the input rows"
    return q * s


def _silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_expert(xrows, w_gate, w_up, w_down) -> np.ndarray:
    """One expert's FFN on a block of token rows ([hotelren §2.1] steps 4-5:
    load the chosen expert's weights and run its matrix products):
    out = (silu(x @ W_gate) * (x @ W_up)) @ W_down."""
    x = _f64(xrows)
    h = _silu(x @ _f64(w_gate)) * (x @ _f64(w_up))
    return h @ _f64(w_down)


# ---------------------------------------------------------------- Layer
@dataclass
class OracleLayer:
    """Layer weights as host arrays (any float dtype; int8 with scales)."""
    w_router: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    top_k: int
    b_router: Optional[np.ndarray] = None
    s_gate: Optional[np.ndarray] = None
    s_up: Optional[np.ndarray] = None
    s_down: Optional[np.ndarray] = None
    w_shared_gate: Optional[np.ndarray] = None
    ws_gate: Optional[np.ndarray] = None
    ws_up: Optional[np.ndarray] = None
    ws_down: Optional[np.ndarray] = None
    group: Optional[int] = None  # int4: input rows per scale (scales [E, in/group, out])
    gate_clamp: bool = False     # clamp the routed logits to [-50, 50] before top-k and softmax
    gate_weighting: str = "softmax"  # "softmax": over the chosen logits; "raw": the chosen logits

    @property
    def n_experts(self) -> int:
        return self.w_gate.shape[0]

    def expert(self, e: int):
        """fp64 (W_gate, W_up, W_down) of expert e."""
        if self.group is not None:
            g = self.group
            return (dequantize_groupwise(self.w_gate[e], self.s_gate[e], g),
                    dequantize_groupwise(self.w_up[e], self.s_up[e], g),
                    dequantize_groupwise(self.w_down[e], self.s_down[e], g))
        if self.s_gate is not None:
            return (dequantize(self.w_gate[e], self.s_gate[e]),
                    dequantize(self.w_up[e], self.s_up[e]),
                    dequantize(self.w_down[e], self.s_down[e]))
        return _f64(self.w_gate[e]), _f64(self.w_up[e]), _f64(self.w_down[e])


def valid_selections(logits_row, k: int, tol: float) -> list:
    """Every top-k choice that a computation within `tol` of these logits could
    make: sets S of k experts with min over S >= max outside S - tol, each in
    slot order (logit desc, id asc). Used for tokens whose k-th/(k+1)-th margin
    is below tol, where more than one answer is correct."""
    l = _f64(logits_row)
    E = l.shape[0]
    order = np.lexsort((np.arange(E), -l))
    kth = l[order[k - 1]]
    cand = [int(e) for e in order if l[e] >= kth - tol]
    out = []
    for S in itertools.combinations(cand, k):
        inside = np.array(S)
        outside = np.setdiff1d(np.arange(E), inside)
        if outside.size and l[inside].min() < l[outside].max() - tol:
            continue
        slot = sorted(S, key=lambda e: (-l[e], e))
        out.append(np.array(slot, dtype=np.int64))
    return out


def _experts_and_gather(x, layer: OracleLayer, idx, w, g_s, sorted_assign, offsets, tokens):
    """Expert Compute and Gather for a routing already scattered: every expert's
    token rows through its SwiGLU FFN, then y[t] = sum_j w[t, j] * o(t, j)
    (+ g_s[t] * S(x[t])) ([hotelren §2.1] steps 4-6, §2.3 combine_kernel)."""
    T = x.shape[0]
    k = idx.shape[1]
    E = layer.n_experts
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    row_of = {int(t): i for i, t in enumerate(rows)}
    y = np.zeros((rows.size, x.shape[1]))
    for e in range(E):
        seg = sorted_assign[offsets[e]:offsets[e + 1]]
        seg = [int(a) for a in seg if int(a) // k in row_of]
        if not seg:
            continue
        wg, wu, wd = layer.expert(e)
        toks = np.array([a // k for a in seg])
        out = swiglu_expert(x[toks], wg, wu, wd)
        # Gather: weighted sum of the k expert outputs ([hotelren §2.3] combine_kernel)
        for r, a in enumerate(seg):
            t, j = divmod(a, k)
            y[row_of[t]] += w[t, j] * out[r]
    if g_s is not None:
        s = swiglu_expert(x[rows], layer.ws_gate, layer.ws_up, layer.ws_down)
        y += g_s[rows, None] * s
    return y


def moe_forward(x, layer: OracleLayer, routing=None, tokens: Optional[Sequence[int]] = None):
    """The whole layer ([hotelren §2.1] six steps; [0539edu §2.2] Gate -> Scatter
    -> Expert Compute -> Gather).

    x[T, d]. `routing` optionally replaces the top-k choice with an idx[T, k]
    the caller built from this module's own valid_selections. `tokens`
    optionally restricts the expert compute and combine to a subset of token
    rows (the gate and scatter still cover all T tokens), so large batches can
    be checked on a sample.

    Returns a dict: logits, idx, margin, w, counts, offsets, sorted_assign,
    g_s (or None), y (fp64, rows in `tokens` order when given).
    """
    x = _f64(x)
    k = layer.top_k
    E = layer.n_experts
    logits = router_logits(x, layer.w_router, layer.b_router)
    if layer.gate_clamp:
        # [0539edu §5.2]: the gate's clip option bounds the logits to [-50, 50] before the
        # softmax; the selection and the weights both use the bounded values
        logits = np.clip(logits, -50.0, 50.0)
    idx, margin = select_topk(logits, k)
    if routing is not None:
        idx = np.asarray(routing, dtype=np.int64)
    if layer.gate_weighting == "softmax":
        w = topk_weights(logits, idx)
    elif layer.gate_weighting == "raw":
        w = topk_raw_weights(logits, idx)
    else:
        raise ValueError("gate_weighting must be 'softmax' or 'raw'")
    counts, offsets, sorted_assign = scatter_stable_sort(idx, E)
    g_s = shared_gate(x, layer.w_shared_gate) if layer.w_shared_gate is not None else None

    y = _experts_and_gather(x, layer, idx, w, g_s, sorted_assign, offsets, tokens)
    return dict(logits=logits, idx=idx, margin=margin, w=w, counts=counts,
                offsets=offsets, sorted_assign=sorted_assign, g_s=g_s, y=y)


def moe_forward_routed(x, layer: OracleLayer, idx, w, g_s=None, tokens: Optional[Sequence[int]] = None):
    """The layer with the routing given instead of computed ([pptc §3.4]: the
    engine consumes routing results made elsewhere, token-major [T][k]).

    idx[T, k] int expert ids, w[T, k] weights used as given, g_s[T] the shared
    expert's scale (layers with a shared expert). An id outside [0, E) is read
    as expert 0 with weight 0 (the library's documented reading: it contributes
    nothing). Returns a dict: idx, w (as read), counts, offsets, sorted_assign,
    y (fp64, rows in `tokens` order when given).
    """
    x = _f64(x)
    E = layer.n_experts
    idx = np.asarray(idx, dtype=np.int64).copy()
    w = _f64(w).copy()
    bad = (idx < 0) | (idx >= E)
    idx[bad] = 0
    w[bad] = 0.0
    if (layer.w_shared_gate is not None) != (g_s is not None):
        raise ValueError("g_s is required exactly when the layer has a shared expert")
    counts, offsets, sorted_assign = scatter_stable_sort(idx, E)
    y = _experts_and_gather(x, layer, idx, w, None if g_s is None else _f64(g_s), sorted_assign, offsets, tokens)
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, sorted_assign=sorted_assign, y=y)
