"""Shared test helpers: build a libmoe layer and its oracle twin from one synthetic
layer, and compare a GPU forward with the oracle under the parity rules.

Parity rules (the tolerances are the layer's contract):
  * tokens whose k-th/(k+1)-th fp64 logit margin is >= 1e-3: top-k indices equal
    the oracle's bit for bit; routing weights within 1e-5;
  * tokens inside the margin: the GPU's choice must be one of the oracle's own
    valid selections (oracle.valid_selections); the oracle is then re-run with
    that selection (chosen from its own list) for weights, scatter and outputs;
  * counts, offsets and the by-expert permutation equal the oracle's bit for bit;
  * outputs: relative Frobenius error <= 1e-2 and max-abs <= 3e-2 * rms(ref) for
    bf16 activations, 1e-4 and 3e-4 * rms(ref) for fp32.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

MARGIN = 1e-3
W_TOL = 1e-5
Y_TOL = {"bf16": (1e-2, 3e-2), "f32": (1e-4, 3e-4)}


def gpu_layer(L: "synth.SynthLayer", max_tokens: int, profile: bool = False, gate_clamp: bool = False,
              gate_weighting: str = "softmax"):
    import moe_layer_forward_gate_amd as moe
    dev = torch.device("cuda", torch.cuda.current_device())
    return moe.MoeLayer(max_tokens=max_tokens, profile=profile, gate_clamp=gate_clamp,
                        gate_weighting=gate_weighting, **synth.layer_kwargs(L, dev))


def _np(t):
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def oracle_layer(L: "synth.SynthLayer", gate_clamp: bool = False) -> oracle.OracleLayer:
    return oracle.OracleLayer(
        w_router=_np(L.w_router), w_gate=_np(L.w_gate), w_up=_np(L.w_up), w_down=_np(L.w_down),
        top_k=L.cfg.top_k, b_router=_np(L.b_router), s_gate=_np(L.s_gate), s_up=_np(L.s_up),
        s_down=_np(L.s_down), w_shared_gate=_np(L.w_shared_gate), ws_gate=_np(L.ws_gate),
        ws_up=_np(L.ws_up), ws_down=_np(L.ws_down),
        group=synth.INT4_GROUP if L.cfg.expert_dtype == "i4" else None, gate_clamp=gate_clamp)


def compare(cfg, x, olay: oracle.OracleLayer, out, sample=None, label=""):
    """Check one GPU forward `out` (RouteResult, scatter outputs filled) against
    the oracle on the same x. `sample`: token rows whose outputs are compared
    (None = all). Returns a dict of the measured errors."""
    xn = _np(x)
    T, k, E = xn.shape[0], cfg.top_k, cfg.n_experts
    ref = oracle.moe_forward(xn, olay, tokens=[] if sample is not None else None)
    gidx = out.topk_idx.cpu().numpy().astype(np.int64)
    gw = out.topk_w.cpu().numpy().astype(np.float64)
    excl = ref["margin"] < MARGIN
    keep = ~excl
    bad = np.nonzero((gidx[keep] != ref["idx"][keep]).any(1))[0]
    assert bad.size == 0, f"{label}: top-k mismatch on {bad.size} tokens outside the margin, first {np.nonzero(keep)[0][bad[:5]]}"
    routing = ref["idx"].copy()
    for t in np.nonzero(excl)[0]:
        alts = oracle.valid_selections(ref["logits"][t], k, MARGIN)
        match = [a for a in alts if np.array_equal(a, gidx[t])]
        assert match, f"{label}: token {t} (margin {ref['margin'][t]:.2e}) chose {gidx[t]}, not a valid selection {alts}"
        routing[t] = match[0]
    rows = np.arange(T) if sample is None else np.asarray(sample)
    if not np.array_equal(routing, ref["idx"]) or sample is not None:
        ref = oracle.moe_forward(xn, olay, routing=routing, tokens=None if sample is None else rows)
    werr = float(np.abs(gw - ref["w"]).max()) if T else 0.0
    assert werr <= W_TOL, f"{label}: routing weight error {werr:.3e}"
    if out.expert_counts is not None:
        assert np.array_equal(out.expert_counts.cpu().numpy(), ref["counts"]), f"{label}: counts differ"
        assert np.array_equal(out.expert_offsets.cpu().numpy(), ref["offsets"]), f"{label}: offsets differ"
        assert np.array_equal(out.sorted_assign.cpu().numpy(), ref["sorted_assign"]), f"{label}: permutation differs"
    if out.shared_gate is not None and ref["g_s"] is not None:
        gerr = float(np.abs(out.shared_gate.cpu().numpy() - ref["g_s"]).max())
        assert gerr <= W_TOL, f"{label}: shared gate error {gerr:.3e}"
    y = _np(out.y).astype(np.float64)[rows]
    yr = ref["y"]
    rel, mabs = Y_TOL[cfg.act_dtype]
    num = np.linalg.norm(y - yr)
    den = np.linalg.norm(yr)
    rms = den / np.sqrt(max(yr.size, 1))
    frob = float(num / den) if den > 0 else float(num)
    mx = float(np.abs(y - yr).max()) if yr.size else 0.0
    assert frob <= rel, f"{label}: relative Frobenius error {frob:.3e} > {rel}"
    assert mx <= mabs * rms, f"{label}: max-abs error {mx:.3e} > {mabs} * rms {rms:.3e}"
    return dict(frob=frob, maxabs_over_rms=mx / rms if rms else 0.0, w_err=werr, excluded=int(excl.sum()))
