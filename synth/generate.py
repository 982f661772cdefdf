"""Seeded draws of MoE layer weights and token batches.

Distributions (one per tensor, independent streams):
  x        ~ N(0, 1)                [T, d_model]      activation dtype
  w_router ~ N(0, 0.02^2)           [d_model, E]      fp32
  b_router  = beta * ln p_pi(e),    p_r ~ r^-s        fp32 (skewed layer only)
  w_gate, w_up ~ N(0, 1/d_model)    [E, d_model, d_ff]
  w_down       ~ N(0, 1/d_ff)       [E, d_ff, d_model]
  w_shared_gate ~ N(0, 0.02^2)      [d_model]         fp32
  ws_gate, ws_up ~ N(0, 1/d_model)  [d_model, Fs]     bf16
  ws_down        ~ N(0, 1/Fs)       [Fs, d_model]     bf16

Draws are made in fp32 and then stored in the target dtype: bf16 by
round-to-nearest-even (torch's conversion), int8 by symmetric
per-output-channel quantisation (scale = max|w| / 127 over the input axis,
q = round-half-even(w / scale) clipped to [-127, 127]; an all-zero channel gets
scale 0 and q 0), or int4 by symmetric group-wise quantisation (one scale per
128 consecutive input rows of each output column, scale = max|w| / 7 over the
group, q = round-half-even(w / scale) clipped to [-7, 7]; an all-zero group gets
scale 0 and q 0). The stored values are the ground truth for every consumer.

Each tensor (and each expert's slice of it) has its own torch.Generator seeded
from (config seed, config name, instance, tensor name, expert), so a layer is
reproducible on any device, and drawing one tensor never shifts another.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass
from typing import Optional

import torch

from .configs import LayerConfig

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _seed(cfg: LayerConfig, *key) -> int:
    s = "|".join([cfg.name] + [str(k) for k in key]).encode()
    return (cfg.seed * 1_000_003 + zlib.crc32(s)) % (2 ** 62)


def _gen(cfg: LayerConfig, device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg, *key))
    return g


def _normal(cfg, device, shape, std, *key) -> torch.Tensor:
    g = _gen(cfg, device, *key)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_per_out_channel(w: torch.Tensor):
    """Symmetric int8 quantisation of w[..., in, out] along its last (output) axis.

    Returns (q int8 of w's shape, scale fp32 of shape w.shape[:-2] + (out,)).
    """
    amax = w.abs().amax(dim=-2)                       # [..., out]
    scale = amax / 127.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = torch.round(w / safe.unsqueeze(-2)).clamp_(-127, 127)
    q = torch.where(scale.unsqueeze(-2) > 0, q, torch.zeros_like(q))
    return q.to(torch.int8), scale.to(torch.float32)


INT4_GROUP = 128  # input rows per int4 scale


def quantize_int4_groupwise(w: torch.Tensor, group: int = INT4_GROUP):
    """Symmetric int4 quantisation of w[..., in, out] in groups of `group` input rows.

    Returns (q int8 of w's shape holding values in [-7, 7], scale fp32 of shape
    w.shape[:-2] + (in / group, out)).
    """
    *lead, n_in, n_out = w.shape
    assert n_in % group == 0, "input axis must be a multiple of the group size"
    wg = w.reshape(*lead, n_in // group, group, n_out)
    scale = wg.abs().amax(dim=-2) / 7.0               # [..., in/group, out]
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = torch.round(wg / safe.unsqueeze(-2)).clamp_(-7, 7)
    q = torch.where(scale.unsqueeze(-2) > 0, q, torch.zeros_like(q))
    return q.reshape(w.shape).to(torch.int8), scale.to(torch.float32)


def pack_int4_pairs(q: torch.Tensor) -> torch.Tensor:
    """Storage of int4 values q[..., in, out] (int8 tensor, values in [-8, 7]) two per
    byte along the input axis: byte [..., i, o] holds q[..., 2i, o] in its low nibble
    and q[..., 2i+1, o] in its high nibble, each as a 4-bit two's complement code."""
    *lead, n_in, n_out = q.shape
    u = (q.to(torch.int16) & 0xF).reshape(*lead, n_in // 2, 2, n_out)
    return (u[..., 0, :] | (u[..., 1, :] << 4)).to(torch.uint8)


@dataclass
class SynthLayer:
    cfg: LayerConfig
    w_router: torch.Tensor                 # [d, E] fp32
    b_router: Optional[torch.Tensor]       # [E] fp32 or None
    w_gate: torch.Tensor                   # [E, d, F]
    w_up: torch.Tensor                     # [E, d, F]
    w_down: torch.Tensor                   # [E, F, d]
    s_gate: Optional[torch.Tensor] = None  # [E, F] fp32 (int8); [E, d/128, F] (int4)
    s_up: Optional[torch.Tensor] = None    # [E, F]; [E, d/128, F]
    s_down: Optional[torch.Tensor] = None  # [E, d]; [E, F/128, d]
    w_shared_gate: Optional[torch.Tensor] = None  # [d] fp32
    ws_gate: Optional[torch.Tensor] = None        # [d, Fs]
    ws_up: Optional[torch.Tensor] = None          # [d, Fs]
    ws_down: Optional[torch.Tensor] = None        # [Fs, d]

    def tensors(self):
        return {k: v for k, v in self.__dict__.items() if isinstance(v, torch.Tensor)}

    def to(self, device) -> "SynthLayer":
        kw = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in self.__dict__.items()}
        return SynthLayer(**kw)


def _expert_stack(cfg, device, name, rows, cols, std, instance):
    """[E, rows, cols] stored in the expert dtype (+ per-column scales for int8, per
    (group, column) scales for int4, whose values are kept one per int8 element)."""
    E = cfg.n_experts
    if cfg.expert_dtype == "i4":
        q = torch.empty((E, rows, cols), dtype=torch.int8, device=device)
        s = torch.empty((E, rows // INT4_GROUP, cols), dtype=torch.float32, device=device)
        for e in range(E):
            w = _normal(cfg, device, (rows, cols), std, instance, name, e)
            q[e], s[e] = quantize_int4_groupwise(w)
            del w
        return q, s
    if cfg.expert_dtype == "i8":
        q = torch.empty((E, rows, cols), dtype=torch.int8, device=device)
        s = torch.empty((E, cols), dtype=torch.float32, device=device)
        for e in range(E):
            w = _normal(cfg, device, (rows, cols), std, instance, name, e)
            q[e], s[e] = quantize_per_out_channel(w)
            del w
        return q, s
    dt = _TORCH_DT[cfg.expert_dtype]
    out = torch.empty((E, rows, cols), dtype=dt, device=device)
    for e in range(E):
        out[e] = _normal(cfg, device, (rows, cols), std, instance, name, e).to(dt)
    return out, None


def zipf_bias(cfg: LayerConfig, device="cpu", instance: int = 0) -> torch.Tensor:
    """b_e = beta * ln p_pi(e), p_r proportional to r^-s for ranks r = 1..E, pi a seeded permutation."""
    E = cfg.n_experts
    r = torch.arange(1, E + 1, dtype=torch.float64)
    p = r.pow(-cfg.zipf_s)
    p = p / p.sum()
    perm = torch.randperm(E, generator=_gen(cfg, "cpu", instance, "zipf_perm"))
    b = torch.empty(E, dtype=torch.float64)
    b[perm] = cfg.zipf_beta * torch.log(p)   # expert perm[r-1] has rank r
    return b.to(torch.float32).to(device)


def make_layer(cfg: LayerConfig, device="cpu", instance: int = 0) -> SynthLayer:
    d, E, F = cfg.d_model, cfg.n_experts, cfg.d_ff
    w_router = _normal(cfg, device, (d, E), 0.02, instance, "w_router")
    b_router = zipf_bias(cfg, device, instance) if cfg.has_bias else None
    w_gate, s_gate = _expert_stack(cfg, device, "w_gate", d, F, d ** -0.5, instance)
    w_up, s_up = _expert_stack(cfg, device, "w_up", d, F, d ** -0.5, instance)
    w_down, s_down = _expert_stack(cfg, device, "w_down", F, d, F ** -0.5, instance)
    layer = SynthLayer(cfg, w_router, b_router, w_gate, w_up, w_down, s_gate, s_up, s_down)
    if cfg.shared_d_ff:
        Fs = cfg.shared_d_ff
        layer.w_shared_gate = _normal(cfg, device, (d,), 0.02, instance, "w_shared_gate")
        layer.ws_gate = _normal(cfg, device, (d, Fs), d ** -0.5, instance, "ws_gate").to(torch.bfloat16)
        layer.ws_up = _normal(cfg, device, (d, Fs), d ** -0.5, instance, "ws_up").to(torch.bfloat16)
        layer.ws_down = _normal(cfg, device, (Fs, d), Fs ** -0.5, instance, "ws_down").to(torch.bfloat16)
    return layer


def make_tokens(cfg: LayerConfig, T: int, device="cpu", instance: int = 0) -> torch.Tensor:
    """x[T, d_model] ~ N(0, 1) in the activation dtype."""
    x = _normal(cfg, device, (T, cfg.d_model), 1.0, instance, "x", T)
    return x.to(_TORCH_DT[cfg.act_dtype])


def make_routing(cfg: LayerConfig, T: int, invalid: float = 0.0, device="cpu", instance: int = 0):
    """A routing drawn without a router, for layers fed a given routing: ids
    [T, top_k] int32 uniform over the experts (repeats within a token allowed), a
    fraction `invalid` of them replaced by ids outside [0, E) (-1 or E); weights
    [T, top_k] fp32 ~ U(0, 1) divided by their sum over the token's slots (the
    router's weights also sum to 1); the shared expert's scale [T] fp32 ~ U(0, 1)
    when the layer has one (else None)."""
    g = _gen(cfg, device, instance, "route", T)
    E = cfg.n_experts
    idx = torch.randint(0, E, (T, cfg.top_k), generator=g, device=device, dtype=torch.int64)
    if invalid > 0:
        bad = torch.rand((T, cfg.top_k), generator=g, device=device) < invalid
        alt = torch.where(torch.rand((T, cfg.top_k), generator=g, device=device) < 0.5, -1, E)
        idx = torch.where(bad, alt, idx)
    w = torch.rand((T, cfg.top_k), generator=g, device=device, dtype=torch.float32)
    w = w / w.sum(dim=1, keepdim=True)
    gs = torch.rand((T,), generator=g, device=device, dtype=torch.float32) if cfg.shared_d_ff else None
    return idx.to(torch.int32), w, gs


def layer_kwargs(L: SynthLayer, device) -> dict:
    """The keyword arguments of the binding's MoeLayer for this layer, its tensors
    moved to `device` (int4 weights stored two to a byte, as the library takes
    them). Marshalling only: no arithmetic of the layer."""
    c = L.cfg
    t = {k: v.to(device).contiguous() for k, v in L.tensors().items()}
    if c.expert_dtype == "i4":
        for k in ("w_gate", "w_up", "w_down"):
            t[k] = pack_int4_pairs(t[k]).contiguous()
    kw = dict(d_model=c.d_model, n_experts=c.n_experts, d_ff=c.d_ff, top_k=c.top_k,
              act_dtype=c.act_dtype, expert_dtype=c.expert_dtype, shared_d_ff=c.shared_d_ff)
    for k in ("w_router", "b_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
              "w_shared_gate", "ws_gate", "ws_up", "ws_down"):
        kw[k] = t.get(k)
    return kw
