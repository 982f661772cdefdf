"""GPU parity of moe_forward_routed: the layer fed a routing drawn without the router
([pptc §3.4]: the engine consumes routing results produced elsewhere, token-major).

Covers: fp32, bf16, int8, int4 and shared-expert layers; T on both sides of the
streaming / tiled switch and of the single / multi-workgroup scatter; repeated
experts within a token and ids outside [0, E) (read as expert 0 at weight 0); the
scatter tables bit for bit; and bit-identity with moe_forward when it is given
moe_forward's own routing.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import moe_layer_forward_gate_amd as moe
from harness import Y_TOL, _np, gpu_layer, oracle_layer

pytestmark = pytest.mark.gpu


def _check(cfg, olay, x, idx, w, gs, out, label):
    ref = oracle.moe_forward_routed(_np(x), olay, idx.numpy(), w.numpy(), None if gs is None else gs.numpy())
    assert np.array_equal(out.expert_counts.cpu().numpy(), ref["counts"]), f"{label}: counts differ"
    assert np.array_equal(out.expert_offsets.cpu().numpy(), ref["offsets"]), f"{label}: offsets differ"
    assert np.array_equal(out.sorted_assign.cpu().numpy(), ref["sorted_assign"]), f"{label}: permutation differs"
    y = _np(out.y).astype(np.float64)
    yr = ref["y"]
    rel, mabs = Y_TOL[cfg.act_dtype]
    den = np.linalg.norm(yr)
    rms = den / np.sqrt(yr.size)
    frob = float(np.linalg.norm(y - yr) / den)
    mx = float(np.abs(y - yr).max())
    assert frob <= rel, f"{label}: relative Frobenius error {frob:.3e} > {rel}"
    assert mx <= mabs * rms, f"{label}: max-abs error {mx:.3e} > {mabs} * rms {rms:.3e}"


def _run(cfg, Ts, invalid=0.1):
    L = synth.make_layer(cfg)
    olay = oracle_layer(L)
    lay = gpu_layer(L, max(Ts))
    for T in Ts:
        label = f"{cfg.name} d={cfg.d_model} E={cfg.n_experts} F={cfg.d_ff} k={cfg.top_k} Fs={cfg.shared_d_ff} T={T}"
        print(f"[routed] {label}", flush=True)
        x = synth.make_tokens(cfg, T)
        idx, w, gs = synth.make_routing(cfg, T, invalid=invalid)
        out = lay.forward_routed(x.cuda(), idx.cuda(), w.cuda(), None if gs is None else gs.cuda(), scatter=True)
        torch.cuda.synchronize()
        _check(cfg, olay, x, idx, w, gs, out, label)
    lay.close()


def test_routed_f32():
    _run(synth.get_config("tiny_f32"), [1, 64, 200])


def test_routed_bf16():
    # streaming (T <= 64), tile-stream (65), LDS-tiled (700, 2100), and the multi-workgroup
    # scatter (T * k > 4095)
    _run(synth.get_config("mixtral_bf16", d_model=256, d_ff=256), [1, 5, 64, 65, 700, 2100])


def test_routed_int8():
    _run(synth.get_config("int8_mixtral22b", d_model=256, d_ff=128), [1, 16, 300])


def test_routed_int4():
    _run(synth.get_config("int4_mixtral22b", d_model=256, d_ff=256), [1, 16, 300])


def test_routed_shared_expert_and_many_experts():
    _run(synth.get_config("shared_fine_bf16", d_model=256, d_ff=64, n_experts=16, top_k=4, shared_d_ff=256),
         [1, 16, 300])
    _run(synth.get_config("skewed_bf16", d_model=256, d_ff=128), [3, 400])


@pytest.mark.parametrize("name,kw", [
    ("mixtral_bf16", dict(d_model=256, d_ff=256)),
    ("shared_fine_bf16", dict(d_model=256, d_ff=64, n_experts=16, top_k=4, shared_d_ff=256)),
    ("int8_mixtral22b", dict(d_model=256, d_ff=128)),
    ("tiny_f32", {}),
])
def test_routed_with_own_routing_is_bit_identical(name, kw):
    cfg = synth.get_config(name, **kw)
    L = synth.make_layer(cfg)
    lay = gpu_layer(L, 300)
    for T in (1, 3, 64, 300):  # fused tiny gate, per-token gate, streaming, tiled (tile-stream or LDS-tiled)
        x = synth.make_tokens(cfg, T).cuda()
        a = lay.forward(x, scatter=True)
        b = lay.forward_routed(x, a.topk_idx, a.topk_w, a.shared_gate, scatter=True)
        torch.cuda.synchronize()
        label = f"{name} T={T}"
        assert torch.equal(a.y, b.y), f"{label}: y differs"
        for f in ("expert_counts", "expert_offsets", "sorted_assign"):
            assert torch.equal(getattr(a, f), getattr(b, f)), f"{label}: {f} differs"
    lay.close()


def test_routed_int4_tile_boundaries():
    # int4 tile-stream at 41-72 rows per expert on average (T = 200, k = 2, E = 8: 50): 80-row
    # up tiles and 64-row down tiles, H written in the down tiling. Experts holding exactly
    # 64, 65, 80 and 81 rows (one tile or two in either tiling), 1 row, and none.
    cfg = synth.get_config("int4_mixtral22b", d_model=256, d_ff=256)
    T, k = 200, cfg.top_k
    counts = [64, 65, 80, 81, 1, 0, 59, 50]
    assert sum(counts) == T * k and len(counts) == cfg.n_experts
    rng = np.random.default_rng(7)
    ids = np.repeat(np.arange(cfg.n_experts), counts)
    rng.shuffle(ids)
    idx = torch.from_numpy(ids.reshape(T, k).astype(np.int32))
    w = torch.from_numpy(rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32))
    L = synth.make_layer(cfg)
    olay = oracle_layer(L)
    lay = gpu_layer(L, T)
    x = synth.make_tokens(cfg, T)
    print(f"[routed] int4 tile boundaries T={T} counts={counts}", flush=True)
    out = lay.forward_routed(x.cuda(), idx.cuda(), w.cuda(), None, scatter=True)
    torch.cuda.synchronize()
    _check(cfg, olay, x, idx, w, None, out, "int4 tile boundaries")
    lay.close()


def test_routed_bf16_tile_stream_tiles():
    # bf16 tile-stream (128-row tiles; T = 214, k = 2 over 8 experts: 53.5 rows on average):
    # experts at 150 (a second tile of 22 rows), 128, 129 (a second tile of one row), 1 and no rows
    cfg = synth.get_config("mixtral_bf16", d_model=256, d_ff=256)
    T, k = 214, cfg.top_k
    counts = [150, 128, 0, 1, 129, 0, 20, 0]
    assert sum(counts) == T * k and len(counts) == cfg.n_experts
    rng = np.random.default_rng(11)
    ids = np.repeat(np.arange(cfg.n_experts), counts)
    rng.shuffle(ids)
    ids = ids.reshape(T, k)
    idx = torch.from_numpy(ids.astype(np.int32))
    w = torch.from_numpy(rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32))
    L = synth.make_layer(cfg)
    olay = oracle_layer(L)
    lay = gpu_layer(L, T)
    x = synth.make_tokens(cfg, T)
    print(f"[routed] bf16 tile-stream tiles T={T} counts={counts}", flush=True)
    out = lay.forward_routed(x.cuda(), idx.cuda(), w.cuda(), None, scatter=True)
    torch.cuda.synchronize()
    _check(cfg, olay, x, idx, w, None, out, "bf16 tile-stream tiles")
    lay.close()


def test_routed_argument_checks():
    cfg = synth.get_config("shared_fine_bf16", d_model=256, d_ff=64, n_experts=8, top_k=2, shared_d_ff=128)
    lay = gpu_layer(synth.make_layer(cfg), 8)
    x = synth.make_tokens(cfg, 4).cuda()
    idx, w, gs = (t.cuda() for t in synth.make_routing(cfg, 4))
    with pytest.raises(moe.MoeError) as e:
        lay.forward_routed(x, idx, w, None)  # the layer has a shared expert
    assert e.value.status == moe.MOE_EINVAL
    lay.close()
    cfg = synth.get_config("mixtral_bf16", d_model=256, d_ff=256)
    lay = gpu_layer(synth.make_layer(cfg), 8)
    x = synth.make_tokens(cfg, 4).cuda()
    idx, w, _ = (None if t is None else t.cuda() for t in synth.make_routing(cfg, 4))
    with pytest.raises(moe.MoeError) as e:
        lay.forward_routed(x, idx, w, torch.ones(4, device="cuda"))  # no shared expert
    assert e.value.status == moe.MOE_EINVAL
    lay.close()
