"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one layer, one moe_forward per batch).

Routing (indices, weights, counts, offsets, permutation) and outputs are
compared for every token at every size, prefill batches included (the oracle
evaluates the whole batch one expert at a time, a few seconds each), so every
row tile and column tile the GEMMs deal out is checked. Layers are drawn on the
GPU with torch's seeded generator to keep set-up short; the oracle gets host
copies of the same tensors.
"""
import numpy as np
import pytest
import torch

import synth
from harness import compare, gpu_layer, oracle_layer

pytestmark = pytest.mark.gpu


def _run(name, Ts):
    cfg = synth.get_config(name)
    print(f"[fullsize] generating {name}", flush=True)
    L = synth.make_layer(cfg, device="cuda")
    olay = oracle_layer(L)
    lay = gpu_layer(L, max(Ts))
    out = {}
    for T in Ts:
        print(f"[fullsize] {name} T={T}", flush=True)
        x = synth.make_tokens(cfg, T, device="cuda")
        r = lay.forward(x, scatter=True)
        torch.cuda.synchronize()
        out[T] = compare(cfg, x, olay, r, label=f"{name} T={T}")
        print(f"[fullsize] {name} T={T} {out[T]}", flush=True)
    lay.close()
    del L, olay
    torch.cuda.empty_cache()
    return out


def test_mixtral_bf16_full():
    # T <= 64 on the streaming kernels, 128 and 384 on the tile-stream ones with 128-row
    # tiles, 512 with 160-row tiles, 4096 on the LDS-tiled GEMMs
    _run("mixtral_bf16", [1, 8, 32, 64, 128, 384, 512, 4096])


def test_shared_fine_bf16_full():
    _run("shared_fine_bf16", [16, 2048])


def test_skewed_bf16_full():
    r = _run("skewed_bf16", [8192])
    assert r[8192]["excluded"] >= 0


def test_int8_mixtral22b_full():
    # T = 1, 16 on the streaming kernels; 64, 256 and 512 on the tile-stream ones (512:
    # experts over one 128-row tile, the down projection's K split four ways)
    _run("int8_mixtral22b", [1, 16, 64, 256, 512])


def test_int4_mixtral22b_full():
    _run("int4_mixtral22b", [1, 16, 64, 256, 512])


def test_mixtral_bf16_routed_full():
    # the given-routing entry at full size: scatter tables bit for bit, outputs on every row
    from harness import Y_TOL, _np
    import oracle
    cfg = synth.get_config("mixtral_bf16")
    L = synth.make_layer(cfg, device="cuda")
    olay = oracle_layer(L)
    lay = gpu_layer(L, 4096)
    for T in (1, 64, 4096):
        print(f"[fullsize] routed mixtral_bf16 T={T}", flush=True)
        x = synth.make_tokens(cfg, T, device="cuda")
        idx, w, _ = synth.make_routing(cfg, T, device="cuda")
        out = lay.forward_routed(x, idx, w, scatter=True)
        torch.cuda.synchronize()
        ref = oracle.moe_forward_routed(_np(x), olay, idx.cpu().numpy(), w.cpu().numpy())
        assert np.array_equal(out.expert_counts.cpu().numpy(), ref["counts"])
        assert np.array_equal(out.expert_offsets.cpu().numpy(), ref["offsets"])
        assert np.array_equal(out.sorted_assign.cpu().numpy(), ref["sorted_assign"])
        y = _np(out.y).astype(np.float64)
        yr = ref["y"]
        rel, mabs = Y_TOL[cfg.act_dtype]
        den = np.linalg.norm(yr)
        rms = den / np.sqrt(yr.size)
        assert np.linalg.norm(y - yr) / den <= rel
        assert np.abs(y - yr).max() <= mabs * rms
    lay.close()
