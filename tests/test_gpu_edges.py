"""GPU parity on edge shapes and degenerate routings, at sizes the oracle evaluates in full.

Covers: k = 1, k = E and k up to the 64-slot limit, expert counts that are not multiples of 8 or 16 (up to the
128-expert limit), the smallest supported widths, T at the max_tokens bound and on
both sides of the streaming / tiled switch, every token routed to one expert, an
expert holding more rows than the streaming row tile (more tiles than active experts), a
shared expert of one and of sixteen d_ff slices, int8 output channels and int4
groups whose scale is zero, the smallest int4 widths, the decode routing paths for routers wider than 16 columns,
int8 token rows of extreme or widely spread magnitudes on both mid-size paths, and decode K loops
that end with steps after their last whole round.
"""
import numpy as np
import pytest
import torch

import synth
import oracle
from harness import MARGIN, Y_TOL, compare, gpu_layer, oracle_layer

pytestmark = pytest.mark.gpu


def _run(cfg, Ts, max_tokens=None, mutate=None):
    L = synth.make_layer(cfg)
    if mutate is not None:
        mutate(L)
    olay = oracle_layer(L)
    lay = gpu_layer(L, max_tokens or max(Ts))
    for T in Ts:
        print(f"[edge] {cfg.name} d={cfg.d_model} E={cfg.n_experts} F={cfg.d_ff} k={cfg.top_k} "
              f"Fs={cfg.shared_d_ff} T={T}", flush=True)
        x = synth.make_tokens(cfg, T).cuda()
        out = lay.forward(x, scatter=True)
        torch.cuda.synchronize()
        compare(cfg, x, olay, out, label=f"{cfg.name} E={cfg.n_experts} k={cfg.top_k} T={T}")
    lay.close()


@pytest.mark.parametrize("k", [1, 8])
def test_top_k_extremes(k):
    # k = 1: every weight is exactly 1; k = E = 8: the dense softmax mixture
    _run(synth.get_config("mixtral_bf16", d_model=256, d_ff=128, top_k=k), [1, 5, 70, 600])


@pytest.mark.parametrize("E,k", [(64, 16), (64, 64), (128, 32), (128, 64)])
def test_large_top_k(E, k):
    # k up to the 64-slot limit: k rounds of the wave maximum over up to 128 keys (two a
    # lane), the softmax over k slots, k*T assignments through the one-wave, one-workgroup
    # and wide scatters
    _run(synth.get_config("mixtral_bf16", d_model=128, d_ff=64, n_experts=E, top_k=k), [1, 3, 40, 300])


@pytest.mark.parametrize("E,k", [(5, 2), (13, 3), (127, 4), (128, 1)])
def test_odd_expert_counts(E, k):
    _run(synth.get_config("mixtral_bf16", d_model=128, d_ff=64, n_experts=E, top_k=k), [3, 64, 65, 700])


def test_smallest_widths():
    _run(synth.get_config("mixtral_bf16", d_model=128, d_ff=64), [1, 2, 64, 65, 513])
    _run(synth.get_config("tiny_f32", d_model=64, d_ff=64), [1, 64, 200])
    _run(synth.get_config("int8_mixtral22b", d_model=128, d_ff=64), [1, 100])


@pytest.mark.parametrize("name,d", [("mixtral_bf16", 8192), ("mixtral_bf16", 8320), ("tiny_f32", 8192), ("tiny_f32", 8320)])
def test_small_gate_width_limit(name, d):
    # the one-workgroup decode gate takes d_model <= 8192 (1024 threads x 8 elements: at 8192
    # every thread loads); 8320 runs the per-token gate instead. T = 1 (the one-token
    # instantiation) and 3 (four token slots)
    _run(synth.get_config(name, d_model=d, d_ff=64, n_experts=8, top_k=2), [1, 3])


def test_max_tokens_bound():
    # T == max_tokens on both sides of the streaming / tiled switch (T <= 64 streams, past it
    # the bf16 tile-stream GEMMs)
    cfg = synth.get_config("mixtral_bf16", d_model=256, d_ff=256)
    _run(cfg, [64], max_tokens=64)
    _run(cfg, [65, 300], max_tokens=300)


def test_every_token_on_one_expert():
    # a large bias on expert 3 puts it in slot 0 of every token: one expert holds T rows
    def bias(L):
        b = torch.zeros(L.cfg.n_experts, dtype=torch.float32)
        b[3] = 50.0
        L.b_router = b
    _run(synth.get_config("mixtral_bf16", d_model=256, d_ff=128), [1, 64, 1000], mutate=bias)


@pytest.mark.parametrize("name", ["mixtral_bf16", "int8_mixtral22b", "int4_mixtral22b"])
def test_streaming_expert_past_one_tile(name):
    # a bias of 2 on expert 3 puts it in slot 0 of (nearly) every token while the slot-1
    # weights stay near 0.2: at T = 32 (and 64 for bf16 weights) expert 3 holds T rows, twice
    # the streaming row tile, so the tiles outnumber the active experts (9 against 8 for this
    # draw); quantised weights take the tile-stream kernels at T = 64, with one expert over
    # its 64-row tile
    def bias(L):
        b = torch.zeros(L.cfg.n_experts, dtype=torch.float32)
        b[3] = 2.0
        L.b_router = b
    _run(synth.get_config(name, d_model=256, d_ff=128), [32, 64], mutate=bias)


@pytest.mark.parametrize("name,d", [("mixtral_bf16", 384), ("mixtral_bf16", 640), ("int8_mixtral22b", 384),
                                    ("int4_mixtral22b", 640)])
def test_streaming_partial_rounds(name, d):
    # the decode streams run their K steps in rounds (8 steps of 32 for the bf16 up
    # projection, 2 otherwise) and the steps left after the last round one at a time:
    # d = 384 and 640 leave 4 steps after one or two bf16 up rounds
    kw = dict(d_model=d, d_ff=256 if name == "int4_mixtral22b" else 128)
    _run(synth.get_config(name, **kw), [1, 3, 16, 32])


@pytest.mark.parametrize("slices", [1, 16])
def test_shared_expert_slices(slices):
    cfg = synth.get_config("shared_fine_bf16", d_model=256, d_ff=64, n_experts=8, top_k=2,
                           shared_d_ff=64 * slices)
    _run(cfg, [1, 16, 300])


def test_int8_zero_scale_channels():
    # output channels quantised from all-zero weights have s = 0 and q = 0
    def zero(L):
        L.w_gate[2, :, 5] = 0
        L.s_gate[2, 5] = 0
        L.w_down[1, :, 7] = 0
        L.s_down[1, 7] = 0
    _run(synth.get_config("int8_mixtral22b", d_model=256, d_ff=128), [1, 300], mutate=zero)


@pytest.mark.parametrize("d_model", [256, 384])
def test_int8_extreme_rows(d_model):
    # int8 experts past the streaming sizes on token rows of extreme magnitude: rows scaled
    # by 1e15 and 1e-15, an all-zero row (its output is exactly zero), and rows spanning 2^20
    # and 2^40 inside themselves. Each row is checked against the oracle on its own scale.
    # d_model = 256: the tile-stream kernels; 384 (a partial last column tile): the
    # LDS-tiled ones.
    cfg = synth.get_config("int8_mixtral22b", d_model=d_model, d_ff=256)
    L = synth.make_layer(cfg)
    olay = oracle_layer(L)
    T = 200
    lay = gpu_layer(L, T)
    x = synth.make_tokens(cfg, T).float()
    x[0] = 0.0
    x[1] *= 1e15
    x[2] *= 1e-15
    x[3, 17] = 1e6
    x[4, 200] = -1e12
    x = x.to(torch.bfloat16).cuda()
    print(f"[edge] int8 token scales d={cfg.d_model} F={cfg.d_ff} T={T}", flush=True)
    out = lay.forward(x)
    torch.cuda.synchronize()
    lay.close()
    xn = x.float().cpu().numpy().astype(np.float64)
    gidx = out.topk_idx.cpu().numpy().astype(np.int64)
    with np.errstate(over="ignore"):  # silu(z) = z / (1 + exp(-z)) at z ~ -1e30: exp overflows, the quotient is -0
        ref = oracle.moe_forward(xn, olay)
    for t in range(T):
        if ref["margin"][t] >= MARGIN:
            assert np.array_equal(gidx[t], ref["idx"][t]), f"token {t}: top-k {gidx[t]} against {ref['idx'][t]}"
        else:
            assert any(np.array_equal(a, gidx[t]) for a in oracle.valid_selections(ref["logits"][t], cfg.top_k, MARGIN))
    with np.errstate(over="ignore"):
        ref = oracle.moe_forward(xn, olay, routing=gidx)
    y = out.y.float().cpu().numpy().astype(np.float64)
    assert np.all(y[0] == 0.0), "an all-zero token row gives exactly zero"
    rel, mabs = Y_TOL["bf16"]
    for t in range(1, T):
        yr = ref["y"][t]
        den = np.linalg.norm(yr)
        rms = den / np.sqrt(yr.size)
        err = y[t] - yr
        assert np.all(np.isfinite(y[t])), f"token {t}: non-finite output"
        assert np.linalg.norm(err) <= rel * den, f"token {t}: relative error {np.linalg.norm(err) / den:.3e}"
        assert np.abs(err).max() <= mabs * rms, f"token {t}: max-abs error {np.abs(err).max() / rms:.3e} rms"


@pytest.mark.parametrize("name", ["int8_mixtral22b", "int4_mixtral22b"])
def test_quantised_every_expert_chosen(name):
    # k = E = 3: every token on every expert, both kernel families
    _run(synth.get_config(name, d_model=256, d_ff=256, n_experts=3, top_k=3), [5, 40, 100])


def test_int4_zero_groups_and_smallest_width():
    # groups quantised from all-zero weights have s = 0 and q = 0; d_model = d_ff = 128
    # is one scale group along each input axis
    def zero(L):
        L.w_gate[2, 128:256, 5] = 0
        L.s_gate[2, 1, 5] = 0
        L.w_down[1, 0:128, 7] = 0
        L.s_down[1, 0, 7] = 0
    _run(synth.get_config("int4_mixtral22b", d_model=256, d_ff=256), [1, 300], mutate=zero)
    _run(synth.get_config("int4_mixtral22b", d_model=128, d_ff=128), [1, 70])


def test_wide_router_decode_paths():
    # more than 16 router columns at T <= 64: the split gate (k <= 8), fp32 tokens included,
    # and the per-token gate kernel when k > 8
    _run(synth.get_config("tiny_f32", d_model=64, d_ff=64, n_experts=32, top_k=4), [1, 8, 64])
    _run(synth.get_config("mixtral_bf16", d_model=128, d_ff=64, n_experts=32, top_k=10), [1, 8, 64])
    # split gate with more than 256 assignments: its scatter runs on the whole workgroup
    _run(synth.get_config("mixtral_bf16", d_model=128, d_ff=64, n_experts=32, top_k=8), [33, 64])


@pytest.mark.parametrize("name,kw,Ts", [
    ("mixtral_bf16", dict(d_model=256, d_ff=128), [1, 5, 300]),       # fused tiny, per-token, MFMA gates
    ("tiny_f32", dict(d_model=64, d_ff=64), [1, 100]),                 # fp32 tokens: fused tiny, tiled gate
    ("mixtral_bf16", dict(d_model=128, d_ff=64, n_experts=32, top_k=4), [32]),  # split decode gate
])
def test_gate_clamp(name, kw, Ts):
    # a bias of 49.9 on three experts puts their logits on both sides of the bound: the
    # clamped ones tie at 50 (lower id first, equal weights)
    cfg = synth.get_config(name, **kw)
    L = synth.make_layer(cfg)
    b = torch.zeros(cfg.n_experts, dtype=torch.float32)
    b[[1, 2, 4]] = 49.9
    L.b_router = b
    olay = oracle_layer(L, gate_clamp=True)
    lay = gpu_layer(L, max(Ts), gate_clamp=True)
    for T in Ts:
        print(f"[edge] gate clamp {cfg.name} E={cfg.n_experts} k={cfg.top_k} T={T}", flush=True)
        x = synth.make_tokens(cfg, T).cuda()
        out = lay.forward(x, scatter=True)
        torch.cuda.synchronize()
        compare(cfg, x, olay, out, label=f"clamp {cfg.name} T={T}")
        # the clamp is active: some token holds two tied experts at equal weights
        w = out.topk_w.cpu()
        assert ((w[:, 0] - w[:, 1]).abs() < 1e-7).any() or T < 32
    lay.close()


@pytest.mark.parametrize("name,kw,Ts,clamp", [
    ("mixtral_bf16", dict(d_model=256, d_ff=128), [1, 5, 300], False),       # fused tiny, per-token, MFMA gates
    ("tiny_f32", dict(d_model=64, d_ff=64), [1, 100], False),                 # fp32 tokens: fused tiny, tiled gate
    ("mixtral_bf16", dict(d_model=128, d_ff=64, n_experts=32, top_k=4), [16], False),  # split decode gate
    ("mixtral_bf16", dict(d_model=128, d_ff=64, n_experts=32, top_k=10), [8], False),  # per-token gate, k > 8
    ("shared_fine_bf16", dict(d_model=256, d_ff=128, shared_d_ff=512), [3, 16, 200], False),  # shared column
    ("int8_mixtral22b", dict(d_model=256, d_ff=128), [2, 70], False),        # int8 streaming and tile-stream experts
    ("mixtral_bf16", dict(d_model=256, d_ff=128), [1, 300], True),           # raw weights of clamped logits
])
def test_gate_raw_weighting(name, kw, Ts, clamp):
    # the routing weights are the chosen logits themselves, on every gate path; the expert
    # kernels and the combine take them as they take softmax weights
    cfg = synth.get_config(name, **kw)
    L = synth.make_layer(cfg)
    if clamp:
        b = torch.zeros(cfg.n_experts, dtype=torch.float32)
        b[[1, 2, 4]] = 49.9
        L.b_router = b
    olay = oracle_layer(L, gate_clamp=clamp)
    olay.gate_weighting = "raw"
    lay = gpu_layer(L, max(Ts), gate_clamp=clamp, gate_weighting="raw")
    for T in Ts:
        print(f"[edge] raw weighting {cfg.name} E={cfg.n_experts} k={cfg.top_k} T={T} clamp={clamp}", flush=True)
        x = synth.make_tokens(cfg, T).cuda()
        out = lay.forward(x, scatter=True)
        torch.cuda.synchronize()
        r = compare(cfg, x, olay, out, label=f"raw {cfg.name} T={T}")
        # raw weights do not sum to one (softmax weights would)
        w = out.topk_w.cpu().double()
        assert (w.sum(1) - 1).abs().max() > 1e-3, r
        if clamp:
            assert (w == 50.0).any()
    lay.close()


@pytest.mark.parametrize("d,T", [(384, 65), (384, 300), (640, 129), (1664, 1000), (256, 7000)])
def test_mfma_gate_slices(d, T):
    # the MFMA gate's (128-token tile, K slice) grid: K of 12, 20, 52 and 8 steps of 32 split
    # into slices of unequal counts, ragged last token tiles, and a shared gate column
    cfg = synth.get_config("shared_fine_bf16", d_model=d, d_ff=128, n_experts=24, top_k=3, shared_d_ff=256)
    _run(cfg, [T])
