"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test targets a plausible slip in the oracle (a dropped bias, a transposed
operand, the wrong SwiGLU branch, a misaligned routing weight, an unstable
grouping, a per-input-channel scale) and checks it against something other than
the oracle's own formula: hand-worked fixtures, closed forms, library routines
(scipy's logistic and softmax, torch's SiLU) and brute force on tiny inputs.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_layer(rng, d, E, F, k, bias=False, shared=0, int8=False):
    wg = rng.standard_normal((E, d, F)) / np.sqrt(d)
    wu = rng.standard_normal((E, d, F)) / np.sqrt(d)
    wd = rng.standard_normal((E, F, d)) / np.sqrt(F)
    kw = {}
    if int8:
        # quantise with the generator's own routine (torch), then hand q and s to the oracle
        qs = [synth.quantize_per_out_channel(torch.from_numpy(w).float()) for w in (wg, wu, wd)]
        (wg, sg), (wu, su), (wd, sd) = [(q.numpy(), s.numpy()) for q, s in qs]
        kw = dict(s_gate=sg, s_up=su, s_down=sd)
    lay = oracle.OracleLayer(w_router=rng.standard_normal((d, E)) * 0.3, w_gate=wg, w_up=wu,
                             w_down=wd, top_k=k, **kw)
    if bias:
        lay.b_router = rng.standard_normal(E)
    if shared:
        lay.w_shared_gate = rng.standard_normal(d) * 0.3
        lay.ws_gate = rng.standard_normal((d, shared)) / np.sqrt(d)
        lay.ws_up = rng.standard_normal((d, shared)) / np.sqrt(d)
        lay.ws_down = rng.standard_normal((shared, d)) / np.sqrt(shared)
    return lay


def _torch_swiglu(x, wg, wu, wd):
    """Textbook SwiGLU with torch's SiLU, float64 on the CPU."""
    x, wg, wu, wd = (torch.as_tensor(np.asarray(a, dtype=np.float64)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg) * (x @ wu) @ wd).numpy()


def _dense_masked(x, lay):
    """Brute force: y_t = sum over ALL experts of 1[e chosen] * w_te * FFN_e(x_t),
    with the choice from a full stable sort and the weights from scipy's softmax."""
    x = np.asarray(x, dtype=np.float64)
    T, E, k = x.shape[0], lay.n_experts, lay.top_k
    logits = x @ np.asarray(lay.w_router, dtype=np.float64)
    if lay.b_router is not None:
        logits = logits + lay.b_router
    y = np.zeros_like(x)
    for t in range(T):
        order = np.argsort(-logits[t], kind="stable")
        chosen = order[:k]
        p = softmax(logits[t][chosen])
        for e in range(E):
            wg, wu, wd = lay.expert(e)
            ffn = _torch_swiglu(x[t:t + 1], wg, wu, wd)[0]
            mask = 1.0 if e in chosen else 0.0
            we = p[list(chosen).index(e)] if e in chosen else 0.0
            y[t] += mask * we * ffn
    if lay.w_shared_gate is not None:
        g = expit(x @ lay.w_shared_gate)
        y += g[:, None] * _torch_swiglu(x, lay.ws_gate, lay.ws_up, lay.ws_down)
    return y


# ------------------------------------------------------------------ Gate
def test_router_logits_table_lookup_and_bias():
    # x rows are unit vectors, so logits[t] must be row i_t of W_r plus b: a
    # transposed W_r (d != E) or a dropped bias fails.
    d, E = 5, 3
    W = np.arange(d * E, dtype=np.float64).reshape(d, E) * 0.5 - 3.0
    b = np.array([10.0, -20.0, 0.25])
    rows = [4, 0, 2, 2, 1]
    x = np.eye(d)[rows]
    got = oracle.router_logits(x, W, b)
    want = np.array([[W[i, e] + b[e] for e in range(E)] for i in rows])
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.router_logits(x, W), W[rows])


def test_topk_hand_fixture():
    g = _load("topk_hand.json")
    for case in g["cases"]:
        L = np.array([case["logits"]])
        idx, _ = oracle.select_topk(L, g["top_k"])
        assert idx[0].tolist() == case["idx"], case
        if "w" in case:
            w = oracle.topk_weights(L, idx)
            assert np.allclose(w[0], case["w"], rtol=0, atol=1e-15)


def test_zero_router_closed_form():
    # all logits equal: the tie rule picks experts 0..k-1 and every weight is 1/k
    rng = np.random.default_rng(1)
    for E, k in [(8, 2), (64, 8), (128, 4), (5, 5)]:
        x = rng.standard_normal((7, 16))
        L = oracle.router_logits(x, np.zeros((16, E)))
        idx, margin = oracle.select_topk(L, k)
        assert (idx == np.arange(k)[None, :]).all()
        assert np.array_equal(oracle.topk_weights(L, idx), np.full((7, k), 1.0 / k))
        if k < E:
            assert (margin == 0).all()


def test_topk_bruteforce_small():
    # exhaustive search over k-subsets and slot orders on tiny E, with ties
    rng = np.random.default_rng(2)
    for trial in range(300):
        E = int(rng.integers(2, 7))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 4, size=E).astype(np.float64)  # many exact ties
        best = None
        for S in itertools.permutations(range(E), k):
            key = [(-l[e], e) for e in S]
            if all(key[i] < key[i + 1] for i in range(k - 1)):
                rest = [e for e in range(E) if e not in S]
                if all((-l[s], s) < (-l[r], r) for s in S for r in rest):
                    best = list(S)
        idx, margin = oracle.select_topk(l[None, :], k)
        assert idx[0].tolist() == best
        srt = sorted(l, reverse=True)
        if k < E:
            assert margin[0] == srt[k - 1] - srt[k]


def test_topk_weights_closed_forms():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 8)) * 2.0
    # k = 2: w0 is the logistic of the logit gap
    idx, _ = oracle.select_topk(L, 2)
    w = oracle.topk_weights(L, idx)
    gap = L[np.arange(50), idx[:, 0]] - L[np.arange(50), idx[:, 1]]
    assert np.allclose(w[:, 0], expit(gap), rtol=0, atol=1e-15)
    # k = 1: weight 1
    idx1, _ = oracle.select_topk(L, 1)
    assert np.array_equal(oracle.topk_weights(L, idx1), np.ones((50, 1)))
    # k = E: the dense softmax in slot order
    idxE, _ = oracle.select_topk(L, 8)
    wE = oracle.topk_weights(L, idxE)
    assert np.allclose(wE, np.take_along_axis(softmax(L, axis=1), idxE, axis=1), atol=1e-15)
    # any k: the full softmax renormalised over the chosen set; sums to 1
    for k in (2, 3, 5):
        idk, _ = oracle.select_topk(L, k)
        wk = oracle.topk_weights(L, idk)
        full = np.take_along_axis(softmax(L, axis=1), idk, axis=1)
        assert np.allclose(wk, full / full.sum(1, keepdims=True), atol=1e-14)
        assert np.abs(wk.sum(1) - 1).max() < 1e-12
        # slot order: weights non-increasing
        assert (np.diff(wk, axis=1) <= 1e-15).all()


def test_forced_routing_pattern():
    # The worked example of [pptc §4] routes token b's slot j to expert
    # (b*k + j) mod E. Force it through one-hot tokens and a descending router row.
    T, E, k = 6, 4, 2
    x = np.eye(T)
    W = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            W[t, (t * k + j) % E] = 10.0 - j
    idx, margin = oracle.select_topk(oracle.router_logits(x, W), k)
    assert idx.tolist() == [[(t * k + j) % E for j in range(k)] for t in range(T)]
    assert (margin == 9.0).all()


def test_shared_gate():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 12))
    assert np.array_equal(oracle.shared_gate(x, np.zeros(12)), np.full(9, 0.5))
    ws = rng.standard_normal(12)
    assert np.allclose(oracle.shared_gate(x, ws), expit(x @ ws), atol=1e-15)


# ------------------------------------------------------------------ Scatter
def test_scatter_hand_fixture():
    g = _load("scatter_hand.json")
    for fn in (oracle.scatter_stable_sort, oracle.scatter_counting):
        c, o, s = fn(np.array(g["idx"]), g["n_experts"])
        assert c.tolist() == g["counts"]
        assert o.tolist() == g["offsets"]
        assert s.tolist() == g["sorted_assign"]


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (64, 8, 2), (333, 64, 8), (1000, 128, 4), (0, 8, 2)])
def test_scatter_formulations_agree_and_invariants(T, E, k):
    rng = np.random.default_rng(T + E)
    L = rng.standard_normal((T, E))
    if T:
        L[: T // 3, 3] += 5.0  # skew
    idx, _ = oracle.select_topk(L, k) if T else (np.zeros((0, k), dtype=np.int64), None)
    c1, o1, s1 = oracle.scatter_stable_sort(idx, E)
    c2, o2, s2 = oracle.scatter_counting(idx, E)
    assert np.array_equal(c1, c2) and np.array_equal(o1, o2) and np.array_equal(s1, s2)
    assert c1.sum() == T * k and o1[0] == 0 and o1[-1] == T * k
    assert (np.diff(o1) == c1).all()
    assert np.array_equal(np.sort(s1), np.arange(T * k))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = s1[o1[e]:o1[e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()  # stable: increasing assignment id


# ------------------------------------------------------------------ Expert compute
def test_swiglu_scalar_closed_form():
    # d = F = 1: y = silu(a) * b * c with silu from scipy's logistic; a != b so a
    # swapped gate/up branch fails, and c != 1 so a dropped down projection fails.
    for a, b, c in [(1.5, -0.7, 3.0), (-2.0, 0.4, -0.5), (0.0, 5.0, 2.0)]:
        got = oracle.swiglu_expert(np.array([[1.0]]), np.array([[a]]), np.array([[b]]), np.array([[c]]))
        assert np.allclose(got, a * expit(a) * b * c, rtol=1e-15, atol=1e-300)


def test_swiglu_matches_torch_textbook():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 24))
    wg, wu = rng.standard_normal((24, 40)), rng.standard_normal((24, 40))
    wd = rng.standard_normal((40, 24))
    assert np.allclose(oracle.swiglu_expert(x, wg, wu, wd), _torch_swiglu(x, wg, wu, wd), rtol=1e-13, atol=1e-13)


def test_dequantize_roundtrip_and_axis():
    # per-output-channel scales that differ by 1000x across columns: a scale
    # applied along the wrong axis breaks the half-step round-trip bound.
    rng = np.random.default_rng(6)
    w = rng.standard_normal((3, 32, 16)) * np.logspace(-3, 0, 16)[None, None, :]
    q, s = synth.quantize_per_out_channel(torch.from_numpy(w).float())
    q, s = q.numpy(), s.numpy()
    assert q.dtype == np.int8 and s.shape == (3, 16)
    assert (np.abs(q).max(axis=1) == 127).all()
    deq = oracle.dequantize(q, s)
    w32 = torch.from_numpy(w).float().double().numpy()
    assert (np.abs(deq - w32) <= s[:, None, :] * 0.5 * (1 + 1e-6)).all()
    # q * s is exact in fp64
    assert np.array_equal(deq, q.astype(np.float64) * s.astype(np.float64)[:, None, :])


# ------------------------------------------------------------------ Layer
def test_dense_masked_bruteforce_tiny_f32_full():
    cfg = synth.get_config("tiny_f32")
    L = synth.make_layer(cfg)
    x = synth.make_tokens(cfg, 64)
    lay = oracle.OracleLayer(L.w_router.numpy(), L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), cfg.top_k)
    out = oracle.moe_forward(x.numpy(), lay)
    ref = _dense_masked(x.numpy(), lay)
    assert np.abs(out["y"] - ref).max() <= 1e-12 * np.abs(ref).max()
    assert out["counts"].sum() == 64 * 2
    assert np.abs(out["w"].sum(1) - 1).max() < 1e-12
    for row in out["idx"]:
        assert len(set(row.tolist())) == len(row)


@pytest.mark.parametrize("bias,shared,int8,k", [(True, 0, False, 3), (False, 48, False, 2), (False, 0, True, 2), (True, 32, True, 4)])
def test_dense_masked_bruteforce_variants(bias, shared, int8, k):
    rng = np.random.default_rng(7 + k)
    lay = _rand_layer(rng, d=20, E=6, F=28, k=k, bias=bias, shared=shared, int8=int8)
    x = rng.standard_normal((11, 20))
    out = oracle.moe_forward(x, lay)
    ref = _dense_masked(x, lay)
    assert np.abs(out["y"] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    # sampled tokens give the same rows as the full evaluation
    sub = oracle.moe_forward(x, lay, tokens=[9, 2, 5])
    assert np.allclose(sub["y"], out["y"][[9, 2, 5]], rtol=0, atol=1e-13)


def test_identical_experts_is_one_swiglu():
    # identical experts: the weights sum to 1, so routing cannot matter
    rng = np.random.default_rng(8)
    d, E, F = 16, 5, 24
    wg, wu, wd = rng.standard_normal((d, F)), rng.standard_normal((d, F)), rng.standard_normal((F, d))
    lay = oracle.OracleLayer(rng.standard_normal((d, E)), np.stack([wg] * E), np.stack([wu] * E),
                             np.stack([wd] * E), top_k=3)
    x = rng.standard_normal((13, d))
    assert np.allclose(oracle.moe_forward(x, lay)["y"], _torch_swiglu(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def test_combine_weight_alignment():
    # expert e's output is (e+1) times a common FFN, so y = (sum_j w_j (idx_j + 1)) FFN_0.
    rng = np.random.default_rng(9)
    d, E, F, k = 12, 6, 10, 3
    wg, wu, wd = rng.standard_normal((d, F)), rng.standard_normal((d, F)), rng.standard_normal((F, d))
    lay = oracle.OracleLayer(rng.standard_normal((d, E)), np.stack([wg] * E), np.stack([wu] * E),
                             np.stack([wd * (e + 1) for e in range(E)]), top_k=k)
    x = rng.standard_normal((17, d))
    out = oracle.moe_forward(x, lay)
    L = x @ lay.w_router
    order = np.argsort(-L, axis=1, kind="stable")[:, :k]
    p = softmax(np.take_along_axis(L, order, axis=1), axis=1)
    scale = (p * (order + 1)).sum(1)
    assert np.allclose(out["y"], scale[:, None] * _torch_swiglu(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def test_zero_and_linear_down_projection():
    rng = np.random.default_rng(10)
    lay = _rand_layer(rng, d=16, E=4, F=8, k=2)
    x = rng.standard_normal((5, 16))
    y1 = oracle.moe_forward(x, lay)["y"]
    lay.w_down = lay.w_down * 2.5
    assert np.allclose(oracle.moe_forward(x, lay)["y"], 2.5 * y1, rtol=1e-14, atol=1e-14)
    lay.w_down = lay.w_down * 0.0
    assert np.array_equal(oracle.moe_forward(x, lay)["y"], np.zeros_like(y1))


def test_shared_expert_alone_is_half_swiglu():
    # w_s = 0 gives gate 1/2; zero routed down projections leave y = S(x) / 2
    rng = np.random.default_rng(11)
    lay = _rand_layer(rng, d=16, E=4, F=8, k=2, shared=24)
    lay.w_shared_gate = np.zeros(16)
    lay.w_down = lay.w_down * 0.0
    x = rng.standard_normal((6, 16))
    out = oracle.moe_forward(x, lay)
    assert np.allclose(out["y"], 0.5 * _torch_swiglu(x, lay.ws_gate, lay.ws_up, lay.ws_down), rtol=1e-13, atol=1e-13)
    assert np.array_equal(out["g_s"], np.full(6, 0.5))


def test_valid_selections_near_tie():
    l = np.array([2.0, 1.0005, 1.0, -3.0])
    alts = oracle.valid_selections(l, 2, 1e-3)
    assert [a.tolist() for a in alts] == [[0, 1], [0, 2]]
    assert [a.tolist() for a in oracle.valid_selections(l, 2, 1e-4)] == [[0, 1]]


def test_skewed_routing_share():
    # the skewed workload's Zipf bias (beta = 3, s = 1.2) concentrates about 90%
    # of the assignments on 4 experts and leaves most experts empty
    cfg = synth.get_config("skewed_bf16")
    x = synth.make_tokens(cfg, 8192).float().numpy()
    # the router weight alone (drawing the whole layer's experts is not needed here)
    wr = synth.generate._normal(cfg, "cpu", (cfg.d_model, cfg.n_experts), 0.02, 0, "w_router").numpy()
    b = synth.zipf_bias(cfg).numpy()
    idx, margin = oracle.select_topk(oracle.router_logits(x, wr, b), cfg.top_k)
    counts, _, _ = oracle.scatter_stable_sort(idx, cfg.n_experts)
    top4 = np.sort(counts)[::-1][:4].sum() / counts.sum()
    assert 0.85 <= top4 <= 0.95, top4
    assert (counts == 0).sum() >= 64
    assert counts.max() <= 8192


# ---------------------------------------------------------------- routing given by the caller
def _routed_bruteforce(x, lay, idx, w, g_s=None):
    """Brute force of the routed layer: token by token, slot by slot, torch's
    textbook SwiGLU of the slot's expert times the given weight; ids outside
    [0, E) add nothing."""
    x = np.asarray(x, dtype=np.float64)
    E = lay.n_experts
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if 0 <= e < E:
                y[t] += w[t, j] * _torch_swiglu(x[t:t + 1], *lay.expert(e))[0]
        if g_s is not None:
            y[t] += g_s[t] * _torch_swiglu(x[t:t + 1], lay.ws_gate, lay.ws_up, lay.ws_down)[0]
    return y


@pytest.mark.parametrize("shared,int8", [(0, False), (16, False), (0, True)])
def test_routed_bruteforce(shared, int8):
    rng = np.random.default_rng(11)
    d, E, F, k, T = 16, 6, 8, 3, 7
    lay = _rand_layer(rng, d, E, F, k, shared=shared, int8=int8)
    x = rng.standard_normal((T, d))
    idx = rng.integers(-2, E + 2, size=(T, k))  # repeats and out-of-range ids included
    w = rng.standard_normal((T, k))
    g_s = rng.random(T) if shared else None
    ref = oracle.moe_forward_routed(x, lay, idx, w, g_s)
    np.testing.assert_allclose(ref["y"], _routed_bruteforce(x, lay, idx, w, g_s), rtol=1e-12, atol=1e-12)
    # the scatter of the ids as read: every slot counted once, ids outside [0, E) under expert 0
    read = np.where((idx < 0) | (idx >= E), 0, idx)
    assert np.array_equal(ref["counts"], np.bincount(read.ravel(), minlength=E))
    assert ref["offsets"][-1] == T * k
    assert np.array_equal(ref["w"][(idx < 0) | (idx >= E)], np.zeros(int(((idx < 0) | (idx >= E)).sum())))


def test_routed_repeated_expert_and_linearity():
    rng = np.random.default_rng(12)
    d, E, F, k, T = 16, 5, 8, 2, 4
    lay = _rand_layer(rng, d, E, F, k)
    x = rng.standard_normal((T, d))
    # the same expert twice with weights a, b equals it once with a + b (the other slot at weight 0)
    idx2 = np.array([[3, 3]] * T)
    w2 = np.array([[0.25, 0.5]] * T)
    idx1 = np.array([[3, 1]] * T)
    w1 = np.array([[0.75, 0.0]] * T)
    y2 = oracle.moe_forward_routed(x, lay, idx2, w2)["y"]
    y1 = oracle.moe_forward_routed(x, lay, idx1, w1)["y"]
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-12)
    # linear in the weights; all-zero weights give y = 0
    idx = rng.integers(0, E, size=(T, k))
    w = rng.standard_normal((T, k))
    ya = oracle.moe_forward_routed(x, lay, idx, w)["y"]
    yb = oracle.moe_forward_routed(x, lay, idx, -2.5 * w)["y"]
    np.testing.assert_allclose(yb, -2.5 * ya, rtol=1e-12, atol=1e-12)
    assert not oracle.moe_forward_routed(x, lay, idx, 0 * w)["y"].any()


def test_routed_with_the_gates_routing_is_the_layer():
    rng = np.random.default_rng(13)
    d, E, F, k, T = 16, 6, 8, 2, 9
    lay = _rand_layer(rng, d, E, F, k, bias=True, shared=8)
    x = rng.standard_normal((T, d))
    ref = oracle.moe_forward(x, lay)
    rt = oracle.moe_forward_routed(x, lay, ref["idx"], ref["w"], ref["g_s"])
    np.testing.assert_allclose(rt["y"], ref["y"], rtol=1e-12, atol=1e-12)
    assert np.array_equal(rt["sorted_assign"], ref["sorted_assign"])
    with pytest.raises(ValueError):
        oracle.moe_forward_routed(x, lay, ref["idx"], ref["w"])  # shared expert needs g_s


# ---------------------------------------------------------------- int4 group-wise weights
def test_dequantize_groupwise_hand_fixture():
    # 4 input rows, 2 output columns, groups of 2 rows: rows 0-1 take scale row 0, rows 2-3 row 1
    q = np.array([[1, -2], [3, 4], [-5, 6], [7, -7]], dtype=np.int8)
    s = np.array([[0.5, 2.0], [0.25, 1.0]], dtype=np.float32)
    want = np.array([[0.5, -4.0], [1.5, 8.0], [-1.25, 6.0], [1.75, -7.0]])
    assert np.array_equal(oracle.dequantize_groupwise(q, s, 2), want)


def test_int4_quantiser_roundtrip_groups_and_axis():
    # scales that differ by 1000x across columns and by 10x between the two K groups:
    # a scale taken from the wrong group or the wrong axis breaks the half-step bound
    rng = np.random.default_rng(21)
    w = rng.standard_normal((2, 256, 16)) * np.logspace(-3, 0, 16)[None, None, :]
    w[:, 128:, :] *= 10.0
    w[1, :128, 3] = 0.0  # an all-zero group
    q, s = synth.quantize_int4_groupwise(torch.from_numpy(w).float())
    q, s = q.numpy(), s.numpy()
    assert q.dtype == np.int8 and s.shape == (2, 2, 16)
    assert q.min() >= -7 and q.max() <= 7
    assert s[1, 0, 3] == 0 and not q[1, :128, 3].any()
    nz = s > 0
    amax = np.abs(q.reshape(2, 2, 128, 16)).max(axis=2)
    assert (amax[nz] == 7).all()  # every nonzero group reaches the end of the range
    deq = oracle.dequantize_groupwise(q, s, 128)
    w32 = torch.from_numpy(w).float().double().numpy()
    bound = np.repeat(s, 128, axis=1) * 0.5 * (1 + 1e-6)
    assert (np.abs(deq - w32) <= bound).all()


def test_int4_storage_encoding():
    # two values per byte along the input axis, low nibble first, 4-bit two's complement
    q = torch.tensor([[[1, -8], [-1, 7], [0, -3], [5, 2]]], dtype=torch.int8)  # [1, in=4, out=2]
    p = synth.pack_int4_pairs(q)
    assert p.dtype == torch.uint8 and tuple(p.shape) == (1, 2, 2)
    assert p.tolist() == [[[0xF1, 0x78], [0x50, 0x2D]]]


def test_dense_masked_bruteforce_int4():
    rng = np.random.default_rng(22)
    d, E, F, k = 256, 5, 128, 2
    ws = [rng.standard_normal((E, a, b)) / np.sqrt(a) for a, b in ((d, F), (d, F), (F, d))]
    qs = [synth.quantize_int4_groupwise(torch.from_numpy(w).float()) for w in ws]
    (wg, sg), (wu, su), (wd, sd) = [(q.numpy(), s.numpy()) for q, s in qs]
    lay = oracle.OracleLayer(w_router=rng.standard_normal((d, E)) * 0.1, w_gate=wg, w_up=wu, w_down=wd,
                             top_k=k, s_gate=sg, s_up=su, s_down=sd, group=128)
    x = rng.standard_normal((5, d))
    out = oracle.moe_forward(x, lay)
    ref = _dense_masked(x, lay)
    assert np.abs(out["y"] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


# ---------------------------------------------------------------- the gate's clamp option
def test_gate_clamp_hand_fixture():
    # zero router, bias [60, 55, 0, -70, 52]: clamped to [50, 50, 0, -50, 50] the three
    # largest tie, so the lower ids win and the weights are equal
    E, d = 5, 4
    w_r = np.zeros((d, E))
    b = np.array([60.0, 55.0, 0.0, -70.0, 52.0])
    wg = np.zeros((E, d, 2)); wd = np.zeros((E, 2, d))
    x = np.ones((1, d))
    for k, clamped, raw in ((2, [0, 1], [0, 1]), (3, [0, 1, 4], [0, 1, 4])):
        lay = oracle.OracleLayer(w_router=w_r, w_gate=wg, w_up=wg, w_down=wd, top_k=k, b_router=b)
        ref = oracle.moe_forward(x, lay)
        assert ref["idx"][0].tolist() == raw
        np.testing.assert_allclose(ref["w"][0], softmax(b[raw]), rtol=1e-15)
        lay.gate_clamp = True
        out = oracle.moe_forward(x, lay)
        assert out["idx"][0].tolist() == clamped
        np.testing.assert_allclose(out["w"][0], np.full(k, 1.0 / k), rtol=1e-15)
        assert out["margin"][0] == 0.0 if k == 2 else out["margin"][0] == 50.0  # tie at 50 / 50 vs 0


def test_gate_clamp_inactive_inside_bounds():
    rng = np.random.default_rng(31)
    lay = _rand_layer(rng, d=16, E=6, F=8, k=2, bias=True)
    x = rng.standard_normal((9, 16))
    a = oracle.moe_forward(x, lay)
    assert np.abs(a["logits"]).max() < 50
    lay.gate_clamp = True
    b = oracle.moe_forward(x, lay)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["y"], b["y"])


# ---------------------------------------------------------------- raw-logit weighting
def _one_token_layer(logits, k, clamp=False):
    """A layer whose router gives `logits` for the token x = ones(1, 1): W_r = 0 and the
    logits as the bias (no experts' work matters here)."""
    E = len(logits)
    z = np.zeros((E, 1, 2))
    return oracle.OracleLayer(w_router=np.zeros((1, E)), w_gate=z, w_up=z, w_down=np.zeros((E, 2, 1)),
                              top_k=k, b_router=np.asarray(logits, dtype=np.float64), gate_clamp=clamp,
                              gate_weighting="raw")


def test_topk_raw_hand_fixture():
    g = _load("topk_raw_hand.json")
    for case in g["cases"]:
        lay = _one_token_layer(case["logits"], case["top_k"], case.get("clamp", False))
        out = oracle.moe_forward(np.ones((1, 1)), lay)
        assert out["idx"][0].tolist() == case["idx"], case
        assert out["w"][0].tolist() == case["w"], case


def _dense_masked_raw(x, lay):
    """Brute force with raw-logit weights: y_t = sum over ALL experts of 1[e chosen] *
    l_te * FFN_e(x_t), the choice from a full stable sort of the logits."""
    x = np.asarray(x, dtype=np.float64)
    T, E, k = x.shape[0], lay.n_experts, lay.top_k
    logits = x @ np.asarray(lay.w_router, dtype=np.float64)
    if lay.b_router is not None:
        logits = logits + lay.b_router
    y = np.zeros_like(x)
    for t in range(T):
        chosen = set(np.argsort(-logits[t], kind="stable")[:k].tolist())
        for e in range(E):
            wg, wu, wd = lay.expert(e)
            y[t] += (logits[t, e] if e in chosen else 0.0) * _torch_swiglu(x[t:t + 1], wg, wu, wd)[0]
    if lay.w_shared_gate is not None:
        y += expit(x @ lay.w_shared_gate)[:, None] * _torch_swiglu(x, lay.ws_gate, lay.ws_up, lay.ws_down)
    return y


@pytest.mark.parametrize("bias,shared,k", [(False, 0, 2), (True, 0, 3), (True, 24, 2)])
def test_raw_weighting_dense_masked_bruteforce(bias, shared, k):
    rng = np.random.default_rng(41 + k)
    lay = _rand_layer(rng, d=18, E=7, F=20, k=k, bias=bias, shared=shared)
    lay.gate_weighting = "raw"
    x = rng.standard_normal((9, 18))
    out = oracle.moe_forward(x, lay)
    ref = _dense_masked_raw(x, lay)
    assert np.abs(out["y"] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_raw_weighting_closed_forms():
    rng = np.random.default_rng(43)
    d, E, F = 14, 6, 10
    wg, wu, wd = rng.standard_normal((d, F)), rng.standard_normal((d, F)), rng.standard_normal((F, d))
    W_r = rng.standard_normal((d, E))
    x = rng.standard_normal((11, d))
    ffn = _torch_swiglu(x, wg, wu, wd)
    # identical experts: y_t = (sum of the k largest logits of token t) * FFN(x_t)
    lay = oracle.OracleLayer(W_r, np.stack([wg] * E), np.stack([wu] * E), np.stack([wd] * E), top_k=3,
                             gate_weighting="raw")
    top3 = -np.sort(-(x @ W_r), axis=1)[:, :3].sum(1)
    np.testing.assert_allclose(oracle.moe_forward(x, lay)["y"], top3[:, None] * ffn, rtol=1e-11, atol=1e-11)
    # k = 1: raw weighting is the softmax layer (weight 1) scaled by the chosen logit
    lay1 = _rand_layer(rng, d=d, E=E, F=F, k=1)
    soft = oracle.moe_forward(x, lay1)
    lay1.gate_weighting = "raw"
    raw = oracle.moe_forward(x, lay1)
    assert np.array_equal(soft["idx"], raw["idx"])
    lmax = (x @ lay1.w_router).max(1)
    np.testing.assert_allclose(raw["y"], lmax[:, None] * soft["y"], rtol=1e-12, atol=1e-12)
    # a positive scale c of router weight and bias keeps the choice and scales y by c
    # (softmax weights would not scale)
    lay2 = _rand_layer(rng, d=d, E=E, F=F, k=2, bias=True)
    lay2.gate_weighting = "raw"
    a = oracle.moe_forward(x, lay2)
    lay2.w_router = lay2.w_router * 2.5
    lay2.b_router = lay2.b_router * 2.5
    b = oracle.moe_forward(x, lay2)
    assert np.array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(b["y"], 2.5 * a["y"], rtol=1e-12, atol=1e-12)


def test_raw_weighting_rejects_unknown_mode():
    lay = _one_token_layer([1.0, 0.0], 1)
    lay.gate_weighting = "sparsemax"
    with pytest.raises(ValueError):
        oracle.moe_forward(np.ones((1, 1)), lay)
