"""bench.py host logic on the CPU: the algorithmic work it prices the kernels with, and its
single-GPU contract."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_bytes_are_the_active_experts_weights():
    # Mixtral-shaped layer, one token on two experts: 2 x 3 x 4096 x 14336 bf16 weights, plus
    # the router (fp32), x and y, and the routing outputs
    cfg = synth.get_config("mixtral_bf16")
    counts = np.array([1, 0, 0, 1, 0, 0, 0, 0])
    up, dn, layer = bench.kernel_work(cfg, counts, 1)
    w = 2 * 3 * 4096 * 14336 * 2
    assert layer["active"] == 2
    assert layer["bytes"] == w + 4096 * 8 * 4 + 2 * 4096 * 2 + 2 * 8
    assert up["bytes"] == 2 * 2 * 4096 * 14336 * 2 + 4096 * 2 + 2 * 14336 * 2
    assert abs(layer["bytes"] / 1e9 - 0.705) < 1e-3


def test_flops_match_the_closed_form():
    # T (2 k 3 d F + 2 d E) routed, + T (6 d Fs + 2 d) for the shared expert
    for name, T in (("mixtral_bf16", 4096), ("shared_fine_bf16", 2048), ("skewed_bf16", 8192)):
        cfg = synth.get_config(name)
        d, F, k, E, Fs = cfg.d_model, cfg.d_ff, cfg.top_k, cfg.n_experts, cfg.shared_d_ff
        counts = np.ones(E, dtype=np.int64)
        _, _, layer = bench.kernel_work(cfg, counts, T)
        want = T * (2 * k * 3 * d * F + 2 * d * E) + (T * (6 * d * Fs + 2 * d) if Fs else 0)
        assert layer["flops"] == want, name
    cfg = synth.get_config("mixtral_bf16")
    _, _, layer = bench.kernel_work(cfg, np.ones(8, dtype=np.int64), 4096)
    assert abs(layer["flops"] / 1e12 - 2.886) < 1e-3


def test_int8_bytes_count_scales():
    cfg = synth.get_config("int8_mixtral22b")
    counts = np.array([0, 1, 0, 0, 0, 0, 1, 0])
    up, dn, _ = bench.kernel_work(cfg, counts, 1)
    d, F = 6144, 16384
    assert up["bytes"] == 2 * (2 * d * F * 1 + 2 * F * 4) + d * 2 + 2 * F * 2
    assert dn["bytes"] == 2 * (F * d * 1 + d * 4) + 2 * F * 2 + 2 * d * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_int4_bytes_count_group_scales():
    # two codes per byte, and one fp32 scale per 128 input rows of every output column
    cfg = synth.get_config("int4_mixtral22b")
    counts = np.array([0, 0, 1, 0, 0, 0, 1, 0])
    up, dn, _ = bench.kernel_work(cfg, counts, 1)
    d, F = 6144, 16384
    assert up["bytes"] == 2 * (2 * d * F // 2 + (d // 128) * 2 * F * 4) + d * 2 + 2 * F * 2
    assert dn["bytes"] == 2 * (F * d // 2 + (F // 128) * d * 4) + 2 * F * 2 + 2 * d * 4


def test_summary_roofline_picks_the_bound_of_the_up_kernel():
    # one token: below the ridge point, priced on HBM bytes; 4096 tokens: on MFMA flops
    cfg = synth.get_config("mixtral_bf16")
    for T, bound in ((1, "hbm"), (4096, "mfma")):
        counts = np.zeros(8, dtype=np.int64)
        counts[:2 if T == 1 else 8] = 1
        res = dict(T=T, ms_per_step=1.0, stage_ms=[0.01, 0.01, 0.5, 0.3, 0.01], counts=counts,
                   step_ms_pct={"p10": 0.9, "p50": 1.0, "p90": 1.1})
        s = bench.summarize(cfg, res)
        rf = s["roofline"]
        up, _, _ = bench.kernel_work(cfg, counts, T)
        want = up["bytes"] / 0.5e-3 / 1e9 if bound == "hbm" else up["flops"] / 0.5e-3 / 1e12
        assert rf["bound"] == bound
        assert abs(rf["achieved"] - want) < 1e-6 * want
        assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
        assert s["tokens_per_s"] == T / 1e-3


def test_only_the_cpu_baseline_leg_imports_the_oracle():
    # the GPU path of the benchmark builds its layers through the binding alone; the
    # oracle (directly or through the test harness) is imported only by the CPU-baseline leg
    import ast
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    allowed = {"_oracle_layer", "cpu_baseline"}
    for fn in [n for n in ast.walk(tree) if isinstance(n, (ast.FunctionDef, ast.Module))]:
        body_nodes = ast.walk(fn) if isinstance(fn, ast.FunctionDef) else fn.body
        for node in body_nodes:
            names = []
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""]
            for m in names:
                assert m.split(".")[0] != "harness", f"bench.py imports the test harness in {getattr(fn, 'name', '<module>')}"
                if m.split(".")[0] == "oracle":
                    assert isinstance(fn, ast.FunctionDef) and fn.name in allowed, \
                        f"bench.py imports the oracle in {getattr(fn, 'name', '<module>')}"
