"""Benchmark of the MoE layer forward (libmoe) on one MI355X.

One step = one moe_forward (gate -> scatter -> expert up -> expert down ->
combine) over one batch of T synthetic tokens, inputs resident in HBM. Layers
rotate round-robin over several independently drawn instances so consecutive
steps never reuse weights from the 256 MB last-level cache.

Prints one JSON line: tokens/s of the main workload (timed with libmoe's stage
events off), the roofline of its dominant kernel (the expert up-projection GEMM;
its average duration comes from libmoe's per-stage HIP events, recorded on the
stream the kernels run on over a second pass of the same steps), the same
figures for every other workload (each layer shape at each of its token counts,
under "workloads"), decode layers on 1 and 8 concurrent streams ("decode_concurrency"),
eager against HIP-graph-replayed decode steps ("hip_graph_replay"), and the CPU oracle
timed on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--tokens T] [--only-main]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
# extra decode measurements of the default run: layers on concurrent streams, and HIP graph replay
CONCURRENCY_CASES = (("mixtral_bf16", 1), ("int8_mixtral22b", 1))
GRAPH_CASE = ("mixtral_bf16", 1)

# HBM traffic per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (scaled by a
# plain-copy calibration), keyed by kernel and workload, valid only while the kernel's
# sources hash to the recorded value.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "expert_gemm": ["expert_gemm.hip", "common.h"],
    "expert_stream": ["expert_stream.hip", "common.h"],
    "expert_tstream": ["expert_tstream.hip", "common.h"],
}


def kernel_sources_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "moe_layer_forward_gate_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def lookup_traffic(kernel, key):
    """Measured HBM bytes per launch of `kernel` on workload `key`, or None when not measured
    or measured on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            tab = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = tab.get("kernels", {}).get(f"{kernel}|{key}")
    if not ent or ent.get("source_sha") != kernel_sources_sha(kernel):
        return None
    return ent.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_bf16")
    ap.add_argument("--tokens", type=int, default=None, help="main workload T (default: largest of the config)")
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--only-main", "--no-sweep", dest="only_main", action="store_true",
                    help="time the main workload only (default: also every layer shape at each of its token "
                         "counts, decode layers on concurrent streams and HIP graph replay)")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="leave out the measured HBM-read and MFMA rates (two microbenchmarks, ~0.3 s)")
    ap.add_argument("--graph", action="store_true", help="replay each step as a captured HIP graph")
    ap.add_argument("--streams", type=int, default=1,
                    help="S > 1: S layer instances forwarded concurrently on S streams (decode throughput)")
    ap.add_argument("--routed", action="store_true",
                    help="time moe_forward_routed on a drawn routing (no gate) instead of moe_forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the batch the oracle runs on (0: the whole batch)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle's pass over the sample until this much time has passed")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure achievable rates: streaming HBM read and bf16 MFMA issue "
                         "microbenchmarks, and hipBLASLt bf16 GEMMs of the expert shapes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB (for HBM counter scaling)")
    return ap.parse_args()


def kernel_work(cfg, counts, T):
    """Algorithmic bytes and flops of the up and down GEMMs for one forward.

    counts: per routed expert assignment counts of this batch. Shared-expert
    slices take all T tokens. Bytes: weights (+ scales) of experts with rows,
    the activations read and the GEMM output written."""
    d, F, k = cfg.d_model, cfg.d_ff, cfg.top_k
    # bytes per weight: int4 packs two in a byte
    welt = {"i8": 1.0, "i4": 0.5, "f32": 4.0}.get(cfg.expert_dtype, 2.0)
    aelt = 4 if cfg.act_dtype == "f32" else 2
    helt = 4 if cfg.expert_dtype == "f32" else 2
    active = int((counts > 0).sum())
    P = T * k
    V = cfg.shared_d_ff // F if cfg.shared_d_ff else 0
    rows = P + V * T
    # fp32 scales: one per output channel (int8), one per 128 input rows of each (int4)
    if cfg.expert_dtype == "i8":
        scale_up, scale_dn = active * 2 * F * 4, active * d * 4
    elif cfg.expert_dtype == "i4":
        scale_up, scale_dn = active * (d // 128) * 2 * F * 4, active * (F // 128) * d * 4
    else:
        scale_up = scale_dn = 0
    up_w = int((active + V) * 2 * d * F * welt) + scale_up
    dn_w = int((active + V) * F * d * welt) + scale_dn
    up = dict(flops=2.0 * rows * d * 2 * F, bytes=up_w + T * d * aelt + rows * F * helt)
    dn = dict(flops=2.0 * rows * F * d, bytes=dn_w + rows * F * helt + rows * d * 4)
    layer_bytes = up_w + dn_w + d * cfg.n_experts * 4 + 2 * T * d * aelt + T * k * 8
    # router GEMM (+ the shared gate's dot per token) and the two expert GEMMs
    layer_flops = 2.0 * T * d * (cfg.n_experts + (1 if V else 0)) + up["flops"] + dn["flops"]
    return up, dn, dict(bytes=layer_bytes, flops=layer_flops, active=active)


def build_layers(cfg, n, max_tokens, torch, synth, moe, keep_layer0=False):
    """n independently drawn layer instances held by libmoe (and, with keep_layer0, a host
    copy of instance 0's tensors for the CPU baseline)."""
    layers, layer0 = [], None
    dev = torch.device("cuda", torch.cuda.current_device())
    for i in range(n):
        L = synth.make_layer(cfg, device="cuda", instance=i)
        layers.append(moe.MoeLayer(max_tokens=max_tokens, **synth.layer_kwargs(L, dev)))
        if i == 0 and keep_layer0:
            layer0 = L.to("cpu")
        del L
        torch.cuda.empty_cache()
    return layers, layer0


def batch_instances(cfg, layers, T, synth, routed=False):
    """(layer, x, outputs) per layer instance for a batch of T tokens; with `routed`, each
    instance's forward is moe_forward_routed on a routing drawn by synth.make_routing."""
    insts = []
    for i, lay in enumerate(layers):
        x = synth.make_tokens(cfg, T, device="cuda", instance=i)
        out = lay.outputs(T, scatter=True)
        if routed:
            idx, w, gs = synth.make_routing(cfg, T, device="cuda", instance=i)
            out.topk_idx, out.topk_w, out.shared_gate = idx, w, gs
            lay = _Routed(lay)
        insts.append((lay, x, out))
    return insts


class _Routed:
    """A layer whose forward(x, out=out) runs moe_forward_routed on out's routing."""

    def __init__(self, lay):
        self.lay = lay

    def forward(self, x, out):
        return self.lay.forward_routed(x, out.topk_idx, out.topk_w, out.shared_gate, out=out)

    def __getattr__(self, name):
        return getattr(self.lay, name)


def run_workload(cfg, T, steps, warmup, layers, torch, synth, graph=False, routed=False):
    """Time `steps` forwards (rotating over the layer instances) with per-stage events off,
    then run the same steps again with libmoe's per-stage HIP events on and average the
    stage times."""
    import numpy as np
    insts = batch_instances(cfg, layers, T, synth, routed=routed)
    n_inst = len(insts)
    for i in range(warmup):
        lay, x, out = insts[i % n_inst]
        lay.forward(x, out=out)
    torch.cuda.synchronize()
    graphs = None
    if graph:
        # one HIP graph per layer instance, each replaying that instance's moe_forward
        graphs = []
        s = torch.cuda.Stream()
        for lay, x, out in insts:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                lay.forward(x, out=out)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if graphs is not None:
            graphs[i % n_inst].replay()
        else:
            lay, x, out = insts[i % n_inst]
            lay.forward(x, out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = []
    for lay, _, _ in insts:
        lay.set_profiling(True)
    for i in range(steps):
        lay, x, out = insts[i % n_inst]
        lay.forward(x, out=out)
        stages.append(lay.stage_times())
    st = np.mean(np.array(stages), axis=0).tolist()
    counts = insts[(steps - 1) % n_inst][2].expert_counts.cpu().numpy()
    # per-step spread from the event pass (gate start to combine end; each stage event adds a few us)
    per_step = np.sum(np.array(stages), axis=1)
    pct = {f"p{q}": float(np.percentile(per_step, q)) for q in (10, 50, 90)}
    res = dict(T=T, ms_per_step=1e3 * wall / steps, stage_ms=st, counts=counts, step_ms_pct=pct)
    for lay, _, _ in insts:
        lay.set_profiling(False)
    res["x0"] = insts[0][1].cpu()
    if routed:
        o = insts[0][2]
        res["routing0"] = (o.topk_idx.cpu(), o.topk_w.cpu(), None if o.shared_gate is None else o.shared_gate.cpu())
    del graphs, insts
    torch.cuda.empty_cache()
    return res


def summarize(cfg, res):
    T = res["T"]
    up, dn, layer = kernel_work(cfg, res["counts"], T)
    gate_ms, scat_ms, up_ms, dn_ms, comb_ms = res["stage_ms"]
    # the up kernel's own roofline: bandwidth-bound below the ridge point (peak flops / peak bytes)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    decode = up["flops"] / up["bytes"] < ridge
    if decode:
        rf = dict(bound="hbm", achieved=up["bytes"] / (up_ms * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        rf = dict(bound="mfma", achieved=up["flops"] / (up_ms * 1e-3) / 1e12, peak=MFMA_BF16_PEAK_TFLOPS,
                  unit="TFLOP/s")
    rf["frac"] = rf["achieved"] / rf["peak"]
    # the up kernel the library's launch plan picks
    quant = cfg.expert_dtype in ("i8", "i4")
    if cfg.expert_dtype == "f32":
        kern = "expert_f32"
    elif T <= (32 if quant else 64):
        kern = "expert_stream"
    elif (2 * cfg.d_ff) % 256 == 0 and cfg.d_model % 256 == 0 and (
            quant or (cfg.shared_d_ff == 0 and T * cfg.top_k <= min(128 * cfg.n_experts, 4096))):
        kern = "expert_tstream"
    else:
        kern = "expert_gemm"
    rf["kernel"] = f"{kern}<up>"
    rf["traffic"] = lookup_traffic(kern, f"up|{cfg.name}|T={T}") if kern in KERNEL_SOURCES else None
    rf["avg_ms"] = up_ms
    layer_s = res["ms_per_step"] * 1e-3
    # the layer against its target: bytes of the active experts against HBM for batches below
    # the ridge point, the grouped GEMM's flops (up + down kernels) against bf16 MFMA above it
    if cfg.act_dtype == "f32":
        target = dict(bound="none", note="fp32 layer: parity only")
    elif decode:
        f = layer["bytes"] / layer_s / 1e9 / HBM_PEAK_GBS
        target = dict(bound="hbm", what="layer, active-expert bytes", frac=f, want=0.70, met=f >= 0.70)
    else:
        f = (up["flops"] + dn["flops"]) / ((up_ms + dn_ms) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
        target = dict(bound="mfma", what="grouped GEMM (up + down kernels)", frac=f, want=0.60, met=f >= 0.60)
    return dict(
        T=T, ms_per_step=res["ms_per_step"], tokens_per_s=T / layer_s,
        stage_ms=dict(gate=gate_ms, scatter=scat_ms, up=up_ms, down=dn_ms, combine=comb_ms),
        layer_GBps=layer["bytes"] / layer_s / 1e9, layer_TFLOPs=layer["flops"] / layer_s / 1e12,
        layer_hbm_frac=layer["bytes"] / layer_s / 1e9 / HBM_PEAK_GBS,
        layer_mfma_frac=layer["flops"] / layer_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        down_frac=(dn["bytes"] / (dn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS) if decode else
        (dn["flops"] / (dn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS),
        active_experts=layer["active"], roofline=rf, step_ms_pct=res["step_ms_pct"], target=target)


def run_streams(cfg, T, steps, warmup, S, torch, synth):
    """S independent layer instances, each on its own HIP stream (default priority), all
    enqueued every step: the decode throughput of concurrent layers (one layer per stream,
    as the library requires). Returns the wall time per step and the algorithmic bytes of
    one step (every instance's expert weights with rows, router, tokens)."""
    import moe_layer_forward_gate_amd as moe
    layers, _ = build_layers(cfg, S, T, torch, synth, moe)
    insts = batch_instances(cfg, layers, T, synth)
    streams = [torch.cuda.Stream() for _ in range(S)]
    cur = torch.cuda.current_stream()
    for st in streams:
        st.wait_stream(cur)  # the inputs were written on the current stream

    def step():
        for (lay, x, out), st in zip(insts, streams):
            lay.forward(x, out=out, stream=st)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_bytes = sum(kernel_work(cfg, out.expert_counts.cpu().numpy(), T)[2]["bytes"] for _, _, out in insts)
    for lay, _, _ in insts:
        lay.close()
    del insts
    torch.cuda.empty_cache()
    return dict(ms_per_step=1e3 * wall / steps, step_bytes=step_bytes)


def _oracle_layer(L):
    """The oracle's layer from a host copy of a synthetic layer (exact stored values)."""
    import oracle
    import synth

    def np_(t):
        return None if t is None else t.float().numpy() if t.is_floating_point() else t.numpy()
    return oracle.OracleLayer(
        w_router=np_(L.w_router), w_gate=np_(L.w_gate), w_up=np_(L.w_up), w_down=np_(L.w_down),
        top_k=L.cfg.top_k, b_router=np_(L.b_router), s_gate=np_(L.s_gate), s_up=np_(L.s_up),
        s_down=np_(L.s_down), w_shared_gate=np_(L.w_shared_gate), ws_gate=np_(L.ws_gate),
        ws_up=np_(L.ws_up), ws_down=np_(L.ws_down),
        group=synth.INT4_GROUP if L.cfg.expert_dtype == "i4" else None)


def cpu_baseline(cfg, layer_cpu, x_cpu, n_tok, min_s, routing=None):
    """The oracle as it stands, on the first n_tok tokens of the same batch, repeated (at most
    4 passes) until min_s seconds have passed (with `routing` (idx, w, g_s): the oracle of
    the layer fed that routing). Then the tiny fp32 layer's whole 64-token batch on one BLAS
    thread, for a single-core figure."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info, threadpool_limits
    olay = _oracle_layer(layer_cpu)
    xs = x_cpu[:n_tok].float().numpy()
    passes = 0
    t0 = time.perf_counter()
    if routing is not None:
        ridx, rw, rgs = (None if t is None else t[:n_tok].numpy() for t in routing)
    while True:
        if routing is None:
            oracle.moe_forward(xs, olay)
        else:
            oracle.moe_forward_routed(xs, olay, ridx, rw, rgs)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or passes == 4:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    # one thread, the tiny fp32 layer (d_model 256, 8 experts, d_ff 512, top-2), T = 64
    tcfg = synth.get_config("tiny_f32")
    tl = _oracle_layer(synth.make_layer(tcfg))
    tx = synth.make_tokens(tcfg, 64).numpy()
    with threadpool_limits(limits=1):
        n1, t1 = 0, time.perf_counter()
        while True:
            oracle.moe_forward(tx, tl)
            n1 += 1
            d1 = time.perf_counter() - t1
            if d1 >= 1.0:
                break
    return dict(value=passes * n_tok / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                host_cpus=os.cpu_count(),
                sample=f"{passes} pass(es) over {n_tok} tokens of the T={x_cpu.shape[0]} batch, whole layer "
                       f"forward in fp64 ({'given routing' if routing is not None else 'gate'}, scatter, "
                       f"{cfg.n_experts} experts, combine), {dt:.1f} s on {threads} BLAS threads",
                single_thread={"config": "tiny_f32", "tokens": 64, "passes": n1,
                               "value": n1 * 64 / d1, "unit": "tokens/s", "cores": 1})


def peaks_lib():
    import ctypes
    P = ctypes.CDLL(os.path.join(ROOT, "moe_layer_forward_gate_amd", "libmoe_peaks.so"))
    for f in ("moe_peak_read_gbps", "moe_peak_read_nt_gbps"):
        getattr(P, f).restype = ctypes.c_double
        getattr(P, f).argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.c_int]
    for f in ("moe_peak_mfma_tflops", "moe_peak_mfma_random_tflops"):
        getattr(P, f).restype = ctypes.c_double
        getattr(P, f).argtypes = [ctypes.c_int, ctypes.c_int]
    return P


def measured_peaks(rf):
    """The two rates measured on this GPU that the kernels can reach, and the dominant kernel's
    achieved rate against the one of its bound: a 4 GiB non-temporal streaming read, and bf16
    MFMA issue on random register operands that change every instruction (about 60 ms, long
    enough for the clock to settle at the power the multipliers draw on real data)."""
    try:
        P = peaks_lib()
    except OSError:
        return None
    hbm = max(P.moe_peak_read_nt_gbps(4 << 30, w, 5) for w in (4096, 8192))
    P.moe_peak_mfma_random_tflops(256, 20000)  # clock settles
    mfma = P.moe_peak_mfma_random_tflops(256, 100000)
    peak = hbm if rf["bound"] == "hbm" else mfma
    return {"hbm_read_GBps": hbm, "mfma_bf16_TFLOPs": mfma,
            "bound_peak": peak, "frac_of_measured": rf["achieved"] / peak if peak > 0 else None,
            "how": "non-temporal streaming read of 4 GiB; v_mfma_f32_16x16x32_bf16 issue on random "
                   "register operands changing every instruction"}


def measure_peaks(torch):
    """Achievable rates on this GPU: libmoe_peaks microbenchmarks (streaming HBM read, bf16
    MFMA issue from registers on constant and on random operands) and, for comparison,
    hipBLASLt bf16 GEMMs of the expert shapes."""
    out = {}
    P = peaks_lib()
    out["read_stream_GBps"] = {w: P.moe_peak_read_gbps(4 << 30, w, 5) for w in (2048, 4096, 8192)}
    out["read_stream_nontemporal_GBps"] = {w: P.moe_peak_read_nt_gbps(4 << 30, w, 5) for w in (2048, 4096, 8192)}
    out["mfma_bf16_TFLOPs"] = {w: P.moe_peak_mfma_tflops(w, 20000) for w in (256, 512)}
    P.moe_peak_mfma_random_tflops(256, 20000)
    out["mfma_bf16_random_operands_TFLOPs"] = {w: P.moe_peak_mfma_random_tflops(w, 50000) for w in (256, 512)}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n = 10
    for M, K, N in ((8192, 8192, 8192), (1024, 4096, 28672), (1024, 14336, 4096)):
        A = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
        B = torch.randn(K, N, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            A @ B
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(n):
            A @ B
        ev[1].record()
        torch.cuda.synchronize()
        out[f"hipblaslt_gemm_{M}x{K}x{N}_TFLOPs"] = 2.0 * M * N * K * n / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        # a plain copy kernel of known size: 1 GiB read + 1 GiB written per launch
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4, "launches": 3}))
        return
    if args.peaks:
        print(json.dumps(measure_peaks(torch)), flush=True)
        return
    import synth
    import moe_layer_forward_gate_amd as moe
    moe.lib()
    torch.cuda.set_device(0)
    cfg = synth.get_config(args.config)
    T = args.tokens or max(cfg.tokens)
    print(f"[bench] {cfg.name} T={T} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    if args.streams > 1:
        r = run_streams(cfg, T, args.steps, args.warmup, args.streams, torch, synth)
        ach = r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
        print(json.dumps({
            "metric": "MoE-layer tokens/s; decode HBM TB/s and prefill MFMA TFLOP/s vs roofline",
            "value": args.streams * T / (r["ms_per_step"] * 1e-3), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": {"bf16": "bf16", "f32": "f32"}[cfg.act_dtype] + {"i8": "+i8w", "i4": "+i4w"}.get(cfg.expert_dtype, ""),
            "data": "synthetic",
            "config": {"workload": f"{cfg.name}: {args.streams} independent layers, one per stream, "
                                   f"{T} tokens each", "tokens": T, "streams": args.streams},
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "traffic": None, "kernel": "whole layers, all streams"}}))
        return
    want_cpu = not args.no_cpu_baseline
    layers, layer0 = build_layers(cfg, args.instances, max(T, max(cfg.tokens)), torch, synth, moe,
                                  keep_layer0=want_cpu)
    res = run_workload(cfg, T, args.steps, args.warmup, layers, torch, synth, graph=args.graph, routed=args.routed)
    main_s = summarize(cfg, res)
    print(f"[bench] main {cfg.name} T={T} {json.dumps(main_s)}", file=sys.stderr, flush=True)
    # every workload: each layer shape at each of its token counts (the main one included,
    # timed again in its turn), layers built once per shape
    workloads = []
    graph_replay = None
    if not args.only_main:
        names = [cfg.name] + [n for n in synth.CONFIGS if n != cfg.name]
        for name in names:
            c = synth.get_config(name)
            if c.name == cfg.name:
                lays = layers
            else:
                print(f"[bench] building {c.name}", file=sys.stderr, flush=True)
                lays, _ = build_layers(c, args.instances, max(c.tokens), torch, synth, moe)
            for Ts in c.tokens:
                r = run_workload(c, Ts, max(args.steps, 20), args.warmup, lays, torch, synth,
                                 graph=args.graph, routed=args.routed)
                s = summarize(c, r)
                s["config"] = c.name
                workloads.append(s)
                print(f"[bench] workload {c.name} T={Ts} {json.dumps(s)}", file=sys.stderr, flush=True)
                if c.name == GRAPH_CASE[0] and Ts == GRAPH_CASE[1] and not args.graph:
                    # the same steps captured once per instance and replayed
                    rg = run_workload(c, Ts, max(args.steps, 50), args.warmup, lays, torch, synth, graph=True)
                    re_ = run_workload(c, Ts, max(args.steps, 50), args.warmup, lays, torch, synth)
                    graph_replay = dict(config=c.name, T=Ts, steps=max(args.steps, 50),
                                        eager_ms=re_["ms_per_step"], graph_ms=rg["ms_per_step"])
                    print(f"[bench] graph {json.dumps(graph_replay)}", file=sys.stderr, flush=True)
            if lays is not layers:
                for lay in lays:
                    lay.close()
                del lays
                torch.cuda.empty_cache()
    for lay in layers:
        lay.close()
    del layers
    torch.cuda.empty_cache()
    # decode layers on concurrent streams: S independent layers, one per stream
    concurrency = []
    if not args.only_main:
        for name, Tc in CONCURRENCY_CASES:
            c = synth.get_config(name)
            for S in (1, 8):
                r = run_streams(c, Tc, max(args.steps, 20), args.warmup, S, torch, synth)
                ach = r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
                concurrency.append(dict(config=name, T=Tc, streams=S, ms_per_step=r["ms_per_step"],
                                        tokens_per_s=S * Tc / (r["ms_per_step"] * 1e-3),
                                        layer_hbm_frac=ach / HBM_PEAK_GBS))
                print(f"[bench] streams {json.dumps(concurrency[-1])}", file=sys.stderr, flush=True)
    cpu = None
    if want_cpu:
        n_tok = T if args.cpu_sample_tokens <= 0 else min(args.cpu_sample_tokens, T)
        cpu = cpu_baseline(cfg, layer0, res["x0"], n_tok, args.cpu_min_seconds, routing=res.get("routing0"))
        print(f"[bench] cpu {json.dumps(cpu)}", file=sys.stderr, flush=True)
    line = {
        "metric": "MoE-layer tokens/s; decode HBM TB/s and prefill MFMA TFLOP/s vs roofline",
        "value": main_s["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32"}[cfg.act_dtype] + {"i8": "+i8w", "i4": "+i4w"}.get(cfg.expert_dtype, ""),
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: MoE layer d_model={cfg.d_model} E={cfg.n_experts} "
                               f"d_ff={cfg.d_ff} top-{cfg.top_k}"
                               + (f" + shared d_ff={cfg.shared_d_ff}" if cfg.shared_d_ff else ""),
                   "tokens": T, "instances": args.instances, "hip_graph": bool(args.graph),
                   "routing": "given" if args.routed else "gate"},
        "roofline": {k: main_s["roofline"][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "roofline_kernel": main_s["roofline"]["kernel"],
        "stage_ms": main_s["stage_ms"],
        "stage_pass_step_ms": main_s["step_ms_pct"],
        "layer": {k: main_s[k] for k in ("layer_GBps", "layer_TFLOPs", "layer_hbm_frac", "layer_mfma_frac",
                                         "down_frac", "active_experts")},
        "target": main_s["target"],
        "workloads": [{k: s[k] for k in ("config", "T", "tokens_per_s", "ms_per_step", "stage_ms", "layer_GBps",
                                         "layer_TFLOPs", "layer_hbm_frac", "layer_mfma_frac", "roofline",
                                         "target", "active_experts")} for s in workloads],
        "decode_concurrency": concurrency,
        "hip_graph_replay": graph_replay,
        "cpu_baseline": cpu,
        "measured_peaks": None if args.no_measured_peaks else measured_peaks(main_s["roofline"]),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
