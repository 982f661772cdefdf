"""GPU parity of libmoe against the CPU oracle, through the C ABI.

Reduced-width layers keep every kernel path (fp32 VALU, bf16 MFMA, int8 and int4 MFMA,
shared expert, skewed routing with empty and overfull experts, ragged row tiles)
at sizes the oracle evaluates in full within seconds. Full-size layers live in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import synth
from harness import compare, gpu_layer, oracle_layer

pytestmark = pytest.mark.gpu


def _run(cfg, T_list, max_tokens=None, instance=0, device="cpu"):
    L = synth.make_layer(cfg, device=device, instance=instance)
    olay = oracle_layer(L)
    lay = gpu_layer(L, max_tokens or max(T_list))
    res = {}
    for T in T_list:
        print(f"[parity] {cfg.name} d={cfg.d_model} E={cfg.n_experts} F={cfg.d_ff} k={cfg.top_k} T={T}", flush=True)
        x = synth.make_tokens(cfg, T, device=device, instance=instance).cuda()
        out = lay.forward(x, scatter=True)
        torch.cuda.synchronize()
        res[T] = compare(cfg, x, olay, out, label=f"{cfg.name} T={T}")
    lay.close()
    return res


def test_tiny_f32_full():
    cfg = synth.get_config("tiny_f32")
    r = _run(cfg, [64, 1, 37, 64])
    assert r[64]["frob"] < 1e-5


def test_mixtral_shape_reduced_bf16():
    # T = 1024 and 3072 run several 256-row tiles per expert (d_ff 1024 is too narrow to split
    # the down projection's K)
    cfg = synth.get_config("mixtral_bf16", d_model=512, d_ff=1024)
    _run(cfg, [1, 8, 64, 300, 1024, 3072])


def test_down_ksplit_reduced_bf16():
    # d_ff >= 4096 and few row tiles: the down projection's K is split in two (partial rows
    # added by the Gather pass)
    cfg = synth.get_config("mixtral_bf16", d_model=256, d_ff=4096)
    _run(cfg, [1024, 2000])


def test_shared_expert_reduced_bf16():
    cfg = synth.get_config("shared_fine_bf16", d_model=512, d_ff=256, shared_d_ff=2048)
    _run(cfg, [16, 200, 1100])


def test_skewed_many_experts_reduced_bf16():
    # 128 experts with a Zipf bias: most experts empty, a few far over one row tile
    cfg = synth.get_config("skewed_bf16", d_model=256, d_ff=128)
    _run(cfg, [1024])


def test_int8_reduced():
    # streaming kernels up to T = 32, tile-stream past it
    cfg = synth.get_config("int8_mixtral22b", d_model=512, d_ff=1024)
    _run(cfg, [1, 16, 32, 33, 64, 256, 1024, 3072])


def test_int4_reduced():
    # int4 group-wise weights: the streaming kernels up to T = 32 (row tiles of 16 and 32 rows,
    # with four experts several 32-row tiles per expert), the tile-stream kernels past it
    # (64-row tiles, several per expert, ragged last tiles of one to four 16-row blocks)
    cfg = synth.get_config("int4_mixtral22b", d_model=512, d_ff=1024)
    _run(cfg, [1, 2, 16, 32, 33, 40, 64, 65, 256, 1000])
    _run(synth.get_config("int4_mixtral22b", d_model=512, d_ff=1024, n_experts=4), [20, 32, 64])


@pytest.mark.parametrize("name,Ts", [
    ("int8_mixtral22b", [40, 100, 130, 200, 260, 330, 400, 470, 520]),
    ("int4_mixtral22b", [40, 80, 130, 200, 250, 520]),
    ("mixtral_bf16", [65, 80, 130, 200, 260, 330, 384, 385, 450, 512, 513]),
])
def test_tile_stream_row_blocks(name, Ts):
    # the tile-stream kernels over every count of 16-row blocks a tile can hold (int8: 64-row
    # tiles up to 32 rows per expert on average, then 128; int4: 64, 80-row up tiles at 41-72;
    # bf16: 128-row tiles from 65 tokens while the experts average at most 96 rows, 160-row
    # ones up to 128, so T = 513 runs the LDS-tiled kernel), each count with its own number of
    # K steps in flight (int8 up projection, 8 K steps: 4 in flight below 5 row blocks, 3 at
    # 5-6 (a partial last round), 2 at 7-8), and experts over one tile
    _run(synth.get_config(name, d_model=512, d_ff=1024), Ts)


@pytest.mark.parametrize("name,E,k,Ts", [
    ("int8_mixtral22b", 64, 8, [40, 300]),
    ("int4_mixtral22b", 128, 4, [40, 700]),
    ("mixtral_bf16", 128, 4, [80, 1000]),
])
def test_tile_stream_many_experts(name, E, k, Ts):
    # the tile-stream kernels (int8, int4, bf16) over 64 and 128 experts: the workgroup's
    # expert is found by ballots over the tile table 64 entries at a time (two passes for
    # 128), most experts hold a few rows, some none
    _run(synth.get_config(name, d_model=256, d_ff=512, n_experts=E, top_k=k), Ts)


def test_quantised_partial_column_tiles():
    # d_model = 384: the down projections' last 256-column tile holds 128 columns (int4: its
    # group scales are read by lanes 0-31 only); d_ff = 192 (int8): the up projection's last
    # tile of gate/up columns holds 128
    _run(synth.get_config("int4_mixtral22b", d_model=384, d_ff=384), [70, 200])
    _run(synth.get_config("int8_mixtral22b", d_model=384, d_ff=192), [70, 200])


def test_bf16_mid_batches_without_whole_column_tiles():
    # bf16 batches in the tile-stream range whose widths leave a half 256-column tile (d_model
    # 384: the down projection; d_ff 192: the up projection's 384 gate/up columns) run the
    # LDS-tiled GEMMs instead; d_model 512, d_ff 640: both whole, the tile-stream kernels
    _run(synth.get_config("mixtral_bf16", d_model=384, d_ff=512), [80, 200])
    _run(synth.get_config("mixtral_bf16", d_model=512, d_ff=192), [80, 200])
    _run(synth.get_config("mixtral_bf16", d_model=512, d_ff=640), [80, 200, 500])


def test_tiny_batches_single_workgroup_route():
    # T <= 4 with at most 16 router columns: gate and scatter run in one workgroup
    _run(synth.get_config("mixtral_bf16", d_model=512, d_ff=1024), [1, 2, 3, 4, 5])
    _run(synth.get_config("shared_fine_bf16", d_model=256, d_ff=128, n_experts=8, top_k=2, shared_d_ff=512),
         [1, 3, 4])
    _run(synth.get_config("tiny_f32"), [1, 4])
    _run(synth.get_config("int8_mixtral22b", d_model=512, d_ff=1024), [2, 4])


def test_deterministic_and_zero_tokens():
    cfg = synth.get_config("shared_fine_bf16", d_model=256, d_ff=128, shared_d_ff=512)
    L = synth.make_layer(cfg)
    lay = gpu_layer(L, 300)
    for T in (300, 16):  # tiled GEMMs, and the streaming kernels
        x = synth.make_tokens(cfg, T).cuda()
        a = lay.forward(x, scatter=True)
        b = lay.forward(x, scatter=True)
        torch.cuda.synchronize()
        for f in ("y", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "sorted_assign", "shared_gate"):
            assert torch.equal(getattr(a, f), getattr(b, f)), (T, f)
    # T = 0 enqueues nothing and leaves the outputs alone
    out = lay.outputs(4, scatter=True)
    out.y.fill_(7)
    lay.forward(x[:0], out=out)
    torch.cuda.synchronize()
    assert (out.y == 7).all()
    lay.close()


def test_zero_router_tie_rule():
    # all logits equal: experts 0..k-1 in order, weights exactly 1/k
    cfg = synth.get_config("mixtral_bf16", d_model=256, d_ff=128, n_experts=8, top_k=3)
    L = synth.make_layer(cfg)
    L.w_router.zero_()
    lay = gpu_layer(L, 70)
    x = synth.make_tokens(cfg, 70).cuda()
    out = lay.forward(x, scatter=True)
    torch.cuda.synchronize()
    assert (out.topk_idx.cpu() == torch.arange(3, dtype=torch.int32)).all()
    assert (out.topk_w.cpu() == 1.0 / 3.0).all()
    compare(cfg, x, oracle_layer(L), out, label="zero router")
    lay.close()


def test_forward_argument_errors():
    import moe_layer_forward_gate_amd as moe
    cfg = synth.get_config("tiny_f32")
    lay = gpu_layer(synth.make_layer(cfg), 16)
    x = synth.make_tokens(cfg, 17).cuda()
    with pytest.raises(moe.MoeError) as ei:
        lay.forward(x)  # T > max_tokens
    assert ei.value.status == moe.MOE_EINVAL
    buf = torch.empty(16 * 256 + 1, dtype=torch.float32, device="cuda")
    xm = buf[1:].view(16, 256)  # 4-byte aligned, not 16
    with pytest.raises(moe.MoeError) as ei:
        lay.forward(xm)
    assert ei.value.status == moe.MOE_EINVAL
    lay.close()


@pytest.mark.parametrize("name,kw", [
    ("shared_fine_bf16", dict(d_model=256, d_ff=128, shared_d_ff=512)),
    ("mixtral_bf16", dict(d_model=256, d_ff=256)),
    ("int8_mixtral22b", dict(d_model=256, d_ff=128)),
    ("int4_mixtral22b", dict(d_model=256, d_ff=256)),
])
def test_hip_graph_replays_match_eager(name, kw):
    # moe_forward only enqueues kernels (no allocation, no host sync, no memset nodes), so it
    # can be captured in a HIP graph; every replay, with eager work and synchronisations in
    # between, must reproduce the eager result bit for bit (prefill and decode plans of the
    # bf16, int8 and int4 kernels: T = 300 runs the LDS-tiled GEMMs on the shared + fine
    # layer, the tile-stream ones on the others)
    cfg = synth.get_config(name, **kw)
    L = synth.make_layer(cfg)
    lay = gpu_layer(L, 300)
    for T in (300, 3, 16):
        x = synth.make_tokens(cfg, T).cuda()
        ref = lay.forward(x, scatter=True)
        torch.cuda.synchronize()
        out = lay.outputs(T, scatter=True)
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            lay.forward(x, out=out, stream=s)
        torch.cuda.synchronize()
        fields = [f for f in ("y", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "sorted_assign",
                              "shared_gate") if getattr(out, f, None) is not None]
        for rep in range(3):
            for f in fields:
                getattr(out, f).fill_(-1) if getattr(out, f).dtype != torch.bfloat16 else getattr(out, f).fill_(7)
            g.replay()
            torch.cuda.synchronize()
            for f in fields:
                assert torch.equal(getattr(out, f), getattr(ref, f)), (T, rep, f)
            lay.forward(x[: max(1, T // 2)], scatter=True)  # eager work between replays
            torch.cuda.synchronize()
        del g
    lay.close()


def test_gate_token_block_shapes():
    # the MFMA gate's workgroup shapes: 16 waves over one 16-token block (T < 8192, up to 80
    # router columns), 8 waves over two blocks (8192 <= T < 16384, up to 128 columns), 4 waves
    # over two (wider routers) or four blocks (T >= 16384); ragged last token blocks
    _run(synth.get_config("mixtral_bf16", d_model=256, d_ff=128), [8200, 16400])
    _run(synth.get_config("shared_fine_bf16", d_model=256, d_ff=128, n_experts=100, top_k=4, shared_d_ff=256),
         [8195])
    _run(synth.get_config("shared_fine_bf16", d_model=256, d_ff=128, n_experts=128, top_k=2, shared_d_ff=256),
         [8200])
