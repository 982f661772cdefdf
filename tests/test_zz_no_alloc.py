"""moe_forward_noalloc (the forward in the library's static device scratch) against
moe_forward through the C ABI: the same launch plan, so every output must be
bit-identical, on two calls in a row with the second batch smaller, for the LDS-tiled
prefill path, the tile-stream path (bf16 and quantised), the weight-streaming decode path
and the split decode gate; and a
batch too large for the scratch is refused before anything is written."""
import ctypes

import pytest
import torch

import moe_layer_forward_gate_amd as moe
import synth

pytestmark = pytest.mark.gpu

FIELDS = ("y", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "sorted_assign", "shared_gate")


def _layer(cfg, max_tokens):
    dev = torch.device("cuda", torch.cuda.current_device())
    return moe.MoeLayer(max_tokens=max_tokens, **synth.layer_kwargs(synth.make_layer(cfg, device="cuda"), dev))


def _route(out):
    p = lambda t: 0 if t is None else int(t.data_ptr())  # noqa: E731
    return moe.MoeRouteOut(p(out.topk_idx), p(out.topk_w), p(out.expert_counts), p(out.expert_offsets),
                           p(out.sorted_assign), p(out.shared_gate))


def _poison(out):
    for f in FIELDS:
        t = getattr(out, f)
        if t is not None:
            t.fill_(7 if t.dtype == torch.bfloat16 else -3)


@pytest.mark.parametrize("name,kw,Ts", [
    ("mixtral_bf16", dict(d_model=512, d_ff=1024), (600, 300, 5)),            # LDS-tiled, tile-stream, streaming
    ("int8_mixtral22b", dict(d_model=512, d_ff=1024), (40, 16, 3)),           # int8 tile-stream, streaming
    ("shared_fine_bf16", dict(d_model=256, d_ff=128, shared_d_ff=512), (20, 2)),  # split gate, shared expert
    ("int4_mixtral22b", dict(d_model=512, d_ff=1024), (250, 70, 9)),          # int4 80/64-row tile-stream, tile-stream, streaming
    ("tiny_f32", {}, (64, 7)),                                                # fp32 experts
])
def test_noalloc_matches_forward(name, kw, Ts):
    cfg = synth.get_config(name, **kw)
    lay = _layer(cfg, max(Ts))
    L = moe.lib()
    s = torch.cuda.current_stream()
    for T in Ts:  # consecutive calls, each batch smaller than the one before
        print(f"[noalloc] {name} T={T}", flush=True)
        x = synth.make_tokens(cfg, T, device="cuda", instance=T)
        ref = lay.forward(x, scatter=True)
        out = lay.outputs(T, scatter=True)
        _poison(out)
        rc = L.moe_forward_noalloc(lay._h, ctypes.c_void_p(x.data_ptr()), T, ctypes.c_void_p(out.y.data_ptr()),
                                   ctypes.byref(_route(out)), ctypes.c_void_p(int(s.cuda_stream)))
        assert rc == moe.MOE_OK, moe.moe_last_error()
        torch.cuda.synchronize()
        for f in FIELDS:
            a, b = getattr(out, f), getattr(ref, f)
            if b is not None:
                assert torch.equal(a, b), (name, T, f)
    lay.close()


def test_noalloc_refuses_a_batch_past_the_scratch():
    # d_model 512, d_ff 8192, T = 4096: H alone needs over 100 MB of padded rows
    cfg = synth.get_config("mixtral_bf16", d_model=512, d_ff=8192)
    lay = _layer(cfg, 4096)
    x = synth.make_tokens(cfg, 4096, device="cuda")
    out = lay.outputs(4096, scatter=True)
    _poison(out)
    torch.cuda.synchronize()
    with pytest.raises(moe.MoeError) as ei:
        lay.forward(x, out=out, noalloc=True)
    assert ei.value.status == moe.MOE_EINVAL
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert (out.y == 7).all() and (out.topk_idx == -3).all()  # nothing was written
    # the same batch through moe_forward, then a decode batch through the scratch
    lay.forward(x, out=out)
    small = synth.make_tokens(cfg, 8, device="cuda")
    a = lay.forward(small, scatter=True)
    b = lay.forward(small, scatter=True, noalloc=True)
    torch.cuda.synchronize()
    for f in FIELDS:
        if getattr(a, f) is not None:
            assert torch.equal(getattr(a, f), getattr(b, f)), f
    lay.close()
