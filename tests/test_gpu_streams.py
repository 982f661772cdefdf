"""Concurrent layers on several HIP streams (one layer per stream, the library's rule for
concurrent calls): every stream's results equal the same layer's results run alone, bit
for bit, and match the oracle."""
import pytest
import torch

import synth
from harness import compare, gpu_layer, oracle_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw,T", [
    ("mixtral_bf16", dict(d_model=512, d_ff=1024), 1),
    ("mixtral_bf16", dict(d_model=512, d_ff=1024), 300),   # tile-stream
    ("mixtral_bf16", dict(d_model=512, d_ff=1024), 600),   # LDS-tiled
    ("int4_mixtral22b", dict(d_model=256, d_ff=256), 16),
])
def test_streams_match_serial(name, kw, T):
    cfg = synth.get_config(name, **kw)
    S = 4
    Ls = [synth.make_layer(cfg, instance=i) for i in range(S)]
    lays = [gpu_layer(L, T) for L in Ls]
    xs = [synth.make_tokens(cfg, T, instance=i).cuda() for i in range(S)]
    print(f"[streams] {name} T={T} serial", flush=True)
    ref = [lay.forward(x, scatter=True) for lay, x in zip(lays, xs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(S)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    print(f"[streams] {name} T={T} concurrent", flush=True)
    outs = []
    for rep in range(3):
        outs = [lay.outputs(T, scatter=True) for lay in lays]
        for lay, x, out, st in zip(lays, xs, outs, streams):
            lay.forward(x, out=out, stream=st)
        torch.cuda.synchronize()
        for i in range(S):
            for f in ("y", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "sorted_assign"):
                assert torch.equal(getattr(outs[i], f), getattr(ref[i], f)), f"stream {i} rep {rep}: {f} differs"
    compare(cfg, xs[1].cpu(), oracle_layer(Ls[1]), outs[1], label=f"{name} T={T} stream 1")
    for lay in lays:
        lay.close()
