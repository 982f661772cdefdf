"""The C ABI on the CPU: libmoe loads, exports every declared symbol, and rejects
bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import moe_layer_forward_gate_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", txt)))


def _decl_comments():
    """{symbol: the block comment right above its MOE_API declaration}."""
    txt = open(HEADER).read()
    out = {}
    for m in re.finditer(r"/\*((?:(?!\*/).)*)\*/\s*MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", txt, re.S):
        out[m.group(2)] = m.group(1)
    return out


# the page keys every citation in the header uses
PAGE_CITE = re.compile(r"\[(0539edu|mhpq|hotelren|trdm|pptc) §\d+(\.\d+)*\]")


# entry points that are not a step of the pages' method: their comment names the callers
# they are for instead of a page passage
NOT_FROM_THE_PAGES = {"moe_forward_noalloc": "callers that cannot allocate"}


def test_every_declaration_cites_a_page_passage():
    com = _decl_comments()
    assert sorted(com) == _declared(), "every MOE_API declaration has a block comment right above it"
    for name, c in com.items():
        if name in NOT_FROM_THE_PAGES:
            assert NOT_FROM_THE_PAGES[name] in " ".join(c.split()), name
            continue
        assert PAGE_CITE.search(c), f"{name}: its comment cites no page passage"


def test_header_declares_binding_names():
    assert _declared() == sorted(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    assert moe.moe_status_str(0) == "MOE_OK"
    assert moe.moe_status_str(-1).startswith("MOE_EINVAL")
    assert moe.moe_status_str(-2).startswith("MOE_EUNSUPPORTED")
    assert moe.moe_status_str(-3).startswith("MOE_ENOMEM")
    assert moe.moe_status_str(-4).startswith("MOE_EHIP")
    assert moe.moe_status_str(5) == "unknown moe status"


def _desc(**kw):
    base = dict(d_model=256, n_experts=8, d_ff=512, top_k=2, max_tokens=64, act_dtype=moe.MOE_BF16,
                expert_dtype=moe.MOE_BF16, shared_d_ff=0, profile=0, gate_clamp=0, gate_weighting=0)
    base.update(kw)
    return moe.MoeDesc(**base)


def _weights(**kw):
    fake = 0x10000  # never dereferenced: every case below fails its checks first
    base = dict(w_router=fake, b_router=0, w_gate=fake, w_up=fake, w_down=fake, s_gate=0, s_up=0, s_down=0,
                w_shared_gate=0, ws_gate=0, ws_up=0, ws_down=0)
    base.update(kw)
    return moe.MoeWeights(**base)


def _create(desc, weights):
    h = ctypes.c_void_p(0xDEAD)
    rc = moe.lib().moe_layer_create(ctypes.byref(desc) if desc is not None else None,
                                    ctypes.byref(weights) if weights is not None else None, ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("desc,weights,status", [
    (None, _weights(), moe.MOE_EINVAL),
    (_desc(), None, moe.MOE_EINVAL),
    (_desc(d_model=0), _weights(), moe.MOE_EINVAL),
    (_desc(max_tokens=-1), _weights(), moe.MOE_EINVAL),
    (_desc(top_k=9), _weights(), moe.MOE_EINVAL),
    (_desc(top_k=0), _weights(), moe.MOE_EINVAL),
    (_desc(profile=2), _weights(), moe.MOE_EINVAL),
    (_desc(gate_clamp=2), _weights(), moe.MOE_EINVAL),
    (_desc(gate_weighting=2), _weights(), moe.MOE_EINVAL),
    (_desc(gate_weighting=-1), _weights(), moe.MOE_EINVAL),
    (_desc(), _weights(w_gate=0), moe.MOE_EINVAL),
    (_desc(), _weights(w_router=0), moe.MOE_EINVAL),
    (_desc(expert_dtype=moe.MOE_I8), _weights(), moe.MOE_EINVAL),            # scales missing
    (_desc(shared_d_ff=1024), _weights(), moe.MOE_EINVAL),                    # shared weights missing
    (_desc(act_dtype=moe.MOE_F32, expert_dtype=moe.MOE_BF16), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(act_dtype=moe.MOE_BF16, expert_dtype=moe.MOE_F32), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(act_dtype=7), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(d_model=192), _weights(), moe.MOE_EUNSUPPORTED),                   # bf16 needs d % 128
    (_desc(d_ff=96), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(n_experts=129, top_k=2), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(n_experts=128, top_k=65), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(shared_d_ff=700), _weights(w_shared_gate=1 << 16, ws_gate=1 << 16, ws_up=1 << 16, ws_down=1 << 16),
     moe.MOE_EUNSUPPORTED),                                                   # not a multiple of d_ff
    (_desc(expert_dtype=moe.MOE_I8, shared_d_ff=1024),
     _weights(s_gate=1 << 16, s_up=1 << 16, s_down=1 << 16, w_shared_gate=1 << 16, ws_gate=1 << 16,
              ws_up=1 << 16, ws_down=1 << 16), moe.MOE_EUNSUPPORTED),
    (_desc(max_tokens=1 << 29, top_k=2), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(expert_dtype=moe.MOE_I4), _weights(), moe.MOE_EINVAL),            # group scales missing
    (_desc(expert_dtype=moe.MOE_I4, d_ff=192), _weights(s_gate=1 << 16, s_up=1 << 16, s_down=1 << 16),
     moe.MOE_EUNSUPPORTED),                                                   # int4 needs d_ff % 128
    (_desc(act_dtype=moe.MOE_F32, expert_dtype=moe.MOE_I4), _weights(), moe.MOE_EUNSUPPORTED),
    (_desc(expert_dtype=moe.MOE_I4, shared_d_ff=512),
     _weights(s_gate=1 << 16, s_up=1 << 16, s_down=1 << 16, w_shared_gate=1 << 16, ws_gate=1 << 16,
              ws_up=1 << 16, ws_down=1 << 16), moe.MOE_EUNSUPPORTED),    # shared expert needs bf16
])
def test_create_rejects(desc, weights, status):
    rc, h = _create(desc, weights)
    assert rc == status, moe.moe_last_error()
    assert h.value is None  # *out set to NULL
    assert moe.moe_last_error() != ""


def test_create_null_out():
    rc = moe.lib().moe_layer_create(ctypes.byref(_desc()), ctypes.byref(_weights()), None)
    assert rc == moe.MOE_EINVAL


def test_forward_rejects_before_gpu():
    L = moe.lib()
    route = moe.MoeRouteOut(0x10000, 0x10000, 0, 0, 0, 0)
    assert L.moe_forward(None, 0x10000, 4, 0x10000, ctypes.byref(route), None) == moe.MOE_EINVAL
    assert "layer" in moe.moe_last_error()


def test_stage_times_profiling_and_destroy_null():
    L = moe.lib()
    ms = (ctypes.c_float * 5)()
    assert L.moe_stage_times(None, ms) == moe.MOE_EINVAL
    assert L.moe_set_profiling(None, 1) == moe.MOE_EINVAL
    L.moe_destroy(None)  # NULL-safe


def test_forward_routed_rejects_before_gpu():
    L = moe.lib()
    fake = 0x10000
    assert L.moe_forward_routed(None, fake, 4, fake, fake, None, fake, None, None) == moe.MOE_EINVAL
    assert "layer" in moe.moe_last_error()


def test_binding_checks_weight_tensors_before_create():
    # the binding checks dtype, shape, device and layout of every weight before the
    # library reads the bytes its layout implies from the pointers
    import torch
    import synth
    cpu = torch.device("cpu")
    for name in ("mixtral_bf16", "int8_mixtral22b", "int4_mixtral22b", "shared_fine_bf16", "skewed_bf16"):
        cfg = synth.get_config(name, d_model=256, d_ff=256, n_experts=8, top_k=2,
                               shared_d_ff=512 if name == "shared_fine_bf16" else 0)
        L = synth.make_layer(cfg)
        kw = synth.layer_kwargs(L, cpu)
        t = {k: kw[k] for k in ("w_router", "b_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                "w_shared_gate", "ws_gate", "ws_up", "ws_down")}
        exp = moe.MoeLayer.expected_weights(cfg.d_model, cfg.n_experts, cfg.d_ff, cfg.act_dtype, cfg.expert_dtype,
                                            cfg.shared_d_ff, has_bias=t["b_router"] is not None)
        moe.check_weight_tensors(t, exp, cpu)  # the generator's layers pass
        bad = dict(t, w_router=t["w_router"].to(torch.bfloat16))
        with pytest.raises(ValueError, match="w_router"):
            moe.check_weight_tensors(bad, exp, cpu)
        bad = dict(t, w_down=t["w_down"][:, :-2])
        with pytest.raises(ValueError, match="w_down"):
            moe.check_weight_tensors(bad, exp, cpu)
        bad = dict(t, w_gate=t["w_gate"].transpose(1, 2))
        with pytest.raises(ValueError, match="w_gate"):
            moe.check_weight_tensors(bad, exp, cpu)
        with pytest.raises(ValueError, match="on meta"):
            moe.check_weight_tensors(t, exp, torch.device("meta"))
        if cfg.expert_dtype in ("i8", "i4"):
            bad = dict(t, s_down=None)
            with pytest.raises(ValueError, match="s_down"):
                moe.check_weight_tensors(bad, exp, cpu)
        else:
            bad = dict(t, s_gate=torch.ones(8))
            with pytest.raises(ValueError, match="s_gate"):
                moe.check_weight_tensors(bad, exp, cpu)
        if cfg.expert_dtype == "i4":  # unpacked int4 (one value a byte) is refused
            bad = dict(t, w_up=L.w_up)
            with pytest.raises(ValueError, match="w_up"):
                moe.check_weight_tensors(bad, exp, cpu)
