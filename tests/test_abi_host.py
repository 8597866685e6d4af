"""The C ABI on the host: the library loads, exports every declared symbol, sizes its
workspace, and rejects bad arguments before any HIP call (CPU only, no kernel launched)."""
import ctypes
import os
import re

import pytest
import torch

from conftest import ROOT

import bit_moe_expert_amd as pkg
from bit_moe_expert_amd import moe

HEADER = os.path.join(ROOT, "include", "moe_int4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|size_t|const char\s*\*)\s+(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    # and nothing of the oracle is linked in
    syms = open(moe.LIB_PATH, "rb").read()
    assert b"oracle_" not in syms


def _dims(d=2048, E=256, k=8, I=512, Is=512, g=64):
    return moe.Dims(d, E, k, I, Is, g)


def test_sizing_helpers():
    d = _dims()
    assert moe.max_tiles(d, 512) == 256 + 4096 // 32 + 16
    assert moe.max_tiles(d, 1) == 8 + 0 + 1
    assert moe.max_tiles(_dims(E=128, I=768, Is=0), 256) == 128 + 64
    ws = moe.workspace_bytes(d, 512)
    # at least the fp16 rows of the down product with their segment exponents, and h
    assert ws % 256 == 0 and ws >= (4096 + 512) * (2048 * 2 + 2048 // 32) + 4096 * 512 * 2
    assert moe.workspace_bytes(d, 0) > 0
    assert moe.workspace_bytes(_dims(g=32), 8) == 0
    # the router's chunk partials hold one [d/64][E] plane per token of a small call
    assert moe.workspace_bytes(d, 8) - moe.workspace_bytes(d, 7) >= (2048 // 64) * 256 * 4
    assert moe.max_tiles(_dims(k=17), 8) == -1


def test_stage_lists():
    L = moe.lib()
    d = _dims()
    n1 = L.moe_num_stages(ctypes.byref(d), 1)
    assert [L.moe_stage_name(ctypes.byref(d), 1, s).decode() for s in range(n1)] == \
        ["router_decode", "gemv_gateup_topk", "gemv_down_combine"]
    n2 = L.moe_num_stages(ctypes.byref(d), 512)
    assert [L.moe_stage_name(ctypes.byref(d), 512, s).decode() for s in range(n2)] == \
        ["router_prefill", "topk_prefill", "route_meta", "gateup_gemm", "down_gemm", "combine"]
    assert L.moe_stage_name(ctypes.byref(d), 512, 6) is None
    big = _dims(k=16, I=2048)  # too much h for the GEMV path: T = 1 runs the grouped GEMM
    assert [L.moe_stage_name(ctypes.byref(big), 1, s).decode() for s in range(L.moe_num_stages(ctypes.byref(big), 1))] \
        == ["router_decode", "decode_topk", "route_meta", "gateup_gemm", "down_gemm", "combine"]
    # calls of up to 32 tokens take the GEMV path; 33 tokens and up the grouped GEMM
    for T in (2, 5, 8, 16, 32):
        assert [L.moe_stage_name(ctypes.byref(d), T, s).decode() for s in range(L.moe_num_stages(ctypes.byref(d), T))] \
            == ["router_decode", "gemv_gateup_topk", "gemv_down_combine"], T
    assert L.moe_stage_name(ctypes.byref(d), 33, 0).decode() == "router_prefill"
    assert L.moe_num_stages(ctypes.byref(d), 33) == 6


class _Fake:
    """Non-null, suitably aligned fake device addresses: validation never dereferences them."""

    def __init__(self):
        self.base = 1 << 40
        self.n = 0

    def __call__(self, align=256):
        self.n += 1
        return self.base + self.n * (1 << 20)


def _ffn(f):
    q = lambda: moe.Q4(f(), f(), f())  # noqa: E731
    return moe.FFNQ4(q(), q(), q())


def _layer_call(dims, T, f, **over):
    a = dict(x=f(), wr=f(), bias=None, routed=_ffn(f), shared=_ffn(f), y=f(), ws=f(), ws_bytes=1 << 40)
    a.update(over)
    L = moe.lib()
    return L.moe_forward_layer(ctypes.byref(dims), T, a["x"], a["wr"], a["bias"],
                               ctypes.byref(a["routed"]) if a["routed"] is not None else None,
                               ctypes.byref(a["shared"]) if a["shared"] is not None else None,
                               a["y"], a["ws"], a["ws_bytes"], None)


def test_validation_codes_before_any_hip_call():
    f = _Fake()
    d = _dims()
    L = moe.lib()
    assert _layer_call(d, 0, f) == moe.MOE_OK  # T = 0: no-op
    assert _layer_call(d, -1, f) == moe.MOE_EINVAL
    assert _layer_call(_dims(g=32), 4, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(_dims(d=100), 4, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(_dims(k=9, E=8), 4, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(_dims(k=17, E=64), 4, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(_dims(E=2048), 4, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(_dims(I=96), 4, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(d, 70000, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(d, 4, f, x=None) == moe.MOE_EINVAL
    assert _layer_call(d, 4, f, x=f() + 2) == moe.MOE_EINVAL          # misaligned
    assert _layer_call(d, 4, f, wr=None) == moe.MOE_EINVAL
    assert _layer_call(d, 4, f, shared=None) == moe.MOE_EINVAL        # d_ff_shared > 0 needs them
    assert _layer_call(_dims(Is=0), 4, f) == moe.MOE_EINVAL            # given but not expected
    assert _layer_call(d, 4, f, y=None) == moe.MOE_EINVAL
    x = f()
    assert _layer_call(d, 4, f, x=x, y=x) == moe.MOE_EINVAL           # y aliases x
    assert _layer_call(d, 4, f, ws=f() + 64) == moe.MOE_EINVAL        # ws alignment
    assert _layer_call(d, 4, f, ws_bytes=1000) == moe.MOE_EWORKSPACE
    bad = _ffn(f)
    bad.down.codes = f() + 8
    assert _layer_call(d, 4, f, routed=bad) == moe.MOE_EINVAL
    assert "codes" in L.moe_last_error().decode()
    assert L.moe_status_str(moe.MOE_EWORKSPACE).decode().startswith("MOE_EWORKSPACE")
    # route and expert_ffn validate the same way
    r = moe.Routing(*[f() for _ in range(8)])
    assert L.moe_route(ctypes.byref(_dims(k=0)), 4, f(), f(), None, ctypes.byref(r), f(), 1 << 40, None) == \
        moe.MOE_EUNSUPPORTED
    r0 = moe.Routing(*([None] + [f() for _ in range(7)]))
    assert L.moe_route(ctypes.byref(d), 4, f(), f(), None, ctypes.byref(r0), f(), 1 << 40, None) == moe.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), 0, f(), f(), None, ctypes.byref(r), f(), 1 << 40, None) == moe.MOE_OK
    rf = _ffn(f)
    assert L.moe_expert_ffn(ctypes.byref(d), 4, f(), ctypes.byref(r), ctypes.byref(rf), None, f(), f(), 1 << 40,
                            None) == moe.MOE_EINVAL
    assert L.moe_expert_ffn(ctypes.byref(d), 0, f(), ctypes.byref(r), ctypes.byref(rf), ctypes.byref(rf), f(), f(),
                            1 << 40, None) == moe.MOE_OK
    q = moe.Q4(f(), f(), f())
    assert L.moe_debug_dequant(ctypes.byref(q), 4, 96, f(), None) == moe.MOE_EUNSUPPORTED
    assert L.moe_debug_dequant(ctypes.byref(q), 0, 128, f(), None) == moe.MOE_OK
    assert L.moe_launch_stage(7, ctypes.byref(d), 4, f(), f(), None, ctypes.byref(rf), ctypes.byref(rf), f(), f(),
                              1 << 40, None) == moe.MOE_EINVAL


def test_binding_refuses_cpu_tensors_and_has_no_fallback():
    import torch
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        moe._ptr(x, torch.bfloat16, "x")
    # the product package never imports the oracle
    src = "".join(open(os.path.join(ROOT, "bit_moe_expert_amd", n)).read() for n in ("moe.py", "__init__.py"))
    assert "oracle" not in src.replace("oracle_", "")
    assert pkg.moe.LIB_PATH.endswith("libmoe_int4.so")


def test_vocab_topk_sizing_and_validation():
    L = moe.lib()
    assert L.moe_vocab_topk_workspace_bytes(256, 262144, 64) == 256 * 512 * 4
    assert L.moe_vocab_topk_workspace_bytes(1, 100, 16) == 256            # one chunk, rounded up
    assert L.moe_vocab_topk_workspace_bytes(3, 1 << 22, 64) == 3 * 8192 * 4
    assert L.moe_vocab_topk_workspace_bytes(3, (1 << 22) + 1, 64) == 0     # more than 8192 chunks
    assert L.moe_vocab_topk_workspace_bytes(3, 1000, 129) == 0
    assert L.moe_vocab_topk_workspace_bytes(3, 10, 11) == 0
    f = _Fake()
    call = lambda R, V, K, **o: L.moe_vocab_topk(R, V, K, o.get("logits", f()), o.get("ids", f()),  # noqa: E731
                                                 o.get("vals", f()), o.get("ws", f()), o.get("ws_bytes", 1 << 30),
                                                 None)
    assert call(0, 1000, 8) == moe.MOE_OK
    assert call(-1, 1000, 8) == moe.MOE_EINVAL
    assert call(2, 1000, 0) == moe.MOE_EUNSUPPORTED
    assert call(2, 1000, 129) == moe.MOE_EUNSUPPORTED
    assert call(2, 8, 9) == moe.MOE_EUNSUPPORTED
    assert call(2, 1000, 8, logits=None) == moe.MOE_EINVAL
    assert call(2, 1000, 8, ids=f() + 2) == moe.MOE_EINVAL
    assert call(2, 1000, 8, ws=f() + 128) == moe.MOE_EINVAL
    assert call(2, 1000, 8, ws_bytes=16) == moe.MOE_EWORKSPACE


def test_code_bits_validation():
    f = _Fake()
    L = moe.lib()

    def dims(bits, **kw):
        d = _dims(**kw)
        d.code_bits = bits
        return d

    assert _layer_call(dims(5), 4, f) == moe.MOE_EUNSUPPORTED
    assert _layer_call(dims(1), 4, f) == moe.MOE_EUNSUPPORTED
    # 3- and 2-bit codes on the grouped-GEMM path (T > 32, or too much h for the GEMV path): the
    # width passes and the checks go on to y
    assert _layer_call(dims(3), 33, f, y=None) == moe.MOE_EINVAL
    assert "y NULL" in L.moe_last_error().decode()
    assert _layer_call(dims(2, k=16, I=2048), 1, f, y=None) == moe.MOE_EINVAL
    assert "y NULL" in L.moe_last_error().decode()
    bad = _ffn(f)
    bad.gate.codes = f() + 4                                         # 4-byte aligned: enough for 3-bit codes only
    assert _layer_call(dims(2), 4, f, routed=bad) == moe.MOE_EINVAL
    assert _layer_call(dims(4), 4, f, routed=bad) == moe.MOE_EINVAL
    bad.gate.codes = f() + 8                                         # 2-bit codes move as 16-byte chunks
    assert _layer_call(dims(2), 4, f, routed=bad) == moe.MOE_EINVAL
    bad.gate.codes = f() + 4
    assert _layer_call(dims(3), 4, f, routed=bad, y=None) == moe.MOE_EINVAL  # the codes passed; y did not
    assert "y NULL" in L.moe_last_error().decode()
    q = moe.Q4(f() + 4, f(), f())
    assert L.moe_debug_dequant_bits(ctypes.byref(q), 4, 128, 5, f(), None) == moe.MOE_EUNSUPPORTED
    assert L.moe_debug_dequant_bits(ctypes.byref(q), 4, 128, 2, f(), None) == moe.MOE_EINVAL


def test_noalloc_and_debug_gemm_validation():
    """moe_forward_layer_noalloc refuses calls whose workspace exceeds the fixed scratch (before any
    HIP call), validates the other arguments like moe_forward_layer; the grouped-GEMM check export
    validates its arguments the same way."""
    f = _Fake()
    d = _dims()
    L = moe.lib()
    hdr = open(HEADER).read()
    assert re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", hdr)
    assert moe.NOALLOC_SCRATCH_BYTES == 64 << 20
    T = 1
    while L.moe_workspace_bytes(ctypes.byref(d), T) <= moe.NOALLOC_SCRATCH_BYTES:
        T += 64
    rf = _ffn(f)

    def na(dims, T, **o):
        return L.moe_forward_layer_noalloc(ctypes.byref(dims), T, o.get("x", f()), o.get("wr", f()), None,
                                           ctypes.byref(rf), ctypes.byref(o.get("sh", rf)) if o.get("sh", rf) else None,
                                           o.get("y", f()), None)
    assert na(d, T) == moe.MOE_EWORKSPACE
    assert "fixed scratch" in L.moe_last_error().decode()
    assert na(d, 0) == moe.MOE_OK
    assert na(d, -3) == moe.MOE_EINVAL
    assert na(d, 8, x=None) == moe.MOE_EINVAL
    assert na(d, 8, y=f() + 2) == moe.MOE_EINVAL
    assert na(d, 8, sh=None) == moe.MOE_EINVAL
    assert na(_dims(g=32), 8) == moe.MOE_EUNSUPPORTED
    r = moe.Routing(*[f() for _ in range(8)])

    def dg(which, **o):
        return L.moe_debug_grouped_gemm(ctypes.byref(o.get("dims", d)), o.get("T", 16), which, o.get("a", f()),
                                        ctypes.byref(r), ctypes.byref(rf), ctypes.byref(rf), o.get("out", f()),
                                        o.get("out2", f()), f(), o.get("ws_bytes", 1 << 40), None)
    assert dg(2) == moe.MOE_EINVAL
    assert dg(0, T=0) == moe.MOE_OK
    assert dg(0, out2=None) == moe.MOE_EINVAL
    assert dg(0, a=f() + 2) == moe.MOE_EINVAL
    assert dg(1, ws_bytes=100) == moe.MOE_EWORKSPACE
    d3 = _dims()
    d3.code_bits = 3                                                 # 3-bit codes pass; the checks go on
    assert dg(0, dims=d3, out2=None) == moe.MOE_EINVAL
    d3.code_bits = 5
    assert dg(0, dims=d3) == moe.MOE_EUNSUPPORTED


def _cpu_ffn(n, I, d, bits=4):
    def proj(out_dim, in_dim):
        return moe.QProj(torch.zeros((n, out_dim, in_dim * bits // 8), dtype=torch.uint8),
                         torch.zeros((n, out_dim, in_dim // 64), dtype=torch.bfloat16),
                         torch.zeros((n, out_dim, in_dim // 64), dtype=torch.bfloat16), bits)
    return moe.QuantFFN(proj(I, d), proj(I, d), proj(d, I))


def _cpu_routing(dims, T):
    k, E = dims.top_k, dims.n_experts
    i32 = dict(dtype=torch.int32)
    return {"topk_ids": torch.zeros((T, k), **i32), "topk_w": torch.zeros((T, k), dtype=torch.float32),
            "counts": torch.zeros(E, **i32), "offsets": torch.zeros(E + 1, **i32),
            "sorted_token": torch.zeros(T * k, **i32), "inv_pos": torch.zeros((T, k), **i32),
            "tiles": torch.zeros((moe.max_tiles(dims, T), 3), **i32), "n_tiles": torch.zeros(1, **i32)}


def _refused(fn, *a, **kw):
    with pytest.raises(moe.MoeError) as ei:
        fn(*a, **kw)
    assert ei.value.status == moe.MOE_EINVAL
    return str(ei.value)


def test_binding_checks_shapes_before_the_library():
    """moe.py refuses tensors whose shapes do not match the layer (the C ABI sees only pointers,
    where a wrong size would turn into out-of-bounds device reads), before any pointer is taken."""
    T, d, E, k, I, Is = 40, 128, 8, 2, 64, 128
    routed, shared = _cpu_ffn(E, I, d), _cpu_ffn(1, Is, d)
    dims = moe.make_dims(d, E, k, I, Is)
    x = torch.zeros((T, d), dtype=torch.bfloat16)
    r = _cpu_routing(dims, T)
    # expert arrays
    bad = _cpu_ffn(E, I, d)
    bad.up.scales = torch.zeros((E, I, d // 64 + 1), dtype=torch.bfloat16)
    assert "up.scales" in _refused(moe.expert_ffn, x, r, bad, shared)
    bad = _cpu_ffn(E, I, d)
    bad.down.codes = torch.zeros((E, d, I // 2 - 1), dtype=torch.uint8)
    assert "down.codes" in _refused(moe.expert_ffn, x, r, bad, shared)
    assert "shared" in _refused(moe.expert_ffn, x, r, routed, _cpu_ffn(2, Is, d))
    assert "shared" in _refused(moe.expert_ffn, x, r, routed, _cpu_ffn(1, Is, 2 * d))
    bad3 = _cpu_ffn(E, I, d, bits=3)
    bad3.gate.codes = torch.zeros((E, I, d // 2), dtype=torch.uint8)  # 4-bit row length with 3-bit codes
    assert "gate.codes" in _refused(moe.expert_ffn, x, r, bad3, None)
    # routing arrays
    for name, t in (("tiles", torch.zeros((moe.max_tiles(dims, T) - 1, 3), dtype=torch.int32)),
                    ("inv_pos", torch.zeros(T * k - 1, dtype=torch.int32)),
                    ("offsets", torch.zeros(E, dtype=torch.int32)),
                    ("counts", torch.zeros(E + 1, dtype=torch.int32)),
                    ("sorted_token", torch.zeros(T * k + 1, dtype=torch.int32))):
        rr = dict(r)
        rr[name] = t
        assert name in _refused(moe.expert_ffn, x, rr, routed, shared)
    rr = dict(r)
    rr["topk_w"] = torch.zeros((T, k + 1), dtype=torch.float32)
    assert "topk_w" in _refused(moe.expert_ffn, x, rr, routed, shared)
    # y, the layer's router and bias
    assert "y has shape" in _refused(moe.expert_ffn, x, r, routed, shared, y=torch.zeros((T, d + 64), dtype=torch.bfloat16))
    assert "w_router" in _refused(moe.Layer, torch.zeros((d, E + 1)), routed, shared, k)
    assert "logit_bias" in _refused(moe.Layer, torch.zeros((d, E)), routed, shared, k, torch.zeros(E - 1))
    assert "w_router" in _refused(moe.route, x, torch.zeros((d + 64, E)), k, I, Is)
    assert "logit_bias" in _refused(moe.route, x, torch.zeros((d, E)), k, I, Is, torch.zeros(E + 1))
    p = routed.gate
    assert "scales" in _refused(moe.debug_dequant, moe.QProj(p.codes, p.scales[:, :, :1].contiguous(), p.biases))
    # the well-formed arguments get past every shape check (and then need a GPU tensor)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.expert_ffn(x, r, routed, shared)


def test_debug_router_logits_validation():
    """moe_debug_router_logits validates like moe_route, before any HIP call."""
    f = _Fake()
    d = _dims()
    L = moe.lib()

    def rl(T=8, **o):
        return L.moe_debug_router_logits(ctypes.byref(o.get("dims", d)), T, o.get("x", f()), o.get("wr", f()),
                                         o.get("bias", None), o.get("out", f()), None)
    assert rl(T=0) == moe.MOE_OK
    assert rl(T=-1) == moe.MOE_EINVAL
    assert rl(x=None) == moe.MOE_EINVAL
    assert rl(wr=f() + 4) == moe.MOE_EINVAL
    assert rl(out=None) == moe.MOE_EINVAL
    assert rl(bias=f() + 2) == moe.MOE_EINVAL
    assert rl(dims=_dims(g=32)) == moe.MOE_EUNSUPPORTED
