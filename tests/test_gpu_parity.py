"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bar: bit-exact routing (ids, counts, offsets, scatter order, inv_pos, block map) and
dequantised weights; gate weights within 1e-5; outputs within 1e-2 * max|ref| + 1e-3.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from workload import gen
from bit_moe_expert_amd import moe
from gpu_inputs import (DEV, bf16_dev, bits_host, check_routing, check_y, f32_dev, f32_of_bits, layer_dev,
                        proj_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need the MI355X"
    yield
    torch.cuda.synchronize()


def _oracle_routing(x, wr, bias, k, has_shared):
    logits = oracle.router_logits(x, wr, bias)
    ids, w = oracle.topk_softmax(logits, k)
    m = oracle.route_meta(ids, wr.shape[1], has_shared)
    m.update(topk_ids=ids, topk_w=w)
    return m


def _custom(T, d, E, k, I, Is, sigma=0.05, seed=0, zipf=False, bits=4):
    return gen.Workload("custom", T, d, E, k, I, Is, sigma, 1, T, zipf=zipf, seed=seed, bits=bits)


# ------------------------------------------------------------------ dequantisation (bit-exact)
def test_dequant_bit_exact_workload_and_exhaustive_scales():
    w = gen.WORKLOADS["prefill"]
    L = gen.expert_weights(w, 0)
    sl = slice(0, 3)
    for name in ("gate", "down"):
        p = {kk: v[sl] for kk, v in L[name].items()}
        got = bits_host(moe.debug_dequant(proj_dev(p)))
        assert (got == oracle.dequant(p["codes"], p["scales"], p["biases"])).all(), name
    # every normal bf16 scale with 16*scale finite, all 16 codes, bias -8*scale and random biases
    sbits = np.arange(0x0080, 0x7D00, dtype=np.uint32).astype(np.uint16)
    n = sbits.size
    q = np.tile(np.arange(16, dtype=np.uint8), 4)
    codes = np.broadcast_to((q[0::2] | (q[1::2] << 4)).astype(np.uint8), (n, 32)).copy()
    sf = (sbits.astype(np.uint32) << 16).view(np.float32)
    b = oracle.round_bf16(-8.0 * sf)
    rng = np.random.default_rng(5)
    # random biases up to 20 scales, clipped to the finite bf16 range (large scales would overflow)
    b2f = np.clip(rng.standard_normal(n) * sf.astype(np.float64) * rng.uniform(0, 20, n), -3.38e38, 3.38e38)
    b2 = oracle.round_bf16(b2f.astype(np.float32))
    for bias in (b, b2):
        p = {"codes": codes, "scales": sbits.reshape(n, 1), "biases": bias.reshape(n, 1)}
        got = bits_host(moe.debug_dequant(proj_dev(p)))
        assert (got == oracle.dequant(codes, p["scales"], p["biases"])).all()


# ------------------------------------------------------------------ routing (bit-exact)
ROUTE_CASES = [("tiny", 0, 0), ("decode", 0, 0), ("decode", 17, 0), ("decode", 39, 0), ("prefill", 0, 0),
               ("long", 0, 0), ("long", 0, 3), ("diffusion", 0, 0), ("diffusion", 29, 0), ("m2", 0, 0),
               ("m8", 3, 0), ("m16", 39, 0)]


@pytest.mark.parametrize("name,layer,chunk", ROUTE_CASES)
def test_route_workloads(name, layer, chunk):
    w = gen.WORKLOADS[name]
    x = gen.tokens(w, layer, chunk)
    wr = gen.router(w, layer)
    bias = gen.logit_bias(w)
    r = moe.route(bf16_dev(x), f32_dev(wr), w.k, w.I, w.Is, f32_dev(bias))
    check_routing(r, _oracle_routing(x, wr, bias, w.k, w.Is > 0), f"{name} layer {layer} chunk {chunk}")


SMALL = [(T, E, k, Is) for T in (1, 2, 3, 8, 33, 257) for E, k in ((1, 1), (2, 1), (2, 2), (4, 2), (16, 1), (16, 4),
                                                                    (16, 16)) for Is in (0, 64)]


@pytest.mark.parametrize("T,E,k,Is", SMALL)
def test_route_small_shapes(T, E, k, Is):
    w = _custom(T, 128, E, k, 64, Is, seed=T * 131 + E * 7 + k)
    x = gen.tokens(w, 0, 0)
    wr = gen.router(w, 0)
    r = moe.route(bf16_dev(x), f32_dev(wr), k, 64, Is)
    check_routing(r, _oracle_routing(x, wr, None, k, Is > 0), f"T={T} E={E} k={k} Is={Is}")


# Calls of more than 32768 pairs take the sliced metadata (per-slice histograms, one scan block,
# per-slice ranks); 32768 pairs and fewer take the single launch. Both sides of the switch, one
# expert, a partial last slice and groups far longer than a slice.
# (T, d, E, Zipf bias): every router block shape (16 tokens x 64 experts, 8 x 64, 8 x 32), one to eight
# staging passes, ragged expert blocks
LOGIT_CASES = [(1, 256, 16, False), (7, 512, 64, False), (64, 320, 300, False), (512, 2048, 256, False),
               (1024, 2048, 256, True), (33, 16384, 8, False), (512, 16384, 256, False), (300, 2048, 1024, True)]


@pytest.mark.parametrize("T,d,E,zipf", LOGIT_CASES)
def test_router_logits_bit_exact(T, d, E, zipf):
    """The grouped path's router logits equal the oracle's fixed-order fp32 chains bit for bit: its fma
    chains run as K = 1 fp32 MFMAs, each step rounded once as fmaf."""
    w = _custom(T, d, E, min(8, E), 64, 0, sigma=0.02, seed=T + d + E, zipf=zipf)
    x = gen.tokens(w, 0, 0)
    wr = gen.router(w, 0)
    bias = gen.logit_bias(w)
    got = moe.debug_router_logits(bf16_dev(x), f32_dev(wr), f32_dev(bias)).cpu().numpy()
    ref = oracle.router_logits(x, wr, bias).astype(np.float32)
    diff = got.view(np.uint32) != ref.view(np.uint32)
    assert not diff.any(), f"{int(diff.sum())} of {diff.size} logits differ, first at {np.argwhere(diff)[0]}"


@pytest.mark.parametrize("T,E,k,Is", [(4096, 256, 8, 64), (4097, 256, 8, 64), (40000, 1, 1, 0), (33000, 300, 5, 64),
                                      (65536, 16, 16, 0)])
def test_route_sliced_metadata(T, E, k, Is):
    w = _custom(T, 64, E, k, 64, Is, seed=T + E)
    x = gen.tokens(w, 0, 0)
    wr = gen.router(w, 0)
    r = moe.route(bf16_dev(x), f32_dev(wr), k, 64, Is)
    check_routing(r, _oracle_routing(x, wr, None, k, Is > 0), f"T={T} E={E} k={k} Is={Is}")


def test_forward_sliced_metadata():
    _forward_check(_custom(4097, 64, 16, 8, 64, 64, seed=11))


def test_route_ties_skew_and_large_groups():
    w = _custom(300, 256, 64, 8, 64, 64, seed=3)
    x = gen.tokens(w, 0, 0)
    wr = gen.router(w, 0)
    wr[:, 5] = wr[:, 2]    # exact ties: expert 2 must win over 5
    wr[:, 40] = wr[:, 9]
    r = moe.route(bf16_dev(x), f32_dev(wr), 8, 64, 64)
    check_routing(r, _oracle_routing(x, wr, None, 8, True), "ties")
    bias = np.zeros(64, np.float32)
    bias[11] = 1e4         # every token picks expert 11 first: one group of 300 rows (3 tiles)
    r = moe.route(bf16_dev(x), f32_dev(wr), 8, 64, 64, f32_dev(bias))
    ref = _oracle_routing(x, wr, bias, 8, True)
    check_routing(r, ref, "one big group")
    assert ref["counts"][11] == 300
    wl = gen.WORKLOADS["long"]
    xb = gen.tokens(wl, 0, 1)
    wrb = gen.router(wl, 0)
    pb = gen.logit_bias(wl, permuted=True)
    r = moe.route(bf16_dev(xb), f32_dev(wrb), 8, 512, 512, f32_dev(pb))
    check_routing(r, _oracle_routing(xb, wrb, pb, 8, True), "permuted zipf")


# ------------------------------------------------------------------ whole layer (tolerance)
def _forward_check(w, layer=0, chunk=0, T=None, sel=None):
    L = gen.layer(w, layer)
    x = gen.tokens(w, layer, chunk, T)
    lay = layer_dev(L, w.k)
    y = lay.forward(bf16_dev(x))
    torch.cuda.synchronize()
    if sel is None:
        ref = oracle.forward_layer(x, L["w_router"], L["routed"], L["shared"], w.k, L["logit_bias"])
        return check_y(y, ref["y"], f"{w.name} layer {layer} chunk {chunk}"), y, x, L
    ref = oracle.forward_tokens(x, L["w_router"], L["routed"], L["shared"], w.k, sel, L["logit_bias"])
    return check_y(y[torch.as_tensor(sel, device=DEV)], ref["y"], f"{w.name} sampled"), y, x, L


def test_forward_tiny():
    _forward_check(gen.WORKLOADS["tiny"])


@pytest.mark.parametrize("layer", [0, 1, 20, 39])
def test_forward_decode_layers(layer):
    _forward_check(gen.WORKLOADS["decode"], layer=layer)


def test_forward_prefill_full():
    _forward_check(gen.WORKLOADS["prefill"])


def test_forward_long_chunks():
    w = gen.WORKLOADS["long"]
    _forward_check(w, chunk=0)
    rng = np.random.default_rng(0)
    for c in (1, 2, 3):
        _forward_check(w, chunk=c, sel=np.sort(rng.choice(w.chunk, 6, replace=False)))


@pytest.mark.parametrize("layer", [0, 29])
def test_forward_diffusion(layer):
    _forward_check(gen.WORKLOADS["diffusion"], layer=layer)


@pytest.mark.parametrize("name,layer", [("m2", 0), ("m2", 39), ("m4", 7), ("m8", 0), ("m8", 39), ("m16", 11),
                                        ("m32", 5), ("m64", 2)])
def test_forward_small_calls(name, layer):
    """2..32 tokens run the GEMV path (a token per wave), 64 the grouped GEMM."""
    _forward_check(gen.WORKLOADS[name], layer=layer)


SHAPES = [
    # (T, d, E, k, I, Is): ragged T, K tails (d or I = 64 mod 128), shared size != routed, no shared
    (1, 256, 16, 4, 128, 128), (1, 192, 8, 2, 192, 64), (2, 256, 16, 4, 128, 128), (3, 192, 4, 2, 192, 0),
    (33, 256, 8, 3, 64, 128), (257, 128, 16, 2, 128, 64), (130, 320, 2, 2, 64, 192), (5, 64, 1, 1, 64, 64),
    (40, 128, 4, 4, 256, 0), (1, 128, 1, 1, 64, 0), (13, 256, 16, 4, 128, 128), (16, 192, 8, 3, 64, 64),
    (31, 192, 8, 3, 64, 0), (32, 256, 16, 4, 128, 128),
    # larger reductions (the prefill router stages d in passes of 2048 inputs), the largest top-k,
    # 1024 experts (the long top-k path), expert counts that are not a multiple of 64
    (40, 4096, 64, 8, 256, 128), (1, 4096, 64, 8, 256, 128), (3, 256, 1024, 16, 64, 64),
    (70, 256, 1024, 16, 64, 0), (64, 128, 300, 5, 192, 64), (2, 128, 300, 5, 192, 64),
    # down reductions of 6 steps or more (one output column block per down work item): whole
    # steps, an odd group count, and a shared size that is not whole steps
    (64, 128, 8, 4, 1024, 1024), (40, 256, 8, 2, 832, 0), (35, 192, 4, 2, 768, 320),
    # enough tokens for the 16-token router blocks, with a partial last token block and a
    # partial last expert block
    (1000, 128, 300, 5, 64, 64),
]


# Large expert groups (hundreds of rows, many whole tiles per group): groups of ~256 rows with a
# shared expert of 1024 rows; a shared expert twice as wide as the routed ones; no shared expert;
# a token count that leaves ragged last tiles.
BIG = [(1024, 512, 8, 2, 512, 512), (700, 1024, 16, 4, 512, 1024), (640, 512, 4, 2, 512, 0), (1000, 512, 8, 4, 512, 512)]


@pytest.mark.parametrize("T,d,E,k,I,Is", BIG)
def test_forward_large_groups(T, d, E, k, I, Is):
    _forward_check(_custom(T, d, E, k, I, Is, seed=T + E))


def test_forward_whole_groups():
    """Logit biases that route every token to one expert (one group of 512 rows, the other groups
    empty), then to one of two experts (two groups of about 256)."""
    w = _custom(512, 512, 4, 1, 512, 512, seed=5)
    L = gen.layer(w, 0)
    x = gen.tokens(w, 0, 0)
    for hot in ([2], [1, 3]):
        bias = np.zeros(4, np.float32)
        bias[hot] = 1e4
        ref = oracle.forward_layer(x, L["w_router"], L["routed"], L["shared"], 1, bias)
        if len(hot) == 1:
            assert (ref["counts"] == np.bincount([2], minlength=4) * 512).all()
        y = layer_dev(dict(L, logit_bias=bias), 1).forward(bf16_dev(x))
        torch.cuda.synchronize()
        check_y(y, ref["y"], f"experts {hot}")


@pytest.mark.parametrize("T,d,E,k,I,Is", SHAPES)
def test_forward_small_shapes(T, d, E, k, I, Is):
    _forward_check(_custom(T, d, E, k, I, Is, seed=T + d + E))


def test_decode_falls_back_to_grouped_gemm_when_h_is_large():
    w = _custom(1, 256, 32, 16, 2048, 0, seed=9)
    lay = layer_dev(gen.layer(w, 0), w.k)
    assert lay.stages(1)[1:3] == ["decode_topk", "route_meta"]
    _forward_check(w)


# ------------------------------------------------------------------ composition and determinism
@pytest.mark.parametrize("name", ["prefill", "decode", "m4", "m8", "diffusion", "long"])
def test_route_then_expert_ffn_equals_forward_and_is_deterministic(name):
    w = gen.WORKLOADS[name]
    L = gen.layer(w, 0)
    x = bf16_dev(gen.tokens(w, 0, 0))
    lay = layer_dev(L, w.k)
    y1 = lay.forward(x)
    y2 = lay.forward(x)
    r = moe.route(x, lay.w_router, w.k, w.I, w.Is, lay.logit_bias)
    y3 = moe.expert_ffn(x, r, lay.routed, lay.shared)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    # the stages launched one by one reproduce the layer
    ws = lay.workspace(x.shape[0])
    y4 = torch.empty_like(x)
    for s in range(len(lay.stages(x.shape[0]))):
        lay.launch_stage(s, x, y4, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y4.view(torch.int16))


# ------------------------------------------------------------------ 3- and 2-bit expert codes
@pytest.mark.parametrize("bits", [2, 3])
def test_lowbit_dequant_bit_exact(bits):
    """The kernels' unpacking of b-bit codes (through moe_debug_dequant_bits) against the oracle:
    random codes and scales, and a projection of the low-bit decode workload."""
    rng = np.random.default_rng(80 + bits)
    for n, out, inn in ((3, 40, 192), (2, 64, 2048)):
        codes = rng.integers(0, 256, (n, out, inn * bits // 8), dtype=np.uint8)
        sc = oracle.round_bf16((np.abs(rng.standard_normal((n, out, inn // 64))) * 0.05).astype(np.float32))
        bi = oracle.round_bf16((rng.standard_normal((n, out, inn // 64)) * 0.1).astype(np.float32))
        want = oracle.dequant(codes, sc, bi, bits)
        got = bits_host(moe.debug_dequant(proj_dev({"codes": codes, "scales": sc, "biases": bi, "bits": bits})))
        assert (got == want).all(), (bits, n, out, inn)
    w = gen.WORKLOADS[f"decode{bits}"]
    p = gen.expert_weights(w, 3)["down"]
    p = {"codes": p["codes"][:4], "scales": p["scales"][:4], "biases": p["biases"][:4], "bits": bits}
    want = oracle.dequant(p["codes"], p["scales"], p["biases"], bits)
    assert (bits_host(moe.debug_dequant(proj_dev(p))) == want).all()


@pytest.mark.parametrize("name,layer", [("tiny3", 0), ("tiny2", 0), ("decode3", 0), ("decode3", 17), ("decode2", 5),
                                        ("m32_3", 1), ("m32_2", 3), ("prefill3", 0), ("diffusion3", 0),
                                        ("diffusion3", 29), ("diffusion2", 0), ("diffusion2", 17)])
def test_forward_lowbit_workloads(name, layer):
    """GEMV path (up to 32 tokens) and grouped-GEMM path (prefill- and diffusion-size calls)."""
    _forward_check(gen.WORKLOADS[name], layer=layer)


@pytest.mark.parametrize("T,d,E,k,I,Is,bits", [(1, 192, 8, 2, 192, 64, 3), (5, 256, 16, 4, 128, 128, 2),
                                               (3, 64, 4, 2, 64, 0, 3), (17, 320, 8, 3, 64, 192, 2),
                                               (32, 128, 4, 2, 256, 64, 3), (1, 2112, 4, 2, 128, 64, 2),
                                               (2, 4096, 1024, 16, 64, 64, 3), (9, 256, 300, 16, 64, 0, 2),
                                               (64, 192, 8, 3, 192, 64, 3), (100, 320, 16, 4, 128, 128, 2),
                                               (33, 256, 8, 2, 832, 0, 3), (48, 2112, 4, 2, 128, 64, 2),
                                               (40, 4096, 300, 16, 64, 64, 3), (200, 128, 3, 2, 320, 0, 2)])
def test_forward_lowbit_shapes(T, d, E, k, I, Is, bits):
    """Ragged K (d = 64 mod 128), no shared expert, d above 2048 (several segments per lane), the
    largest top-k over 1024 experts, an expert count that is not a multiple of 64; calls of more
    than 32 tokens take the grouped GEMM (groups of more than 32 rows in the last two)."""
    _forward_check(_custom(T, d, E, k, I, Is, seed=T + d + bits, bits=bits))


@pytest.mark.parametrize("name", ["decode3", "m32_2", "prefill3", "diffusion2"])
def test_lowbit_route_then_expert_ffn_equals_forward(name):
    w = gen.WORKLOADS[name]
    L = gen.layer(w, 2)
    x = bf16_dev(gen.tokens(w, 2, 0))
    lay = layer_dev(L, w.k)
    y1 = lay.forward(x)
    r = moe.route(x, lay.w_router, w.k, w.I, w.Is, lay.logit_bias)
    y2 = moe.expert_ffn(x, r, lay.routed, lay.shared)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_zero_tokens_is_a_noop():
    w = gen.WORKLOADS["tiny"]
    lay = layer_dev(gen.layer(w, 0), w.k)
    x = torch.empty((0, w.d), dtype=torch.bfloat16, device=DEV)
    y = lay.forward(x, ws=lay.workspace(1))
    assert y.shape == (0, w.d)


# ------------------------------------------------------------------ large magnitudes
def _times_pow2_bf16(bits: np.ndarray, m: int) -> np.ndarray:
    """bf16 values (as bits) times 2^m, exactly: m is added to the exponent of every nonzero value."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    return np.where((b & 0x7FFF) == 0, b, b + (m << 7)).astype(np.uint16)


@pytest.mark.parametrize("T,d,E,k,I,Is,m", [(96, 256, 16, 4, 128, 128, 13), (96, 256, 16, 4, 128, 128, 16),
                                            (130, 320, 2, 1, 192, 64, 16), (40, 128, 8, 2, 64, 0, 15)])
def test_grouped_rows_beyond_fp16_range(T, d, E, k, I, Is, m):
    """Down scales and biases times 2^m (exact in bf16) put the grouped down GEMM's rows and the
    outputs beyond the fp16 range (up to about 1e6); the layer must still match the oracle, so the
    rows' fp16 storage must carry their range in its per-segment power-of-two exponents."""
    w = _custom(T, d, E, k, I, Is, seed=m + T)
    L = gen.layer(w, 0)
    for f in (L["routed"], L["shared"]):
        if f is not None:
            f["down"] = dict(f["down"], scales=_times_pow2_bf16(f["down"]["scales"], m),
                             biases=_times_pow2_bf16(f["down"]["biases"], m))
    x = gen.tokens(w, 0, 0)
    ref = oracle.forward_layer(x, L["w_router"], L["routed"], L["shared"], k, L["logit_bias"])
    assert np.abs(f32_of_bits(ref["y"])).max() > 65504.0  # the rows really leave the fp16 range
    y = layer_dev(L, k).forward(bf16_dev(x))
    torch.cuda.synchronize()
    check_y(y, ref["y"], f"down weights x 2^{m}")
