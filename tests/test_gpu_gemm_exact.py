"""GPU parity of the grouped GEMMs at the bit level, through the check export
moe_debug_grouped_gemm (the same kernels, LDS stages, code unpacking and scale/bias slots as the
layer's grouped path, with fp32 results written before the activation).

1. Exact-arithmetic inputs (integer activations, per-group power-of-two scales, biases that are
   small multiples of the scale): every product and partial sum is exact in fp32 whatever the
   order of the matrix cores, so the gate/up pre-activations and the down rows must equal the
   oracle's double-precision sums exactly. A wrong code, nibble, row, group's scale or bias, tile
   row or shared-row offset changes at least one value.
2. One-hot activations over the workload's own weights: the gate/up product of row e_c is the
   weight column c as the GEMM reconstructs it (scale * code + bias in fp32). For these weights
   (bias = -2^(b-1) * scale) that is exact, so rounded to bf16 it must equal the oracle's
   dequantised weights bit for bit: the dequantisation export of the grouped path, for 4-, 3- and
   2-bit codes.

Equality is of values: -0 and +0 compare equal (the sign of an exact zero depends on the order).
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from workload import gen
from bit_moe_expert_amd import moe
from gpu_inputs import DEV, bf16_dev, check_routing, f32_dev, ffn_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need the MI355X"
    yield
    torch.cuda.synchronize()


def _oracle_routing(L, k):
    logits = oracle.router_logits(L["x"], L["w_router"], L["logit_bias"])
    ids, w = oracle.topk_softmax(logits, k)
    m = oracle.route_meta(ids, L["w_router"].shape[1], L["shared"] is not None)
    m.update(topk_ids=ids, topk_w=w)
    return m


def _assert_exact(got: np.ndarray, want: np.ndarray, what: str):
    assert (want.astype(np.float32).astype(np.float64) == want).all(), f"{what}: inputs not exact"
    bad = got.astype(np.float64) != want
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} differ, first at {np.argwhere(bad)[0]}: " \
                          f"{got[tuple(np.argwhere(bad)[0])]} vs {want[tuple(np.argwhere(bad)[0])]}"


# (T, d, E, k, I, Is, zipf, bits): the prefill shape; a K tail (d and I = 64 mod 128) with a
# shared expert of another size; groups of ~150 rows; the skewed long shape (groups of up to ~250
# rows); a down reduction of 13 groups (one output column block per work item, odd group count);
# then the 3- and 2-bit codes on the prefill and diffusion shapes and on the ragged ones; last,
# groups of 200-500 rows (many whole tiles per group), with a shared expert twice as wide and
# with skewed groups
CASES = [
    (512, 2048, 256, 8, 512, 512, False, 4),
    (100, 192, 8, 3, 192, 64, False, 4),
    (300, 256, 4, 2, 128, 128, False, 4),
    (256, 2048, 256, 8, 512, 512, True, 4),
    (40, 256, 8, 2, 832, 0, False, 4),
    (512, 2048, 256, 8, 512, 512, False, 3),
    (256, 2048, 128, 8, 768, 0, False, 3),
    (256, 2048, 128, 8, 768, 0, False, 2),
    (100, 192, 8, 3, 192, 64, False, 3),
    (100, 192, 8, 3, 192, 64, False, 2),
    (300, 256, 4, 2, 128, 128, False, 2),
    (40, 256, 8, 2, 832, 0, False, 3),
    (40, 320, 8, 2, 832, 0, False, 2),
    (1024, 512, 8, 2, 512, 512, False, 4),
    (640, 1024, 4, 2, 512, 1024, True, 4),
]


def _setup(T, d, E, k, I, Is, zipf, bits):
    L = gen.exact_layer(T, d, E, k, I, Is, seed=T + d + I, zipf=zipf, bits=bits)
    ref = _oracle_routing(L, k)
    r = moe.route(bf16_dev(L["x"]), f32_dev(L["w_router"]), k, I, Is, f32_dev(L["logit_bias"]))
    check_routing(r, ref, "exact layer routing")
    return L, ref, r


@pytest.mark.parametrize("T,d,E,k,I,Is,zipf,bits", CASES)
def test_gateup_preactivations_bit_exact(T, d, E, k, I, Is, zipf, bits):
    L, ref, r = _setup(T, d, E, k, I, Is, zipf, bits)
    if zipf:
        assert ref["counts"].max() > 128, "the skewed case must hold a group of more than 128 rows"
    g, u = moe.debug_grouped_gemm(0, bf16_dev(L["x"]), r, ffn_dev(L["routed"]), ffn_dev(L["shared"]))
    torch.cuda.synchronize()
    wg, wu, wgs, wus = oracle.gateup_preact(L["x"], L["routed"], L["shared"], k, ref["offsets"], ref["sorted_token"])
    P = T * k
    g, u = g.cpu().numpy(), u.cpu().numpy()
    _assert_exact(g[:P * I].reshape(P, I), wg, "routed gate")
    _assert_exact(u[:P * I].reshape(P, I), wu, "routed up")
    if Is:
        _assert_exact(g[P * I:].reshape(T, Is), wgs, "shared gate")
        _assert_exact(u[P * I:].reshape(T, Is), wus, "shared up")


@pytest.mark.parametrize("T,d,E,k,I,Is,zipf,bits", CASES)
def test_down_rows_bit_exact(T, d, E, k, I, Is, zipf, bits):
    L, ref, r = _setup(T, d, E, k, I, Is, zipf, bits)
    P = T * k
    h = gen.small_ints_bf16(gen.key(T, d, 77), P * I).reshape(P, I)
    hs = gen.small_ints_bf16(gen.key(T, d, 78), T * Is).reshape(T, Is) if Is else None
    a = h.reshape(-1) if not Is else np.concatenate([h.reshape(-1), hs.reshape(-1)])
    y = moe.debug_grouped_gemm(1, bf16_dev(a), r, ffn_dev(L["routed"]), ffn_dev(L["shared"]))
    torch.cuda.synchronize()
    want = oracle.down_rows(h, hs, L["routed"], L["shared"], k, ref["offsets"])
    _assert_exact(y.cpu().numpy(), want, "down rows")


def _onehot_routing(experts, rows_per_expert, E):
    """Host-made routing of k = 1: token t goes to experts[t // rows_per_expert] (ascending, so
    grouped row order is token order); the block map from the oracle's metadata."""
    ids = np.repeat(np.asarray(experts, np.int32), rows_per_expert).reshape(-1, 1)
    m = oracle.route_meta(ids, E, False)
    cap = moe.max_tiles(moe.make_dims(64, E, 1, 64, 0), ids.shape[0])
    tiles = np.zeros((cap, 3), np.int32)
    tiles[:m["n_tiles"]] = m["tiles"]
    r = {"topk_ids": ids, "topk_w": np.ones(ids.shape, np.float32), "counts": m["counts"], "offsets": m["offsets"],
         "sorted_token": m["sorted_token"], "inv_pos": m["inv_pos"], "tiles": tiles,
         "n_tiles": np.array([m["n_tiles"]], np.int32)}
    assert (m["sorted_token"] == np.arange(ids.shape[0])).all()
    return {kk: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for kk, v in r.items()}


def _exact_weights(p, e):
    """s * q + b in float64 (exact here), codes unpacked from each row's little-endian bit stream
    with numpy: [out][in]."""
    bits = p.get("bits", 4)
    st = np.unpackbits(np.ascontiguousarray(p["codes"][e], np.uint8), axis=-1, bitorder="little").astype(np.int64)
    q = (st.reshape(p["codes"].shape[1], -1, bits) << np.arange(bits, dtype=np.int64)).sum(axis=-1)
    s = np.repeat(oracle.bf16_to_f32(p["scales"][e]).astype(np.float64), 64, axis=1)
    b = np.repeat(oracle.bf16_to_f32(p["biases"][e]).astype(np.float64), 64, axis=1)
    return s * q + b


@pytest.mark.parametrize("wname,experts", [("prefill", [0, 137, 255]), ("prefill3", [0, 77, 255]),
                                          ("diffusion2", [0, 64, 127])])
def test_dequant_export_through_the_grouped_gemm(wname, experts):
    """Workload weights (layer 0), three experts: the GEMMs' reconstruction of every gate, up and
    down weight, rounded to bf16, equals the oracle's dequantised weight (4-, 3- and 2-bit codes)."""
    w = gen.WORKLOADS[wname]
    W = gen.expert_weights(w, 0)
    routed = ffn_dev(W)
    d, I, E = w.d, w.I, w.E
    # gate/up: token t is the one-hot row of input t % d
    r = _onehot_routing(experts, d, E)
    x = np.zeros((len(experts) * d, d), np.uint16)
    x[np.arange(len(experts) * d), np.arange(len(experts) * d) % d] = 0x3F80  # 1.0
    g, u = moe.debug_grouped_gemm(0, bf16_dev(x), r, routed, None)
    # down: grouped row j of an expert is the one-hot h row of intermediate unit j % I
    rd = _onehot_routing(experts, I, E)
    h = np.zeros((len(experts) * I, I), np.uint16)
    h[np.arange(len(experts) * I), np.arange(len(experts) * I) % I] = 0x3F80
    y = moe.debug_grouped_gemm(1, bf16_dev(h), rd, routed, None)
    torch.cuda.synchronize()
    g = g.cpu().numpy().reshape(len(experts), d, I)
    u = u.cpu().numpy().reshape(len(experts), d, I)
    y = y.cpu().numpy().reshape(len(experts), I, d)
    for n, e in enumerate(experts):
        for name, got in (("gate", g[n].T), ("up", u[n].T), ("down", y[n].T)):
            p = W[name]
            want_bits = oracle.dequant(p["codes"][e], p["scales"][e], p["biases"][e], w.bits)
            assert (oracle.round_bf16(got) == want_bits).all(), f"expert {e} {name}: bf16 weights differ"
            assert (got.astype(np.float64) == _exact_weights(p, e)).all(), f"expert {e} {name}: fp32 weights differ"
