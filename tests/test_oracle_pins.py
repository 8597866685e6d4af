"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each test checks an oracle function against something other than the oracle itself:
exact integer arithmetic, closed forms, values the pages print, brute force, or a
different implementation of the same definition. A plausible mistake (dropped term,
wrong sign or index, swapped operand, wrong nibble order or group index, wrong
rounding mode, a missing shared expert) fails at least one of them.
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

from conftest import ROOT, load_golden
from oracle import oracle
from workload import gen

F32 = np.float32


# ------------------------------------------------------------------ exact rounding helpers
def _split(v: float):
    """Exact (N, e) with v = N * 2**e."""
    m, ex = math.frexp(v)
    return int(m * (1 << 53)), ex - 53


def _rne(N: int, e: int, p: int):
    """Round N * 2**e to p significant bits, ties to even (normal range assumed)."""
    if N == 0:
        return 0, 0
    s = -1 if N < 0 else 1
    N = abs(N)
    sh = N.bit_length() - p
    if sh <= 0:
        return s * N, e
    q, r = divmod(N, 1 << sh)
    half = 1 << (sh - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return s * q, e + sh


def _val(N, e):
    return math.ldexp(N, e)


def _bf16_bits_of_exact(v: float) -> int:
    """bf16 bits of a value that is exactly representable in bf16."""
    b = int(np.array([v], F32).view(np.uint32)[0])
    assert b & 0xFFFF == 0
    return b >> 16


def _bits_to_f(b):
    return float(oracle.bf16_to_f32(np.array([b], np.uint16))[0])


def _pack(q: np.ndarray) -> np.ndarray:
    """[..., in] codes -> [..., in/2] bytes, even input in the low nibble."""
    q = q.astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def _bf16(v) -> np.ndarray:
    return oracle.round_bf16(np.asarray(v, F32))


# ------------------------------------------------------------------ bf16 rounding
def test_round_bf16_known_values():
    one = 1.0
    cases = {
        1.0: 0x3F80, -2.5: 0xC020, 0.0: 0x0000,
        one + 2.0 ** -8: 0x3F80,              # exact tie -> even (down)
        one + 3 * 2.0 ** -8: 0x3F82,          # exact tie -> even (up)
        one + 2.0 ** -8 + 2.0 ** -20: 0x3F81,  # just above the tie
        one + 2.0 ** -8 - 2.0 ** -20: 0x3F80,  # just below the tie
        65504.0: 0x4780,                      # 65504 = 0x477FE000 rounds up to 65536
    }
    for v, bits in cases.items():
        assert int(_bf16([v])[0]) == bits, (v, hex(int(_bf16([v])[0])), hex(bits))


def test_round_bf16_random_vs_exact_integer_rounding():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(F32)
    got = _bf16(v)
    for x, g in zip(v.tolist(), got.tolist()):
        N, e = _rne(*_split(x), 8)
        assert g == _bf16_bits_of_exact(_val(N, e)), x


# ------------------------------------------------------------------ dequantisation
def test_dequant_nibble_order_and_affine_form():
    # byte 0x21 holds code 1 for input 0 (low nibble) and code 2 for input 1 (high nibble)
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0x21
    codes[0, 1] = 0xF3
    one = _bf16([1.0])
    zero = _bf16([0.0])
    w = oracle.bf16_to_f32(oracle.dequant(codes, one.reshape(1, 1), zero.reshape(1, 1)))[0]
    assert w[:4].tolist() == [1.0, 2.0, 3.0, 15.0] and not w[4:].any()
    # w = scale * q + bias: scale 0.5, bias -3 -> q=0 gives the bias, q=15 gives 15*s + b
    s, b = _bf16([0.5]), _bf16([-3.0])
    codes = _pack(np.array([[0, 15] + [1] * 62]))
    w = oracle.bf16_to_f32(oracle.dequant(codes, s.reshape(1, 1), b.reshape(1, 1)))[0]
    assert w[0] == -3.0 and w[1] == 4.5 and (w[2:] == -2.5).all()


def test_dequant_group_index():
    # one code per input = 1, bias 0, scale of group g = 2**-g: weight of input c is 2**-(c // 64)
    G = 5
    codes = _pack(np.ones((2, 64 * G), np.uint8))
    sc = np.stack([_bf16([2.0 ** -g for g in range(G)]), _bf16([3 * 2.0 ** -g for g in range(G)])])
    bi = np.stack([_bf16([0.0] * G), _bf16([1.0] * G)])
    w = oracle.bf16_to_f32(oracle.dequant(codes, sc, bi))
    c = np.arange(64 * G)
    assert (w[0] == 2.0 ** -(c // 64)).all()
    assert (w[1] == 3 * 2.0 ** -(c // 64) + 1.0).all()


def test_dequant_exhaustive_workload_identities():
    """All 16 codes x every positive normal bf16 scale with 16*scale finite, bias = -8*scale."""
    sbits = np.arange(0x0080, 0x7D00, dtype=np.uint32).astype(np.uint16)  # exponent 1..249
    n = sbits.size
    s = oracle.bf16_to_f32(sbits).astype(np.float64)
    b = _bf16(-8.0 * s)
    assert (oracle.bf16_to_f32(b) == -8.0 * s).all()  # the bias is exact
    q = np.tile(np.arange(16, dtype=np.uint8), 4)
    codes = np.broadcast_to(_pack(q[None, :]), (n, 32)).copy()
    got = oracle.dequant(codes, sbits.reshape(n, 1), b.reshape(n, 1))  # [n][64]
    # exact: s*(q-8) = m*2^e*(q-8) with m the 8-bit significand; round to 8 bits by integers
    m = ((sbits.astype(np.int64) & 0x7F) | 0x80)
    e = ((sbits.astype(np.int64) >> 7) & 0xFF) - 127 - 7
    prod = m[:, None] * (q.astype(np.int64)[None, :] - 8)  # |prod| < 2^11
    mag = np.abs(prod)
    nbits = np.where(mag > 0, np.floor(np.log2(np.maximum(mag, 1))).astype(np.int64) + 1, 0)
    sh = np.maximum(nbits - 8, 0)
    qq = mag >> sh
    r = mag - (qq << sh)
    half = np.where(sh > 0, 1 << np.maximum(sh - 1, 0), 0)
    up = (sh > 0) & ((r > half) | ((r == half) & (qq & 1).astype(bool)))
    qq = qq + up
    exact = np.sign(prod) * np.ldexp(qq.astype(np.float64), (e[:, None] + sh))
    want = (exact.astype(F32).view(np.uint32) >> 16).astype(np.uint16)
    assert (got == want).all()
    # codes whose q-8 needs no rounding reproduce s*(q-8) exactly
    wf = oracle.bf16_to_f32(got)
    exact_cols = np.isin(q.astype(np.int64) - 8, [0, 1, -1, 2, -2, 4, -4, -8])
    assert (wf[:, exact_cols] == (s[:, None] * (q[exact_cols].astype(np.float64) - 8))).all()
    # (w32 - b) / s recovers the code where no bf16 rounding happened
    assert (np.rint((wf[:, exact_cols] - oracle.bf16_to_f32(b)[:, None]) / s[:, None]) == q[exact_cols]).all()
    # some codes do need rounding: truncation or a missing rounding would be caught
    assert (got != (exact.astype(F32).view(np.uint32) >> 16)).sum() == 0
    assert up.any()


def test_dequant_general_bias_two_step_rounding():
    """General bias: w = bf16(fp32(s*q + b)); checked by exact integer arithmetic."""
    rng = np.random.default_rng(7)
    n = 4000
    sb = _bf16(np.abs(rng.standard_normal(n)) * 0.02)
    bb = _bf16(rng.standard_normal(n) * 0.3 * np.exp(rng.uniform(-8, 3, n)))
    q = rng.integers(0, 16, (n, 64)).astype(np.uint8)
    got = oracle.dequant(_pack(q), sb.reshape(n, 1), bb.reshape(n, 1))
    sf = oracle.bf16_to_f32(sb)
    bf = oracle.bf16_to_f32(bb)
    for i in range(0, n, 7):
        for c in range(0, 64, 5):
            Ns, es = _split(float(sf[i]))
            Nb, eb = _split(float(bf[i]))
            lo = min(es, eb)
            N = Ns * int(q[i, c]) * (1 << (es - lo)) + Nb * (1 << (eb - lo))
            N32, e32 = _rne(N, lo, 24)
            N16, e16 = _rne(N32, e32, 8)
            assert int(got[i, c]) == _bf16_bits_of_exact(_val(N16, e16)), (i, c)


def test_dequant_quantisation_round_trip():
    """Affine 4-bit quantisation (bias = group minimum, scale = range / 15) dequantises back
    within half a step plus bf16 rounding: a swapped scale/bias or a sign error fails."""
    rng = np.random.default_rng(3)
    W = rng.standard_normal((16, 256)) * 0.05
    G = W.reshape(16, 4, 64)
    lo, hi = G.min(-1), G.max(-1)
    s = _bf16((hi - lo) / 15)
    b = _bf16(lo)
    sf, bf = oracle.bf16_to_f32(s).astype(np.float64), oracle.bf16_to_f32(b).astype(np.float64)
    q = np.clip(np.rint((G - bf[..., None]) / sf[..., None]), 0, 15).astype(np.uint8).reshape(16, 256)
    w = oracle.bf16_to_f32(oracle.dequant(_pack(q), s, b)).astype(np.float64)
    step = np.repeat(sf, 64, axis=1)
    assert (np.abs(w - W) <= 0.5 * step + np.abs(W) * 2.0 ** -7 + 2 * step * 2.0 ** -8).all()


def test_storage_ratio_matches_pages():
    g = load_golden("pages_storage.txt")
    bits_per_weight = 4 + 2 * 16 / g["group_size"]  # 4-bit code + bf16 scale and bias per group
    assert bits_per_weight == 4.5
    assert abs(g["params"] * 2 / 1e9 - g["bf16_gb"]) < 1e-9
    q4_gb = g["params"] * bits_per_weight / 8 / 1e9
    assert abs(q4_gb - g["q4_gb"]) / g["q4_gb"] < 0.03
    w = gen.WORKLOADS["decode"]
    assert w.expert_bytes * 8 / (3 * w.d * w.I) == bits_per_weight


# ------------------------------------------------------------------ router logits
def test_router_integer_exact():
    rng = np.random.default_rng(5)
    T, d, E = 6, 256, 16
    xi = rng.integers(-8, 9, (T, d))
    wi = rng.integers(-8, 9, (d, E))
    bias = rng.integers(-5, 6, E).astype(F32)
    x = _bf16(xi.astype(F32))
    got = oracle.router_logits(x, wi.astype(F32), bias)
    assert (got == (xi @ wi + bias).astype(F32)).all()


def test_router_summation_order_is_chunked():
    """Chunk partials (64 inputs each) are summed after each chunk is reduced."""
    d, E = 128, 1
    x = np.zeros((1, d), F32)
    w = np.zeros((d, E), F32)
    x[0, 0], w[0, 0] = 2.0 ** 12, 2.0 ** 12   # 2^24 in chunk 0
    x[0, 1], w[1, 0] = 1.0, 1.0               # +1 in chunk 0 is lost (tie to even)
    x[0, 64], w[64, 0] = 1.0, 1.0             # chunk 1 adds up to 2 before joining
    x[0, 65], w[65, 0] = 1.0, 1.0
    got = oracle.router_logits(_bf16(x), w)
    assert got[0, 0] == 2.0 ** 24 + 2


def test_router_random_within_error_bound_and_bias_last():
    rng = np.random.default_rng(9)
    T, d, E = 4, 512, 32
    x = _bf16(rng.standard_normal((T, d)))
    w = (rng.standard_normal((d, E)) * 0.02).astype(F32)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    got = oracle.router_logits(x, w)
    exact = xf @ w.astype(np.float64)
    bound = (d + 2) * 2.0 ** -24 * (np.abs(xf) @ np.abs(w.astype(np.float64)))
    assert (np.abs(got - exact) <= bound).all()
    bias = (rng.standard_normal(E)).astype(F32)
    gb = oracle.router_logits(x, w, bias)
    assert (gb == (got + bias).astype(F32)).all()


# ------------------------------------------------------------------ top-k and gate weights
def test_topk_matches_full_sort_and_ties():
    rng = np.random.default_rng(11)
    T, E, k = 50, 40, 6
    l = rng.standard_normal((T, E)).astype(F32)
    l[:, 7] = l[:, 3]          # exact ties: the lower index must come first
    l[:5] = 0.25               # all equal
    ids, w = oracle.topk_softmax(l, k)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(l[t, e]), e))[:k]
        assert ids[t].tolist() == order
    assert (ids[:5] == np.arange(k)).all()
    assert np.allclose(w[:5], 1.0 / k, rtol=0, atol=2.0 ** -24)


def test_gate_weights_closed_forms():
    rng = np.random.default_rng(12)
    l = rng.standard_normal((200, 16)).astype(F32)
    ids, w = oracle.topk_softmax(l, 1)
    assert (w == 1.0).all()
    ids, w = oracle.topk_softmax(l, 2)
    for t in range(200):
        delta = float(l[t, ids[t, 1]]) - float(l[t, ids[t, 0]])
        assert abs(float(w[t, 0]) - 1.0 / (1.0 + math.exp(delta))) <= 2.0 ** -24
    k = 8
    ids, w = oracle.topk_softmax(l, k)
    assert (np.abs(w.astype(np.float64).sum(1) - 1.0) <= 4 * k * 2.0 ** -24).all()
    assert (np.diff(w, axis=1) <= 0).all()
    # the other reading of the gate: softmax over all experts, renormalised over the picked ones
    p = np.exp(l.astype(np.float64) - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    sel = np.take_along_axis(p, ids, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=0, atol=2.0 ** -23)


# ------------------------------------------------------------------ histogram, scan, scatter, block map
def _check_meta(ids, E, has_shared, m):
    T, k = ids.shape
    P = T * k
    assert m["counts"].sum() == P and m["offsets"][0] == 0 and m["offsets"][E] == P
    assert (m["counts"] == np.bincount(ids.ravel(), minlength=E)).all()
    assert (np.diff(m["offsets"]) == m["counts"]).all()
    order = sorted(range(P), key=lambda p: int(ids.flat[p]))  # textbook stable sort by expert
    assert (m["sorted_token"] == np.array(order) // k).all()
    inv = np.empty(P, np.int64)
    inv[np.array(order)] = np.arange(P)
    assert (m["inv_pos"].ravel() == inv).all()
    # tiles partition the grouped rows in order, never cross a group, at most 32 rows
    tiles = m["tiles"]
    rows = np.concatenate([np.arange(s, s + n) for _, s, n in tiles]) if len(tiles) else np.zeros(0)
    assert (rows == np.arange(P + (T if has_shared else 0))).all()
    for e, s, n in tiles:
        assert 1 <= n <= 32
        if e < E:
            assert m["offsets"][e] <= s and s + n <= m["offsets"][e + 1]
        else:
            assert e == E and has_shared and s >= P
    assert m["n_tiles"] <= oracle.max_tiles(T, E, k, has_shared)


def test_route_meta_invariants_random_and_skewed():
    rng = np.random.default_rng(13)
    for T, E, k, sh in [(37, 16, 4, True), (300, 8, 1, False), (1, 256, 8, True), (513, 64, 8, True)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        _check_meta(ids, E, sh, oracle.route_meta(ids, E, sh))
    ids = np.full((300, 1), 3, np.int32)  # every token to one expert: nine tiles of 32, then 12
    m = oracle.route_meta(ids, 8, False)
    _check_meta(ids, 8, False, m)
    assert m["tiles"].tolist() == [[3, 32 * i, 32] for i in range(9)] + [[3, 288, 12]]


def test_route_meta_worked_instance_from_pages():
    g = load_golden("pages_routing_counts.txt")
    T, k, E = int(g["qwen_prompt_tokens"]), int(g["qwen_top_k"]), int(g["qwen_experts"])
    rng = np.random.default_rng(17)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    m = oracle.route_meta(ids, E, True)
    assert m["counts"].sum() == g["qwen_assignments"]
    assert m["counts"].mean() == g["qwen_rows_per_expert_mean"]
    T, k, E = int(g["diffusion_canvas"]), int(g["diffusion_top_k"]), int(g["diffusion_experts"])
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    m = oracle.route_meta(ids, E, False)
    assert m["offsets"][E] == g["diffusion_pairs"]


# ------------------------------------------------------------------ the FFN
def _q4_from_int(Wint: np.ndarray, scale: float = 1.0, bias: float = 0.0):
    """Exact packing of integer weights in [0, 15] (bias 0) as one or more matrices."""
    Wint = np.asarray(Wint)
    shp = Wint.shape
    G = shp[-1] // 64
    return {"codes": _pack(Wint.astype(np.uint8)),
            "scales": np.full(shp[:-1] + (G,), int(_bf16([scale])[0]), np.uint16),
            "biases": np.full(shp[:-1] + (G,), int(_bf16([bias])[0]), np.uint16)}


def _silu(z):
    return z / (1.0 + math.exp(-z))


def test_ffn_closed_form_with_permutation_weights():
    """Gate = permutation sigma, up = 2 * sigma, down = permutation pi (all exact in 4 bits):
    y[o] = bf16(silu(x_j) * 2 x_j) with j = sigma(pi(o)). Swapping gate and up, transposing a
    matrix or dropping the bf16 rounding of h gives other values."""
    d = I = 64
    rng = np.random.default_rng(19)
    sig, pi = rng.permutation(I), rng.permutation(d)
    Pg = np.zeros((1, I, d), np.int64)
    Pg[0, np.arange(I), sig] = 1
    Pd = np.zeros((1, d, I), np.int64)
    Pd[0, np.arange(d), pi] = 1
    routed = {"gate": _q4_from_int(Pg), "up": _q4_from_int(2 * Pg), "down": _q4_from_int(Pd)}
    x = _bf16(np.concatenate([[1.0, -1.0, 0.0, 2.0], rng.standard_normal(d - 4)]).reshape(1, d))
    out = oracle.forward_layer(x, np.ones((d, 1), F32), routed, None, 1)
    xf = oracle.bf16_to_f32(x)[0].astype(np.float64)
    y = oracle.bf16_to_f32(out["y"])[0]
    for o in range(d):
        j = sig[pi[o]]
        assert y[o] == oracle.bf16_to_f32(_bf16([_silu(xf[j]) * 2 * xf[j]]))[0]
    # worked value: x = 1 gives 2 * silu(1) = 2e / (e + 1) = 1.46211..., which is 1.4609375 in bf16
    o1 = int(np.where(sig[pi] == 0)[0][0])
    assert y[o1] == 1.4609375


def test_shared_expert_is_ungated_and_added():
    """Routed experts all zero, shared expert = the closed form above: y = shared(x)."""
    d = I = 64
    Pg = np.eye(I, d, dtype=np.int64)[None]
    zero = np.zeros((3, I, d), np.int64)
    routed = {"gate": _q4_from_int(zero), "up": _q4_from_int(zero), "down": _q4_from_int(np.zeros((3, d, I)))}
    shared = {"gate": _q4_from_int(Pg), "up": _q4_from_int(3 * Pg), "down": _q4_from_int(Pg)}
    rng = np.random.default_rng(23)
    x = _bf16(rng.standard_normal((5, d)))
    out = oracle.forward_layer(x, (rng.standard_normal((d, 3)) * 0.1).astype(F32), routed, shared, 2)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    want = np.vectorize(lambda v: _silu(v) * 3 * v)(xf)
    assert (out["y"] == _bf16(want)).all()


def test_expert_selection_uses_the_routed_experts_weights():
    """Three experts with gate = up = c_e * I (c_e = 1, 2, 3), down = I; a router bias forces
    each token's expert (k = 1): y = bf16(silu(c x) * c x) of the chosen expert."""
    d = I = 64
    Id = np.eye(I, d, dtype=np.int64)
    routed = {"gate": _q4_from_int(np.stack([c * Id for c in (1, 2, 3)])),
              "up": _q4_from_int(np.stack([c * Id for c in (1, 2, 3)])),
              "down": _q4_from_int(np.stack([Id] * 3))}
    rng = np.random.default_rng(29)
    x = _bf16(rng.standard_normal((3, d)) * 0.5)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    for e in range(3):
        bias = np.full(3, -100.0, F32)
        bias[e] = 100.0
        out = oracle.forward_layer(x, np.zeros((d, 3), F32), routed, None, 1, bias=bias)
        assert (out["topk_ids"] == e).all()
        c = e + 1
        want = np.vectorize(lambda v: _silu(c * v) * c * v)(xf)
        assert (out["y"] == _bf16(want)).all()


def _random_layer(rng, T, d, E, k, I, Is, bits=4):
    def proj(n, o, i):
        p = {"codes": rng.integers(0, 256, (n, o, i * bits // 8), dtype=np.uint8),
             "scales": _bf16(np.abs(rng.standard_normal((n, o, i // 64))) * 0.02),
             "biases": _bf16(rng.standard_normal((n, o, i // 64)) * 0.1)}
        if bits != 4:
            p["bits"] = bits
        return p
    routed = {"gate": proj(E, I, d), "up": proj(E, I, d), "down": proj(E, d, I)}
    shared = {"gate": proj(1, Is, d), "up": proj(1, Is, d), "down": proj(1, d, Is)} if Is else None
    x = _bf16(rng.standard_normal((T, d)))
    wr = (rng.standard_normal((d, E)) * 0.05).astype(F32)
    return x, wr, routed, shared


def _python_dense_forward(x, routed, shared, ids, w):
    """Brute force: per token, dense evaluation of the chosen experts, no grouping.
    Own dequantisation (Python ints and floats), double sums in ascending order."""
    T, d = x.shape
    xf = oracle.bf16_to_f32(x).astype(np.float64)

    def deq(m, mat, row, c, in_dim):
        bits = m.get("bits", 4)
        if bits == 4:
            byte = int(m["codes"][mat, row, c // 2])
            q = (byte >> 4) if (c & 1) else (byte & 15)
        else:  # the row's bytes as one little-endian integer, code c at bits [bits*c, bits*c + bits)
            q = (int.from_bytes(bytes(m["codes"][mat, row]), "little") >> (bits * c)) & ((1 << bits) - 1)
        s = np.float32(_bits_to_f(int(m["scales"][mat, row, c // 64])))
        b = np.float32(_bits_to_f(int(m["biases"][mat, row, c // 64])))
        return _bits_to_f(int(_bf16([np.float32(s * np.float32(q)) + b])[0]))

    def ffn(W, mat, xrow):
        I = W["gate"]["codes"].shape[1]
        h = []
        for i in range(I):
            g = u = 0.0
            for c in range(d):
                g += xrow[c] * deq(W["gate"], mat, i, c, d)
                u += xrow[c] * deq(W["up"], mat, i, c, d)
            h.append(_bits_to_f(int(_bf16([(g / (1.0 + math.exp(-g))) * u])[0])))
        out = []
        for o in range(d):
            acc = 0.0
            for i in range(I):
                acc += h[i] * deq(W["down"], mat, o, i, I)
            out.append(acc)
        return out

    y = np.empty((T, d), np.uint16)
    for t in range(T):
        rows = [ffn(routed, int(e), xf[t]) for e in ids[t]]
        sh = ffn(shared, 0, xf[t]) if shared else None
        for o in range(d):
            acc = 0.0
            for j in range(ids.shape[1]):
                acc += float(w[t, j]) * rows[j][o]
            if sh:
                acc += sh[o]
            y[t, o] = int(_bf16([acc])[0])
    return y


def test_grouped_forward_equals_dense_brute_force():
    rng = np.random.default_rng(31)
    T, d, E, k, I, Is = 5, 64, 4, 2, 64, 64
    x, wr, routed, shared = _random_layer(rng, T, d, E, k, I, Is)
    out = oracle.forward_layer(x, wr, routed, shared, k)
    ids, w = oracle.topk_softmax(oracle.router_logits(x, wr), k)
    assert (out["topk_ids"] == ids).all() and (out["topk_w"] == w).all()
    assert (out["y"] == _python_dense_forward(x, routed, shared, ids, w)).all()


@pytest.mark.parametrize("bits", [2, 3])
def test_lowbit_grouped_forward_equals_dense_brute_force(bits):
    rng = np.random.default_rng(50 + bits)
    T, d, E, k, I, Is = 3, 64, 4, 2, 64, 64
    x, wr, routed, shared = _random_layer(rng, T, d, E, k, I, Is, bits=bits)
    out = oracle.forward_layer(x, wr, routed, shared, k)
    ids, w = oracle.topk_softmax(oracle.router_logits(x, wr), k)
    assert (out["y"] == _python_dense_forward(x, routed, shared, ids, w)).all()


def _pack_codes(codes, bits):
    """Independent packer: codes [rows][n] -> bytes [rows][n * bits / 8], code i at bits
    [bits * i, bits * i + bits) of the row read as a little-endian integer."""
    rows, n = codes.shape
    out = np.zeros((rows, n * bits // 8), np.uint8)
    for r in range(rows):
        v = 0
        for i in range(n - 1, -1, -1):
            v = (v << bits) | int(codes[r, i])
        out[r] = np.frombuffer(v.to_bytes(n * bits // 8, "little"), np.uint8)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lowbit_unpack_round_trip(bits):
    rng = np.random.default_rng(60 + bits)
    codes = rng.integers(0, 1 << bits, (5, 192))
    ones = np.full((5, 3), 0x3F80, np.uint16)  # scale 1.0
    zeros = np.zeros((5, 3), np.uint16)
    w = oracle.bf16_to_f32(oracle.dequant(_pack_codes(codes, bits), ones, zeros, bits))
    assert (w == codes).all()
    if bits == 4:  # the bit-stream reading is the nibble order of the 4-bit format
        assert (_pack_codes(codes, 4)[:, 0] == (codes[:, 0] | (codes[:, 1] << 4))).all()


@pytest.mark.parametrize("bits", [2, 3])
def test_lowbit_affine_identities(bits):
    """bias = -2^(bits-1) * scale, as the generator draws it: w32 = s * (q - 2^(bits-1)) exactly,
    and the bf16 result is the round-to-nearest-even of that exact product."""
    rng = np.random.default_rng(70 + bits)
    rows = 64
    codes = rng.integers(0, 1 << bits, (rows, 64))
    s = _bf16(np.abs(rng.standard_normal(rows)) * 0.05).reshape(rows, 1)
    b = _bf16(-(2.0 ** (bits - 1)) * oracle.bf16_to_f32(s).astype(np.float64)).reshape(rows, 1)
    assert (oracle.bf16_to_f32(b) == -(2.0 ** (bits - 1)) * oracle.bf16_to_f32(s)).all()  # exact
    w = oracle.bf16_to_f32(oracle.dequant(_pack_codes(codes, bits), s, b, bits)).astype(np.float64)
    exact = oracle.bf16_to_f32(s).astype(np.float64) * (codes - 2 ** (bits - 1))
    assert (w == oracle.bf16_to_f32(_bf16(exact))).all()


def test_sampled_tokens_equal_grouped_rows():
    rng = np.random.default_rng(37)
    x, wr, routed, shared = _random_layer(rng, 40, 128, 8, 3, 64, 128)
    full = oracle.forward_layer(x, wr, routed, shared, 3)
    sel = [0, 7, 39, 7]
    s = oracle.forward_tokens(x, wr, routed, shared, 3, sel)
    assert (s["y"] == full["y"][sel]).all() and (s["topk_ids"] == full["topk_ids"][sel]).all()


def test_identical_experts_make_routing_irrelevant():
    """All experts equal: y = bf16(sum_j w_j r + s) with sum_j w_j = 1, so it matches the
    E = k = 1 layer to within one bf16 step."""
    rng = np.random.default_rng(41)
    x, wr, routed, shared = _random_layer(rng, 9, 128, 1, 1, 64, 64)
    many = {n: {kk: np.repeat(v, 6, axis=0) for kk, v in routed[n].items()} for n in routed}
    y1 = oracle.bf16_to_f32(oracle.forward_layer(x, wr, routed, shared, 1)["y"]).astype(np.float64)
    wr6 = (rng.standard_normal((128, 6)) * 0.3).astype(F32)
    y6 = oracle.bf16_to_f32(oracle.forward_layer(x, wr6, many, shared, 4)["y"]).astype(np.float64)
    assert (np.abs(y6 - y1) <= 2.0 ** -7 * np.abs(y1) + 1e-30).all()


def test_token_permutation_and_expert_relabelling():
    rng = np.random.default_rng(43)
    x, wr, routed, shared = _random_layer(rng, 12, 128, 8, 3, 64, 64)
    base = oracle.forward_layer(x, wr, routed, shared, 3)
    perm = rng.permutation(12)
    pt = oracle.forward_layer(x[perm], wr, routed, shared, 3)
    assert (pt["y"] == base["y"][perm]).all()
    lab = rng.permutation(8)  # new expert e' = lab[e]
    inv = np.argsort(lab)
    routed2 = {n: {kk: v[inv] for kk, v in routed[n].items()} for n in routed}
    rl = oracle.forward_layer(x, wr[:, inv], routed2, shared, 3)
    assert (rl["y"] == base["y"]).all()
    assert (inv[rl["topk_ids"]] == base["topk_ids"]).all()


def test_oracle_is_thread_count_invariant():
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from workload import gen; from oracle import oracle; import hashlib\n"
        "w = gen.WORKLOADS['tiny']; L = gen.layer(w, 0); x = gen.tokens(w, 0, 0, T=33)\n"
        "o = oracle.forward_layer(x, L['w_router'], L['routed'], L['shared'], w.k)\n"
        "print(hashlib.sha256(o['y'].tobytes() + o['topk_w'].tobytes()).hexdigest())\n" % ROOT)
    outs = []
    for nt in ("1", "5"):
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                                   check=True).stdout.strip())
    assert outs[0] == outs[1] and len(outs[0]) == 64


# ------------------------------------------------------------------ exact top-K of logit rows
def _brute_topk(row, K):
    order = sorted(range(len(row)), key=lambda i: (-float(row[i]), i))[:K]
    return np.array(order, np.int32), row[order]


def _chunk_max_topk(row, K, C, lower_chunk_first=True):
    """The pages' hierarchical selection, written from their description: chunk maxima, the K
    chunks with the largest maxima, then the top K inside the chosen chunks."""
    V = len(row)
    nch = (V + C - 1) // C
    cmax = [max(float(v) for v in row[c * C:(c + 1) * C]) for c in range(nch)]
    tie = (lambda c: c) if lower_chunk_first else (lambda c: -c)
    chosen = sorted(range(nch), key=lambda c: (-cmax[c], tie(c)))[:K]
    cand = [i for c in chosen for i in range(c * C, min(V, (c + 1) * C))]
    cand.sort(key=lambda i: (-float(row[i]), i))
    return np.array(cand[:K], np.int32)


def test_vocab_topk_closed_forms():
    V, K = 1000, 16
    ids, vals = oracle.vocab_topk(np.zeros((1, V), np.float32), K)           # all equal: lowest indices
    assert (ids[0] == np.arange(K)).all() and (vals == 0).all()
    ids, _ = oracle.vocab_topk(-np.arange(V, dtype=np.float32)[None], K)      # decreasing ramp
    assert (ids[0] == np.arange(K)).all()
    ids, vals = oracle.vocab_topk(np.arange(V, dtype=np.float32)[None], K)    # increasing ramp
    assert (ids[0] == np.arange(V - 1, V - 1 - K, -1)).all() and (vals[0] == ids[0]).all()
    ids, _ = oracle.vocab_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), 2)  # -0 == +0: index order
    assert ids.tolist() == [[0, 1]]
    ids, vals = oracle.vocab_topk(np.array([[1.0, np.inf, -np.inf, 2.0]], np.float32), 4)
    assert ids.tolist() == [[1, 3, 0, 2]]


def test_vocab_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for V, K in ((1, 1), (7, 7), (300, 1), (513, 64), (2000, 100)):
        x = rng.integers(-6, 6, size=(3, V)).astype(np.float32) * 0.5  # heavy ties
        x[1] = rng.normal(size=V).astype(np.float32)
        ids, vals = oracle.vocab_topk(x, K)
        for r in range(3):
            bi, bv = _brute_topk(x[r], K)
            assert (ids[r] == bi).all() and (vals[r] == bv).all(), (V, K, r)


def test_chunk_max_selection_is_exact_as_the_pages_state():
    """[DIFFGEMMA "The optimizations that worked"]: a value in the global top-K has fewer than K
    chunk maxima above it, so its chunk is among the K chosen. With equal maxima the lower chunk
    must win (the values tied with it that it displaces come first); adversarial rows check both."""
    rng = np.random.default_rng(12)
    V = 1000
    rows = [rng.normal(size=V).astype(np.float32)]
    r = rng.normal(size=V).astype(np.float32) - 10.0
    r[200:264] = 5.0 + rng.random(64).astype(np.float32)  # the whole top-K inside one chunk
    rows.append(r)
    rows.append(np.repeat(rng.integers(0, 4, V // 8 + 1), 8)[:V].astype(np.float32))  # ties across chunks
    r = np.zeros(V, np.float32)
    r[::50] = 1.0  # one maximum per chunk of 50, equal everywhere
    rows.append(r)
    for row in rows:
        for K in (1, 5, 16, 64):
            want, _ = oracle.vocab_topk(row[None], K)
            for C in (50, 64, 128, 333):
                assert (_chunk_max_topk(row, K, C) == want[0]).all(), (K, C)
    # the tie rule matters: taking the higher chunk among equal maxima loses lower-index entries
    row = np.zeros(V, np.float32)
    assert not (_chunk_max_topk(row, 4, 100, lower_chunk_first=False) == oracle.vocab_topk(row[None], 4)[0][0]).all()


def test_vocab_topk_full_size_row_against_lexsort():
    """One row of the pages' size (262,144 logits, K = 64) against numpy's lexsort."""
    rng = np.random.default_rng(13)
    x = (rng.normal(size=(2, 262144)) * 3).astype(np.float32)
    x[1, 1000:1100] = x[0].max() + 1.0  # a tied block at the top
    ids, vals = oracle.vocab_topk(x, 64)
    for r in range(2):
        order = np.lexsort((np.arange(x.shape[1]), -x[r].astype(np.float64)))[:64]
        assert (ids[r] == order).all() and (vals[r] == x[r][order]).all()


# ------------------------------------------------------------------ the two grouped products alone
def _numpy_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """[out][in * bits / 8] bytes -> [out][in] codes: each row a little-endian bit stream (numpy's
    unpackbits, least significant bit first), code i = the bits [bits i, bits i + bits)."""
    st = np.unpackbits(np.ascontiguousarray(codes, np.uint8), axis=-1, bitorder="little").astype(np.int64)
    st = st.reshape(codes.shape[0], -1, bits)
    return (st << np.arange(bits, dtype=np.int64)).sum(axis=-1)


def _numpy_weights(p, mat):
    """Independent dequantisation of an exact-arithmetic projection (numpy bit unpacking, float64):
    w = s * q + b, codes a little-endian bit stream per row (for 4 bits the even input in the low
    nibble); exact in float64 and in bf16 here."""
    q = _numpy_codes(p["codes"][mat], p.get("bits", 4))
    s = np.repeat(oracle.bf16_to_f32(p["scales"][mat]).astype(np.float64), 64, axis=1)
    b = np.repeat(oracle.bf16_to_f32(p["biases"][mat]).astype(np.float64), 64, axis=1)
    return s * q + b


def _routing_of(L, k):
    ids, _ = oracle.topk_softmax(oracle.router_logits(L["x"], L["w_router"], L["logit_bias"]), k)
    return oracle.route_meta(ids, L["w_router"].shape[1], L["shared"] is not None)


@pytest.mark.parametrize("T,d,E,k,I,Is,bits", [(9, 192, 4, 2, 128, 64, 4), (6, 128, 3, 3, 64, 0, 4),
                                               (9, 192, 4, 2, 128, 64, 3), (6, 128, 3, 3, 64, 64, 2)])
def test_gateup_preact_exact_against_numpy_matmul(T, d, E, k, I, Is, bits):
    """Exact-arithmetic inputs: the oracle's pre-activations equal a float64 matmul of numpy-made
    weights row for row (token of each grouped row, expert of each group, gate vs up, shared last)."""
    L = gen.exact_layer(T, d, E, k, I, Is, seed=T + d, bits=bits)
    m = _routing_of(L, k)
    g, u, gs, us = oracle.gateup_preact(L["x"], L["routed"], L["shared"], k, m["offsets"], m["sorted_token"])
    xf = oracle.bf16_to_f32(L["x"]).astype(np.float64)
    for e in range(E):
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        xs = xf[m["sorted_token"][r0:r1]]
        assert (g[r0:r1] == xs @ _numpy_weights(L["routed"]["gate"], e).T).all()
        assert (u[r0:r1] == xs @ _numpy_weights(L["routed"]["up"], e).T).all()
    if Is:
        assert (gs == xf @ _numpy_weights(L["shared"]["gate"], 0).T).all()
        assert (us == xf @ _numpy_weights(L["shared"]["up"], 0).T).all()
    # every value is exactly representable in fp32 (the property the GPU comparison relies on)
    for a in (g, u, gs, us):
        assert (a.astype(np.float32).astype(np.float64) == a).all()


def test_gateup_preact_gives_the_forward_layers_h():
    """On random (inexact) inputs the pre-activations, through silu(g) * u rounded to bf16, give
    the h of the whole-layer oracle, and they match a float64 matmul of the oracle's weights."""
    rng = np.random.default_rng(44)
    T, d, E, k, I, Is = 7, 128, 4, 2, 64, 128
    x, wr, routed, shared = _random_layer(rng, T, d, E, k, I, Is)
    out = oracle.forward_layer(x, wr, routed, shared, k, want_h=True)
    g, u, gs, us = oracle.gateup_preact(x, routed, shared, k, out["offsets"], out["sorted_token"])
    silu = lambda z: z / (1.0 + np.exp(-z))  # noqa: E731
    assert (_bf16((silu(g) * u).astype(F32)) == out["h"]).all()
    assert (_bf16((silu(gs) * us).astype(F32)) == out["h_shared"]).all()
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    for e in range(E):
        r0, r1 = out["offsets"][e], out["offsets"][e + 1]
        W = oracle.bf16_to_f32(oracle.dequant(routed["gate"]["codes"][e], routed["gate"]["scales"][e],
                                              routed["gate"]["biases"][e])).astype(np.float64)
        np.testing.assert_allclose(g[r0:r1], xf[out["sorted_token"][r0:r1]] @ W.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,d,E,k,I,Is,bits", [(9, 192, 4, 2, 128, 64, 4), (6, 128, 3, 3, 192, 0, 4),
                                               (9, 192, 4, 2, 128, 64, 2), (6, 128, 3, 3, 192, 64, 3)])
def test_down_rows_exact_against_numpy_matmul(T, d, E, k, I, Is, bits):
    L = gen.exact_layer(T, d, E, k, I, Is, seed=3 * T + d, bits=bits)
    m = _routing_of(L, k)
    P = T * k
    h = gen.small_ints_bf16(gen.key(7, 0, 1), P * I).reshape(P, I)
    hs = gen.small_ints_bf16(gen.key(7, 0, 2), T * Is).reshape(T, Is) if Is else None
    y = oracle.down_rows(h, hs, L["routed"], L["shared"], k, m["offsets"])
    assert y.shape == (P + (T if Is else 0), d)
    hf = oracle.bf16_to_f32(h).astype(np.float64)
    for e in range(E):
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        assert (y[r0:r1] == hf[r0:r1] @ _numpy_weights(L["routed"]["down"], e).T).all()
    if Is:
        assert (y[P:] == oracle.bf16_to_f32(hs).astype(np.float64) @ _numpy_weights(L["shared"]["down"], 0).T).all()
    assert (y.astype(np.float32).astype(np.float64) == y).all()


def test_down_rows_combine_to_the_forward_layers_output():
    """The whole-layer oracle's output is the combine of its own h through down_rows: y[t] =
    bf16(sum_j w[t][j] * y_row(t, j) + y_shared(t)), j ascending."""
    rng = np.random.default_rng(45)
    T, d, E, k, I, Is = 6, 128, 4, 3, 64, 64
    x, wr, routed, shared = _random_layer(rng, T, d, E, k, I, Is)
    out = oracle.forward_layer(x, wr, routed, shared, k, want_h=True)
    yr = oracle.down_rows(out["h"], out["h_shared"], routed, shared, k, out["offsets"])
    P = T * k
    acc = np.zeros((T, d), np.float64)
    for j in range(k):
        acc += out["topk_w"][:, j:j + 1].astype(np.float64) * yr[out["inv_pos"][:, j]]
    acc += yr[P:]
    assert (_bf16(acc.astype(F32)) == out["y"]).all()
