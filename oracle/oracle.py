"""Python binding of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE: only the tests, the package smoke check and the benchmark's CPU
baseline leg use this module. The GPU library and its binding never import it.

Arrays are numpy: bf16 values travel as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "moe_oracle.c")
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wno-unknown-pragmas", src, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Q4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("bits", ctypes.c_int32)]


class _FFN(ctypes.Structure):
    _fields_ = [("gate", _Q4), ("up", _Q4), ("down", _Q4)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.oracle_round_bf16.argtypes = [i64, vp, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_router_logits.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.oracle_topk_softmax.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_route_meta.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp]
        L.oracle_dequant.argtypes = [i64, i32, vp, vp, vp, vp]
        L.oracle_dequant_bits.argtypes = [i64, i32, i32, vp, vp, vp, vp]
        L.oracle_forward_layer.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, ctypes.POINTER(_FFN),
                                           ctypes.POINTER(_FFN), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.oracle_forward_tokens.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, ctypes.POINTER(_FFN),
                                            ctypes.POINTER(_FFN), i32, vp, vp, vp, vp]
        L.oracle_vocab_topk.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_gateup_preact.argtypes = [i32, i32, i32, i32, i32, i32, vp, ctypes.POINTER(_FFN),
                                           ctypes.POINTER(_FFN), vp, vp, vp, vp]
        L.oracle_down_rows.argtypes = [i32, i32, i32, i32, i32, i32, vp, ctypes.POINTER(_FFN),
                                       ctypes.POINTER(_FFN), vp, vp]
        for f in ("oracle_router_logits", "oracle_topk_softmax", "oracle_route_meta", "oracle_dequant",
                  "oracle_forward_layer", "oracle_forward_tokens", "oracle_vocab_topk", "oracle_dequant_bits",
                  "oracle_gateup_preact", "oracle_down_rows"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().oracle_num_threads()


def _p(a: Optional[np.ndarray]) -> Optional[int]:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _ffn(w: Optional[dict]):
    """dict(gate|up|down -> dict(codes, scales, biases)) -> (struct, keep-alive list)."""
    if w is None:
        return None, []
    keep = []
    q = {}
    for name in ("gate", "up", "down"):
        c = _c(w[name]["codes"], np.uint8)
        s = _c(w[name]["scales"], np.uint16)
        b = _c(w[name]["biases"], np.uint16)
        keep += [c, s, b]
        q[name] = _Q4(_p(c), _p(s), _p(b), int(w[name].get("bits", 4)))
    return _FFN(q["gate"], q["up"], q["down"]), keep


def round_bf16(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_round_bf16(a.size, _p(a), _p(out))
    return out


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (a format conversion, not arithmetic)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def router_logits(x, w_router, bias=None) -> np.ndarray:
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E = w_router.shape[1]
    out = np.empty((T, E), np.float32)
    rc = lib().oracle_router_logits(T, d, E, _p(x), _p(w_router), _p(bias), _p(out))
    if rc:
        raise ValueError(f"oracle_router_logits rc={rc}")
    return out


def topk_softmax(logits, k: int):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = lib().oracle_topk_softmax(T, E, k, _p(logits), _p(ids), _p(w))
    if rc:
        raise ValueError(f"oracle_topk_softmax rc={rc}")
    return ids, w


def max_tiles(T: int, E: int, k: int, has_shared: bool) -> int:
    P = T * k
    return min(E, P) + P // 32 + ((T + 31) // 32 if has_shared else 0)


def route_meta(ids, E: int, has_shared: bool):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    P = T * k
    cap = max_tiles(T, E, k, has_shared) + 1
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_token = np.empty(P, np.int32)
    inv_pos = np.empty((T, k), np.int32)
    tiles = np.zeros((cap, 3), np.int32)
    n = np.zeros(1, np.int32)
    rc = lib().oracle_route_meta(T, E, k, int(has_shared), _p(ids), _p(counts), _p(offsets), _p(sorted_token),
                                 _p(inv_pos), _p(tiles), cap, _p(n))
    if rc:
        raise ValueError(f"oracle_route_meta rc={rc}")
    return {"counts": counts, "offsets": offsets, "sorted_token": sorted_token, "inv_pos": inv_pos,
            "tiles": tiles[: n[0]].copy(), "n_tiles": int(n[0])}


def dequant(codes, scales, biases, bits: int = 4) -> np.ndarray:
    """codes [..., out, in * bits / 8] -> bf16 bits [..., out, in]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    in_dim = codes.shape[-1] * 8 // bits
    rows = codes.size // codes.shape[-1]
    out = np.empty(codes.shape[:-1] + (in_dim,), np.uint16)
    rc = lib().oracle_dequant_bits(rows, in_dim, bits, _p(codes), _p(scales), _p(biases), _p(out))
    if rc:
        raise ValueError(f"oracle_dequant rc={rc}")
    return out


def forward_layer(x, w_router, routed: dict, shared: Optional[dict], k: int, bias=None, want_h: bool = False):
    """Whole layer on all tokens. Returns dict with y (bf16 bits [T][d]) and the routing."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E = w_router.shape[1]
    I = routed["gate"]["codes"].shape[-2]
    Is = 0 if shared is None else shared["gate"]["codes"].shape[-2]
    P = T * k
    cap = max_tiles(T, E, k, Is > 0) + 1
    r_ffn, keep_r = _ffn(routed)
    s_ffn, keep_s = _ffn(shared)
    out = {
        "y": np.empty((T, d), np.uint16), "logits": np.empty((T, E), np.float32),
        "topk_ids": np.empty((T, k), np.int32), "topk_w": np.empty((T, k), np.float32),
        "counts": np.empty(E, np.int32), "offsets": np.empty(E + 1, np.int32),
        "sorted_token": np.empty(P, np.int32), "inv_pos": np.empty((T, k), np.int32),
        "tiles": np.zeros((cap, 3), np.int32),
    }
    n = np.zeros(1, np.int32)
    h = np.empty((P, I), np.uint16) if want_h else None
    hs = np.empty((T, Is), np.uint16) if (want_h and Is) else None
    rc = lib().oracle_forward_layer(
        T, d, E, k, I, Is, _p(x), _p(w_router), _p(bias), ctypes.byref(r_ffn),
        ctypes.byref(s_ffn) if s_ffn is not None else None,
        _p(out["y"]), _p(out["logits"]), _p(out["topk_ids"]), _p(out["topk_w"]), _p(out["counts"]),
        _p(out["offsets"]), _p(out["sorted_token"]), _p(out["inv_pos"]), _p(out["tiles"]), cap, _p(n), _p(h), _p(hs))
    del keep_r, keep_s
    if rc:
        raise ValueError(f"oracle_forward_layer rc={rc}")
    out["n_tiles"] = int(n[0])
    out["tiles"] = out["tiles"][: out["n_tiles"]].copy()
    if want_h:
        out["h"] = h
        out["h_shared"] = hs
    return out


def forward_tokens(x, w_router, routed: dict, shared: Optional[dict], k: int, sel, bias=None):
    """Output rows of the listed tokens only, evaluated token by token."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    bias = _c(bias, np.float32)
    sel = _c(sel, np.int32)
    T, d = x.shape
    E = w_router.shape[1]
    I = routed["gate"]["codes"].shape[-2]
    Is = 0 if shared is None else shared["gate"]["codes"].shape[-2]
    r_ffn, keep_r = _ffn(routed)
    s_ffn, keep_s = _ffn(shared)
    y = np.empty((sel.size, d), np.uint16)
    ids = np.empty((sel.size, k), np.int32)
    w = np.empty((sel.size, k), np.float32)
    rc = lib().oracle_forward_tokens(T, d, E, k, I, Is, _p(x), _p(w_router), _p(bias), ctypes.byref(r_ffn),
                                     ctypes.byref(s_ffn) if s_ffn is not None else None, sel.size, _p(sel),
                                     _p(y), _p(ids), _p(w))
    del keep_r, keep_s
    if rc:
        raise ValueError(f"oracle_forward_tokens rc={rc}")
    return {"y": y, "topk_ids": ids, "topk_w": w}


def _dims_of(routed: dict, shared: Optional[dict], d: int):
    E = routed["gate"]["codes"].shape[0]
    I = routed["gate"]["codes"].shape[-2]
    Is = 0 if shared is None else shared["gate"]["codes"].shape[-2]
    return E, I, Is


def gateup_preact(x, routed: dict, shared: Optional[dict], k: int, offsets, sorted_token):
    """Gate and up products of every grouped row before the activation, in double:
    (g, u), each [T*k][I] (grouped row order) and, with a shared expert, [T][Is] (g_s, u_s)."""
    x = _c(x, np.uint16)
    offsets = _c(offsets, np.int32)
    sorted_token = _c(sorted_token, np.int32)
    T, d = x.shape
    E, I, Is = _dims_of(routed, shared, d)
    P = T * k
    r_ffn, keep_r = _ffn(routed)
    s_ffn, keep_s = _ffn(shared)
    g = np.empty(P * I + T * Is, np.float64)
    u = np.empty(P * I + T * Is, np.float64)
    rc = lib().oracle_gateup_preact(T, d, E, k, I, Is, _p(x), ctypes.byref(r_ffn),
                                    ctypes.byref(s_ffn) if s_ffn is not None else None, _p(offsets),
                                    _p(sorted_token), _p(g), _p(u))
    del keep_r, keep_s
    if rc:
        raise ValueError(f"oracle_gateup_preact rc={rc}")
    return (g[: P * I].reshape(P, I), u[: P * I].reshape(P, I), g[P * I:].reshape(T, Is), u[P * I:].reshape(T, Is))


def down_rows(h, h_shared, routed: dict, shared: Optional[dict], k: int, offsets):
    """Down products of given bf16 rows in double: h [T*k][I] (grouped order), h_shared [T][Is]
    (or None) -> y [T*k + T][d] (shared rows last; [T*k][d] without a shared expert)."""
    h = _c(h, np.uint16)
    offsets = _c(offsets, np.int32)
    P = h.shape[0]
    T = P // k
    d = routed["down"]["codes"].shape[-2]
    E, I, Is = _dims_of(routed, shared, d)
    hh = h.reshape(-1) if not Is else np.concatenate([h.reshape(-1), _c(h_shared, np.uint16).reshape(-1)])
    r_ffn, keep_r = _ffn(routed)
    s_ffn, keep_s = _ffn(shared)
    y = np.empty((P + (T if Is else 0), d), np.float64)
    rc = lib().oracle_down_rows(T, d, E, k, I, Is, _p(hh), ctypes.byref(r_ffn),
                                ctypes.byref(s_ffn) if s_ffn is not None else None, _p(offsets), _p(y))
    del keep_r, keep_s
    if rc:
        raise ValueError(f"oracle_down_rows rc={rc}")
    return y


def vocab_topk(logits, K: int):
    """Exact top-K of each row by (value desc, index asc): (ids [R][K] int32, vals [R][K] fp32)."""
    logits = _c(logits, np.float32)
    R, V = logits.shape
    ids = np.empty((R, K), np.int32)
    vals = np.empty((R, K), np.float32)
    rc = lib().oracle_vocab_topk(R, V, K, _p(logits), _p(ids), _p(vals))
    if rc:
        raise ValueError(f"oracle_vocab_topk rc={rc}")
    return ids, vals
