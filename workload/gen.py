"""Seeded synthetic inputs for the routed int4 MoE layer workloads.

Only input generation lives here (random draws and their storage format); none of
the method's arithmetic does. The generator itself is C (``moe_gen.c``, which states
its exact definition); this file names the workloads and lays the drawn values out in
the layouts the library and the oracle both take:

* ``x``            [T][d]       bf16 bits (uint16), N(0, 1)
* ``w_router``     [d][E]       fp32, N(0, sigma_r^2)
* ``logit_bias``   [E]          fp32 or None (Zipf-like 1.5 * ln(1/rank) for the skewed workload)
* per projection   codes [n_mat][out][in/2] uint8 (two 4-bit codes per byte, the even
                   input index in the low nibble), scales and biases [n_mat][out][in/64]
                   bf16 bits; scale = |N(0, 0.02^2)|, bias = -8 * scale
* gate, up: out = I, in = d;  down: out = d, in = I;  the shared expert has n_mat = 1.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gen.so")

# tensor ids of the streams of one layer
T_ROUTER = 1
T_GATE_CODES, T_GATE_SB = 2, 3
T_UP_CODES, T_UP_SB = 4, 5
T_DOWN_CODES, T_DOWN_SB = 6, 7
T_SH_GATE_CODES, T_SH_GATE_SB = 8, 9
T_SH_UP_CODES, T_SH_UP_SB = 10, 11
T_SH_DOWN_CODES, T_SH_DOWN_SB = 12, 13
T_PERM = 14
T_X = 100  # + chunk index
T_LOGITS = 1000  # + step index (logit rows of the top-K workload)
T_EXACT = 2000  # + tensor offset: inputs whose products and sums are exact in fp32

QUANT_SIGMA = 0.02
GROUP = 64

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the generator with gcc (OpenMP, -O2, IEEE semantics)."""
    import subprocess

    src = os.path.join(_HERE, "moe_gen.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           src, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        L.gen_stream_key.restype = u64
        L.gen_stream_key.argtypes = [u64, u64, u64]
        L.gen_word.restype = u64
        L.gen_word.argtypes = [u64, u64]
        L.gen_bytes.argtypes = [u64, u64, i64, vp]
        L.gen_normal_bf16.argtypes = [u64, u64, i64, dbl, vp]
        L.gen_normal_f32.argtypes = [u64, u64, i64, dbl, vp]
        L.gen_scale_bias_bf16.argtypes = [u64, u64, i64, dbl, vp, vp]
        L.gen_zipf_bias.argtypes = [i32, dbl, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(seed: int, layer: int, tensor: int) -> int:
    return lib().gen_stream_key(seed, layer, tensor)


def rand_bytes(k: int, n: int, start: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    out = np.empty(n, np.uint8) if out is None else out
    assert out.dtype == np.uint8 and out.size == n
    lib().gen_bytes(k, start, n, _ptr(out))
    return out


def normal_bf16(k: int, n: int, sigma: float, start: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    out = np.empty(n, np.uint16) if out is None else out
    assert out.dtype == np.uint16 and out.size == n
    lib().gen_normal_bf16(k, start, n, sigma, _ptr(out))
    return out


def normal_f32(k: int, n: int, sigma: float, start: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    out = np.empty(n, np.float32) if out is None else out
    assert out.dtype == np.float32 and out.size == n
    lib().gen_normal_f32(k, start, n, sigma, _ptr(out))
    return out


def scale_bias(k: int, n: int, sigma: float = QUANT_SIGMA, start: int = 0, out_s=None, out_b=None):
    s = np.empty(n, np.uint16) if out_s is None else out_s
    b = np.empty(n, np.uint16) if out_b is None else out_b
    lib().gen_scale_bias_bf16(k, start, n, sigma, _ptr(s), _ptr(b))
    return s, b


def zipf_bias(n_experts: int, alpha: float = 1.5, rank: Optional[np.ndarray] = None) -> np.ndarray:
    out = np.empty(n_experts, np.float32)
    if rank is not None:
        rank = np.ascontiguousarray(rank, dtype=np.int32)
        assert rank.size == n_experts
    lib().gen_zipf_bias(n_experts, alpha, None if rank is None else _ptr(rank), _ptr(out))
    return out


def permutation(k: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 driven by the stream's words (j = word % (i + 1))."""
    p = np.arange(n, dtype=np.int32)
    for i in range(n - 1, 0, -1):
        j = lib().gen_word(k, n - 1 - i) % (i + 1)
        p[i], p[j] = p[j], p[i]
    return p


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens per pass of the workload
    d: int            # hidden size
    E: int            # routed experts
    k: int            # experts per token
    I: int            # routed expert intermediate size
    Is: int           # shared expert intermediate size (0 = no shared expert)
    router_sigma: float
    layers: int       # distinct layers the workload cycles through
    chunk: int        # tokens per call (T is processed in T // chunk sequential calls)
    zipf: bool = False
    seed: int = 0
    bits: int = 4     # bits per expert weight code (4, or the 3- and 2-bit variants)

    @property
    def calls(self) -> int:
        return self.T // self.chunk

    @property
    def expert_bytes(self) -> int:
        """Packed bytes of one routed expert (codes + bf16 scales + bf16 biases, 3 matrices)."""
        return 3 * self.d * self.I * self.bits // 8 + 3 * 2 * 2 * self.d * self.I // GROUP

    @property
    def shared_bytes(self) -> int:
        return 3 * self.d * self.Is * self.bits // 8 + 3 * 2 * 2 * self.d * self.Is // GROUP


WORKLOADS: Dict[str, Workload] = {
    # T=8, d=256, 16 experts top-4 + shared (I_s = I = 128), router N(0, 0.05^2)
    "tiny": Workload("tiny", 8, 256, 16, 4, 128, 128, 0.05, 1, 8),
    # batch-1 decode over 40 distinct layers, 256 experts top-8 + shared, I = 512
    "decode": Workload("decode", 1, 2048, 256, 8, 512, 512, 0.02, 40, 1),
    # 512-token prefill through one layer of the decode shapes
    "prefill": Workload("prefill", 512, 2048, 256, 8, 512, 512, 0.02, 1, 512),
    # 4096 tokens in 4 chunks of 1024 with a Zipf-like logit bias
    "long": Workload("long", 4096, 2048, 256, 8, 512, 512, 0.02, 1, 1024, zipf=True),
    # diffusion canvas: 256 positions x 30 layers, 128 experts top-8, I = 768, no shared expert
    "diffusion": Workload("diffusion", 256, 2048, 128, 8, 768, 0, 0.02, 30, 256),
    # small-M calls (2..64 tokens, e.g. a few decode streams or speculative rows) at the decode
    # shapes, over the same 40 layers
    "m2": Workload("m2", 2, 2048, 256, 8, 512, 512, 0.02, 40, 2),
    "m4": Workload("m4", 4, 2048, 256, 8, 512, 512, 0.02, 40, 4),
    "m8": Workload("m8", 8, 2048, 256, 8, 512, 512, 0.02, 40, 8),
    "m16": Workload("m16", 16, 2048, 256, 8, 512, 512, 0.02, 40, 16),
    "m32": Workload("m32", 32, 2048, 256, 8, 512, 512, 0.02, 40, 32),
    "m64": Workload("m64", 64, 2048, 256, 8, 512, 512, 0.02, 40, 64),
    # the 3- and 2-bit expert variants at the decode shapes (same layers, fewer bits per weight)
    "decode3": Workload("decode3", 1, 2048, 256, 8, 512, 512, 0.02, 40, 1, bits=3),
    "decode2": Workload("decode2", 1, 2048, 256, 8, 512, 512, 0.02, 40, 1, bits=2),
    "m32_3": Workload("m32_3", 32, 2048, 256, 8, 512, 512, 0.02, 40, 32, bits=3),
    "m32_2": Workload("m32_2", 32, 2048, 256, 8, 512, 512, 0.02, 40, 32, bits=2),
    "tiny3": Workload("tiny3", 8, 256, 16, 4, 128, 128, 0.05, 1, 8, bits=3),
    "tiny2": Workload("tiny2", 8, 256, 16, 4, 128, 128, 0.05, 1, 8, bits=2),
    # the same variants on the grouped-GEMM path: the diffusion canvas at 3 and 2 bits, and a
    # prefill-size 3-bit call
    "diffusion3": Workload("diffusion3", 256, 2048, 128, 8, 768, 0, 0.02, 30, 256, bits=3),
    "diffusion2": Workload("diffusion2", 256, 2048, 128, 8, 768, 0, 0.02, 30, 256, bits=2),
    "prefill3": Workload("prefill3", 512, 2048, 256, 8, 512, 512, 0.02, 1, 512, bits=3),
}


def _proj(seed: int, layer: int, t_codes: int, t_sb: int, n_mat: int, out_dim: int, in_dim: int,
          out: Optional[dict] = None, bits: int = 4) -> dict:
    """Codes are uniform random bits (so every b-bit code is uniform in [0, 2^b)); a row's codes
    are a little-endian bit stream. scale = |N(0, 0.02^2)| * 2^(4 - b) and bias = -2^(b-1) * scale,
    so the weights s * (q - 2^(b-1)) cover the same range at every b; the bias is then -8 times the
    4-bit scale, the same bits as for 4-bit codes."""
    n_codes = n_mat * out_dim * in_dim * bits // 8
    n_sb = n_mat * out_dim * in_dim // GROUP
    if out is None:
        out = {"codes": np.empty(n_codes, np.uint8), "scales": np.empty(n_sb, np.uint16),
               "biases": np.empty(n_sb, np.uint16)}
    rand_bytes(key(seed, layer, t_codes), n_codes, out=out["codes"].reshape(-1))
    scale_bias(key(seed, layer, t_sb), n_sb, out_s=out["scales"].reshape(-1), out_b=out["biases"].reshape(-1))
    if bits != 4:  # times 2^(4 - b): an exact exponent step for these normal bf16 values
        sc = out["scales"].reshape(-1)
        sc += np.uint16((4 - bits) << 7)
    out["codes"] = out["codes"].reshape(n_mat, out_dim, in_dim * bits // 8)
    out["scales"] = out["scales"].reshape(n_mat, out_dim, in_dim // GROUP)
    out["biases"] = out["biases"].reshape(n_mat, out_dim, in_dim // GROUP)
    if bits != 4:  # (absent: 4-bit codes)
        out["bits"] = bits
    return out


def expert_weights(w: Workload, layer: int, shared: bool = False, out: Optional[dict] = None) -> dict:
    """Packed gate/up/down of all routed experts (or of the shared expert) of one layer."""
    seed = w.seed
    if shared:
        n, I, ids = 1, w.Is, (T_SH_GATE_CODES, T_SH_GATE_SB, T_SH_UP_CODES, T_SH_UP_SB, T_SH_DOWN_CODES, T_SH_DOWN_SB)
    else:
        n, I, ids = w.E, w.I, (T_GATE_CODES, T_GATE_SB, T_UP_CODES, T_UP_SB, T_DOWN_CODES, T_DOWN_SB)
    out = out or {}
    return {
        "gate": _proj(seed, layer, ids[0], ids[1], n, I, w.d, out.get("gate"), w.bits),
        "up": _proj(seed, layer, ids[2], ids[3], n, I, w.d, out.get("up"), w.bits),
        "down": _proj(seed, layer, ids[4], ids[5], n, w.d, I, out.get("down"), w.bits),
    }


def router(w: Workload, layer: int) -> np.ndarray:
    return normal_f32(key(w.seed, layer, T_ROUTER), w.d * w.E, w.router_sigma).reshape(w.d, w.E)


def logit_bias(w: Workload, permuted: bool = False) -> Optional[np.ndarray]:
    if not w.zipf:
        return None
    rank = None
    if permuted:
        rank = permutation(key(w.seed, 0, T_PERM), w.E) + 1
    return zipf_bias(w.E, 1.5, rank)


def tokens(w: Workload, layer: int, chunk: int, T: Optional[int] = None) -> np.ndarray:
    T = w.chunk if T is None else T
    return normal_bf16(key(w.seed, layer, T_X + chunk), T * w.d, 1.0).reshape(T, w.d)


@dataclasses.dataclass(frozen=True)
class VocabWorkload:
    """Rows of logits whose exact top-K a sampler needs: R positions over a V-entry vocabulary."""
    name: str
    R: int
    V: int
    K: int
    sigma: float    # spread of the raw logits
    softcap: float  # logits are softcap * tanh(z / softcap), z ~ N(0, sigma^2), as a softcapped head gives
    steps: int = 1  # distinct logit matrices the benchmark cycles
    seed: int = 0


VOCAB_WORKLOADS: Dict[str, VocabWorkload] = {
    "vocab_tiny": VocabWorkload("vocab_tiny", 5, 3000, 16, 3.0, 30.0),
    # a 256-position canvas over a 262,144-entry vocabulary, top-64 per position
    "vocab": VocabWorkload("vocab", 256, 262144, 64, 3.0, 30.0, steps=4),
}


def vocab_logits(w: VocabWorkload, step: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """fp32 logits [R][V] of one step (the first `rows` rows when given)."""
    R = w.R if rows is None else rows
    z = normal_f32(key(w.seed, 0, T_LOGITS + step), R * w.V, w.sigma)
    np.tanh(z * np.float32(1.0 / w.softcap), out=z)
    z *= np.float32(w.softcap)
    return z.reshape(R, w.V)


def layer(w: Workload, layer_idx: int = 0) -> dict:
    """All inputs of one layer except the activations."""
    return {
        "w_router": router(w, layer_idx),
        "logit_bias": logit_bias(w),
        "routed": expert_weights(w, layer_idx),
        "shared": expert_weights(w, layer_idx, shared=True) if w.Is > 0 else None,
    }


# ------------------------------------------------------------------ exact-arithmetic inputs
# Inputs on which every product and every partial sum of the expert FFN's two matrix products is
# exactly representable in fp32, whatever the summation order: integer activations in [-4, 4]
# (bf16), and per group a power-of-two scale 2^-m (m in 3..7) with a bias of -c * 2^-m (c in
# 0..16). A weight s * q + b = (q - c) * 2^-m then has at most 5 significant bits (exact in
# bf16), and a sum over d <= 4096 inputs stays below 2^24 units of 2^-7. Only bit patterns are
# drawn here; the values follow from the bf16 format.
def _f32_bits_to_bf16(v: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(v, np.float32).view(np.uint32)
    assert not (b & 0xFFFF).any(), "value not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


def small_ints_bf16(k: int, n: int, lo: int = -4, hi: int = 4, start: int = 0) -> np.ndarray:
    """bf16 bits of integers drawn from [lo, hi] (byte of the stream modulo the range size)."""
    r = rand_bytes(k, n, start).astype(np.int32) % (hi - lo + 1) + lo
    return _f32_bits_to_bf16(r.astype(np.float32))


def exact_proj(seed: int, layer: int, tensor: int, n_mat: int, out_dim: int, in_dim: int, bits: int = 4) -> dict:
    """Codes of `bits` bits (uniform random bytes of the rows' bit streams), exact scales/biases."""
    n_sb = n_mat * out_dim * in_dim // GROUP
    codes = rand_bytes(key(seed, layer, T_EXACT + 3 * tensor), n_mat * out_dim * in_dim * bits // 8)
    sb = rand_bytes(key(seed, layer, T_EXACT + 3 * tensor + 1), 2 * n_sb).reshape(n_sb, 2).astype(np.int32)
    m = 3 + sb[:, 0] % 5
    c = sb[:, 1] % 17
    scale = np.ldexp(np.float32(1.0), -m).astype(np.float32)
    out = {"codes": codes.reshape(n_mat, out_dim, in_dim * bits // 8),
           "scales": _f32_bits_to_bf16(scale).reshape(n_mat, out_dim, in_dim // GROUP),
           "biases": _f32_bits_to_bf16((-c * scale).astype(np.float32)).reshape(n_mat, out_dim, in_dim // GROUP)}
    if bits != 4:
        out["bits"] = bits
    return out


def exact_layer(T: int, d: int, E: int, k: int, I: int, Is: int, seed: int = 0, layer: int = 0,
                router_sigma: float = 0.02, zipf: bool = False, bits: int = 4) -> dict:
    """A layer (as layer()) plus its activations "x", all with exact-arithmetic values; the router
    is N(0, router_sigma^2) in fp32, with the skewed workload's logit bias when zipf is set."""
    def ffn(base, n, Ie):
        return {"gate": exact_proj(seed, layer, base, n, Ie, d, bits),
                "up": exact_proj(seed, layer, base + 1, n, Ie, d, bits),
                "down": exact_proj(seed, layer, base + 2, n, d, Ie, bits)}
    return {
        "x": small_ints_bf16(key(seed, layer, T_EXACT + 99), T * d).reshape(T, d),
        "w_router": normal_f32(key(seed, layer, T_EXACT + 98), d * E, router_sigma).reshape(d, E),
        "logit_bias": zipf_bias(E, 1.5) if zipf else None,
        "routed": ffn(0, E, I),
        "shared": ffn(3, 1, Is) if Is > 0 else None,
    }
