"""Python binding of libmoe_int4.so (the routed int4 MoE FFN for MI355X).

Argument marshalling only: tensors are checked for device, dtype and contiguity, then
their data pointers and torch's current HIP stream go to the C ABI (include/moe_int4.h).
Every step of the computation runs in the library's gfx950 kernels; there is no CPU
fallback, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import torch  # imported first: the library must bind to the HIP runtime torch already loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_int4.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES: the fixed scratch of moe_forward_layer_noalloc


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: Optional[str] = None):
        L = lib()
        detail = L.moe_last_error().decode() if detail is None else detail
        super().__init__(f"{where}: {L.moe_status_str(status).decode()} ({detail})")
        self.status = status


def _shape_error(where: str, detail: str) -> MoeError:
    """A shape mismatch caught before the library is called: the C ABI sees only pointers, so a
    tensor of the wrong size would become out-of-bounds device accesses."""
    return MoeError(MOE_EINVAL, where, detail)


class Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("code_bits", ctypes.c_int32)]


class Q4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class FFNQ4(ctypes.Structure):
    _fields_ = [("gate", Q4), ("up", Q4), ("down", Q4)]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_ids", "topk_w", "counts", "offsets", "sorted_token", "inv_pos", "tiles", "n_tiles")]


_lib = None


def lib():
    """Load the library once. Raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with bit_moe_expert_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, vp, i32, i64, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_max_tiles.argtypes = [P(Dims), i32]
        L.moe_max_tiles.restype = i32
        L.moe_workspace_bytes.argtypes = [P(Dims), i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_route.argtypes = [P(Dims), i32, vp, vp, vp, P(Routing), vp, sz, vp]
        L.moe_expert_ffn.argtypes = [P(Dims), i32, vp, P(Routing), P(FFNQ4), P(FFNQ4), vp, vp, sz, vp]
        L.moe_forward_layer.argtypes = [P(Dims), i32, vp, vp, vp, P(FFNQ4), P(FFNQ4), vp, vp, sz, vp]
        L.moe_forward_layer_noalloc.argtypes = [P(Dims), i32, vp, vp, vp, P(FFNQ4), P(FFNQ4), vp, vp]
        L.moe_debug_dequant.argtypes = [P(Q4), i64, i32, vp, vp]
        L.moe_debug_dequant_bits.argtypes = [P(Q4), i64, i32, i32, vp, vp]
        L.moe_debug_grouped_gemm.argtypes = [P(Dims), i32, i32, vp, P(Routing), P(FFNQ4), P(FFNQ4), vp, vp, vp, sz, vp]
        L.moe_debug_router_logits.argtypes = [P(Dims), i32, vp, vp, vp, vp, vp]
        L.moe_num_stages.argtypes = [P(Dims), i32]
        L.moe_num_stages.restype = i32
        L.moe_stage_name.argtypes = [P(Dims), i32, i32]
        L.moe_stage_name.restype = ctypes.c_char_p
        L.moe_launch_stage.argtypes = [i32, P(Dims), i32, vp, vp, vp, P(FFNQ4), P(FFNQ4), vp, vp, sz, vp]
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_vocab_topk_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_vocab_topk_workspace_bytes.restype = sz
        L.moe_vocab_topk.argtypes = [i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_vocab_topk_stage.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        for f in ("moe_route", "moe_expert_ffn", "moe_forward_layer", "moe_forward_layer_noalloc",
                  "moe_debug_dequant", "moe_debug_dequant_bits",
                  "moe_launch_stage", "moe_debug_grouped_gemm",
                  "moe_vocab_topk", "moe_vocab_topk_stage"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def make_dims(d: int, E: int, k: int, I: int, Is: int, bits: int = 4) -> Dims:
    return Dims(d, E, k, I, Is, 64, bits)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype, name: str, device=None) -> Optional[int]:
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


@dataclasses.dataclass
class QProj:
    """One projection of n experts: codes [n][out][in * bits / 8] uint8, scales/biases [n][out][in/64] bf16."""
    codes: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor
    bits: int = 4

    def struct(self, device=None) -> Q4:
        return Q4(_ptr(self.codes, torch.uint8, "codes", device), _ptr(self.scales, torch.bfloat16, "scales", device),
                  _ptr(self.biases, torch.bfloat16, "biases", device))


@dataclasses.dataclass
class QuantFFN:
    gate: QProj
    up: QProj
    down: QProj

    def struct(self, device=None) -> FFNQ4:
        return FFNQ4(self.gate.struct(device), self.up.struct(device), self.down.struct(device))

    @property
    def n_experts(self) -> int:
        return self.gate.codes.shape[0]

    @property
    def d_ff(self) -> int:
        return self.gate.codes.shape[1]

    @property
    def d_model(self) -> int:
        return self.down.codes.shape[1]

    @property
    def bits(self) -> int:
        if not self.gate.bits == self.up.bits == self.down.bits:
            raise ValueError("gate, up and down must use the same code width")
        return self.gate.bits

    def check(self, d: int, what: str) -> None:
        """Every array's shape against (n experts, d_ff, d_model = d, code width)."""
        n, I, b = self.n_experts, self.d_ff, self.bits
        for name, p, out_dim, in_dim in (("gate", self.gate, I, d), ("up", self.up, I, d), ("down", self.down, d, I)):
            if in_dim % 64 or (in_dim * b) % 8:
                raise _shape_error(what, f"{name}: input dimension {in_dim} is not a multiple of 64")
            want = {"codes": (n, out_dim, in_dim * b // 8), "scales": (n, out_dim, in_dim // 64),
                    "biases": (n, out_dim, in_dim // 64)}
            for arr, shape in want.items():
                got = tuple(getattr(p, arr).shape)
                if got != shape:
                    raise _shape_error(what, f"{name}.{arr} has shape {got}, expected {shape}")


def _bits_of(routed: QuantFFN, shared: Optional[QuantFFN]) -> int:
    if shared is not None and shared.bits != routed.bits:
        raise ValueError("routed and shared experts must use the same code width")
    return routed.bits


def _dims_for(d: int, routed: QuantFFN, shared: Optional[QuantFFN], k: int, where: str) -> Dims:
    """The dims of a layer of d_model = d, with every expert array's shape checked."""
    routed.check(d, where + " (routed)")
    if shared is not None:
        if shared.n_experts != 1:
            raise _shape_error(where, f"the shared expert has {shared.n_experts} matrices, expected 1")
        shared.check(d, where + " (shared)")
    return make_dims(d, routed.n_experts, k, routed.d_ff, 0 if shared is None else shared.d_ff,
                     _bits_of(routed, shared))


def _check_routing(r: Dict[str, torch.Tensor], dims: Dims, T: int, where: str) -> None:
    """Every routing array's size against (T, k, E) and the block map's bound."""
    k, E = dims.top_k, dims.n_experts
    want = {"topk_ids": T * k, "topk_w": T * k, "counts": E, "offsets": E + 1, "sorted_token": T * k,
            "inv_pos": T * k, "tiles": 3 * max(max_tiles(dims, T), 1), "n_tiles": 1}
    for name, n in want.items():
        if name not in r:
            raise _shape_error(where, f"routing has no {name}")
        got = r[name].numel()
        if got < n if name == "tiles" else got != n:
            raise _shape_error(where, f"routing {name} holds {got} values, expected {'at least ' if name == 'tiles' else ''}{n}")
    if tuple(r["topk_ids"].shape) != (T, k) or tuple(r["topk_w"].shape) != (T, k):
        raise _shape_error(where, f"topk_ids / topk_w must be [{T}][{k}]")


def max_tiles(dims: Dims, T: int) -> int:
    return lib().moe_max_tiles(ctypes.byref(dims), T)


def workspace_bytes(dims: Dims, T: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(dims), T)


def new_workspace(dims: Dims, T: int, device) -> torch.Tensor:
    """Workspace of the size the library asks for (zero-filled, though the ABI does not need it)."""
    n = workspace_bytes(dims, T)
    if n == 0:
        raise MoeError(MOE_EUNSUPPORTED, "workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def new_routing(dims: Dims, T: int, device) -> Dict[str, torch.Tensor]:
    k, E = dims.top_k, dims.n_experts
    i32 = dict(dtype=torch.int32, device=device)
    return {
        "topk_ids": torch.empty((T, k), **i32), "topk_w": torch.empty((T, k), dtype=torch.float32, device=device),
        "counts": torch.empty(E, **i32), "offsets": torch.empty(E + 1, **i32),
        "sorted_token": torch.empty(T * k, **i32), "inv_pos": torch.empty((T, k), **i32),
        "tiles": torch.empty((max(max_tiles(dims, T), 1), 3), **i32), "n_tiles": torch.empty(1, **i32),
    }


def _routing_struct(r: Dict[str, torch.Tensor], device) -> Routing:
    return Routing(*[_ptr(r[n], torch.float32 if n == "topk_w" else torch.int32, n, device)
                     for n, _ in Routing._fields_])


def route(x: torch.Tensor, w_router: torch.Tensor, k: int, d_ff: int, d_ff_shared: int,
          logit_bias: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """moe_route: top-k, gate weights and the routing metadata of T tokens."""
    if x.dim() != 2 or w_router.dim() != 2 or w_router.shape[0] != x.shape[1]:
        raise _shape_error("moe_route", f"x {tuple(x.shape)} and w_router {tuple(w_router.shape)} must be [T][d] and [d][E]")
    T, d = x.shape
    dims = make_dims(d, w_router.shape[1], k, d_ff, d_ff_shared)
    if logit_bias is not None and logit_bias.numel() != dims.n_experts:
        raise _shape_error("moe_route", f"logit_bias holds {logit_bias.numel()} values, expected {dims.n_experts}")
    dev = x.device
    ws = new_workspace(dims, T, dev) if ws is None else ws
    r = new_routing(dims, T, dev)
    rs = _routing_struct(r, dev)
    rc = lib().moe_route(ctypes.byref(dims), T, _ptr(x, torch.bfloat16, "x", dev),
                         _ptr(w_router, torch.float32, "w_router", dev), _ptr(logit_bias, torch.float32, "logit_bias", dev),
                         ctypes.byref(rs), _ptr(ws, torch.uint8, "ws", dev), ws.numel(), _stream(dev))
    _check(rc, "moe_route")
    return r


def expert_ffn(x: torch.Tensor, routing: Dict[str, torch.Tensor], routed: QuantFFN, shared: Optional[QuantFFN],
               ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_expert_ffn: the expert FFN of routed tokens (GEMV path for calls of up to 32 tokens, grouped GEMM above)."""
    if x.dim() != 2:
        raise _shape_error("moe_expert_ffn", "x must be [T][d]")
    T, d = x.shape
    k = routing["topk_ids"].shape[1] if routing["topk_ids"].dim() == 2 else -1
    dims = _dims_for(d, routed, shared, k, "moe_expert_ffn")
    _check_routing(routing, dims, T, "moe_expert_ffn")
    dev = x.device
    ws = new_workspace(dims, T, dev) if ws is None else ws
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev) if y is None else y
    if tuple(y.shape) != (T, d):
        raise _shape_error("moe_expert_ffn", f"y has shape {tuple(y.shape)}, expected {(T, d)}")
    rs = _routing_struct(routing, dev)
    rf = routed.struct(dev)
    sf = shared.struct(dev) if shared is not None else None
    rc = lib().moe_expert_ffn(ctypes.byref(dims), T, _ptr(x, torch.bfloat16, "x", dev), ctypes.byref(rs),
                              ctypes.byref(rf), ctypes.byref(sf) if sf is not None else None,
                              _ptr(y, torch.bfloat16, "y", dev), _ptr(ws, torch.uint8, "ws", dev), ws.numel(),
                              _stream(dev))
    _check(rc, "moe_expert_ffn")
    return y


class Layer:
    """Marshalled arguments of moe_forward_layer for one layer, reusable across calls."""

    def __init__(self, w_router: torch.Tensor, routed: QuantFFN, shared: Optional[QuantFFN], k: int,
                 logit_bias: Optional[torch.Tensor] = None):
        self.dev = w_router.device
        self.w_router, self.routed, self.shared, self.k, self.logit_bias = w_router, routed, shared, k, logit_bias
        self.dims = _dims_for(routed.d_model, routed, shared, k, "moe_forward_layer")
        if w_router.shape != (self.dims.d_model, self.dims.n_experts):
            raise _shape_error("moe_forward_layer", f"w_router shape {tuple(w_router.shape)} does not match the experts")
        if logit_bias is not None and logit_bias.numel() != self.dims.n_experts:
            raise _shape_error("moe_forward_layer", f"logit_bias holds {logit_bias.numel()} values")
        self._wr = _ptr(w_router, torch.float32, "w_router", self.dev)
        self._bias = _ptr(logit_bias, torch.float32, "logit_bias", self.dev)
        self._rf = routed.struct(self.dev)
        self._sf = shared.struct(self.dev) if shared is not None else None

    def _io(self, x: torch.Tensor, y: torch.Tensor):
        T = x.shape[0]
        if x.dim() != 2 or x.shape[1] != self.dims.d_model or y.shape != x.shape:
            raise _shape_error("moe_forward_layer", f"x {tuple(x.shape)} / y {tuple(y.shape)} must both be [T][{self.dims.d_model}]")
        return (ctypes.byref(self.dims), T, _ptr(x, torch.bfloat16, "x", self.dev), self._wr, self._bias,
                ctypes.byref(self._rf), ctypes.byref(self._sf) if self._sf is not None else None,
                _ptr(y, torch.bfloat16, "y", self.dev))

    def args(self, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor):
        return self._io(x, y) + (_ptr(ws, torch.uint8, "ws", self.dev), ws.numel(), _stream(self.dev))

    def workspace(self, T: int) -> torch.Tensor:
        return new_workspace(self.dims, T, self.dev)

    def forward(self, x: torch.Tensor, ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None):
        T = x.shape[0]
        ws = self.workspace(T) if ws is None else ws
        y = torch.empty_like(x) if y is None else y
        _check(lib().moe_forward_layer(*self.args(x, y, ws)), "moe_forward_layer")
        return y

    def forward_noalloc(self, x: torch.Tensor, y: Optional[torch.Tensor] = None):
        """moe_forward_layer_noalloc: the layer with the library's fixed device scratch as workspace."""
        y = torch.empty_like(x) if y is None else y
        _check(lib().moe_forward_layer_noalloc(*self._io(x, y), _stream(self.dev)), "moe_forward_layer_noalloc")
        return y

    def stages(self, T: int):
        L = lib()
        n = L.moe_num_stages(ctypes.byref(self.dims), T)
        return [L.moe_stage_name(ctypes.byref(self.dims), T, s).decode() for s in range(n)]

    def launch_stage(self, stage: int, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor) -> None:
        _check(lib().moe_launch_stage(stage, *self.args(x, y, ws)), "moe_launch_stage")


def forward_layer(x: torch.Tensor, w_router: torch.Tensor, routed: QuantFFN, shared: Optional[QuantFFN], k: int,
                  logit_bias: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_forward_layer: route + expert FFN + combine for T tokens."""
    return Layer(w_router, routed, shared, k, logit_bias).forward(x, ws, y)


def debug_router_logits(x: torch.Tensor, w_router: torch.Tensor,
                        logit_bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_debug_router_logits: fp32 logits [T][E] from the router kernel of calls of more than 32
    tokens, whatever T (for bit-for-bit comparison)."""
    if x.dim() != 2 or w_router.dim() != 2 or w_router.shape[0] != x.shape[1]:
        raise _shape_error("moe_debug_router_logits", f"x {tuple(x.shape)} and w_router {tuple(w_router.shape)} "
                           "must be [T][d] and [d][E]")
    T, d = x.shape
    E = w_router.shape[1]
    dims = make_dims(d, E, 1, 64, 0)
    if logit_bias is not None and logit_bias.numel() != E:
        raise _shape_error("moe_debug_router_logits", f"logit_bias holds {logit_bias.numel()} values, expected {E}")
    dev = x.device
    out = torch.empty((T, E), dtype=torch.float32, device=dev)
    rc = lib().moe_debug_router_logits(ctypes.byref(dims), T, _ptr(x, torch.bfloat16, "x", dev),
                                       _ptr(w_router, torch.float32, "w_router", dev),
                                       _ptr(logit_bias, torch.float32, "logit_bias", dev), _ptr(out, torch.float32, "out", dev),
                                       _stream(dev))
    _check(rc, "moe_debug_router_logits")
    return out


def debug_dequant(p: QProj) -> torch.Tensor:
    """moe_debug_dequant_bits: bf16 expansion of a projection, with the GEMV kernels' unpacking of the
    codes (seg_pairs). The grouped GEMM's own unpacking is checked through debug_grouped_gemm."""
    codes = p.codes
    in_dim = codes.shape[-1] * 8 // p.bits
    rows = codes.numel() // codes.shape[-1]
    if p.scales.shape != codes.shape[:-1] + (in_dim // 64,) or p.biases.shape != p.scales.shape:
        raise _shape_error("moe_debug_dequant", f"scales {tuple(p.scales.shape)} / biases {tuple(p.biases.shape)} do not "
                           f"match codes {tuple(codes.shape)}")
    dev = codes.device
    out = torch.empty(tuple(codes.shape[:-1]) + (in_dim,), dtype=torch.bfloat16, device=dev)
    q = p.struct(dev)
    rc = lib().moe_debug_dequant_bits(ctypes.byref(q), rows, in_dim, p.bits, _ptr(out, torch.bfloat16, "out", dev),
                                      _stream(dev))
    _check(rc, "moe_debug_dequant")
    return out


def debug_grouped_gemm(which: int, a: torch.Tensor, routing: Dict[str, torch.Tensor], routed: QuantFFN,
                       shared: Optional[QuantFFN], ws: Optional[torch.Tensor] = None):
    """moe_debug_grouped_gemm: one grouped-GEMM kernel alone, fp32 results before the activation.
    which = 0: a = x [T][d]; returns (g, u), each [T*k*I + T*Is] fp32 (grouped rows, shared last).
    which = 1: a = h [T*k*I + T*Is] bf16 (same layout); returns y rows [T*k (+ T)][d] fp32."""
    k = routing["topk_ids"].shape[1]
    T = routing["topk_ids"].shape[0]
    dev = a.device
    d = routed.d_model
    dims = _dims_for(d, routed, shared, k, "moe_debug_grouped_gemm")
    _check_routing(routing, dims, T, "moe_debug_grouped_gemm")
    P, I, Is = T * k, dims.d_ff, dims.d_ff_shared
    if which == 0:
        if tuple(a.shape) != (T, d):
            raise ValueError("x must be [T][d]")
        out = torch.empty(P * I + T * Is, dtype=torch.float32, device=dev)
        out2 = torch.empty_like(out)
    else:
        if a.numel() != P * I + T * Is:
            raise ValueError("h must hold T*k*d_ff + T*d_ff_shared values")
        out = torch.empty((P + (T if Is else 0), d), dtype=torch.float32, device=dev)
        out2 = None
    ws = new_workspace(dims, T, dev) if ws is None else ws
    rs = _routing_struct(routing, dev)
    rf = routed.struct(dev)
    sf = shared.struct(dev) if shared is not None else None
    rc = lib().moe_debug_grouped_gemm(ctypes.byref(dims), T, which, _ptr(a, torch.bfloat16, "a", dev), ctypes.byref(rs),
                                      ctypes.byref(rf), ctypes.byref(sf) if sf is not None else None,
                                      _ptr(out, torch.float32, "out", dev),
                                      _ptr(out2, torch.float32, "out2", dev) if out2 is not None else None,
                                      _ptr(ws, torch.uint8, "ws", dev), ws.numel(), _stream(dev))
    _check(rc, "moe_debug_grouped_gemm")
    return (out, out2) if which == 0 else out


def vocab_topk_workspace_bytes(R: int, V: int, K: int) -> int:
    return lib().moe_vocab_topk_workspace_bytes(R, V, K)


def vocab_topk(logits: torch.Tensor, K: int, ws: Optional[torch.Tensor] = None, ids: Optional[torch.Tensor] = None,
               vals: Optional[torch.Tensor] = None, stage: int = -1):
    """moe_vocab_topk: exact top-K of each row of fp32 logits [R][V] by (value desc, index asc).
    Returns (ids [R][K] int32, vals [R][K] fp32). stage 0 / 1 runs one of its two kernels alone
    (moe_vocab_topk_stage, for timing)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [R][V]")
    R, V = logits.shape
    dev = logits.device
    n = vocab_topk_workspace_bytes(R, V, K)
    if n == 0:
        raise MoeError(MOE_EUNSUPPORTED, "moe_vocab_topk_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if ws is None else ws
    ids = torch.empty((R, K), dtype=torch.int32, device=dev) if ids is None else ids
    vals = torch.empty((R, K), dtype=torch.float32, device=dev) if vals is None else vals
    rc = lib().moe_vocab_topk_stage(stage, R, V, K, _ptr(logits, torch.float32, "logits", dev),
                                    _ptr(ids, torch.int32, "ids", dev), _ptr(vals, torch.float32, "vals", dev),
                                    _ptr(ws, torch.uint8, "ws", dev), ws.numel(), _stream(dev))
    _check(rc, "moe_vocab_topk" if stage < 0 else f"moe_vocab_topk_stage({stage})")
    return ids, vals
