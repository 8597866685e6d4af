"""Move seeded workload inputs (numpy, from workload.gen) onto the GPU as the binding's types,
and compare GPU results with oracle results. Marshalling and comparison only."""
from typing import Optional

import numpy as np
import torch

from bit_moe_expert_amd import moe

DEV = torch.device("cuda:0")


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_of_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def proj_dev(p: dict) -> moe.QProj:
    return moe.QProj(torch.from_numpy(np.ascontiguousarray(p["codes"])).to(DEV), bf16_dev(p["scales"]),
                     bf16_dev(p["biases"]), p.get("bits", 4))


def ffn_dev(f: Optional[dict]) -> Optional[moe.QuantFFN]:
    if f is None:
        return None
    return moe.QuantFFN(proj_dev(f["gate"]), proj_dev(f["up"]), proj_dev(f["down"]))


def f32_dev(a: Optional[np.ndarray]) -> Optional[torch.Tensor]:
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def layer_dev(L: dict, k: int) -> moe.Layer:
    return moe.Layer(f32_dev(L["w_router"]), ffn_dev(L["routed"]), ffn_dev(L["shared"]), k, f32_dev(L["logit_bias"]))


def check_y(y_gpu: torch.Tensor, y_ref_bits: np.ndarray, what: str = "") -> float:
    """Per element |gpu - ref| <= 1e-2 * max|ref| + 1e-3 (max over this call's output).
    Returns the worst error as a fraction of the allowance."""
    g = f32_of_bits(bits_host(y_gpu)).astype(np.float64)
    r = f32_of_bits(y_ref_bits).astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    tol = 1e-2 * np.abs(r).max() + 1e-3
    err = np.abs(g - r)
    worst = float(err.max() / tol) if err.size else 0.0
    assert worst <= 1.0, f"{what}: max |gpu-ref| = {err.max():.4g} > tol {tol:.4g} at {np.unravel_index(err.argmax(), err.shape)}"
    return worst


def check_routing(r_gpu: dict, ref: dict, what: str = "") -> None:
    """Bit-exact ids, counts, offsets, scatter order, inv_pos and block map; gate weights to 1e-5."""
    h = {k: v.cpu().numpy() for k, v in r_gpu.items()}
    assert (h["topk_ids"] == ref["topk_ids"]).all(), f"{what}: topk_ids differ"
    assert np.abs(h["topk_w"] - ref["topk_w"]).max() <= 1e-5, f"{what}: topk_w off by {np.abs(h['topk_w'] - ref['topk_w']).max()}"
    assert (h["counts"] == ref["counts"]).all(), f"{what}: counts differ"
    assert (h["offsets"] == ref["offsets"]).all(), f"{what}: offsets differ"
    assert (h["sorted_token"] == ref["sorted_token"]).all(), f"{what}: sorted_token differs"
    assert (h["inv_pos"] == ref["inv_pos"]).all(), f"{what}: inv_pos differs"
    n = int(h["n_tiles"][0])
    assert n == ref["n_tiles"], f"{what}: n_tiles {n} vs {ref['n_tiles']}"
    assert (h["tiles"][:n] == ref["tiles"]).all(), f"{what}: tiles differ"
