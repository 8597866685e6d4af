"""moe_forward_layer_noalloc (the layer with the library's fixed device scratch instead of a caller
workspace) against moe_forward_layer on the same inputs: two calls in a row, the second smaller,
each bit-identical to the workspace entry point (same kernels, deterministic); sizes past the
fixed scratch are refused before any launch."""
import pytest
import torch

from oracle import oracle
from workload import gen
from gpu_inputs import bf16_dev, check_y, layer_dev

pytestmark = pytest.mark.gpu


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


# a call of more than 32768 token-expert pairs (4097 x top-8) routes through the sliced metadata,
# whose per-slice histograms then live in the fixed scratch too; its second call takes the single
# launch
SLICED = gen.Workload("sliced", 4097, 128, 64, 8, 64, 64, 0.05, 1, 4097, seed=7)


@pytest.mark.parametrize("name,T2", [("prefill", 64), ("decode", 1), ("sliced", 64)])
def test_noalloc_matches_workspace_entry_point(name, T2):
    torch.cuda.synchronize()
    w = SLICED if name == "sliced" else gen.WORKLOADS[name]
    L = gen.layer(w, 0)
    lay = layer_dev(L, w.k)
    x1 = gen.tokens(w, 0, 0)
    # first call: the workload's own size; second call: fewer tokens (a prefix of other tokens)
    x2 = gen.tokens(w, 0, 1, T=max(T2, 1))
    for x in (x1, x2):
        xd = bf16_dev(x)
        y_ref = lay.forward(xd)
        y = torch.full_like(xd, float("nan"))
        lay.forward_noalloc(xd, y)
        torch.cuda.synchronize()
        assert _same(y, y_ref), f"{name}: T = {x.shape[0]} differs from moe_forward_layer"
    # and the oracle's bar on the smaller call
    ref = oracle.forward_layer(x2, L["w_router"], L["routed"], L["shared"], w.k, L["logit_bias"])
    check_y(y, ref["y"], f"{name} noalloc T={x2.shape[0]}")
