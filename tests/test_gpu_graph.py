"""GPU: the layer captured in a HIP graph (torch.cuda.graph) and replayed.

Each replay must reproduce, bit for bit, an eager call on the same input: the path is
deterministic (the same kernels in the same order, no atomics whose order reaches a result).
Between replays the test rewrites the captured input and runs eager calls of its own on other
inputs and buffers, so a replay that depended on state an earlier call left behind (in the
workspace, or in the fixed device scratch of the allocation-free entry point) would differ.
The eager results are tied to the oracle first. Cases: the single-token path (T <= 32), the
grouped GEMM with and without a shared expert and with 3-bit codes, the routing metadata in
slices (T*k above 32768), and the allocation-free entry point.
"""
import pytest
import torch

from oracle import oracle
from workload import gen
from gpu_inputs import bf16_dev, check_y, layer_dev

pytestmark = pytest.mark.gpu

# (id, T, d, E, k, I, Is, code bits, allocation-free entry point)
CASES = [
    ("single-token T=1", 1, 512, 64, 8, 256, 256, 4, False),
    ("single-token T=20", 20, 256, 16, 4, 128, 128, 4, False),
    ("grouped T=200", 200, 512, 32, 4, 256, 128, 4, False),
    ("grouped T=130 no shared 3-bit", 130, 320, 8, 2, 192, 0, 3, False),
    ("sliced metadata T=4200 k=8", 4200, 128, 64, 8, 64, 64, 4, False),
    ("allocation-free T=96", 96, 256, 16, 4, 128, 128, 4, True),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need the MI355X"
    yield
    torch.cuda.synchronize()


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(case):
    _, T, d, E, k, I, Is, bits, noalloc = case
    w = gen.Workload("custom", T, d, E, k, I, Is, 0.05, 1, T, seed=T + E + bits, bits=bits)
    L = gen.layer(w, 0)
    lay = layer_dev(L, k)
    xs_host = [gen.tokens(w, 0, c) for c in range(3)]
    xs = [bf16_dev(a) for a in xs_host]

    def call(x, ws, y):
        return lay.forward_noalloc(x, y) if noalloc else lay.forward(x, ws, y)

    # eager results on the three inputs, the first checked against the oracle
    ws_e = None if noalloc else lay.workspace(T)
    eager = [call(x, ws_e, torch.empty_like(x)).clone() for x in xs]
    torch.cuda.synchronize()
    ref = oracle.forward_layer(xs_host[0], L["w_router"], L["routed"], L["shared"], k, L["logit_bias"])
    check_y(eager[0], ref["y"], f"eager T={T}")

    # capture one call on static buffers (warmed once on the capture stream)
    x_g = xs[0].clone()
    y_g = torch.empty_like(x_g)
    ws_g = None if noalloc else lay.workspace(T)
    dev = x_g.device
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        call(x_g, ws_g, y_g)
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(x_g, ws_g, y_g)
    torch.cuda.synchronize()

    y_other = torch.empty_like(x_g)
    for rep, c in enumerate([0, 1, 2, 1, 0]):
        x_g.copy_(xs[c])
        y_g.fill_(0)
        # eager work of the program's own between replays, on another input
        call(xs[(c + 1) % 3], ws_e, y_other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y_g), _bits(eager[c])), f"replay {rep} (input {c}) differs from the eager call"
        assert torch.equal(_bits(y_other), _bits(eager[(c + 1) % 3])), f"eager call after replay {rep} changed"
    del g
