"""GPU: calls on two streams at once. The library keeps no state between calls apart from the fixed
scratch of the allocation-free entry point (not used here), so calls on different streams with
different workspaces may run concurrently: each output must equal, bit for bit, the same call
made alone. The calls mix the single-token path and the grouped GEMM, and two layers of
different shapes, so kernels of both streams overlap on the GPU.
"""
import pytest
import torch

from workload import gen
from gpu_inputs import bf16_dev, layer_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need the MI355X"
    yield
    torch.cuda.synchronize()


def test_two_streams_match_calls_made_alone():
    shapes = [(1, 512, 64, 8, 256, 256), (200, 512, 32, 4, 256, 128), (24, 256, 16, 4, 128, 0), (130, 320, 8, 2, 192, 64)]
    cases = []
    for i, (T, d, E, k, I, Is) in enumerate(shapes):
        w = gen.Workload("custom", T, d, E, k, I, Is, 0.05, 1, T, seed=100 + i)
        lay = layer_dev(gen.layer(w, 0), k)
        xs = [bf16_dev(gen.tokens(w, 0, c)) for c in range(2)]
        cases.append((lay, xs, T))
    # alone: one call at a time on the default stream
    alone = []
    for lay, xs, T in cases:
        for x in xs:
            alone.append(lay.forward(x).clone())
            torch.cuda.synchronize()
    # together: the calls alternate between two streams, each with its own workspaces and outputs
    dev = alone[0].device
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    ws = [[lay.workspace(T) for _ in streams] for lay, _, T in cases]
    outs = [torch.empty_like(a) for a in alone]
    torch.cuda.synchronize()
    for rep in range(3):
        n = 0
        for ci, (lay, xs, T) in enumerate(cases):
            for xi, x in enumerate(xs):
                si = (n + rep) % 2
                with torch.cuda.stream(streams[si]):
                    lay.forward(x, ws[ci][si], outs[n])
                n += 1
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, alone)):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"call {i} differs (repetition {rep})"
            got.fill_(0)
        torch.cuda.synchronize()
