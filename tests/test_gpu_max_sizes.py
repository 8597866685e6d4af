"""GPU parity at the largest sizes the C ABI accepts, one dimension at a time: d_model 16384,
d_ff and d_ff_shared 8192, the largest top-k of the single-token path, and T = 65536 tokens (with
1024 experts at top-16, so P = T k = 1,048,576 routed rows).

Bar as in test_gpu_parity: bit-exact routing, outputs within 1e-2 * max|ref| + 1e-3. Calls of
65536 tokens compare the whole routing and the outputs of sampled tokens (the oracle computes
them one by one), since the oracle's whole layer at that size takes minutes.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from workload import gen
from bit_moe_expert_amd import moe
from gpu_inputs import DEV, bf16_dev, check_routing, check_y, f32_dev, layer_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need the MI355X"
    yield
    torch.cuda.synchronize()


def _w(T, d, E, k, I, Is, bits=4, seed=0):
    return gen.Workload("custom", T, d, E, k, I, Is, 0.05, 1, T, seed=seed, bits=bits)


def _layer_check(w, sel=None):
    L = gen.layer(w, 0)
    x = gen.tokens(w, 0, 0)
    lay = layer_dev(L, w.k)
    y = lay.forward(bf16_dev(x))
    torch.cuda.synchronize()
    what = f"T={w.T} d={w.d} E={w.E} k={w.k} I={w.I} Is={w.Is} bits={w.bits}"
    if sel is None:
        ref = oracle.forward_layer(x, L["w_router"], L["routed"], L["shared"], w.k, L["logit_bias"])
        return check_y(y, ref["y"], what)
    ref = oracle.forward_tokens(x, L["w_router"], L["routed"], L["shared"], w.k, sel, L["logit_bias"])
    return check_y(y[torch.as_tensor(sel, device=DEV)], ref["y"], what + " sampled")


# d_model 16384: the router reduces over 8 passes of 2048 inputs, the gate/up GEMM over 128 steps,
# the down GEMM writes 128 column blocks; 1-3 tokens take the single-token path, 40 the GEMM.
@pytest.mark.parametrize("T,bits", [(1, 4), (3, 4), (40, 4), (40, 3), (33, 2), (2, 3)])
def test_max_d_model(T, bits):
    _layer_check(_w(T, 16384, 8, 2, 128, 64, bits=bits, seed=T + bits))


# d_ff and d_ff_shared 8192: the down GEMM reduces over 128 groups; one token with an h this long
# runs the grouped GEMM (its h does not fit the single-token down kernel).
@pytest.mark.parametrize("T,bits", [(40, 4), (1, 4), (65, 3), (40, 2)])
def test_max_d_ff(T, bits):
    _layer_check(_w(T, 128, 4, 2, 8192, 8192, bits=bits, seed=T + bits))


# the largest h the single-token path keeps in LDS: top-16 of 1024-wide experts plus a 1024-wide
# shared expert
@pytest.mark.parametrize("T", [1, 32])
def test_largest_single_token_h(T):
    _layer_check(_w(T, 256, 64, 16, 1024, 1024, seed=T))


# T = 65536: the whole routing bit-exact, sampled outputs
@pytest.mark.parametrize("d,E,k,I,Is", [(64, 1024, 16, 64, 0), (128, 64, 8, 64, 64)])
def test_max_tokens(d, E, k, I, Is):
    w = _w(65536, d, E, k, I, Is, seed=E + k)
    x = gen.tokens(w, 0, 0)
    wr = gen.router(w, 0)
    bias = gen.logit_bias(w)
    r = moe.route(bf16_dev(x), f32_dev(wr), k, I, Is, f32_dev(bias))
    logits = oracle.router_logits(x, wr, bias)
    ids, tw = oracle.topk_softmax(logits, k)
    ref = oracle.route_meta(ids, E, Is > 0)
    ref.update(topk_ids=ids, topk_w=tw)
    check_routing(r, ref, f"T=65536 E={E} k={k}")
    del r
    rng = np.random.default_rng(E)
    sel = np.sort(np.concatenate([[0, 65535], rng.choice(np.arange(1, 65535), 62, replace=False)]))
    _layer_check(w, sel)
