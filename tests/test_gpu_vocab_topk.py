"""GPU parity of the exact top-K of logit rows (moe_vocab_topk) against the oracle's full sort.

Bar: ids and values bit-exact (the selection is exact and copies the input values).
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from workload import gen
from bit_moe_expert_amd import moe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check(x: np.ndarray, K: int, what: str, rows=None):
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    ids, vals = moe.vocab_topk(xt, K)
    torch.cuda.synchronize()
    ids, vals = ids.cpu().numpy(), vals.cpu().numpy()
    sel = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    want_i, want_v = oracle.vocab_topk(x[sel], K)
    bad = np.nonzero((ids[sel] != want_i).any(axis=1))[0]
    assert bad.size == 0, f"{what}: ids differ in rows {sel[bad][:5]} (first: {ids[sel][bad[0]][:8]} vs {want_i[bad[0]][:8]})"
    assert (vals[sel].view(np.uint32) == want_v.view(np.uint32)).all(), f"{what}: values differ"


def test_vocab_topk_tiny_workload():
    w = gen.VOCAB_WORKLOADS["vocab_tiny"]
    _check(gen.vocab_logits(w), w.K, "vocab_tiny")


@pytest.mark.parametrize("R,V,K", [(3, 4096, 64), (2, 5000, 64), (2, 1000, 1), (2, 7, 7), (4, 3001, 16),
                                   (2, 70000, 128), (2, 262143, 33), (1, 511, 64), (3, 100000, 32)])
def test_vocab_topk_shapes(R, V, K):
    """Several chunks, all chunks (V/C <= K), K = 1, K = V, ragged rows (V % 4 != 0 uses scalar
    loads), the largest K, a chunk size boundary (K = 32 | 33)."""
    rng = np.random.default_rng(R * 7919 + V + K)
    x = (rng.normal(size=(R, V)) * 3).astype(np.float32)
    _check(x, K, f"R={R} V={V} K={K}")


def test_vocab_topk_ties_and_clusters():
    rng = np.random.default_rng(5)
    V = 20000
    rows = []
    rows.append(np.zeros(V, np.float32))                                         # everything tied
    rows.append(rng.integers(-3, 4, V).astype(np.float32))                       # few distinct values
    r = (rng.normal(size=V) - 20).astype(np.float32)
    r[3000:3070] = 10 + rng.random(70).astype(np.float32)                        # the whole top-64 in one chunk
    rows.append(r)
    r = np.zeros(V, np.float32)
    r[::512] = 1.0                                                               # equal maxima in every chunk
    rows.append(r)
    r = np.repeat(rng.integers(0, 5, V // 300 + 1), 300)[:V].astype(np.float32)  # tied runs across chunk edges
    rows.append(r)
    r = rng.normal(size=V).astype(np.float32)
    r[r > 2.0] = 2.0                                                             # a plateau at the top
    rows.append(r)
    r = np.full(V, -0.0, np.float32)
    r[1::2] = 0.0                                                                # -0 and +0 alternate
    rows.append(r)
    x = np.stack(rows)
    for K in (1, 17, 64, 128):
        _check(x, K, f"ties K={K}")


def test_vocab_topk_full_size_sampled_rows():
    """The pages' size: 256 positions over 262,144 logits, top-64; 24 rows checked one by one."""
    w = gen.VOCAB_WORKLOADS["vocab"]
    x = gen.vocab_logits(w, 0)
    rows = np.random.default_rng(0).choice(w.R, 24, replace=False)
    _check(x, w.K, "vocab full size", rows=rows)


def test_vocab_topk_zero_rows_and_repeat():
    x = torch.zeros((0, 1000), dtype=torch.float32, device=DEV)
    ids, vals = moe.vocab_topk(x, 8)
    assert ids.shape == (0, 8)
    rng = np.random.default_rng(9)
    xt = torch.from_numpy((rng.normal(size=(8, 50000))).astype(np.float32)).to(DEV)
    a = moe.vocab_topk(xt, 64)
    b = moe.vocab_topk(xt, 64)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_vocab_topk_full_width_ties_take_the_general_path():
    """Rows of the pages' width whose maximum is shared by every chunk (zeros; four values): more
    than 128 chunks reach the K-th largest chunk maximum, so the three-level path runs."""
    rng = np.random.default_rng(21)
    V = 262144
    x = np.stack([np.zeros(V, np.float32), rng.integers(0, 4, V).astype(np.float32),
                  np.repeat(rng.integers(0, 3, V // 1000 + 1), 1000)[:V].astype(np.float32)])
    for K in (64, 128):
        _check(x, K, f"full-width ties K={K}")
