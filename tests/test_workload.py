"""The seeded input generator: published SplitMix64 outputs, counter-based sub-ranges,
determinism and the value distributions the workloads state (CPU only)."""
import numpy as np

from oracle import oracle
from workload import gen


def test_splitmix64_published_sequence():
    # SplitMix64 started from state 0 (Steele, Lea, Flood 2014; the reference C of Vigna's
    # splitmix64.c) gives these first three outputs.
    got = [gen.lib().gen_word(0, n) for n in range(3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_subranges_and_determinism():
    k = gen.key(0, 3, gen.T_GATE_CODES)
    full = gen.rand_bytes(k, 4099)
    for s in (0, 1, 7, 8, 13, 4000):
        assert (gen.rand_bytes(k, 4099 - s, start=s) == full[s:]).all()
    assert (gen.rand_bytes(k, 4099) == full).all()
    assert not (gen.rand_bytes(gen.key(0, 4, gen.T_GATE_CODES), 4099) == full).all()
    n = gen.normal_bf16(k, 1000, 1.0)
    assert (gen.normal_bf16(k, 990, 1.0, start=10) == n[10:]).all()
    s, b = gen.scale_bias(k, 500)
    s2, b2 = gen.scale_bias(k, 400, start=100)
    assert (s2 == s[100:]).all() and (b2 == b[100:]).all()


def test_distributions():
    k = gen.key(0, 0, gen.T_X)
    x = oracle.bf16_to_f32(gen.normal_bf16(k, 200000, 1.0))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    w = gen.normal_f32(k, 200000, 0.02)
    assert abs(w.std() - 0.02) < 0.0003
    s, b = gen.scale_bias(k, 100000)
    sf, bf = oracle.bf16_to_f32(s), oracle.bf16_to_f32(b)
    assert (sf >= 0).all() and (bf == -8 * sf).all()
    assert abs(sf.mean() - 0.02 * np.sqrt(2 / np.pi)) < 0.0003
    codes = gen.rand_bytes(k, 200000)
    q = np.concatenate([codes & 15, codes >> 4])
    cnt = np.bincount(q, minlength=16)
    assert cnt.min() > 0.95 * q.size / 16 and cnt.max() < 1.05 * q.size / 16


def test_zipf_bias_and_workload_shapes():
    b = gen.zipf_bias(256)
    assert b[0] == 0.0 and abs(b[9] - 1.5 * np.log(1 / 10)) < 1e-6 and (np.diff(b) < 0).all()
    w = gen.WORKLOADS["tiny"]
    L = gen.layer(w, 0)
    assert L["w_router"].shape == (256, 16) and L["logit_bias"] is None
    assert L["routed"]["gate"]["codes"].shape == (16, 128, 128)
    assert L["routed"]["down"]["scales"].shape == (16, 256, 2)
    assert L["shared"]["up"]["biases"].shape == (1, 128, 4)
    assert gen.WORKLOADS["diffusion"].Is == 0 and gen.WORKLOADS["long"].calls == 4
    p = gen.permutation(gen.key(0, 0, gen.T_PERM), 256)
    assert sorted(p.tolist()) == list(range(256))
