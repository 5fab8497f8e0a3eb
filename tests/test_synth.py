"""The seeded input generator: definition, determinism, distributions."""
import numpy as np

import synth
from synth import configs


def test_splitmix64_reference_vector():
    # First five outputs of SplitMix64 seeded with 1234567, as printed by the
    # reference C implementation of the generator (Vigna, splitmix64.c).
    assert [int(v) for v in synth.draws(1234567, 0, 5)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_counter_based_random_access():
    key = synth.stream_key(3, synth.T_QUP, 7, 123)
    seq = synth.draws(key, 0, 1000)
    idx = np.array([0, 1, 17, 500, 999])
    assert np.array_equal(synth.draws_at(key, idx), seq[idx])
    assert np.array_equal(synth.draws(key, 400, 100), seq[400:500])


def test_streams_are_distinct():
    keys = {synth.stream_key(s, t, l, e) for s in (0, 1) for t in (1, 2, 3) for l in (0, 1, 47)
            for e in (0, 1, 511, synth.SHARED_EXPERT)}
    assert len(keys) == 2 * 3 * 3 * 4


def test_expert_arrays_deterministic_and_in_range():
    cfg = configs.TINY
    a = synth.expert_arrays(cfg, 0, 3)
    b = synth.expert_arrays(cfg, 0, 3)
    c = synth.expert_arrays(cfg, 0, 4)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["qg"], c["qg"])
    assert a["qg"].shape == (128, 256) and a["qd"].shape == (256, 128)
    assert a["sg"].shape == (128, 4) and a["sd"].shape == (256, 2)
    assert a["qg"].max() <= 15
    s = synth.bf16_bits_to_f32(a["sg"])
    b_ = synth.bf16_bits_to_f32(a["bd"])
    assert s.min() >= 0.0099 and s.max() <= 0.0501
    assert b_.min() >= -0.4005 and b_.max() <= 0.0


def test_distribution_moments():
    cfg = configs.DECODE_80B
    a = synth.expert_arrays(cfg, 1, 2)
    q = a["qg"].astype(np.float64)
    assert abs(q.mean() - 7.5) < 0.02 and abs(q.var() - 21.25) < 0.1
    s = synth.bf16_bits_to_f32(a["su"]).astype(np.float64)
    assert abs(s.mean() - 0.03) < 5e-4 and abs(s.var() - 0.04 ** 2 / 12) < 2e-5
    b = synth.bf16_bits_to_f32(a["bu"]).astype(np.float64)
    assert abs(b.mean() + 0.2) < 3e-3
    q8 = synth.expert_arrays(configs.BATCHED_80B_INT8, 0, 0)["qd"].astype(np.float64)
    assert q8.max() == 255 and abs(q8.mean() - 127.5) < 0.5
    w = synth.router_weight(cfg, 0).astype(np.float64)
    assert abs(w.mean()) < 1e-3 and abs(w.std() * np.sqrt(2048) - 1.0) < 0.01
    x = synth.activations(configs.DECODE_35B, variant=3)
    assert x.shape == (1, 2048) and abs(x.std() - 1.0) < 0.05
    # bf16 activations are exactly bf16 values
    assert np.all(x.view(np.uint32) & 0xFFFF == 0)


def test_zipf_router_bias():
    cfg = configs.BATCHED_80B
    b = synth.router_bias(cfg, 0).astype(np.float64)
    ranks = np.exp(-b / 1.1)
    assert np.allclose(np.sort(ranks), np.arange(1, 513), rtol=1e-5)
    assert synth.router_bias(configs.DECODE_80B, 0) is None


def test_slot_table_permutation():
    cfg = configs.DECODE_35B
    st = synth.slot_table(cfg, 2)
    assert np.array_equal(st, 2 * 256 + np.arange(256))
    sp = synth.slot_table(cfg, 2, permute_seed=9)
    assert sorted(sp.tolist()) == st.tolist() and not np.array_equal(sp, st)


def test_c_generator_matches_numpy_definition():
    import pytest
    if synth._host_lib() is None:
        pytest.skip("libsynth_host.so not built")
    for bits in (4, 8):
        key = synth.stream_key(5, synth.T_QDOWN, 3, 9)
        ref = synth.codes_from_draws(synth.draws(key, 0, 100003), bits)
        assert np.array_equal(synth.codes_c(key, 100003, bits), ref)
    key = synth.stream_key(1, synth.T_BUP, 0, 4)
    for lo, hi in ((synth.SCALE_LO, synth.SCALE_HI), (synth.BIAS_LO, synth.BIAS_HI)):
        ref = synth.uniform_bf16_from_draws(synth.draws(key, 0, 70001), lo, hi)
        assert np.array_equal(synth.uniform_bf16_c(key, 70001, lo, hi), ref)
