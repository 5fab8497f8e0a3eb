"""Pins of the mixer oracle (oracle/mixer_oracle.py) to facts outside it.

Gated DeltaNet step: the delta rule's own identities (beta = 0 only decays the
state; with alpha = beta = 1 and a unit key e_j the state's column j becomes v;
for any inputs S' k = (1 - beta) alpha S k + beta v), unit norms, and scalar
brute force.  Gated GQA attention: equal keys give the mean of V, one dominant
key gives its V, a single position gives V_0, the group mapping, and scalar
brute force with math.fsum.  The last tests plant mistakes in the oracle (on
the CPU) and check that a pin catches each.
"""
import math

import numpy as np
import pytest

from oracle import mixer_oracle as mx


def _gdn_case(rng, B=2, Hk=2, Hv=4, dk=8, dv=6):
    S = rng.uniform(-0.5, 0.5, (B, Hv, dv, dk))
    q = rng.standard_normal((B, Hk, dk))
    k = rng.standard_normal((B, Hk, dk))
    v = rng.standard_normal((B, Hv, dv))
    g = rng.uniform(-1.0, -0.01, (B, Hv))
    beta = rng.uniform(0.05, 0.95, (B, Hv))
    return S, q, k, v, g, beta


# ---------------------------------------------------------------------------
# Gated DeltaNet


def test_l2norm_unit_and_scale_free(rng):
    x = rng.standard_normal((5, 16)) * 3
    n = mx.l2norm(x, 0.0)
    assert np.allclose(np.sum(n * n, -1), 1.0, rtol=1e-14)
    assert np.allclose(mx.l2norm(7.5 * x, 0.0), n, rtol=1e-14)
    # eps inside the square root
    assert mx.l2norm(np.array([[3.0, 4.0]]), 11.0)[0, 0] == 3.0 / 6.0


def test_gdn_zero_beta_only_decays(rng):
    S, q, k, v, g, beta = _gdn_case(rng)
    beta[:] = 0.0
    S2, o = mx.gdn_step(S, q, k, v, g, beta)
    alpha = np.exp(g)[:, :, None, None]
    assert np.allclose(S2, alpha * S, rtol=1e-15, atol=0)
    qn = mx.l2norm(q, 1e-6) / math.sqrt(S.shape[-1])
    rep = S.shape[1] // q.shape[1]
    for b in range(S.shape[0]):
        for h in range(S.shape[1]):
            assert np.allclose(o[b, h], alpha[b, h, 0, 0] * S[b, h] @ qn[b, h // rep], rtol=1e-13)


def test_gdn_unit_key_overwrites_one_column(rng):
    """alpha = 1, beta = 1, k = e_j: S' = S (I - e_j e_j^T) + v e_j^T, so column
    j of S' is v and every other column is unchanged (eps = 0 keeps k a unit
    vector exactly)."""
    S, q, k, v, g, beta = _gdn_case(rng, B=1, Hk=1, Hv=1)
    g[:] = 0.0
    beta[:] = 1.0
    j = 5
    k[:] = 0.0
    k[0, 0, j] = 2.5          # normalised to e_j
    S2, _ = mx.gdn_step(S, q, k, v, g, beta, eps=0.0)
    # S + (v - S) rounds: equal to v within one rounding of the O(1) values
    assert np.allclose(S2[0, 0][:, j], v[0, 0], rtol=0, atol=1e-15)
    others = [c for c in range(S.shape[-1]) if c != j]
    assert np.array_equal(S2[0, 0][:, others], S[0, 0][:, others])


def test_gdn_delta_identity(rng):
    """For any inputs, with k the normalised key (|k| = 1 when eps = 0):
    S' k = alpha S k + beta (v - alpha S k) = (1 - beta) alpha S k + beta v."""
    S, q, k, v, g, beta = _gdn_case(rng)
    S2, _ = mx.gdn_step(S, q, k, v, g, beta, eps=0.0)
    kn = mx.l2norm(k, 0.0)
    rep = S.shape[1] // k.shape[1]
    for b in range(S.shape[0]):
        for h in range(S.shape[1]):
            kh = kn[b, h // rep]
            a = math.exp(g[b, h])
            ref = (1 - beta[b, h]) * a * (S[b, h] @ kh) + beta[b, h] * v[b, h]
            assert np.allclose(S2[b, h] @ kh, ref, rtol=1e-12, atol=1e-13)


def test_gdn_bruteforce(rng):
    """Scalar loops over every element, including the head mapping (value
    head h reads key/query head h // 2)."""
    S, q, k, v, g, beta = _gdn_case(rng, B=1, Hk=2, Hv=4, dk=4, dv=3)
    S2, o = mx.gdn_step(S, q, k, v, g, beta, eps=1e-6)
    dk, dv = 4, 3
    for h in range(4):
        kh, qh = k[0, h // 2], q[0, h // 2]
        nk = math.sqrt(math.fsum(x * x for x in kh) + 1e-6)
        nq = math.sqrt(math.fsum(x * x for x in qh) + 1e-6)
        kk = [x / nk for x in kh]
        qq = [x / nq / math.sqrt(dk) for x in qh]
        a = math.exp(g[0, h])
        for i in range(dv):
            sk = math.fsum(S[0, h, i, j] * kk[j] for j in range(dk))
            u = v[0, h, i] - a * sk
            row = [a * S[0, h, i, j] + beta[0, h] * u * kk[j] for j in range(dk)]
            for j in range(dk):
                assert abs(S2[0, h, i, j] - row[j]) <= 1e-14
            assert abs(o[0, h, i] - math.fsum(row[j] * qq[j] for j in range(dk))) <= 1e-14


# ---------------------------------------------------------------------------
# gated GQA attention


def _att_case(rng, B=2, Hq=4, Hkv=2, D=8, n=7):
    q = rng.standard_normal((B, Hq, D))
    gate = rng.standard_normal((B, Hq, D))
    K = rng.uniform(-2, 2, (B, Hkv, n, D))
    V = rng.uniform(-2, 2, (B, Hkv, n, D))
    return q, gate, K, V


def test_attn_equal_keys_give_mean_value(rng):
    q, gate, K, V = _att_case(rng)
    K[:] = K[:, :, :1, :]
    out = mx.attn_decode(q, gate, lambda b, h, n: (K[b, h, :n], V[b, h, :n]), [7, 5], 2)
    for b, n in ((0, 7), (1, 5)):
        for h in range(4):
            ref = V[b, h // 2, :n].mean(0) * mx.sigmoid(gate[b, h])
            assert np.allclose(out[b, h], ref, rtol=1e-13, atol=1e-14)


def test_attn_dominant_key_and_single_position(rng):
    q, gate, K, V = _att_case(rng, B=1, Hq=2, Hkv=1, n=6)
    K[0, 0, 3] = 400.0 * q[0, 0] / np.linalg.norm(q[0, 0])   # score far above the rest
    out = mx.attn_decode(q, gate, lambda b, h, n: (K[b, h, :n], V[b, h, :n]), [6], 1)
    assert np.allclose(out[0, 0], V[0, 0, 3] * mx.sigmoid(gate[0, 0]), rtol=1e-12)
    one = mx.attn_decode(q, gate, lambda b, h, n: (K[b, h, :n], V[b, h, :n]), [1], 1)
    for h in range(2):
        assert np.allclose(one[0, h], V[0, 0, 0] * mx.sigmoid(gate[0, h]), rtol=1e-15)


def test_attn_bruteforce(rng):
    q, gate, K, V = _att_case(rng, B=1, Hq=4, Hkv=2, D=5, n=4)
    out = mx.attn_decode(q, gate, lambda b, h, n: (K[b, h, :n], V[b, h, :n]), [4], 2)
    D = 5
    for h in range(4):
        kv = h // 2
        s = [math.fsum(q[0, h, d] * K[0, kv, j, d] for d in range(D)) / math.sqrt(D)
             for j in range(4)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = math.fsum(e)
        for d in range(D):
            o = math.fsum(e[j] / z * V[0, kv, j, d] for j in range(4))
            ref = o / (1.0 + math.exp(-gate[0, h, d]))
            assert abs(out[0, h, d] - ref) <= 1e-14 * max(1.0, abs(ref))


# ---------------------------------------------------------------------------
# planted mistakes


def _head_step_no_decay_in_delta(S, q, k, v, g, beta):
    S = np.asarray(S, np.float64)
    alpha = np.exp(g)
    u = np.asarray(v) - S @ np.asarray(k)                   # wrong: S k not decayed
    S2 = alpha * S + beta * np.outer(u, k)
    return S2, S2 @ q


def _head_step_wrong_sign(S, q, k, v, g, beta):
    S = np.asarray(S, np.float64)
    alpha = np.exp(g)
    u = np.asarray(v) + alpha * (S @ np.asarray(k))         # wrong sign
    S2 = alpha * S + beta * np.outer(u, k)
    return S2, S2 @ q


def _attn_head_no_scale(q, K, V, gate, scale):
    return mx.softmax(np.asarray(K) @ np.asarray(q)) @ np.asarray(V) * mx.sigmoid(gate)


@pytest.mark.parametrize("name,bad,pin", [
    ("gdn_head_step", _head_step_no_decay_in_delta, test_gdn_delta_identity),
    ("gdn_head_step", _head_step_wrong_sign, test_gdn_unit_key_overwrites_one_column),
    ("attn_head", _attn_head_no_scale, test_attn_bruteforce),
])
def test_planted_mistake_is_caught(monkeypatch, rng, name, bad, pin):
    monkeypatch.setattr(mx, name, bad)
    import inspect
    args = [rng] if "rng" in inspect.signature(pin).parameters else []
    with pytest.raises(AssertionError):
        pin(*args)


def test_planted_group_mapping_is_caught(monkeypatch, rng):
    """Query head h reading kv head h % n_kv_heads instead of h // group."""
    def bad_decode(q, gate, get_kv, lengths, n_kv_heads, scale=None):
        q = np.asarray(q, np.float64)
        B, Hq, D = q.shape
        scale = 1.0 / np.sqrt(D) if scale is None else scale
        out = np.empty((B, Hq, D))
        for b in range(B):
            for h in range(Hq):
                K, V = get_kv(b, h % n_kv_heads, int(lengths[b]))
                out[b, h] = mx.attn_head(q[b, h], K, V, gate[b, h], scale)
        return out
    monkeypatch.setattr(mx, "attn_decode", bad_decode)
    with pytest.raises(AssertionError):
        test_attn_bruteforce(rng)
