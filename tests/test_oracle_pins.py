"""Pins of the fp64 oracle to facts outside the oracle itself.

The pages print no worked example of the layer, so each oracle function is
pinned by brute force on tiny inputs (plain Python loops over scalars), closed
forms, exact special cases or invariants.  Every pin runs against both
implementations of the oracle: the numpy module and the C++ library
(``oracle/moe_oracle.cpp``).  The last tests plant a mistake in each oracle
(on the CPU; a separate build of the C++ file for its planted copies) and
check that some pin catches it.
"""
import itertools
import math
import struct

import numpy as np
import pytest

import oracle
from oracle import moe_oracle as mo


@pytest.fixture(params=["numpy", "cpp"])
def O(request):
    """The oracle implementation under test: the numpy module or the C++
    library behind the same API.  Every pin runs against both."""
    if request.param == "numpy":
        return mo
    from oracle import cpp
    return cpp.default()

# ---------------------------------------------------------------------------
# independent scalar helpers (struct / math based; no numpy vectorisation)


def bf16_struct(bits: int) -> float:
    return struct.unpack(">f", struct.pack(">I", (int(bits) & 0xFFFF) << 16))[0]


def f32_bits(v: float) -> int:
    return struct.unpack(">I", struct.pack(">f", v))[0]


def bf16_bits_of_value(v: float) -> int:
    """bf16 bit pattern of a value known to be exactly representable."""
    b = f32_bits(v)
    assert b & 0xFFFF == 0
    return b >> 16


def nearest_bf16_bruteforce(v: float) -> float:
    """Nearest bf16 to a float that is exactly an fp32, ties to even, by
    comparing the two neighbouring bf16 patterns."""
    b = f32_bits(v)
    lo = b & 0xFFFF0000
    hi = lo + 0x10000
    flo = struct.unpack(">f", struct.pack(">I", lo))[0]
    fhi = struct.unpack(">f", struct.pack(">I", hi))[0]
    dlo, dhi = abs(v - flo), abs(fhi - v)
    if dlo < dhi:
        return flo
    if dhi < dlo:
        return fhi
    return flo if ((lo >> 16) & 1) == 0 else fhi


def silu_scalar(g: float) -> float:
    if g < -700:
        return 0.0
    return g / (1.0 + math.exp(-g))


def ffn_bruteforce(x, a, group):
    """SwiGLU expert by scalar loops over the logical arrays."""
    I, H = a["qg"].shape

    def w(q, s, b, r, c):
        return bf16_struct(s[r][c // group]) * float(q[r][c]) + bf16_struct(b[r][c // group])

    ys = []
    for xt in x:
        h = []
        for r in range(I):
            g = sum(w(a["qg"], a["sg"], a["bg"], r, c) * float(xt[c]) for c in range(H))
            u = sum(w(a["qu"], a["su"], a["bu"], r, c) * float(xt[c]) for c in range(H))
            h.append(silu_scalar(g) * u)
        y = [sum(w(a["qd"], a["sd"], a["bd"], r, c) * h[c] for c in range(I)) for r in range(H)]
        ys.append(y)
    return np.array(ys)


def rand_bf16_bits(rng, shape, lo, hi):
    v = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return np.vectorize(lambda z: f32_bits(float(z)) >> 16)(v).astype(np.uint16)


def rand_expert(rng, H, I, bits=4, group=64):
    nq = 1 << bits
    return {
        "qg": rng.integers(0, nq, (I, H)).astype(np.uint8),
        "qu": rng.integers(0, nq, (I, H)).astype(np.uint8),
        "qd": rng.integers(0, nq, (H, I)).astype(np.uint8),
        "sg": rand_bf16_bits(rng, (I, H // group), 0.01, 0.05),
        "bg": rand_bf16_bits(rng, (I, H // group), -0.4, 0.0),
        "su": rand_bf16_bits(rng, (I, H // group), 0.01, 0.05),
        "bu": rand_bf16_bits(rng, (I, H // group), -0.4, 0.0),
        "sd": rand_bf16_bits(rng, (H, I // group), 0.01, 0.05),
        "bd": rand_bf16_bits(rng, (H, I // group), -0.4, 0.0),
    }


# ---------------------------------------------------------------------------
# number formats


def test_bf16_widening_all_patterns(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(bits)
    for b in range(0, 65536, 1):
        ref = bf16_struct(b)
        g = got[b]
        if math.isnan(ref):
            assert math.isnan(g)
        else:
            assert g == ref, hex(b)


def test_round_to_bf16_ties_and_neighbours(O, rng):
    # exact ties at 1.0: spacing 2**-7
    assert O.round_to_bf16(1 + 2 ** -8) == 1.0
    assert O.round_to_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert O.round_to_bf16(-(1 + 2 ** -8)) == -1.0
    assert O.round_to_bf16(0.0) == 0.0
    assert O.round_to_bf16(255.5) == 256.0      # 255.5 is a tie between 255 and 256
    vals = rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 8, 20000)
    got = O.round_to_bf16(vals.astype(np.float64))
    for v, g in zip(vals[:4000], got[:4000]):
        assert g == nearest_bf16_bruteforce(float(v))
    # every result is a bf16 value
    assert np.all(got.astype(np.float32).view(np.uint32) & 0xFFFF == 0)


# ---------------------------------------------------------------------------
# dequantisation  (w = scale * q + bias per group of 64 along the input axis)


def test_dequantize_bruteforce(O, rng):
    for bits in (4, 8):
        q = rng.integers(0, 1 << bits, (3, 192)).astype(np.uint8)
        s = rand_bf16_bits(rng, (3, 3), 0.01, 0.05)
        b = rand_bf16_bits(rng, (3, 3), -0.4, 0.0)
        W = O.dequantize(q, s, b, 64)
        for r in range(3):
            for c in range(192):
                ref = bf16_struct(s[r][c // 64]) * int(q[r][c]) + bf16_struct(b[r][c // 64])
                assert W[r, c] == ref          # exact: 8-bit x 8-bit products in fp64


@pytest.mark.parametrize("bits", [4, 8])
def test_dequantize_every_code(O, bits):
    from fractions import Fraction
    codes = np.arange(1 << bits, dtype=np.uint8)[None, :]
    cols = codes.shape[1]
    pad = (-cols) % 64
    q = np.concatenate([codes, np.zeros((1, pad), np.uint8)], axis=1)
    G = q.shape[1] // 64
    s = np.full((1, G), bf16_bits_of_value(0.03125), np.uint16)
    b = np.full((1, G), bf16_bits_of_value(-0.25), np.uint16)
    W = O.dequantize(q, s, b, 64)
    for c in range(1 << bits):
        assert Fraction(W[0, c]) == Fraction(c, 32) - Fraction(1, 4)


def test_dequantize_group_and_row_indexing(O):
    rows, cols = 3, 256
    q = np.ones((rows, cols), np.uint8)
    s = np.zeros((rows, cols // 64), np.uint16)
    for r in range(rows):
        for g in range(cols // 64):
            s[r, g] = bf16_bits_of_value(2.0 ** (r + 4 * g))
    b = np.zeros_like(s)
    W = O.dequantize(q, s, b, 64)
    for r in range(rows):
        for c in range(cols):
            assert W[r, c] == 2.0 ** (r + 4 * (c // 64))


# ---------------------------------------------------------------------------
# router, softmax, top-k, renormalisation


def test_router_logits_one_hot(O, rng):
    E, H = 16, 256
    Wr = rng.standard_normal((E, H)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    for c in (0, 7, 255):
        x = np.zeros((1, H))
        x[0, c] = 1.0
        l = O.router_logits(x, Wr)
        assert np.array_equal(l[0], Wr[:, c].astype(np.float64))
        lb = O.router_logits(x, Wr, bias)
        assert np.array_equal(lb[0], Wr[:, c].astype(np.float64) + bias.astype(np.float64))


def test_router_logits_bruteforce(O, rng):
    E, H = 5, 64
    Wr = rng.standard_normal((E, H)).astype(np.float32)
    x = rng.standard_normal((2, H))
    l = O.router_logits(x, Wr)
    for t in range(2):
        for e in range(E):
            ref = math.fsum(float(Wr[e, c]) * float(x[t, c]) for c in range(H))
            assert abs(l[t, e] - ref) <= 1e-12 * (1 + abs(ref))


def test_dense_q4_router_bruteforce(O, rng):
    """The 4-bit dense path: logits from router rows given as int4 codes with
    bf16 (scale, bias) per group of 64 equal a scalar loop over the codes
    (w = s q + b, then the dot product), and the shared gate reads row E."""
    E, H, G = 3, 128, 2
    q = rng.integers(0, 16, (E + 1, H)).astype(np.uint8)
    s = mo.round_to_bf16(rng.uniform(0.001, 0.01, (E + 1, G)))
    b = mo.round_to_bf16(rng.uniform(-0.08, 0.0, (E + 1, G)))
    bits = lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    rows = O.dequantize(q, bits(s), bits(b), 64)
    x = rng.standard_normal((2, H))
    l = O.router_logits(x, rows[:E])
    gam = O.shared_gate(x, rows[E])
    for t in range(2):
        for e in range(E + 1):
            ref = math.fsum((float(s[e, c // 64]) * int(q[e, c]) + float(b[e, c // 64])) * float(x[t, c])
                            for c in range(H))
            if e < E:
                assert abs(l[t, e] - ref) <= 1e-12 * (1 + abs(ref))
            else:
                assert abs(gam[t] - 1.0 / (1.0 + math.exp(-ref))) <= 1e-12


def test_topk_matches_best_subset(O, rng):
    for trial in range(40):
        E = int(rng.integers(3, 13))
        k = int(rng.integers(1, E + 1))
        l = rng.standard_normal(E)
        sel, gap = O.topk(l, k)
        best = max(itertools.combinations(range(E), k), key=lambda S: math.fsum(l[i] for i in S))
        assert set(sel.tolist()) == set(best)
        # ordered by logit, descending
        assert all(l[sel[i]] > l[sel[i + 1]] for i in range(k - 1))
        srt = sorted(l.tolist(), reverse=True)
        assert gap == (math.inf if k == E else srt[k - 1] - srt[k])


def test_topk_ties_to_lower_index(O):
    sel, gap = O.topk(np.zeros(16), 4)
    assert sel.tolist() == [0, 1, 2, 3] and gap == 0.0
    sel, _ = O.topk(np.array([1.0, 2.0, 2.0, 0.0]), 1)
    assert sel.tolist() == [1]
    sel, _ = O.topk(np.array([1.0, 2.0, 2.0, 0.0]), 2)
    assert sel.tolist() == [1, 2]
    sel, _ = O.topk(np.array([3.0, 1.0, 3.0, 1.0, 1.0]), 3)
    assert sel.tolist() == [0, 2, 1]


def test_all_zero_router_gives_uniform_weights(O):
    E, H, k = 16, 64, 4
    l, idx, w, gap = O.route(np.ones((3, H)), np.zeros((E, H)), None, k)
    assert idx.tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(w == 0.25)


def test_renormalised_weights_closed_forms(O, rng):
    # k = 2: w_0 is the logistic function of the logit gap
    for _ in range(50):
        l = rng.standard_normal(9) * 3
        _, idx, w, _ = O.route(np.ones((1, 9)), np.diag(l), None, 2)
        a, b = l[idx[0, 0]], l[idx[0, 1]]
        assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-14
    # general k: w_j = exp(l_j) / sum_{i in S} exp(l_i), and sum = 1
    for _ in range(50):
        E, k = 12, 5
        l = rng.standard_normal(E) * 4
        _, idx, w, _ = O.route(np.ones((1, E)), np.diag(l), None, k)
        den = math.fsum(math.exp(l[i]) for i in idx[0])
        for j, e in enumerate(idx[0]):
            assert abs(w[0, j] - math.exp(l[e]) / den) < 1e-13
        assert abs(w[0].sum() - 1.0) < 1e-12


def test_k_equals_E_is_full_softmax(O, rng):
    E = 7
    l = rng.standard_normal(E)
    _, idx, w, gap = O.route(np.ones((1, E)), np.diag(l), None, E)
    assert gap == math.inf
    den = math.fsum(math.exp(v) for v in l)
    for j, e in enumerate(idx[0]):
        assert abs(w[0, j] - math.exp(l[e]) / den) < 1e-14


def test_softmax_shift_and_sum(O, rng):
    l = rng.standard_normal((4, 10)) * 50
    p = O.softmax(l)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-14)
    assert np.allclose(O.softmax(l + 1234.5), p, atol=1e-14)


# ---------------------------------------------------------------------------
# experts


def test_silu_closed_forms(O):
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu(-2.0) - (-2.0 / (1.0 + math.exp(2.0)))) < 1e-16
    assert O.silu(-1000.0) == 0.0         # no inf/inf
    assert O.silu(1000.0) == 1000.0
    assert O.sigmoid(0.0) == 0.5


@pytest.mark.parametrize("bits", [4, 8])
def test_expert_ffn_bruteforce(O, rng, bits):
    H, I = 128, 64
    a = rand_expert(rng, H, I, bits)
    x = rng.standard_normal((2, H))
    y = O.expert_ffn(x, a, 64)
    ref = ffn_bruteforce(x, a, 64)
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_expert_ffn_zero_weights(O, rng):
    a = rand_expert(rng, 128, 64)
    a["qd"][:] = 0
    a["bd"][:] = 0
    assert np.all(O.expert_ffn(rng.standard_normal((3, 128)), a, 64) == 0.0)


def test_expert_ffn_constant_closed_form(O, rng):
    H, I = 128, 64
    a = rand_expert(rng, H, I)
    cg, cu, cd = 3, 11, 5
    sg, bg, su, bu, sd, bd = 0.03125, -0.125, 0.015625, -0.25, 0.0625, -0.0625
    a["qg"][:], a["qu"][:], a["qd"][:] = cg, cu, cd
    for key, v in (("sg", sg), ("bg", bg), ("su", su), ("bu", bu), ("sd", sd), ("bd", bd)):
        a[key][:] = bf16_bits_of_value(v)
    x = rng.standard_normal((2, H))
    y = O.expert_ffn(x, a, 64)
    for t in range(2):
        X = math.fsum(x[t])
        g = (sg * cg + bg) * X
        u = (su * cu + bu) * X
        h = silu_scalar(g) * u
        yr = (sd * cd + bd) * I * h
        assert np.allclose(y[t], yr, rtol=1e-12)


def _tiny_layer(rng, E=8, H=128, I=64, k=3, T=5):
    experts = [rand_expert(rng, H, I) for _ in range(E)]
    shared = rand_expert(rng, H, I)
    Wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    wsg = (rng.standard_normal(H) * 0.1).astype(np.float32)
    x = rng.standard_normal((T, H))
    return experts, shared, Wr, wsg, x, k


def test_identity_and_scaled_copies_combine(O, rng):
    experts, shared, Wr, wsg, x, k = _tiny_layer(rng)
    base = experts[0]
    # identical experts: output independent of routing
    same = lambda e: base  # noqa: E731
    r = O.moe_layer(x, Wr, None, wsg, same, shared, k, 64)
    dense = O.expert_ffn(x, base, 64)
    ys = O.expert_ffn(x, shared, 64)
    gamma = O.shared_gate(x, wsg)
    assert np.allclose(r["out"], dense + gamma[:, None] * ys, rtol=1e-12, atol=1e-9)
    # scaled copies: expert e's down scale and bias times c_e = 2**m_e (exact in bf16)
    m = [0, 1, -1, 2, 3, -2, 1, 4]

    def scaled(e):
        a = dict(base)
        for key in ("sd", "bd"):
            v = O.bf16_to_f64(base[key]) * 2.0 ** m[e]
            a[key] = np.vectorize(lambda z: bf16_bits_of_value(float(z)))(v).astype(np.uint16)
        return a

    r2 = O.moe_layer(x, Wr, None, wsg, scaled, shared, k, 64)
    for t in range(x.shape[0]):
        c = math.fsum(r2["w"][t, j] * 2.0 ** m[r2["idx"][t, j]] for j in range(k))
        assert np.allclose(r2["out"][t], c * dense[t] + gamma[t] * ys[t], rtol=1e-11, atol=1e-8)


def test_shared_gate_zero_weight_and_zero_shared(O, rng):
    experts, shared, Wr, wsg, x, k = _tiny_layer(rng)
    g = O.shared_gate(x, np.zeros_like(wsg))
    assert np.all(g == 0.5)
    zero = dict(shared)
    zero["qd"] = np.zeros_like(shared["qd"])
    zero["bd"] = np.zeros_like(shared["bd"])
    get = lambda e: experts[e]  # noqa: E731
    with_zero = O.moe_layer(x, Wr, None, wsg, get, zero, k, 64)["out"]
    without = O.moe_layer(x, Wr, None, wsg, get, None, k, 64)["out"]
    assert np.array_equal(with_zero, without)


def test_layer_bruteforce(O, rng):
    """Whole layer on tiny sizes against scalar loops for every step."""
    E, H, I, k, T = 4, 64, 64, 2, 2
    experts = [rand_expert(rng, H, I) for _ in range(E)]
    shared = rand_expert(rng, H, I)
    Wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
    wsg = (rng.standard_normal(H) * 0.1).astype(np.float32)
    x = rng.standard_normal((T, H))
    r = O.moe_layer(x, Wr, bias, wsg, lambda e: experts[e], shared, k, 64)
    for t in range(T):
        l = [math.fsum(float(Wr[e, c]) * x[t, c] for c in range(H)) + float(bias[e]) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        assert r["idx"][t].tolist() == order
        den = math.fsum(math.exp(l[e]) for e in order)
        w = [math.exp(l[e]) / den for e in order]
        gam = 1.0 / (1.0 + math.exp(-math.fsum(float(wsg[c]) * x[t, c] for c in range(H))))
        ref = np.zeros(H)
        for j, e in enumerate(order):
            ref += w[j] * ffn_bruteforce(x[t:t + 1], experts[e], 64)[0]
        ref += gam * ffn_bruteforce(x[t:t + 1], shared, 64)[0]
        assert np.allclose(r["out"][t], ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


def test_token_independence(O, rng):
    experts, shared, Wr, wsg, x, k = _tiny_layer(rng)
    get = lambda e: experts[e]  # noqa: E731
    full = O.moe_layer(x, Wr, None, wsg, get, shared, k, 64)
    for t in range(x.shape[0]):
        one = O.moe_layer(x[t:t + 1], Wr, None, wsg, get, shared, k, 64)
        assert one["idx"][0].tolist() == full["idx"][t].tolist()
        assert np.allclose(one["out"][0], full["out"][t], rtol=1e-13, atol=1e-10)


def test_forward_with_given_routing(O, rng):
    experts, shared, Wr, wsg, x, k = _tiny_layer(rng)
    get = lambda e: experts[e]  # noqa: E731
    T = x.shape[0]
    idx = np.array([[7, 0, 3]] * T)
    w = np.array([[0.5, 0.25, 0.25]] * T)
    r = O.moe_layer(x, Wr, None, wsg, get, None, k, 64, routing=(idx, w))
    ref = (0.5 * O.expert_ffn(x, experts[7], 64) + 0.25 * O.expert_ffn(x, experts[0], 64)
           + 0.25 * O.expert_ffn(x, experts[3], 64))
    assert np.allclose(r["out"], ref, rtol=1e-13, atol=1e-10)


# ---------------------------------------------------------------------------
# chain prologue / epilogue and bucketing


def test_rmsnorm_closed_forms(O, rng):
    H = 64
    x = np.array([[1.0, -1.0] * (H // 2)])
    eps = 1e-6
    assert np.allclose(O.rmsnorm(x, eps), x / math.sqrt(1 + eps), rtol=1e-15)
    c = 3.5
    assert np.allclose(O.rmsnorm(np.full((1, H), c), eps), c / math.sqrt(c * c + eps), rtol=1e-15)
    y = rng.standard_normal((3, H))
    assert np.allclose(O.rmsnorm(7.25 * y, 0.0), O.rmsnorm(y, 0.0), rtol=1e-14)
    z = O.rmsnorm(y, 0.0)
    assert np.allclose(np.mean(z * z, -1), 1.0, rtol=1e-14)


def test_chain_epilogue_rounds_to_act(O):
    x = np.array([[1.0, 256.0, -3.0]])
    out = np.array([[2 ** -8, 1.0, 2 ** -30]])
    got = O.chain_epilogue(x, out, "bf16")
    assert got.tolist() == [[1.0, 256.0, -3.0]]      # 1+2^-8 ties to 1; 257 -> 256 (even)
    got32 = O.chain_epilogue(x, out, "f32")
    assert got32.tolist() == [[1.0 + 2 ** -8, 257.0, -3.0]]


def test_bucket_bruteforce(O, rng):
    for T, E, k in ((1, 16, 2), (64, 512, 10), (100, 8, 3)):
        idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
        counts, offsets, pairs = O.bucket(idx, E)
        lists = [[] for _ in range(E)]
        for t in range(T):
            for j in range(k):
                lists[idx[t, j]].append((t, j))
        flat = [p for lst in lists for p in lst]
        assert [tuple(p) for p in pairs.tolist()] == flat
        assert counts.tolist() == [len(lst) for lst in lists]
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert all(offsets[e + 1] - offsets[e] == counts[e] for e in range(E))


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above


def _bad_group_index(q, s, b, group):
    q = np.asarray(q, np.float64)
    cg = np.arange(q.shape[1]) % (q.shape[1] // group)   # wrong: c mod G instead of c // 64
    return mo.bf16_to_f64(s)[:, cg] * q + mo.bf16_to_f64(b)[:, cg]


def _dropped_bias(q, s, b, group):
    q = np.asarray(q, np.float64)
    cg = np.arange(q.shape[1]) // group
    return mo.bf16_to_f64(s)[:, cg] * q


def _wrong_silu_sign(g):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(g))


def _topk_ascending_ties(l_row, k):
    l_row = np.asarray(l_row, np.float64)
    order = np.lexsort((-np.arange(len(l_row)), -l_row))     # ties to the higher index
    gap = np.inf if k == len(l_row) else float(l_row[order[k - 1]] - l_row[order[k]])
    return order[:k], gap


def _renorm_over_all(p_row, sel):
    return np.asarray(p_row, np.float64)[np.asarray(sel)]     # forgot to renormalise


def _rms_of_sum(x, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)   # sum, not mean


# (function planted in the numpy oracle, its bad version, the C++ build's
#  ORACLE_PLANT number of the same mistake, the pin that must catch it)
PLANTED = [
    ("dequantize", _bad_group_index, 1, test_dequantize_group_and_row_indexing),
    ("dequantize", _dropped_bias, 2, test_dequantize_bruteforce),
    ("silu", _wrong_silu_sign, 3, test_silu_closed_forms),
    ("topk", _topk_ascending_ties, 4, test_topk_ties_to_lower_index),
    ("renormalize", _renorm_over_all, 5, test_renormalised_weights_closed_forms),
    ("rmsnorm", _rms_of_sum, 6, test_rmsnorm_closed_forms),
]


def _run_pin(pin, O, rng):
    import inspect
    args = [O] + ([rng] if "rng" in inspect.signature(pin).parameters else [])
    pin(*args)


@pytest.mark.parametrize("name,bad,plant,pin", PLANTED, ids=[f"{p[0]}-{p[2]}" for p in PLANTED])
def test_planted_mistake_is_caught_numpy(monkeypatch, rng, name, bad, plant, pin):
    monkeypatch.setattr(mo, name, bad)
    with pytest.raises(AssertionError):
        _run_pin(pin, mo, rng)


@pytest.mark.parametrize("name,bad,plant,pin", PLANTED, ids=[f"{p[0]}-{p[2]}" for p in PLANTED])
def test_planted_mistake_is_caught_cpp(tmp_path, rng, name, bad, plant, pin):
    """The same mistakes planted in the C++ oracle (a build of moe_oracle.cpp
    with -DORACLE_PLANT=n): the pin that catches the numpy version catches it."""
    from oracle import build as obuild
    from oracle.cpp import CppOracle
    path = obuild.build(out=str(tmp_path / f"liboracle_plant{plant}.so"), plant=plant)
    with pytest.raises(AssertionError):
        _run_pin(pin, CppOracle(path), rng)


def test_cpp_and_numpy_oracles_agree(rng):
    """Both implementations of the definition on one small layer: the same
    routing and outputs equal to fp64 summation-order differences."""
    from oracle import cpp
    experts, shared, Wr, wsg, x, k = _tiny_layer(rng, E=12, H=192, I=128, k=4, T=9)
    get = lambda e: experts[e]  # noqa: E731
    bias = (rng.standard_normal(12) * 0.5).astype(np.float32)
    a = mo.moe_layer(x, Wr, bias, wsg, get, shared, k, 64)
    b = cpp.default().moe_layer(x, Wr, bias, wsg, get, shared, k, 64)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.allclose(a["w"], b["w"], rtol=1e-14, atol=0)
    assert np.allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12 * np.abs(a["out"]).max())


def test_cpp_oracle_thread_count_does_not_change_results(rng):
    """Each output element is computed by one thread in a fixed order: one
    thread and all threads give the same bits."""
    from oracle import cpp
    O = cpp.default()
    experts, shared, Wr, wsg, x, k = _tiny_layer(rng, E=8, H=128, I=64, k=3, T=6)
    get = lambda e: experts[e]  # noqa: E731
    n = O.num_threads()
    try:
        O.set_num_threads(1)
        one = O.moe_layer(x, Wr, None, wsg, get, shared, k, 64)["out"]
    finally:
        O.set_num_threads(n)
    many = O.moe_layer(x, Wr, None, wsg, get, shared, k, 64)["out"]
    assert np.array_equal(one, many)
