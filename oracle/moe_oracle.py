"""fp64 CPU oracle of one sparse MoE layer with int4/int8 group-quantized experts.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP product path
never calls it and shares no code with it.

It computes the plain definition of the layer, step by step, in float64:

* Expert routing of each token to the top-k of E experts (10 of 512 for the
  80B-A3B family, 8 of 256 for the 35B-A3B family) with a resident router and
  an always-active shared expert: page "Paquets Swiftlet 80B Qwen ..." (xix.ai),
  4th paragraph; page "Swiftlet — Swift + Metal рантайм" (news.bugfactory.tech),
  3rd paragraph.
* MLX-style int4/int8 group quantisation of the expert weights: xix.ai page,
  last paragraph.  The affine form ``w = scale * q + bias`` per group of 64
  consecutive input columns, SwiGLU experts, the sigmoid-gated shared expert
  and softmax -> top-k -> renormalise are the workload definition of this
  project; the pages do not print them.

Readings the pages leave open (numbered as in the design notes):
R1  codes are unsigned (0..15 / 0..255) and groups run along the input axis.
R2  scale and bias are bf16, widened exactly.
R5  softmax over all E, then top-k, then renormalise over the k selected.
R6  top-k ordered by logit descending, ties to the lower expert index.
R7  activations are stored in the activation dtype (bf16 rounds to nearest
    even); the oracle widens stored values exactly.
R9  chained layers: x_hat = act(rmsnorm(x)) (unit weight) before the layer,
    x_next = act(x + out) after it.
All functions are pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# number formats (the oracle's own; nothing shared with the HIP path)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the high 16 bits of an IEEE fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), exactly.

    Done in exact arithmetic on the float64 representation: the bf16 spacing at
    the value's binade is 2**(e-7); np.round rounds half to even.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    m, e = np.frexp(v[nz])            # v = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: |m| * 2**8 in [128, 256)
    q = np.round(m * 256.0)           # half-to-even on exact float64 values
    out[nz] = np.ldexp(q / 256.0, e)
    return out


def round_act(v, act: str) -> np.ndarray:
    """Store a float64 result in the activation dtype and widen it back."""
    if act == "bf16":
        return round_to_bf16(v)
    if act == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(act)


# ---------------------------------------------------------------------------
# the layer, step by step


def dequantize(q, scale_bits, bias_bits, group: int) -> np.ndarray:
    """W[r, c] = s[r, c // group] * q[r, c] + b[r, c // group]   (R1, R2).

    ``q``: [rows x cols] unsigned codes; ``scale_bits``/``bias_bits``:
    [rows x cols/group] bf16 bit patterns.
    """
    q = np.asarray(q, dtype=np.float64)
    rows, cols = q.shape
    s = bf16_to_f64(scale_bits)
    b = bf16_to_f64(bias_bits)
    assert s.shape == (rows, cols // group) and b.shape == s.shape
    col_group = np.arange(cols) // group
    return s[:, col_group] * q + b[:, col_group]


def router_logits(x_hat, router_w, router_bias=None) -> np.ndarray:
    """l[t, e] = sum_c Wr[e, c] * x_hat[t, c]  (+ b_e)."""
    l = np.asarray(x_hat, np.float64) @ np.asarray(router_w, np.float64).T
    if router_bias is not None:
        l = l + np.asarray(router_bias, np.float64)[None, :]
    return l


def softmax(l) -> np.ndarray:
    """Softmax over the last axis (shifted by the row maximum)."""
    l = np.asarray(l, np.float64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def topk(l_row, k: int):
    """Indices of the k largest logits of one token, ordered by logit
    descending with ties to the lower expert index (R6), and the gap
    l_(k) - l_(k+1) between the k-th and (k+1)-th largest (inf when k == E)."""
    l_row = np.asarray(l_row, np.float64)
    E = l_row.shape[0]
    # lexsort: last key is primary -> sort by -l, then by index
    order = np.lexsort((np.arange(E), -l_row))
    sel = order[:k]
    gap = np.inf if k == E else float(l_row[order[k - 1]] - l_row[order[k]])
    return sel.astype(np.int64), gap


def renormalize(p_row, sel) -> np.ndarray:
    """w_j = p[S_j] / sum_{i in S} p[i]."""
    ps = np.asarray(p_row, np.float64)[np.asarray(sel)]
    return ps / ps.sum()


def silu(g) -> np.ndarray:
    """g * sigmoid(g), written g / (1 + exp(-g)) so that g -> -inf gives 0."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def sigmoid(v) -> np.ndarray:
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def expert_ffn(x_hat, arrays: dict, group: int) -> np.ndarray:
    """SwiGLU expert on int codes: g = Wg x, u = Wu x, h = silu(g) * u,
    y = Wd h.  ``x_hat``: [n x hidden] -> y: [n x hidden]."""
    Wg = dequantize(arrays["qg"], arrays["sg"], arrays["bg"], group)   # [I x H]
    Wu = dequantize(arrays["qu"], arrays["su"], arrays["bu"], group)   # [I x H]
    Wd = dequantize(arrays["qd"], arrays["sd"], arrays["bd"], group)   # [H x I]
    x = np.asarray(x_hat, np.float64)
    g = x @ Wg.T
    u = x @ Wu.T
    h = silu(g) * u
    return h @ Wd.T


def shared_gate(x_hat, w_sg) -> np.ndarray:
    """gamma[t] = sigmoid(w_sg . x_hat[t])   (R4)."""
    return sigmoid(np.asarray(x_hat, np.float64) @ np.asarray(w_sg, np.float64))


def route(x_hat, router_w, router_bias, k: int):
    """Router + softmax + top-k + renormalise for every token.

    Returns (logits [T x E], idx [T x k], w [T x k], gap [T])."""
    l = router_logits(x_hat, router_w, router_bias)
    p = softmax(l)
    T = l.shape[0]
    idx = np.zeros((T, k), np.int64)
    w = np.zeros((T, k), np.float64)
    gap = np.zeros(T, np.float64)
    for t in range(T):
        idx[t], gap[t] = topk(l[t], k)
        w[t] = renormalize(p[t], idx[t])
    return l, idx, w, gap


def combine(x_hat, idx, w, get_expert, group: int, gamma=None, shared=None) -> np.ndarray:
    """out[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x_hat[t]) + gamma[t] * FFN_s(x_hat[t]).

    ``get_expert(e)`` returns the logical arrays of routed expert e; each
    routed expert is dequantised once and applied to the tokens that chose it.
    ``shared``: logical arrays of the shared expert, or None for no shared expert.
    """
    x = np.asarray(x_hat, np.float64)
    idx = np.asarray(idx)
    out = np.zeros_like(x)
    for e in np.unique(idx):
        tok, j = np.nonzero(idx == e)
        y = expert_ffn(x[tok], get_expert(int(e)), group)
        out[tok] += np.asarray(w, np.float64)[tok, j][:, None] * y
    if shared is not None:
        out += np.asarray(gamma, np.float64)[:, None] * expert_ffn(x, shared, group)
    return out


def moe_layer(x_hat, router_w, router_bias, w_sg, get_expert, shared, k: int, group: int,
              routing=None) -> dict:
    """One MoE layer on the (already normalised) input ``x_hat`` [T x H].

    ``routing=(idx, w)`` runs the experts with a given routing instead of the
    router's ("forward with given routing").  Returns a dict with the logits,
    idx, w, gap, gamma and the float64 output."""
    logits, idx, w, gap = route(x_hat, router_w, router_bias, k)
    if routing is not None:
        idx, w = np.asarray(routing[0]), np.asarray(routing[1], np.float64)
    gamma = shared_gate(x_hat, w_sg) if shared is not None else None
    out = combine(x_hat, idx, w, get_expert, group, gamma, shared)
    return {"logits": logits, "idx": idx, "w": w, "gap": gap, "gamma": gamma, "out": out}


# ---------------------------------------------------------------------------
# the chain around the layer (R9)


def rmsnorm(x, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps), unit weight, per token."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def chain_prologue(x, eps: float, act: str) -> np.ndarray:
    """x_hat = act(rmsnorm(x))."""
    return round_act(rmsnorm(x, eps), act)


def chain_epilogue(x, out, act: str) -> np.ndarray:
    """x_next = act(x + out)."""
    return round_act(np.asarray(x, np.float64) + np.asarray(out, np.float64), act)


# ---------------------------------------------------------------------------
# token -> expert bucketing of a batch


def bucket(idx, n_experts: int):
    """Group the (token, j) pairs of a batch by expert.

    Returns (counts [E], offsets [E+1], pairs [T*k x 2]) where pairs lists
    (token, j) sorted by expert, then by token; offsets[e] is the first pair of
    expert e (exclusive prefix sum of counts)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    tok = np.repeat(np.arange(T), k)
    j = np.tile(np.arange(k), T)
    e = idx.ravel()
    order = np.lexsort((tok, e))
    pairs = np.stack([tok[order], j[order]], axis=1)
    return counts, offsets, pairs
