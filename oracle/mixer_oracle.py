"""fp64 CPU oracle of the two token mixers of the hybrid layers.

TEST INFRASTRUCTURE ONLY: the test suite and the benchmark's CPU-baseline leg
are its only users; the HIP product path never imports it and it imports
nothing from that path.

* Gated DeltaNet decode step.  75% of the layers of the hybrid models use
  Gated DeltaNet linear attention with a fixed-size recurrent state (page
  "Paquets Swiftlet 80B Qwen ..." on xix.ai, 5th paragraph; Swiftlet news item
  on news.bugfactory.tech, 3rd paragraph).  The pages print no formula; the
  reading used here is the gated delta rule as published (Yang, Kautz and
  Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule",
  2024): per value head, with state S [d_v x d_k],
      S' = alpha S (I - beta k k^T) + beta v k^T,   o = S' q,
  alpha = exp(g) the decay gate, beta the write strength, q and k L2-normalised
  (q also scaled by 1/sqrt(d_k)); v head h reads query/key head
  h // (n_v_heads / n_k_heads).  (Readings G1-G4 in the design notes.)
* Gated GQA attention decode.  The remaining layers use gated GQA attention
  (xix.ai page, last paragraph; news.bugfactory.tech item, 5th paragraph).
  Reading: one new query token per sequence; query head h reads kv head
  h // (n_q_heads / n_kv_heads); scores q . K_j / sqrt(D) over the sequence's
  valid positions, softmax, o = sum_j p_j V_j, and the output gate
  o * sigmoid(gate) elementwise.  (Readings A1-A3.)

Everything in float64, step by step; pinned by tests/test_mixer_pins.py.
"""
from __future__ import annotations

import numpy as np


def l2norm(x, eps: float) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(v) -> np.ndarray:
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def gdn_head_step(S, q, k, v, g: float, beta: float):
    """One value head, one token: (S', o) with S [d_v x d_k], q, k [d_k]
    already normalised (q scaled), v [d_v]:
        u = v - alpha S k,  S' = alpha S + beta u k^T,  o = S' q."""
    S = np.asarray(S, np.float64)
    alpha = np.exp(np.float64(g))
    u = np.asarray(v, np.float64) - alpha * (S @ np.asarray(k, np.float64))
    S2 = alpha * S + np.float64(beta) * np.outer(u, np.asarray(k, np.float64))
    return S2, S2 @ np.asarray(q, np.float64)


def gdn_step(S, q, k, v, g, beta, eps: float = 1e-6, scale: float | None = None):
    """Gated DeltaNet decode step for a batch of sequences.

    S [B, Hv, d_v, d_k], q, k [B, Hk, d_k], v [B, Hv, d_v], g, beta [B, Hv].
    Returns (S' [B, Hv, d_v, d_k], o [B, Hv, d_v]), float64."""
    S = np.asarray(S, np.float64)
    B, Hv, dv, dk = S.shape
    Hk = np.asarray(q).shape[1]
    rep = Hv // Hk
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    qn = l2norm(q, eps) * scale
    kn = l2norm(k, eps)
    S2 = np.empty_like(S)
    o = np.empty((B, Hv, dv), np.float64)
    for b in range(B):
        for h in range(Hv):
            S2[b, h], o[b, h] = gdn_head_step(S[b, h], qn[b, h // rep], kn[b, h // rep],
                                              np.asarray(v, np.float64)[b, h],
                                              float(np.asarray(g)[b, h]),
                                              float(np.asarray(beta)[b, h]))
    return S2, o


def softmax(s) -> np.ndarray:
    s = np.asarray(s, np.float64)
    z = np.exp(s - s.max())
    return z / z.sum()


def attn_head(q, K, V, gate, scale: float):
    """One query head over n cache rows K, V [n x D]: sigmoid(gate) * sum_j
    softmax(K q * scale)_j V_j."""
    s = np.asarray(K, np.float64) @ np.asarray(q, np.float64) * scale
    p = softmax(s)
    return (p @ np.asarray(V, np.float64)) * sigmoid(gate)


def attn_decode(q, gate, get_kv, lengths, n_kv_heads: int, scale: float | None = None):
    """Gated GQA attention decode for a batch.

    q, gate [B, Hq, D]; get_kv(b, kv_head, n) -> (K, V) [n x D] the first n
    cache rows of sequence b; lengths [B].  Returns out [B, Hq, D] float64."""
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    group = Hq // n_kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), np.float64)
    for b in range(B):
        n = int(lengths[b])
        for kvh in range(n_kv_heads):
            K, V = get_kv(b, kvh, n)
            for h in range(kvh * group, (kvh + 1) * group):
                out[b, h] = attn_head(q[b, h], K, V, np.asarray(gate, np.float64)[b, h], scale)
    return out
