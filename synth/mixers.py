"""Seeded synthetic inputs for the two token mixers of the hybrid layers: the
Gated DeltaNet decode step and gated GQA attention decode.

Like the rest of ``synth`` this only draws inputs (normals and uniforms from
the counter-based generator, rounded to their storage dtype); it holds none of
the mixers' arithmetic.  Shapes follow the hybrid Qwen3-Next / Qwen3.5 family
the pages describe (75% of the layers use Gated DeltaNet linear attention with
a fixed-size recurrent state, the rest gated GQA attention: page "Paquets
Swiftlet 80B Qwen ..." on xix.ai, 5th and last paragraphs).  Head counts and
sizes are not on the pages; they are the workload definitions of this
project.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from . import (NO_EXPERT, bf16_bits_to_f32, draws, draws_at, f32_to_bf16_bits, normal_f64,
               stream_key, uniform_bf16_from_draws)

# stream "tensor" ids of the mixers
T_GDN_Q, T_GDN_K, T_GDN_V, T_GDN_G, T_GDN_B, T_GDN_S = 20, 21, 22, 23, 24, 25
T_ATT_Q, T_ATT_GATE, T_ATT_K, T_ATT_V, T_ATT_LEN = 26, 27, 28, 29, 30


def _bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, np.float32)))


def uniform_bf16_values(seed: int, tensor: int, layer: int, start: int, n: int, lo: float,
                        hi: float) -> np.ndarray:
    """Elements [start, start + n) of a bf16-uniform stream as fp32 values (the
    device fill ``synth.device.fill_uniform_bf16`` writes the same bits)."""
    key = stream_key(seed, tensor, layer, NO_EXPERT)
    d = draws_at(key, np.arange(start, start + n, dtype=np.uint64))
    return bf16_bits_to_f32(uniform_bf16_from_draws(d, lo, hi))


def _uniform_f32(key: int, n: int, lo: float, hi: float) -> np.ndarray:
    u = (draws(key, 0, n) >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    return (np.float32(lo) + np.float32(np.float32(hi) - np.float32(lo)) * u).astype(np.float32)


# ---------------------------------------------------------------------------
# Gated DeltaNet decode step


@dataclass(frozen=True)
class GdnConfig:
    name: str
    seed: int
    n_seqs: int          # sequences, one new token each
    n_k_heads: int       # query/key heads
    n_v_heads: int       # value heads (a multiple of n_k_heads)
    d_k: int
    d_v: int
    steps: int = 1       # decode steps chained through the state
    state_amp: float = 0.5   # initial state ~ U(-state_amp, state_amp), bf16 values

    def with_(self, **kw) -> "GdnConfig":
        return replace(self, **kw)


GDN_TINY = GdnConfig("gdn_tiny", seed=10, n_seqs=3, n_k_heads=2, n_v_heads=4, d_k=64, d_v=16,
                     steps=4)
GDN_80B = GdnConfig("gdn_80b", seed=11, n_seqs=1, n_k_heads=16, n_v_heads=32, d_k=128, d_v=128)
GDN_BATCHED = GDN_80B.with_(name="gdn_batched", seed=12, n_seqs=64)

GDN_CONFIGS = {c.name: c for c in (GDN_TINY, GDN_80B, GDN_BATCHED)}


def gdn_inputs(cfg: GdnConfig, step: int = 0) -> dict:
    """One decode step's inputs: q, k [B, Hk, dk] and v [B, Hv, dv] ~ N(0, 1)
    stored bf16 (fp32 values), the log-decay g ~ U(-1, -0.01) and the write
    strength beta ~ U(0.05, 0.95) [B, Hv] fp32."""
    B, Hk, Hv, dk, dv = cfg.n_seqs, cfg.n_k_heads, cfg.n_v_heads, cfg.d_k, cfg.d_v

    def normal(t, shape):
        key = stream_key(cfg.seed, t, step, NO_EXPERT)
        return _bf16(normal_f64(key, int(np.prod(shape))).astype(np.float32).reshape(shape))

    return {
        "q": normal(T_GDN_Q, (B, Hk, dk)),
        "k": normal(T_GDN_K, (B, Hk, dk)),
        "v": normal(T_GDN_V, (B, Hv, dv)),
        "g": _uniform_f32(stream_key(cfg.seed, T_GDN_G, step, NO_EXPERT), B * Hv, -1.0,
                          -0.01).reshape(B, Hv),
        "beta": _uniform_f32(stream_key(cfg.seed, T_GDN_B, step, NO_EXPERT), B * Hv, 0.05,
                             0.95).reshape(B, Hv),
    }


def gdn_state_spec(cfg: GdnConfig):
    """(seed, tensor, layer, n, lo, hi) of the initial state's bf16-uniform
    stream, element order [B, Hv, dv, dk]."""
    n = cfg.n_seqs * cfg.n_v_heads * cfg.d_v * cfg.d_k
    return cfg.seed, T_GDN_S, 0, n, -cfg.state_amp, cfg.state_amp


def gdn_state(cfg: GdnConfig, seqs=None) -> np.ndarray:
    """Initial recurrent state [B, Hv, dv, dk] fp32 ~ U(-state_amp, state_amp)
    with bf16 values; ``seqs``: only these sequences (sampled checks)."""
    seed, t, layer, _, lo, hi = gdn_state_spec(cfg)
    per = cfg.n_v_heads * cfg.d_v * cfg.d_k
    seqs = range(cfg.n_seqs) if seqs is None else seqs
    return np.stack([uniform_bf16_values(seed, t, layer, b * per, per, lo, hi) for b in seqs]
                    ).reshape(len(seqs), cfg.n_v_heads, cfg.d_v, cfg.d_k)


# ---------------------------------------------------------------------------
# gated GQA attention decode


@dataclass(frozen=True)
class AttnConfig:
    name: str
    seed: int
    n_seqs: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    max_len: int         # KV cache capacity per sequence (positions)
    ragged: bool = False  # per-sequence lengths drawn in [1, max_len]

    def with_(self, **kw) -> "AttnConfig":
        return replace(self, **kw)


ATT_TINY = AttnConfig("att_tiny", seed=20, n_seqs=3, n_q_heads=4, n_kv_heads=2, head_dim=64,
                      max_len=300, ragged=True)
ATT_80B = AttnConfig("att_80b", seed=21, n_seqs=1, n_q_heads=16, n_kv_heads=2, head_dim=256,
                     max_len=32768)
ATT_BATCHED = ATT_80B.with_(name="att_batched", seed=22, n_seqs=64, max_len=4096, ragged=True)

ATT_CONFIGS = {c.name: c for c in (ATT_TINY, ATT_80B, ATT_BATCHED)}


def attn_lengths(cfg: AttnConfig) -> np.ndarray:
    """Valid cache positions per sequence (int32 [B]): max_len, or drawn
    uniformly in [1, max_len] when ragged."""
    if not cfg.ragged:
        return np.full(cfg.n_seqs, cfg.max_len, np.int32)
    d = draws(stream_key(cfg.seed, T_ATT_LEN, 0, NO_EXPERT), 0, cfg.n_seqs)
    return (1 + (d % np.uint64(cfg.max_len))).astype(np.int32)


KV_AMP = 2.0  # cache entries ~ U(-2, 2)


def attn_query(cfg: AttnConfig, step: int = 0) -> dict:
    """q and the output gate [B, Hq, D] ~ N(0, 1) stored bf16 (fp32 values)."""
    B, Hq, D = cfg.n_seqs, cfg.n_q_heads, cfg.head_dim

    def normal(t):
        key = stream_key(cfg.seed, t, step, NO_EXPERT)
        return _bf16(normal_f64(key, B * Hq * D).astype(np.float32).reshape(B, Hq, D))

    return {"q": normal(T_ATT_Q), "gate": normal(T_ATT_GATE)}


def attn_cache_spec(cfg: AttnConfig, which: str):
    """(seed, tensor, layer, n, lo, hi) of the K or V cache's bf16-uniform
    stream, element order [B, Hkv, max_len, D]."""
    n = cfg.n_seqs * cfg.n_kv_heads * cfg.max_len * cfg.head_dim
    return cfg.seed, (T_ATT_K if which == "k" else T_ATT_V), 0, n, -KV_AMP, KV_AMP


def attn_cache(cfg: AttnConfig, which: str, seq: int, kv_head: int, n: int) -> np.ndarray:
    """Positions [0, n) of one sequence's and kv head's K or V cache rows
    [n, D] (fp32 values of the stored bf16)."""
    seed, t, layer, _, lo, hi = attn_cache_spec(cfg, which)
    start = ((seq * cfg.n_kv_heads + kv_head) * cfg.max_len) * cfg.head_dim
    return uniform_bf16_values(seed, t, layer, start, n * cfg.head_dim, lo, hi).reshape(
        n, cfg.head_dim)
