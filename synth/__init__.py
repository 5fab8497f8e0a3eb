"""Seeded synthetic inputs for the int4/int8 group-quantized MoE layer.

This module only *draws* inputs.  It holds none of the layer's arithmetic
(no dequantisation, no routing, no expert math): it produces the logical
arrays -- integer codes, bf16 scale/bias bit patterns, fp32 router weights,
activations -- from which both the fp64 oracle (``oracle/``) and the HIP
product path (``int4_group_quantized_moe_amd``) are fed.  It is the only code
the two sides share.

Generator definition (counter-based, so any element can be regenerated on its
own, on the host or on the device):

* ``mix64`` is the SplitMix64 output finaliser (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31`` (all mod 2**64).
* A stream is identified by ``(seed, tensor, layer, expert)`` packed into one
  64-bit word ``id = seed<<48 | tensor<<40 | layer<<24 | expert`` and keyed
  by ``key = mix64(id)``.
* Element ``i`` of a stream is the ``i``-th SplitMix64 output from state
  ``key``: ``draw(i) = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)``.
* int4 code = ``draw >> 60``; int8 code = ``draw >> 56``.
* uniform u in [0,1) = ``(draw >> 40) * 2**-24`` (exact in fp32).
  ``U(a, b)`` = ``fl32(a + fl32(fl32(b - a) * u))`` in fp32 with separate
  roundings (no fused multiply-add), then rounded to bf16 (round to nearest
  even) when stored as bf16.
* normal: Box--Muller on draws ``2i`` and ``2i+1`` in fp64:
  ``u1 = ((d0 >> 11) + 1) * 2**-53``, ``u2 = (d1 >> 11) * 2**-53``,
  ``z = sqrt(-2 ln u1) * cos(2 pi u2)``.  Normals are only drawn on the host.

The device fill (``synth/synth_fill.hip``) implements the integer codes and the
bf16 uniforms with exactly the same definition; a GPU test checks the two
bit-equal on sampled elements.
"""
from __future__ import annotations

import numpy as np

from .configs import CONFIGS, MoeConfig  # noqa: F401

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

# stream "tensor" ids
T_QGATE, T_QUP, T_QDOWN = 1, 2, 3
T_SGATE, T_BGATE, T_SUP, T_BUP, T_SDOWN, T_BDOWN = 4, 5, 6, 7, 8, 9
T_ROUTER_W, T_ROUTER_BIAS, T_SHARED_GATE_W, T_X = 10, 11, 12, 13
T_DENSE_Q, T_DENSE_S, T_DENSE_B = 14, 15, 16  # 4-bit dense rows (router + shared gate)
SHARED_EXPERT = 0xFFFFFF  # expert field of the shared expert's streams
NO_EXPERT = 0xFFFFFE      # expert field of per-layer dense tensors

# scale / bias distributions of the quantised weights (all configs)
SCALE_LO, SCALE_HI = 0.01, 0.05
BIAS_LO, BIAS_HI = -0.4, 0.0


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wraps mod 2**64)."""
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor: int, layer: int, expert: int) -> int:
    assert 0 <= seed < (1 << 16) and 0 <= tensor < (1 << 8)
    assert 0 <= layer < (1 << 16) and 0 <= expert < (1 << 24)
    sid = (seed << 48) | (tensor << 40) | (layer << 24) | expert
    return _mix64_int(sid)


def draws(key: int, start: int, n: int) -> np.ndarray:
    """Elements ``start .. start+n-1`` of the stream with the given key."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    return mix64(np.uint64(key) + i * GOLDEN)


def draws_at(key: int, idx: np.ndarray) -> np.ndarray:
    """Elements at arbitrary indices of the stream (for sampled checks)."""
    i = np.asarray(idx, dtype=np.uint64) + np.uint64(1)
    return mix64(np.uint64(key) + i * GOLDEN)


def codes_from_draws(d: np.ndarray, bits: int) -> np.ndarray:
    return (d >> np.uint64(64 - bits)).astype(np.uint8)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + rounding) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniform_bf16_from_draws(d: np.ndarray, lo: float, hi: float) -> np.ndarray:
    u = (d >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    width = np.float32(np.float32(hi) - np.float32(lo))
    t = (width * u).astype(np.float32)           # rounded product
    v = (np.float32(lo) + t).astype(np.float32)  # rounded sum
    return f32_to_bf16_bits(v)


def normal_f64(key: int, n: int) -> np.ndarray:
    d = draws(key, 0, 2 * n)
    d0, d1 = d[0::2], d[1::2]
    u1 = ((d0 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (d1 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


# ---------------------------------------------------------------------------
# optional C implementation of the same definition (synth_host.c), used for
# speed when built; tests check it bit-equal to the numpy definition above.

_clib = None


def _host_lib():
    global _clib
    if _clib is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth_host.so")
        if not os.path.exists(path):
            _clib = False
        else:
            h = ctypes.CDLL(path)
            h.synth_host_codes.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_void_p]
            h.synth_host_uniform_bf16.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_float,
                                                  ctypes.c_float, ctypes.c_void_p]
            _clib = h
    return _clib or None


def codes_c(key: int, n: int, bits: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    _host_lib().synth_host_codes(key, n, bits, out.ctypes.data)
    return out


def uniform_bf16_c(key: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, np.uint16)
    _host_lib().synth_host_uniform_bf16(key, n, lo, hi, out.ctypes.data)
    return out


# ---------------------------------------------------------------------------
# logical tensors of one configuration


def quant_codes(seed: int, tensor: int, layer: int, expert: int, rows: int, cols: int,
                bits: int) -> np.ndarray:
    key = stream_key(seed, tensor, layer, expert)
    if _host_lib() is not None:
        return codes_c(key, rows * cols, bits).reshape(rows, cols)
    return codes_from_draws(draws(key, 0, rows * cols), bits).reshape(rows, cols)


def quant_sb(seed: int, tensor: int, layer: int, expert: int, rows: int, groups: int,
             lo: float, hi: float) -> np.ndarray:
    key = stream_key(seed, tensor, layer, expert)
    if _host_lib() is not None:
        return uniform_bf16_c(key, rows * groups, lo, hi).reshape(rows, groups)
    return uniform_bf16_from_draws(draws(key, 0, rows * groups), lo, hi).reshape(rows, groups)


def expert_arrays(cfg: "MoeConfig", layer: int, expert: int) -> dict:
    """Logical int codes (one per byte) and bf16 scale/bias bits of one expert.

    gate/up: [inter x hidden] codes, [inter x hidden/group] scale and bias;
    down: [hidden x inter] codes, [hidden x inter/group] scale and bias.
    ``expert == SHARED_EXPERT`` gives the shared expert (``shared_inter`` rows).
    """
    s, H, G, bits = cfg.seed, cfg.hidden, cfg.group, cfg.bits
    inter = cfg.shared_inter if expert == SHARED_EXPERT else cfg.inter
    return {
        "qg": quant_codes(s, T_QGATE, layer, expert, inter, H, bits),
        "qu": quant_codes(s, T_QUP, layer, expert, inter, H, bits),
        "qd": quant_codes(s, T_QDOWN, layer, expert, H, inter, bits),
        "sg": quant_sb(s, T_SGATE, layer, expert, inter, H // G, SCALE_LO, SCALE_HI),
        "bg": quant_sb(s, T_BGATE, layer, expert, inter, H // G, BIAS_LO, BIAS_HI),
        "su": quant_sb(s, T_SUP, layer, expert, inter, H // G, SCALE_LO, SCALE_HI),
        "bu": quant_sb(s, T_BUP, layer, expert, inter, H // G, BIAS_LO, BIAS_HI),
        "sd": quant_sb(s, T_SDOWN, layer, expert, H, inter // G, SCALE_LO, SCALE_HI),
        "bd": quant_sb(s, T_BDOWN, layer, expert, H, inter // G, BIAS_LO, BIAS_HI),
    }


def router_weight(cfg: "MoeConfig", layer: int) -> np.ndarray:
    """fp32 [n_experts x hidden], N(0, router_std^2)."""
    key = stream_key(cfg.seed, T_ROUTER_W, layer, NO_EXPERT)
    z = normal_f64(key, cfg.n_experts * cfg.hidden)
    return (z * cfg.router_std).astype(np.float32).reshape(cfg.n_experts, cfg.hidden)


def router_bias(cfg: "MoeConfig", layer: int):
    """fp32 [n_experts] additive router bias, or None.

    Zipf(s) reading: ``b_e = -s * ln(rank_e)`` with ``rank`` a seeded
    permutation of 1..E, so ``softmax(b)`` is the Zipf pmf over experts.
    """
    if not cfg.zipf_s:
        return None
    key = stream_key(cfg.seed, T_ROUTER_BIAS, layer, NO_EXPERT)
    d = draws(key, 0, cfg.n_experts)
    order = np.argsort(d, kind="stable")           # seeded permutation
    rank = np.empty(cfg.n_experts, dtype=np.int64)
    rank[order] = np.arange(1, cfg.n_experts + 1)
    return (-cfg.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


def shared_gate_weight(cfg: "MoeConfig", layer: int) -> np.ndarray:
    """fp32 [hidden] weight of the shared expert's sigmoid gate, N(0, 0.02^2)."""
    key = stream_key(cfg.seed, T_SHARED_GATE_W, layer, NO_EXPERT)
    return (normal_f64(key, cfg.hidden) * 0.02).astype(np.float32)


def dense_q4_arrays(cfg: "MoeConfig", layer: int) -> dict:
    """The layer's dense rows in 4 bits: the E router rows and, with a shared
    expert, its gate vector as row E.  Codes uniform 0..15, scale
    ~U(0.8 c, 1.2 c) and bias ~U(-8.5 c, -6.5 c) per group of 64, c =
    router_std / 4.61 (the standard deviation of q - 7.5), so that the rows
    have about the fp32 router's spread and mean 0.

    q: [rows x hidden] codes (one per byte); s, b: [rows x hidden/64] bf16 bits.
    """
    rows = cfg.n_experts + (1 if cfg.shared_inter > 0 else 0)
    c = cfg.router_std / 4.61
    G = cfg.hidden // cfg.group
    return {
        "q": quant_codes(cfg.seed, T_DENSE_Q, layer, NO_EXPERT, rows, cfg.hidden, 4),
        "s": quant_sb(cfg.seed, T_DENSE_S, layer, NO_EXPERT, rows, G, 0.8 * c, 1.2 * c),
        "b": quant_sb(cfg.seed, T_DENSE_B, layer, NO_EXPERT, rows, G, -8.5 * c, -6.5 * c),
    }


def activations(cfg: "MoeConfig", variant: int = 0, n_tokens: int | None = None) -> np.ndarray:
    """Layer input x ~ N(0,1) [n_tokens x hidden] as fp32 values exactly
    representable in the activation dtype (bf16 configs round to nearest even).
    ``variant`` selects one of several independent input batches."""
    T = cfg.n_tokens if n_tokens is None else n_tokens
    key = stream_key(cfg.seed, T_X, variant, NO_EXPERT)
    x = normal_f64(key, T * cfg.hidden).astype(np.float32).reshape(T, cfg.hidden)
    if cfg.act == "bf16":
        x = bf16_bits_to_f32(f32_to_bf16_bits(x))
    return x


def slot_table(cfg: "MoeConfig", layer: int, permute_seed: int | None = None) -> np.ndarray:
    """Expert -> slab slot table of one layer.  Default: slot = layer*E + e.
    With ``permute_seed`` the layer's slots are permuted among themselves."""
    E = cfg.n_experts
    base = layer * E
    if permute_seed is None:
        return (base + np.arange(E)).astype(np.int32)
    key = stream_key(permute_seed & 0xFFFF, 0xFE, layer, NO_EXPERT)
    perm = np.argsort(draws(key, 0, E), kind="stable")
    return (base + perm).astype(np.int32)
