"""Feeds the oracle with one layer of a synthetic workload.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The inputs come from
the seeded generator ``synth``; the logical arrays are read directly, never a
packed expert slab.
"""
from __future__ import annotations

import functools

import numpy as np

import synth

from . import moe_oracle


class LayerInputs:
    """Router, shared expert and (lazily, cached) routed experts of one layer."""

    def __init__(self, cfg, layer: int, overrides: dict | None = None, dense_q4: bool = False):
        self.cfg = cfg
        self.layer = layer
        ov = overrides or {}
        if dense_q4:
            # router rows and shared gate in 4 bits: the values they encode
            # (w = s q + b per group), row E the gate vector
            a = synth.dense_q4_arrays(cfg, layer)
            rows = moe_oracle.dequantize(a["q"], a["s"], a["b"], cfg.group)
            ov = {"router_w": rows[:cfg.n_experts], "w_sg": rows[cfg.n_experts], **ov}
        self.router_w = ov.get("router_w", synth.router_weight(cfg, layer))
        self.router_bias = ov.get("router_bias", synth.router_bias(cfg, layer))
        self.w_sg = ov.get("w_sg", synth.shared_gate_weight(cfg, layer))
        self.shared = ov.get("shared", synth.expert_arrays(cfg, layer, synth.SHARED_EXPERT))
        self._expert_override = ov.get("get_expert")

    @functools.lru_cache(maxsize=None)
    def expert(self, e: int) -> dict:
        if self._expert_override is not None:
            return self._expert_override(e)
        return synth.expert_arrays(self.cfg, self.layer, e)


def implementation(impl: str = "cpp"):
    """The oracle implementation: "cpp" (the C++ library, the default) or
    "numpy"; both have the same functions and are pinned by the same tests."""
    if impl == "numpy":
        return moe_oracle
    if impl == "cpp":
        from . import cpp
        return cpp.default()
    raise ValueError(impl)


def oracle_layer(inputs: LayerInputs, x_hat: np.ndarray, routing=None, impl: str = "cpp") -> dict:
    """Run the oracle on one layer with input ``x_hat`` [T x H] (stored values)."""
    cfg = inputs.cfg
    return implementation(impl).moe_layer(x_hat, inputs.router_w, inputs.router_bias, inputs.w_sg,
                                          inputs.expert, inputs.shared, cfg.top_k, cfg.group,
                                          routing=routing)
