"""The five synthetic workloads of the MoE layer (shapes and distributions only).

Shapes follow the two model families the pages describe: routing 8 of 256
experts (Qwen3.5/3.6-35B-A3B) and 10 of 512 experts (Qwen3-Next-80B-A3B),
per layer and per token.  Hidden size, expert intermediate size, group size
and value distributions are not on the pages; they are the workload
definitions this project measures on.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoeConfig:
    name: str
    seed: int
    n_tokens: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    bits: int = 4
    group: int = 64
    act: str = "bf16"          # activation dtype: "f32" or "bf16"
    layers: int = 1            # distinct layers chained with pre-RMSNorm + residual
    router_std: float = 0.02   # router weight N(0, std^2)
    zipf_s: float = 0.0        # >0: additive Zipf(s) router bias
    rms_eps: float = 1e-6

    def with_(self, **kw) -> "MoeConfig":
        return replace(self, **kw)

    @property
    def chained(self) -> bool:
        return self.layers > 1


TINY = MoeConfig(name="tiny", seed=0, n_tokens=4, hidden=256, n_experts=16, top_k=2,
                 inter=128, shared_inter=128, act="f32", layers=1, router_std=0.02)

DECODE_35B = MoeConfig(name="decode_35b", seed=1, n_tokens=1, hidden=2048, n_experts=256,
                       top_k=8, inter=512, shared_inter=512, layers=40, router_std=0.02)

DECODE_80B = MoeConfig(name="decode_80b", seed=2, n_tokens=1, hidden=2048, n_experts=512,
                       top_k=10, inter=512, shared_inter=512, layers=48,
                       router_std=1.0 / math.sqrt(2048))

BATCHED_80B = MoeConfig(name="batched_80b", seed=3, n_tokens=64, hidden=2048, n_experts=512,
                        top_k=10, inter=512, shared_inter=512, layers=48,
                        router_std=1.0 / math.sqrt(2048), zipf_s=1.1)

BATCHED_80B_INT8 = BATCHED_80B.with_(name="batched_80b_int8", bits=8)

PREFILL_35B = MoeConfig(name="prefill_35b", seed=4, n_tokens=4096, hidden=2048, n_experts=256,
                        top_k=8, inter=512, shared_inter=512, layers=1,
                        router_std=1.0 / math.sqrt(2048))

CONFIGS = {c.name: c for c in (TINY, DECODE_35B, DECODE_80B, BATCHED_80B, BATCHED_80B_INT8,
                               PREFILL_35B)}
