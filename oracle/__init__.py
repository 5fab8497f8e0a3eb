"""fp64 CPU oracle of the int4/int8 group-quantized MoE layer.

Two implementations of the same definition, pinned by the same tests: the
plain C++ library ``moe_oracle.cpp`` (OpenMP over the host cores; reached
through ``oracle.cpp``, the default of ``oracle_layer``) and the numpy module
``moe_oracle`` (whose functions this package re-exports).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The HIP product path
(``int4_group_quantized_moe_amd``) never imports, links or runs anything here,
and this package imports nothing from it.
"""
from .moe_oracle import (  # noqa: F401
    bf16_to_f64, round_to_bf16, round_act, dequantize, router_logits, softmax, topk,
    renormalize, silu, sigmoid, expert_ffn, shared_gate, route, combine, moe_layer,
    rmsnorm, chain_prologue, chain_epilogue, bucket,
)
from .workloads import LayerInputs, implementation, oracle_layer  # noqa: F401
