"""Seeded synthetic inputs for the offloaded MoE layer.

Test infrastructure and benchmark input: this module only draws random
numbers and lays them out as bytes.  It holds none of the layer's
arithmetic (routing, cache replay, dequantisation, FFN); both the CPU
oracle and the GPU library consume what it writes.

Workload recipe (the pages measure on real prompts that are not
available here; these streams stand in for them as the source of temporal
expert reuse):

* hidden states: per stream an AR(1) process ``x_0 ~ N(0, I)``,
  ``x_t = 0.9 x_{t-1} + 0.436 eps_t``; independent streams for a batch;
* router weights ``W_r[l] ~ N(0, 1/sqrt(H))`` (standard deviation), fp32;
* expert weights ``~ N(0, 0.02)`` before quantisation into the packed
  expert block (see ``block_layout``); a shared expert's ``~ N(0, 0.01)``,
  so that a 48-layer residual chain without normalisation stays bounded.

Randomness: NumPy PCG64 seeded through ``SeedSequence(seed, spawn_key=...)``
so that any (layer, expert) block or any stream can be drawn on its own,
in any order and in parallel, with the same bytes.
"""
from .gen import (  # noqa: F401
    QUANT_F32, QUANT_INT4_G32, QUANT_E2M1_G16, QUANT_NAMES,
    expert_bytes, block_layout, ar1_streams, router_weights,
    expert_block, shared_expert_blocks, fill_expert_store, fill_blocks, alias_index, quantize_int4_g32, quantize_e2m1_g16,
    prefill_prompt,
)
