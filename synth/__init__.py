"""Seeded synthetic workloads for the CONF-KV decode step.

This module is shared by the tests, the benchmark and the smoke check. It
holds only shapes, policy constants and seeded random draws; it performs none
of the method's arithmetic (no softmax, no confidence, no quantisation).

Workload shapes follow the decode configurations used for CONF-KV
(CONF-KV paper summary, "Experimental results"/"Throughput and latency";
structured review, "Reproduction": tau=0.7, P, alpha=0.65, W, B=128).
The datasets the pages evaluate on (WikiText-2, Needle-in-a-Haystack,
VisualWebArena) are not used; seeded Gaussian tensors of the same shapes
stand in for them.
"""
from .configs import Config, Policy, CONFIGS, get_config  # noqa: F401
from .gen import (  # noqa: F401
    logits_for_step,
    decode_inputs,
    prefill_kv,
    step_rng,
)
