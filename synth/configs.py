"""Named workload configurations (shapes and policy constants only)."""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Policy:
    """CONF-KV hyper-parameters.

    tau, N_high (tight budget when confident), N_low (loose budget), P
    (protected newest tokens), alpha (rank mix), W (FP16 window), lambda (EMA
    decay) and the confidence weights (w_H, w_m, w_p) = (0.4, 0.3, 0.3).
    """
    tau: float = 0.7
    alpha: float = 0.65
    lam: float = 0.9
    w_h: float = 0.4
    w_m: float = 0.3
    w_p: float = 0.3
    n_high: int = 256
    n_low: int = 512
    protect: int = 32
    window: int = 64
    block: int = 0     # 0: token eviction; B: whole blocks of B tokens
    order: int = 0     # token eviction: 0 keeps position order (stable gather), 1 fills INT8 holes from the tail


@dataclass(frozen=True)
class Config:
    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    vocab: int
    prefill: int          # tokens in the cache before the first decode step
    steps: int            # decode steps of the full workload
    policy: Policy
    logit_scales: Tuple[float, ...] = (0.5, 2.0, 8.0)
    sinks: int = 0        # number of high-norm keys placed among the first 16 positions
    sink_gain: float = 4.0
    # per-layer budgets (CONF-KV-L); None means uniform budgets
    layer_n_low: Optional[Tuple[int, ...]] = None
    layer_n_high: Optional[Tuple[int, ...]] = None
    # "confkv": the method; "full_kv": comparison run keeping every token in
    # FP16 (attention output only, then the append)
    mode: str = "confkv"
    # planted key (a stand-in for needle retrieval): sequence b holds, at
    # position round(plant_depths[b] * prefill), the key plant_beta * u in
    # every layer and kv head (u a seeded unit vector per layer and kv head),
    # and every decode query is plant_gamma * u plus N(0, 1) noise
    plant_depths: Tuple[float, ...] = ()
    plant_beta: float = 0.0
    plant_gamma: float = 0.0

    @property
    def cap(self) -> int:
        """Token slots per (layer, sequence).

        A cache holds at most max(prefill, N_low + 1) tokens before a step
        (after a step it holds at most N + 1), and the step needs one more
        slot for the new token.
        """
        n_low = max(self.layer_n_low) if self.layer_n_low else self.policy.n_low
        return max(self.prefill, n_low + 1) + 1

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


def _pyramid(layers: int, top: int, bottom: int):
    # budgets fall linearly with depth from `top` (layer 0) to `bottom` (last layer)
    lo = []
    for l in range(layers):
        num = top * (layers - 1) - (top - bottom) * l
        q, r = divmod(num, layers - 1)
        lo.append(q + (1 if 2 * r >= layers - 1 else 0))
    hi = [x // 2 for x in lo]
    return tuple(lo), tuple(hi)


_PYR_LO, _PYR_HI = _pyramid(64, 4096, 1024)

CONFIGS = {
    # Single decode layer, GPT-2-small shape, 1024 cached tokens (newest 64 FP16)
    "gpt2_layer": Config(
        name="gpt2_layer", layers=1, batch=1, hq=12, hkv=12, d=64, vocab=50257,
        prefill=1024, steps=64,
        policy=Policy(n_high=256, n_low=512, protect=32, window=64)),
    # GPT-2-small full stack from an empty cache
    "gpt2_stack": Config(
        name="gpt2_stack", layers=12, batch=1, hq=12, hkv=12, d=64, vocab=50257,
        prefill=0, steps=2048,
        policy=Policy(n_high=256, n_low=512, protect=64, window=128), sinks=4),
    # Qwen-14B shape, GQA 5:1
    "qwen14b": Config(
        name="qwen14b", layers=48, batch=8, hq=40, hkv=8, d=128, vocab=152064,
        prefill=8192, steps=1024,
        policy=Policy(n_high=2048, n_low=4096, protect=64, window=256)),
    # Qwen-32B shape, GQA 5:1, batch 8 (the throughput workload)
    "qwen32b": Config(
        name="qwen32b", layers=64, batch=8, hq=40, hkv=8, d=128, vocab=152064,
        prefill=2048, steps=4096,
        policy=Policy(n_high=1024, n_low=2048, protect=64, window=256)),
    # Comparison runs on the Qwen-32B shape: every token kept in FP16 over the
    # workload's 4096 generated tokens (window and budget cover the 6144
    # tokens of prefill + generation, so nothing is evicted or quantised) ...
    "qwen32b_fullkv": Config(
        name="qwen32b_fullkv", layers=64, batch=8, hq=40, hkv=8, d=128, vocab=152064,
        prefill=2048, steps=4096,
        policy=Policy(n_high=6144, n_low=6144, protect=64, window=6144), mode="full_kv"),
    # ... and a sliding window of the newest 512 tokens (recency-only rank)
    "qwen32b_sw512": Config(
        name="qwen32b_sw512", layers=64, batch=8, hq=40, hkv=8, d=128, vocab=152064,
        prefill=2048, steps=4096,
        policy=Policy(alpha=0.0, n_high=512, n_low=512, protect=64, window=256)),
    # The Qwen-32B workload with block eviction: whole blocks of 128 tokens
    # leave (coarse eviction for paged layouts), same budgets
    "qwen32b_block128": Config(
        name="qwen32b_block128", layers=64, batch=8, hq=40, hkv=8, d=128, vocab=152064,
        prefill=2048, steps=4096,
        policy=Policy(n_high=1024, n_low=2048, protect=64, window=256, block=128)),
    # The Qwen-32B workload with the hole-filling survivor order (the INT8
    # holes below the new INT8 length take the INT8 tail), same budgets
    "qwen32b_fill": Config(
        name="qwen32b_fill", layers=64, batch=8, hq=40, hkv=8, d=128, vocab=152064,
        prefill=2048, steps=4096,
        policy=Policy(n_high=1024, n_low=2048, protect=64, window=256, order=1)),
    # Long-context pyramid with one planted key per sequence at depths
    # 10/30/50/70/90 % of the prefill (five sequences, one per depth)
    "qwen32b_niah": Config(
        name="qwen32b_niah", layers=64, batch=5, hq=40, hkv=8, d=128, vocab=152064,
        prefill=32768, steps=512,
        policy=Policy(n_high=_PYR_HI[0], n_low=_PYR_LO[0], protect=64, window=256),
        layer_n_low=_PYR_LO, layer_n_high=_PYR_HI,
        plant_depths=(0.1, 0.3, 0.5, 0.7, 0.9), plant_beta=2.0 * 128 ** 0.5, plant_gamma=4.0),
    # The same with a weak needle (a stand-in for the over-confident
    # rare-entity lookups the pages name as a failure mode): the planted key
    # has the norm of the other keys (beta = sqrt(d)) and the queries lean
    # only gamma = 1 toward it, so its score is N(1, 1) against N(0, 1) for
    # the others; retention can and does fail, most at the oldest depths
    "qwen32b_niah_weak": Config(
        name="qwen32b_niah_weak", layers=64, batch=5, hq=40, hkv=8, d=128, vocab=152064,
        prefill=32768, steps=512,
        policy=Policy(n_high=_PYR_HI[0], n_low=_PYR_LO[0], protect=64, window=256),
        layer_n_low=_PYR_LO, layer_n_high=_PYR_HI,
        plant_depths=(0.1, 0.3, 0.5, 0.7, 0.9), plant_beta=128 ** 0.5, plant_gamma=1.0),
    # One decode layer of the Qwen-32B shape at batch 1 over a 32000-token
    # cache whose budgets cover it (nothing is evicted; the cache grows by one
    # token per step): eight long units, the shape where attention splits
    # each unit's keys over several workgroups
    "long32k_layer": Config(
        name="long32k_layer", layers=1, batch=1, hq=40, hkv=8, d=128, vocab=152064,
        prefill=32000, steps=64,
        policy=Policy(n_high=32768, n_low=32768, protect=64, window=256)),
    # Long-context pyramid (CONF-KV-L), Qwen-32B layer shape, batch 1
    "qwen32b_pyramid": Config(
        name="qwen32b_pyramid", layers=64, batch=1, hq=40, hkv=8, d=128, vocab=152064,
        prefill=32768, steps=512,
        policy=Policy(n_high=_PYR_HI[0], n_low=_PYR_LO[0], protect=64, window=256),
        layer_n_low=_PYR_LO, layer_n_high=_PYR_HI),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
