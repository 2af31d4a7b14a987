"""CONF-KV decode step on AMD MI355X: Python binding of libconfk.

The work of every step runs in libconfk's HIP kernels; this package only
allocates device memory through PyTorch and passes pointers and the current
stream to the C ABI (include/confk.h). It raises if the library is missing.
"""
from ._lib import (  # noqa: F401
    Cache, Policy, ConfkError, load, check, LIB_PATH, EXPORTS,
    OK, ERR_INVALID_ARG, ERR_BUDGET, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_LAUNCH,
    STATUS_NONFINITE_LOGITS, STATUS_CAPACITY, QUANT_STEP, QUANT_PREFILL,
    META_N, META_N8, META_BASE8, META_BASE16, META_CALIB, META_SAT, META_EVICTED,
    META_MOVED, META_MOVED16, META_MASSROWS, META_WORDS,
)
from .engine import (  # noqa: F401
    make_policy, DeviceCache, DecodeEngine, confidence, attn_decode, confidence_attn_decode, decode_step, ema_rank,
    compact, quantize,
)
