"""Seeded generators. Each draw is keyed by (seed, purpose, step) so that any
single step can be regenerated without replaying the others."""
import numpy as np

_PURPOSE = {"prefill": 1, "logits": 2, "decode": 3, "scale": 4, "sink": 5, "plant": 6}


def step_rng(seed: int, purpose: str, step: int = 0, extra: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, _PURPOSE[purpose], step, extra]))


def logit_scale(cfg, seed: int, step: int) -> np.ndarray:
    """Per-sequence standard deviation of this step's logits, drawn from cfg.logit_scales."""
    r = step_rng(seed, "scale", step)
    return np.asarray(cfg.logit_scales, dtype=np.float64)[r.integers(0, len(cfg.logit_scales), size=cfg.batch)]


def logits_for_step(cfg, seed: int, step: int) -> np.ndarray:
    """fp32 [B, V] logits, N(0, s_b) with s_b drawn per (step, sequence)."""
    s = logit_scale(cfg, seed, step)
    r = step_rng(seed, "logits", step)
    z = r.standard_normal((cfg.batch, cfg.vocab), dtype=np.float32)
    return (z * s[:, None].astype(np.float32)).astype(np.float32)


def decode_inputs(cfg, seed: int, step: int):
    """q fp16 [L,B,Hq,d], k_new/v_new fp16 [L,B,Hkv,d] for one decode step (N(0,1);
    queries aligned with the planted key when the config has one)."""
    r = step_rng(seed, "decode", step)
    L, B = cfg.layers, cfg.batch
    q = r.standard_normal((L, B, cfg.hq, cfg.d), dtype=np.float32)
    k = r.standard_normal((L, B, cfg.hkv, cfg.d), dtype=np.float32).astype(np.float16)
    v = r.standard_normal((L, B, cfg.hkv, cfg.d), dtype=np.float32).astype(np.float16)
    return plant_queries(cfg, seed, q).astype(np.float16), k, v


def sink_positions(cfg, seed: int):
    """Positions (among the first 16) whose keys are scaled by cfg.sink_gain."""
    if cfg.sinks == 0:
        return np.zeros(0, dtype=np.int64)
    r = step_rng(seed, "sink")
    return np.sort(r.choice(16, size=cfg.sinks, replace=False)).astype(np.int64)


def apply_sinks(cfg, seed: int, step: int, k_new: np.ndarray) -> np.ndarray:
    """High-norm keys at the seeded sink positions (used by the empty-cache stack)."""
    if step in set(sink_positions(cfg, seed).tolist()):
        k_new = (k_new.astype(np.float32) * cfg.sink_gain).astype(np.float16)
    return k_new


def prefill_kv(cfg, seed: int, layer0: int = 0, nlayers: int = None):
    """Prefill K/V, fp16 [nl,B,Hkv,L0,d] (N(0,1))."""
    nl = cfg.layers - layer0 if nlayers is None else nlayers
    shape = (nl, cfg.batch, cfg.hkv, cfg.prefill, cfg.d)
    out_k = np.empty(shape, dtype=np.float16)
    out_v = np.empty(shape, dtype=np.float16)
    for i in range(nl):
        r = step_rng(seed, "prefill", 0, layer0 + i)
        out_k[i] = r.standard_normal(shape[1:], dtype=np.float32).astype(np.float16)
        out_v[i] = r.standard_normal(shape[1:], dtype=np.float32).astype(np.float16)
    plant_prefill(cfg, seed, out_k, layer0)
    return out_k, out_v


def prefill_kv_device(cfg, seed: int, device, layer0: int = 0, nlayers: int = None):
    """Prefill K/V, fp16 [nl,B,Hkv,L0,d] N(0,1), drawn on the device with a
    seeded torch generator (fast for the large workloads). The oracle reads
    the same tensors back through a host copy."""
    import torch
    nl = cfg.layers - layer0 if nlayers is None else nlayers
    shape = (cfg.batch, cfg.hkv, cfg.prefill, cfg.d)
    k = torch.empty((nl,) + shape, dtype=torch.float16, device=device)
    v = torch.empty((nl,) + shape, dtype=torch.float16, device=device)
    gen = torch.Generator(device=device)
    for i in range(nl):
        gen.manual_seed(seed * 1_000_003 + (layer0 + i) * 7919 + 1)
        k[i] = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).half()
        v[i] = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).half()
    plant_prefill(cfg, seed, k, layer0)
    return k, v


def decode_inputs_device(cfg, seed: int, step: int, device):
    """q, k_new, v_new for one step drawn on the device (throughput runs)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + step * 104729 + 2)
    L, B = cfg.layers, cfg.batch
    q = torch.randn((L, B, cfg.hq, cfg.d), generator=gen, device=device).half()
    k = torch.randn((L, B, cfg.hkv, cfg.d), generator=gen, device=device).half()
    v = torch.randn((L, B, cfg.hkv, cfg.d), generator=gen, device=device).half()
    plant_queries(cfg, seed, q)
    return q, k, v


def logits_device(cfg, seed: int, step: int, device):
    """fp32 [B, V] logits N(0, s_b) drawn on the device, s_b from logit_scale()."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + step * 15485863 + 3)
    s = torch.as_tensor(logit_scale(cfg, seed, step), dtype=torch.float32, device=device)
    return torch.randn((cfg.batch, cfg.vocab), generator=gen, device=device) * s[:, None]


# ---------------------------------------------------------------- planted key

def plant_positions(cfg) -> np.ndarray:
    """Position of the planted key of each sequence (int64 [B]), or empty."""
    if not cfg.plant_depths:
        return np.zeros(0, dtype=np.int64)
    assert len(cfg.plant_depths) == cfg.batch
    return np.asarray([min(cfg.prefill - 1, int(round(x * cfg.prefill))) for x in cfg.plant_depths],
                      dtype=np.int64)


def plant_directions(cfg, seed: int, layer0: int = 0, nlayers: int = None) -> np.ndarray:
    """Unit vectors u [nl, Hkv, d] (float32) of the planted key per layer and kv head."""
    nl = cfg.layers - layer0 if nlayers is None else nlayers
    out = np.empty((nl, cfg.hkv, cfg.d), dtype=np.float32)
    for i in range(nl):
        u = step_rng(seed, "plant", 0, layer0 + i).standard_normal((cfg.hkv, cfg.d))
        out[i] = (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32)
    return out


def plant_prefill(cfg, seed: int, k, layer0: int = 0):
    """Writes the planted keys into prefill keys k [nl, B, Hkv, L0, d] (numpy
    or torch, in place)."""
    if not cfg.plant_depths:
        return k
    pos = plant_positions(cfg)
    u = plant_directions(cfg, seed, layer0, k.shape[0]) * np.float32(cfg.plant_beta)
    for b, p in enumerate(pos.tolist()):
        if isinstance(k, np.ndarray):
            k[:, b, :, p, :] = u.astype(k.dtype)
        else:
            import torch
            k[:, b, :, p, :] = torch.as_tensor(u, device=k.device).to(k.dtype)
    return k


def plant_queries(cfg, seed: int, q, layer0: int = 0):
    """Adds plant_gamma * u to every decode query q [nl, B, Hq, d] (in place)."""
    if not cfg.plant_depths:
        return q
    g = cfg.hq // cfg.hkv
    u = np.repeat(plant_directions(cfg, seed, layer0, q.shape[0]), g, axis=1) * np.float32(cfg.plant_gamma)
    if isinstance(q, np.ndarray):
        q[...] = (q.astype(np.float32) + u[:, None]).astype(q.dtype)
    else:
        import torch
        q += torch.as_tensor(u, device=q.device)[:, None].to(q.dtype)
    return q
