"""The allocation-free compaction entry point against the workspace one.

confk_ema_compact_static keeps its scratch in a static device array of the
library instead of a caller workspace. Through the C ABI, two engines run the
same seeded steps: one calls confk_ema_compact with its workspace, the other
confk_ema_compact_static; after every call the two caches and step outputs
must be identical bit for bit (both run the same kernels, so the bar for the
integer and byte state and for the fp32 EMA and scores is exact equality).
Two calls in a row on different caches, the second smaller than the first,
show that the array's leftover contents from a larger call do not leak into
a smaller one; a call beyond the array's limit is rejected before any launch.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _cfg(name, layers, batch, hq, hkv, d, vocab, prefill, n_high, n_low, protect, window, **kw):
    pol = synth.Policy(n_high=n_high, n_low=n_low, protect=protect, window=window, **kw)
    return synth.Config(name=name, layers=layers, batch=batch, hq=hq, hkv=hkv, d=d, vocab=vocab,
                        prefill=prefill, steps=0, policy=pol)


def _same(a, b, what):
    import mixed_precision_attention_amd as M
    for name in ("meta", "k8", "v8", "k16", "v16", "kscale", "vscale", "status"):
        assert torch.equal(getattr(a.cache, name), getattr(b.cache, name)), (what, name)
    nlen = a.cache.meta[..., M.META_N].cpu().numpy()
    for l in range(nlen.shape[0]):
        for bb in range(nlen.shape[1]):
            n = int(nlen[l, bb])
            for name in ("ema", "pos"):
                x, y = getattr(a.cache, name)[l, bb, :n], getattr(b.cache, name)[l, bb, :n]
                assert torch.equal(x, y), (what, name, l, bb)
            assert torch.equal(a.score[l, bb, :n], b.score[l, bb, :n]), (what, "score", l, bb)
    assert torch.equal(a.evicted, b.evicted), (what, "evicted")


def _pair(cfg, seed):
    import mixed_precision_attention_amd as M
    dev = torch.device("cuda")
    ws_eng, st_eng = M.DecodeEngine(cfg, dev), M.DecodeEngine(cfg, dev)
    kp, vp = synth.prefill_kv(cfg, seed)
    kp, vp = torch.from_numpy(kp).to(dev), torch.from_numpy(vp).to(dev)
    for e in (ws_eng, st_eng):
        e.prefill(kp, vp)
    return ws_eng, st_eng


def _step(ws_eng, st_eng, cfg, seed, i):
    import mixed_precision_attention_amd as M
    dev = torch.device("cuda")
    lg = torch.from_numpy(synth.logits_for_step(cfg, seed, i)).to(dev)
    q, kn, vn = (torch.from_numpy(x).to(dev) for x in synth.decode_inputs(cfg, seed, i))
    t = cfg.prefill + i
    for e in (ws_eng, st_eng):
        e.step_confidence(lg)
        e.step_attention(q, kn, vn)
    ws_eng.step_ema_compact(t, kn, vn, fuse_quantize=True)
    M.engine.ema_compact_static(st_eng.cache, st_eng.mass, st_eng.pol, t, st_eng.score, st_eng.budget,
                                st_eng.budget_stride, kn, vn, st_eng.evicted, fuse_quantize=True)
    torch.cuda.synchronize()
    return int((ws_eng.evicted > 0).sum())


def test_static_scratch_matches_workspace_on_two_calls_second_smaller():
    import mixed_precision_attention_amd as M
    M.load()
    # call 1: a larger cache (2 layers x 3 sequences, GQA 5, d128, 301 slots;
    # the first step evicts about 100 tokens per sequence and moves rows)
    big = _cfg("na_big", 2, 3, 10, 2, 128, 1000, 300, 96, 200, 16, 64)
    # call 2: a smaller one (1 layer x 2 sequences, MHA d64, 151 slots)
    small = _cfg("na_small", 1, 2, 4, 4, 64, 777, 150, 40, 80, 8, 32)
    assert M.engine.workspace_bytes(M._lib.WS_COMPACT, M.DeviceCache.for_config(small, "cuda"), nlayers=1) < \
        M.engine.workspace_bytes(M._lib.WS_COMPACT, M.DeviceCache.for_config(big, "cuda"), nlayers=2)
    print("[no-alloc] call 1 (larger cache)", flush=True)
    a1, b1 = _pair(big, 3)
    ev = _step(a1, b1, big, 3, 0)
    assert ev > 0 and int(b1.cache.meta[..., M.META_MOVED].max()) > 0  # rows moved in the static call
    _same(a1, b1, "call 1")
    print("[no-alloc] call 2 (smaller cache)", flush=True)
    a2, b2 = _pair(small, 4)
    ev = _step(a2, b2, small, 4, 0)
    assert ev > 0
    _same(a2, b2, "call 2")
    # a few more steps on the smaller pair keep agreeing (the window step and
    # later evictions through the static array)
    for i in range(1, 6):
        _step(a2, b2, small, 4, i)
        _same(a2, b2, f"call 2 step {i}")


def test_static_scratch_rejects_calls_beyond_its_limit():
    import ctypes
    import mixed_precision_attention_amd as M
    lib = M.load()
    # 64 layers x 8 sequences x 32770 slots need far more than 64 MiB
    cfg = _cfg("na_huge", 64, 8, 8, 8, 64, 100, 32769, 16, 32, 8, 16)
    c = M._lib.Cache(cfg.layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d, cfg.cap, cfg.policy.window + 1,
                     *([0x1000] * 10))
    need = lib.confk_workspace_size(M._lib.WS_COMPACT, ctypes.byref(c), cfg.layers, 0, 0)
    assert need > M._lib.STATIC_SCRATCH_BYTES
    pol = M.engine.make_policy(cfg.policy)
    fake = ctypes.c_void_p(0x1000)
    code = lib.confk_ema_compact_static(ctypes.byref(c), 0, cfg.layers, fake, ctypes.byref(pol), 5, fake, fake,
                                        0, fake, fake, None, 0, None)
    assert code == M.ERR_WORKSPACE
