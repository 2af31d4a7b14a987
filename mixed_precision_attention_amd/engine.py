"""Device memory (PyTorch) and the call sequence of one CONF-KV decode step.

Algorithm 1 of the CONF-KV review ("方法步骤详情"): confidence and budget from
the logits, attention with per-key mass, EMA and rank, eviction/compaction
with the append of the new token, and quantisation of the token that left
the FP16 window. Each function below forwards pointers, sizes and the
current HIP stream to one C-ABI entry point; nothing is computed here.
"""
import ctypes
import dataclasses

import numpy as np
import torch

from . import _lib as L


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_policy(p) -> L.Policy:
    """C policy struct from any object with tau, alpha, lam, w_h, w_m, w_p,
    n_high, n_low, protect, window and (optionally) block and order attributes."""
    return L.Policy(float(p.tau), float(p.alpha), float(p.lam), float(p.w_h), float(p.w_m),
                    float(p.w_p), int(p.n_high), int(p.n_low), int(p.protect), int(p.window),
                    int(getattr(p, "block", 0)), int(getattr(p, "order", 0)))


class DeviceCache:
    """The cache tensors of include/confk.h, owned by PyTorch."""

    def __init__(self, layers, batch, hq, hkv, d, cap, cap16, device="cuda"):
        self.layers, self.batch, self.hq, self.hkv, self.d = layers, batch, hq, hkv, d
        self.cap, self.cap16 = cap, cap16
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
        self.k8 = z((layers, batch, hkv, cap, d), torch.int8)
        self.v8 = z((layers, batch, hkv, cap, d), torch.int8)
        self.k16 = z((layers, batch, hkv, cap16, d), torch.float16)
        self.v16 = z((layers, batch, hkv, cap16, d), torch.float16)
        self.kscale = z((layers, batch, hkv, d), torch.float32)
        self.vscale = z((layers, batch, hkv, d), torch.float32)
        self.ema = z((layers, batch, cap), torch.float32)
        self.pos = z((layers, batch, cap), torch.int32)
        self.meta = z((layers, batch, L.META_WORDS), torch.int32)
        self.status = z((1,), torch.int32)
        self.struct = L.Cache(layers, batch, hq, hkv, d, cap, cap16,
                              self.k8.data_ptr(), self.v8.data_ptr(), self.k16.data_ptr(),
                              self.v16.data_ptr(), self.kscale.data_ptr(), self.vscale.data_ptr(),
                              self.ema.data_ptr(), self.pos.data_ptr(), self.meta.data_ptr(),
                              self.status.data_ptr())

    @classmethod
    def for_config(cls, cfg, device="cuda"):
        return cls(cfg.layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d, cfg.cap, cfg.policy.window + 1,
                   device)

    def ref(self):
        return ctypes.byref(self.struct)

    # -------------------------------------------------------- inspection
    def lengths(self):
        m = self.meta.cpu().numpy()
        return m[..., L.META_N], m[..., L.META_N8]

    def mass_rows(self):
        """Rows of partial mass sums of each (layer, sequence) from the last
        attention call (the meta word; 0 in a fresh cache reads as hkv)."""
        r = self.meta[..., L.META_MASSROWS].cpu().numpy()
        return np.where((r >= 1) & (r <= self.hkv), r, self.hkv)

    def snapshot(self, l, b):
        """Host copy of one (layer, sequence) in logical order (INT8 part first)."""
        m = self.meta[l, b].cpu().numpy()
        n, n8, b8, b16 = int(m[L.META_N]), int(m[L.META_N8]), int(m[L.META_BASE8]), int(m[L.META_BASE16])
        f = n - n8
        i8 = torch.as_tensor((b8 + np.arange(n8)) % self.cap, device=self.k8.device, dtype=torch.long)
        i16 = torch.as_tensor((b16 + np.arange(f)) % self.cap16, device=self.k8.device, dtype=torch.long)
        g = lambda t, idx: t[l, b].index_select(1, idx).permute(1, 0, 2).cpu().numpy()  # noqa: E731
        return dict(
            n=n, n8=n8, base8=b8, base16=b16, calibrated=bool(m[L.META_CALIB]),
            saturated=int(m[L.META_SAT]), evicted=int(m[L.META_EVICTED]), moved=int(m[L.META_MOVED]),
            k8=g(self.k8, i8), v8=g(self.v8, i8), k16=g(self.k16, i16), v16=g(self.v16, i16),
            ks=self.kscale[l, b].cpu().numpy(), vs=self.vscale[l, b].cpu().numpy(),
            ema=self.ema[l, b, :n].cpu().numpy(), pos=self.pos[l, b, :n].cpu().numpy(),
        )


# ------------------------------------------------------------------ calls

def confidence(logits, pol, c_out, budget_out, status, ws, layer_n_high=None, layer_n_low=None,
               token_out=None, temperature=0.0, uniform=None):
    lib = L.load()
    nbl = 1 if layer_n_high is None else int(layer_n_high.numel())
    L.check("confk_confidence", lib.confk_confidence(
        _p(logits), logits.stride(0), logits.shape[0], logits.shape[1], ctypes.byref(pol),
        _p(layer_n_high), _p(layer_n_low), nbl, _p(c_out), _p(budget_out), _p(status),
        _p(uniform), float(temperature), _p(token_out), _p(ws), ws.numel() * ws.element_size(),
        _stream()))


def confidence_attn_decode(logits, pol, c_out, budget_out, status, conf_ws, cache, q, k_new, v_new, out,
                           mass, attn_ws, layer_n_high=None, layer_n_low=None, token_out=None,
                           temperature=0.0, uniform=None, layer0=0, nlayers=None):
    """confk_confidence_attn_decode: confidence then attention in two launches
    (the confidence merge runs in the attention launch), same results."""
    lib = L.load()
    nbl = 1 if layer_n_high is None else int(layer_n_high.numel())
    nl = cache.layers - layer0 if nlayers is None else nlayers
    awsb = 0 if attn_ws is None else attn_ws.numel() * attn_ws.element_size()
    L.check("confk_confidence_attn_decode", lib.confk_confidence_attn_decode(
        _p(logits), logits.stride(0), logits.shape[0], logits.shape[1], ctypes.byref(pol),
        _p(layer_n_high), _p(layer_n_low), nbl, _p(c_out), _p(budget_out), _p(status),
        _p(uniform), float(temperature), _p(token_out), _p(conf_ws), conf_ws.numel() * conf_ws.element_size(),
        cache.ref(), layer0, nl, _p(q), _p(k_new), _p(v_new), _p(out), _p(mass), _p(attn_ws), awsb,
        _stream()))


def decode_step(logits, pol, c_out, budget_out, cache, t, q, k_new, v_new, out, mass, score, conf_ws, attn_ws,
                compact_ws, layer_n_high=None, layer_n_low=None, token_out=None, temperature=0.0, uniform=None,
                evicted=None, fuse_quantize=True, layer0=0, nlayers=None):
    """confk_decode_step: confidence, attention, EMA + rank + compaction (and
    the window step) in three launches, same results as the five calls."""
    lib = L.load()
    nbl = 1 if layer_n_high is None else int(layer_n_high.numel())
    nl = cache.layers - layer0 if nlayers is None else nlayers
    wsb = lambda w: 0 if w is None else w.numel() * w.element_size()  # noqa: E731
    L.check("confk_decode_step", lib.confk_decode_step(
        _p(logits), logits.stride(0), logits.shape[1], ctypes.byref(pol), _p(layer_n_high), _p(layer_n_low), nbl,
        _p(c_out), _p(budget_out), _p(uniform), float(temperature), _p(token_out), cache.ref(), layer0, nl, int(t),
        _p(q), _p(k_new), _p(v_new), _p(out), _p(mass), _p(score), _p(evicted),
        L.FUSE_QUANTIZE if fuse_quantize else 0, _p(conf_ws), wsb(conf_ws), _p(attn_ws), wsb(attn_ws),
        _p(compact_ws), wsb(compact_ws), _stream()))


def attn_decode(cache, q, k_new, v_new, out, mass, ws, layer0=0, nlayers=None):
    lib = L.load()
    nl = cache.layers - layer0 if nlayers is None else nlayers
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    L.check("confk_attn_decode", lib.confk_attn_decode(
        cache.ref(), layer0, nl, _p(q), _p(k_new), _p(v_new), _p(out), _p(mass), _p(ws), wsb,
        _stream()))


def ema_rank(cache, mass, pol, t, score, layer0=0, nlayers=None):
    lib = L.load()
    nl = cache.layers - layer0 if nlayers is None else nlayers
    L.check("confk_ema_rank", lib.confk_ema_rank(
        cache.ref(), layer0, nl, _p(mass), ctypes.byref(pol), int(t), _p(score), _stream()))


def compact(cache, budget, budget_stride, score, pol, k_new, v_new, ws, evicted=None, layer0=0,
            nlayers=None):
    lib = L.load()
    nl = cache.layers - layer0 if nlayers is None else nlayers
    L.check("confk_compact", lib.confk_compact(
        cache.ref(), layer0, nl, _p(budget), int(budget_stride), _p(score), ctypes.byref(pol),
        _p(k_new), _p(v_new), _p(evicted), _p(ws), ws.numel() * ws.element_size(), _stream()))


def ema_compact(cache, mass, pol, t, score, budget, budget_stride, k_new, v_new, ws, evicted=None,
                layer0=0, nlayers=None, fuse_quantize=False):
    """confk_ema_compact: ema_rank and compact in one launch (and, with
    fuse_quantize, the window step of quantize after the append)."""
    lib = L.load()
    nl = cache.layers - layer0 if nlayers is None else nlayers
    L.check("confk_ema_compact", lib.confk_ema_compact(
        cache.ref(), layer0, nl, _p(mass), ctypes.byref(pol), int(t), _p(score), _p(budget),
        int(budget_stride), _p(k_new), _p(v_new), _p(evicted), L.FUSE_QUANTIZE if fuse_quantize else 0, _p(ws),
        ws.numel() * ws.element_size(), _stream()))


def ema_compact_static(cache, mass, pol, t, score, budget, budget_stride, k_new, v_new, evicted=None,
                       layer0=0, nlayers=None, fuse_quantize=False):
    """confk_ema_compact_static: ema_compact with the library's static
    scratch instead of a workspace (for callers that cannot allocate)."""
    lib = L.load()
    nl = cache.layers - layer0 if nlayers is None else nlayers
    L.check("confk_ema_compact_static", lib.confk_ema_compact_static(
        cache.ref(), layer0, nl, _p(mass), ctypes.byref(pol), int(t), _p(score), _p(budget),
        int(budget_stride), _p(k_new), _p(v_new), _p(evicted), L.FUSE_QUANTIZE if fuse_quantize else 0,
        _stream()))


def quantize(cache, pol, t, mode=L.QUANT_STEP, k_src=None, v_src=None, n_src=0, layer0=0,
             nlayers=None):
    lib = L.load()
    nl = cache.layers - layer0 if nlayers is None else nlayers
    L.check("confk_quantize", lib.confk_quantize(
        cache.ref(), layer0, nl, int(t), ctypes.byref(pol), int(mode), _p(k_src), _p(v_src),
        int(n_src), _stream()))


def read_probe(buf, sink):
    """One streaming read of the device buffer `buf` (a measurement aid, in
    libconfk_probe.so); `sink` (device uint32 [1]) is XOR-ed with the XOR of
    its 32-bit words."""
    lib = L.load_probe()
    L.check("confk_read_probe", lib.confk_read_probe(
        _p(buf), buf.numel() * buf.element_size(), _p(sink), _stream()))


def workspace_bytes(which, cache=None, nlayers=0, batch=0, vocab=0):
    lib = L.load()
    ref = cache.ref() if cache is not None else None
    return int(lib.confk_workspace_size(which, ref, nlayers, batch, vocab))


class DecodeEngine:
    """Buffers of one decode step for a workload config, and the step itself."""

    def __init__(self, cfg, device="cuda", overlap=False, split_keys=True):
        self.cfg = cfg
        # split_keys=False sizes the attention workspace without the split
        # exchange area, so every attention launch runs one workgroup per
        # (layer, sequence, kv head) (or two kv heads per workgroup) instead
        # of spreading a unit's keys over several workgroups when the launch
        # would leave most of the GPU idle.
        # overlap=True: confidence reads only the logits and feeds only the
        # compaction, so step() may run it on a second stream (default
        # priority) beside the attention launch. Off by default: in a model the
        # logits of a step come out of that step's forward pass, after its
        # attention.
        self.side = torch.cuda.Stream(device=device) if overlap else None
        self.conf_done = torch.cuda.Event() if overlap else None
        self.pol = make_policy(cfg.policy)
        self.cache = DeviceCache.for_config(cfg, device)
        Lr, B = cfg.layers, cfg.batch
        self.layer_n_low = self.layer_n_high = None
        nbl = 1
        if cfg.layer_n_low is not None:
            self.layer_n_low = torch.tensor(cfg.layer_n_low, dtype=torch.int32, device=device)
            self.layer_n_high = torch.tensor(cfg.layer_n_high, dtype=torch.int32, device=device)
            nbl = Lr
            # the host checks capacity and protection against the largest budgets
            self.pol = make_policy(dataclasses.replace(
                cfg.policy, n_low=max(cfg.layer_n_low), n_high=max(cfg.layer_n_high)))
        self.budget_stride = B if nbl > 1 else 0
        self.c = torch.zeros(B, dtype=torch.float32, device=device)
        self.budget = torch.zeros((nbl, B), dtype=torch.int32, device=device)
        cws = workspace_bytes(L.WS_CONFIDENCE, batch=B, vocab=cfg.vocab)
        self.conf_ws = torch.zeros(max(cws, 4), dtype=torch.uint8, device=device)
        aws = workspace_bytes(L.WS_ATTENTION if split_keys else L.WS_ATTENTION_NOSPLIT, self.cache, nlayers=Lr)
        self.attn_ws = torch.zeros(aws, dtype=torch.uint8, device=device) if aws else None
        kws = workspace_bytes(L.WS_COMPACT, self.cache, nlayers=Lr)
        self.compact_ws = torch.zeros(kws, dtype=torch.uint8, device=device)
        self.out = torch.zeros((Lr, B, cfg.hq, cfg.d), dtype=torch.float16, device=device)
        self.mass = torch.zeros((Lr, B, cfg.hkv, cfg.cap), dtype=torch.float32, device=device)
        self.score = torch.zeros((Lr, B, cfg.cap), dtype=torch.float32, device=device)
        self.evicted = torch.zeros((Lr, B), dtype=torch.int32, device=device)
        self.token = torch.zeros(B, dtype=torch.int32, device=device)
        if cfg.mode == "full_kv":
            self.budget.fill_(cfg.policy.n_low)

    def prefill(self, k_src, v_src):
        """k_src, v_src fp16 [L, B, Hkv, L0, d] on the device (L0 may be 0)."""
        n_src = 0 if k_src is None else k_src.shape[3]
        quantize(self.cache, self.pol, 0, L.QUANT_PREFILL, k_src, v_src, n_src)

    # the five calls of one step, in the order of the method
    def step_confidence(self, logits, temperature=None, uniform=None):
        """Confidence and budgets; with temperature given (0 = greedy) also the
        next token of every sequence into self.token, in the same pass."""
        confidence(logits, self.pol, self.c, self.budget, self.cache.status, self.conf_ws,
                   self.layer_n_high, self.layer_n_low,
                   token_out=None if temperature is None else self.token,
                   temperature=0.0 if temperature is None else temperature, uniform=uniform)

    def step_attention(self, q, k_new, v_new):
        attn_decode(self.cache, q, k_new, v_new, self.out, self.mass, self.attn_ws)

    def step_confidence_attention(self, logits, q, k_new, v_new, temperature=None, uniform=None):
        """step_confidence then step_attention as one call (two launches: the
        confidence merge runs inside the attention launch), same results."""
        confidence_attn_decode(logits, self.pol, self.c, self.budget, self.cache.status, self.conf_ws,
                               self.cache, q, k_new, v_new, self.out, self.mass, self.attn_ws,
                               self.layer_n_high, self.layer_n_low,
                               token_out=None if temperature is None else self.token,
                               temperature=0.0 if temperature is None else temperature, uniform=uniform)

    def step_ema_rank(self, t):
        ema_rank(self.cache, self.mass, self.pol, t, self.score)

    def step_compact(self, k_new, v_new):
        compact(self.cache, self.budget, self.budget_stride, self.score, self.pol, k_new, v_new,
                self.compact_ws, self.evicted)

    def step_ema_compact(self, t, k_new, v_new, fuse_quantize=False):
        """EMA, rank scores and compaction in one launch (same state as
        step_ema_rank followed by step_compact; with fuse_quantize, also as
        step_quantize after them)."""
        ema_compact(self.cache, self.mass, self.pol, t, self.score, self.budget, self.budget_stride,
                    k_new, v_new, self.compact_ws, self.evicted, fuse_quantize=fuse_quantize)

    def step_quantize(self, t):
        quantize(self.cache, self.pol, t)

    def step_attention_layerwise(self, q, k_new, v_new):
        """step_attention as one launch per layer, in layer order, as a
        model's forward pass issues it. A launch over one layer has few
        units, so at batch 1 it may split each unit's keys over several
        workgroups."""
        for l in range(self.cfg.layers):
            attn_decode(self.cache, q[l:], k_new[l:], v_new[l:], self.out[l:], self.mass[l:], self.attn_ws,
                        layer0=l, nlayers=1)

    def capture_attention_layerwise(self, q, k_new, v_new):
        """A HIP graph of step_attention_layerwise over the buffers q, k_new
        and v_new (the caller copies each step's inputs into them before a
        replay): 64 one-layer launches cost one graph launch from the host.
        The launches record no memory-set node, and split keys keep their
        exchange words valid across replays (a per-unit epoch in device
        memory). Call after a warm-up step, which makes the library's
        one-time device queries outside the capture."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step_attention_layerwise(q, k_new, v_new)
        return graph

    def step_layerwise(self, logits, q, k_new, v_new, t):
        """One step with attention issued per layer: the confidence pass, one
        attention launch per layer, then the EMA, rank scores, compaction and
        window step as one launch over all layers (the review's Algorithm 1
        runs the per-layer eviction loop after the forward pass)."""
        self.step_confidence(logits)
        self.step_attention_layerwise(q, k_new, v_new)
        self.step_ema_compact(t, k_new, v_new, fuse_quantize=True)

    def step(self, logits, q, k_new, v_new, t):
        if self.cfg.mode == "full_kv":
            # comparison run: attention output only, then the append (the
            # budget covers every token, so nothing is evicted or quantised).
            # With no attention mass the rank call writes only the new
            # token's metadata slot (position t), which the append stores.
            attn_decode(self.cache, q, k_new, v_new, self.out, None, None)
            ema_rank(self.cache, None, self.pol, t, self.score)
            self.step_compact(k_new, v_new)
            return
        if self.side is None:  # one stream: the whole-step call (three launches)
            decode_step(logits, self.pol, self.c, self.budget, self.cache, t, q, k_new, v_new, self.out,
                        self.mass, self.score, self.conf_ws, self.attn_ws, self.compact_ws,
                        self.layer_n_high, self.layer_n_low, evicted=self.evicted)
            return
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)  # the logits, and the previous step's use of the budget
        with torch.cuda.stream(self.side):
            self.step_confidence(logits)
        self.conf_done.record(self.side)
        self.step_attention(q, k_new, v_new)
        main.wait_event(self.conf_done)
        self.step_ema_compact(t, k_new, v_new, fuse_quantize=True)
