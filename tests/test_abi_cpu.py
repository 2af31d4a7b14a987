"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import mixed_precision_attention_amd as M
from mixed_precision_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "confk.h")
PROBE_HEADER = os.path.join(ROOT, "include", "confk_probe.h")


def declared(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(confk_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_five_calls():
    names = declared()
    for n in ("confk_confidence", "confk_attn_decode", "confk_ema_rank", "confk_compact", "confk_quantize"):
        assert n in names
    assert set(names) == set(_lib.EXPORTS)


def test_every_header_is_covered():
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["confk.h", "confk_probe.h"]
    assert declared(PROBE_HEADER) == sorted(_lib.PROBE_EXPORTS)
    assert not set(declared()) & set(declared(PROBE_HEADER))


def test_probe_library_exports_its_symbol():
    probe = _lib.load_probe()
    for n in declared(PROBE_HEADER):
        assert hasattr(probe, n), n


def test_product_library_does_not_export_the_probe(lib):
    assert not hasattr(lib, "confk_read_probe")


def test_library_exports_every_declared_symbol(lib):
    for n in declared():
        assert hasattr(lib, n), n
    assert lib.confk_version() == 107
    assert lib.confk_strerror(-1) == b"invalid argument"
    assert lib.confk_strerror(12345) == b"unknown error"


def test_binding_constants_match_header():
    """Every constant the binding mirrors (status bits, workspace selectors,
    modes) has the header's value."""
    import re
    vals = dict(re.findall(r"#define CONFK_(\w+) (-?\d+)u?\b", open(HEADER).read()))
    mirrored = [n for n in vals if hasattr(_lib, n)]
    assert {"STATUS_SPLIT_WAIT", "WS_ATTENTION", "WS_ATTENTION_NOSPLIT", "WS_COMPACT"} <= set(mirrored)
    for n in mirrored:
        assert getattr(_lib, n) == int(vals[n]), n


def test_struct_layout_matches_header():
    # 7 int32 dims, 4 bytes padding, 10 pointers
    assert ctypes.sizeof(_lib.Cache) == 7 * 4 + 4 + 10 * 8
    assert _lib.Cache.k8.offset == 32
    assert ctypes.sizeof(_lib.Policy) == 12 * 4
    assert _lib.Policy.block.offset == 40
    assert _lib.Policy.order.offset == 44


def _fake_cache(**kw):
    dims = dict(layers=2, batch=3, hq=10, hkv=2, d=128, cap=100, cap16=65)
    dims.update(kw)
    c = _lib.Cache(dims["layers"], dims["batch"], dims["hq"], dims["hkv"], dims["d"], dims["cap"],
                   dims["cap16"], *([0x1000] * 10))
    return c


def _pol(**kw):
    p = dict(tau=0.7, alpha=0.65, lam=0.9, w_h=0.4, w_m=0.3, w_p=0.3, n_high=24, n_low=48,
             protect=8, window=64, block=0, order=0)
    p.update(kw)
    return _lib.Policy(p["tau"], p["alpha"], p["lam"], p["w_h"], p["w_m"], p["w_p"], p["n_high"],
                       p["n_low"], p["protect"], p["window"], p["block"], p["order"])


FAKE = ctypes.c_void_p(0x1000)


def test_confidence_validation(lib):
    pol = _pol()
    ok_args = dict(logits=FAKE, ld=10, batch=2, vocab=10, nbl=1, ws=FAKE, wsb=1 << 20, uniform=None,
                   temperature=0.0, token=None)

    def call(**kw):
        a = dict(ok_args)
        a.update(kw)
        return lib.confk_confidence(a["logits"], a["ld"], a["batch"], a["vocab"], ctypes.byref(pol),
                                    None, None, a["nbl"], FAKE, FAKE, None, a["uniform"], a["temperature"],
                                    a["token"], a["ws"], a["wsb"], None)
    assert call(logits=None) == M.ERR_INVALID_ARG
    assert call(vocab=1) == M.ERR_INVALID_ARG
    assert call(ld=5) == M.ERR_INVALID_ARG
    assert call(batch=0) == M.ERR_INVALID_ARG
    assert call(nbl=2) == M.ERR_INVALID_ARG          # per-layer count without arrays
    assert call(ws=None) == M.ERR_WORKSPACE
    assert call(wsb=4) == M.ERR_WORKSPACE
    assert call(temperature=-1.0) == M.ERR_INVALID_ARG
    assert call(temperature=float("nan")) == M.ERR_INVALID_ARG
    assert call(temperature=float("inf")) == M.ERR_INVALID_ARG
    assert call(temperature=0.8, token=FAKE) == M.ERR_INVALID_ARG   # sampling needs uniforms
    assert lib.confk_confidence(FAKE, 10, 2, 10, ctypes.byref(pol), FAKE, None, 2, FAKE, FAKE, None,
                                None, 0.0, None, FAKE, 1 << 20, None) == M.ERR_INVALID_ARG


def test_attention_validation(lib):
    c = _fake_cache()
    r = lambda cc, l0=0, nl=2, ws=FAKE, wsb=1 << 30: lib.confk_attn_decode(  # noqa: E731
        ctypes.byref(cc), l0, nl, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)
    assert r(_fake_cache(d=96)) == M.ERR_UNSUPPORTED
    assert r(_fake_cache(hq=40, hkv=2)) == M.ERR_UNSUPPORTED     # group of 20 > 16
    assert r(_fake_cache(hq=9, hkv=2)) == M.ERR_INVALID_ARG      # not a multiple
    assert r(c, l0=1, nl=2) == M.ERR_INVALID_ARG
    assert r(c, nl=0) == M.ERR_INVALID_ARG
    bad = _fake_cache()
    bad.meta = None
    assert r(bad) == M.ERR_INVALID_ARG
    assert lib.confk_attn_decode(ctypes.byref(c), 0, 2, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) \
        == M.ERR_INVALID_ARG


def test_fused_confidence_attention_validation(lib):
    """Each argument set of confk_confidence_attn_decode is validated as in
    its own call, before anything is launched."""
    pol = _pol()
    c = _fake_cache()

    def call(logits=FAKE, vocab=10, conf_ws=FAKE, conf_wsb=1 << 20, cache=c, nl=2, q=FAKE, temperature=0.0,
             token=None, uniform=None):
        return lib.confk_confidence_attn_decode(
            logits, 10, 3, vocab, ctypes.byref(pol), None, None, 1, FAKE, FAKE, None, uniform, temperature,
            token, conf_ws, conf_wsb, ctypes.byref(cache), 0, nl, q, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert call(logits=None) == M.ERR_INVALID_ARG
    assert call(vocab=1) == M.ERR_INVALID_ARG
    assert call(conf_ws=None) == M.ERR_WORKSPACE
    assert call(conf_wsb=4) == M.ERR_WORKSPACE
    assert call(temperature=0.8, token=FAKE) == M.ERR_INVALID_ARG   # sampling needs uniforms
    assert call(q=None) == M.ERR_INVALID_ARG
    assert call(nl=3) == M.ERR_INVALID_ARG
    assert call(cache=_fake_cache(d=96)) == M.ERR_UNSUPPORTED


def test_decode_step_validation(lib):
    """confk_decode_step validates the three calls' argument sets (and its
    own) before anything is launched."""
    pol = _pol()
    c = _fake_cache()
    big = 1 << 30

    def call(logits=FAKE, nbl=1, lnh=None, lnl=None, mass=FAKE, t=5, flags=0, conf_ws=FAKE, attn_ws=FAKE,
             compact_ws=FAKE, cwsb=big, q=FAKE, score=FAKE, cache=c, nl=2):
        return lib.confk_decode_step(
            logits, 10, 10, ctypes.byref(pol), lnh, lnl, nbl, FAKE, FAKE, None, 0.0, None, ctypes.byref(cache), 0,
            nl, t, q, FAKE, FAKE, FAKE, mass, score, None, flags, conf_ws, big, attn_ws, big, compact_ws, cwsb,
            None)
    assert call(logits=None) == M.ERR_INVALID_ARG
    assert call(mass=None) == M.ERR_INVALID_ARG
    assert call(t=-1) == M.ERR_INVALID_ARG
    assert call(flags=4) == M.ERR_INVALID_ARG
    assert call(nbl=3, lnh=FAKE, lnl=FAKE) == M.ERR_INVALID_ARG   # neither 1 nor nlayers
    assert call(conf_ws=None) == M.ERR_WORKSPACE
    assert call(compact_ws=None) == M.ERR_WORKSPACE
    assert call(cwsb=4) == M.ERR_WORKSPACE
    assert call(q=None) == M.ERR_INVALID_ARG
    assert call(score=None) == M.ERR_INVALID_ARG
    assert call(nl=3) == M.ERR_INVALID_ARG
    assert call(cache=_fake_cache(d=96)) == M.ERR_UNSUPPORTED


def _split_words(g, d):
    # per unit: the epoch word and a spare, 16 splits x 16 heads x (max,
    # normaliser), 16 output partials of g x d values; 8 bytes each
    return 2 + 16 * 32 + 16 * g * d


def test_attention_workspace_sizes(lib):
    """The attention workspace is the score spill area (caches too long for
    on-chip memory), then the split exchange area for min(units, 64) (layer,
    sequence, kv head) units at the next 256-byte boundary."""
    ws = lambda c, nl, which=M._lib.WS_ATTENTION: lib.confk_workspace_size(which, ctypes.byref(c), nl, 0, 0)  # noqa: E731
    small = _fake_cache(cap=300)  # 2 x 3 x 2 units, g = 5, d = 128; no spill
    assert ws(small, 2, M._lib.WS_ATTENTION_NOSPLIT) == 0
    assert ws(small, 2) == 12 * _split_words(5, 128) * 8
    big = _fake_cache(cap=40000, hq=40, hkv=8)  # 48 units whose scores spill
    spill = ws(big, 2, M._lib.WS_ATTENTION_NOSPLIT)
    assert spill > 0
    assert ws(big, 2) == (spill + 255) // 256 * 256 + 48 * _split_words(5, 128) * 8
    many = _fake_cache(layers=64, batch=8, hq=40, hkv=8, cap=2050)  # 4096 units, no spill
    assert ws(many, 64, M._lib.WS_ATTENTION_NOSPLIT) == 0
    assert ws(many, 64) == 64 * _split_words(5, 128) * 8
    wide = _fake_cache(layers=64, batch=2, hq=128, hkv=8, d=64, cap=300)  # g = 16, 1024 units, no spill
    assert ws(wide, 64, M._lib.WS_ATTENTION_NOSPLIT) == 0
    assert ws(wide, 64) == 64 * _split_words(16, 64) * 8
    assert lib.confk_attn_decode(ctypes.byref(big), 0, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, spill - 4,
                                 None) == M.ERR_WORKSPACE
    assert lib.confk_workspace_size(M._lib.WS_CONFIDENCE, None, 0, 8, 152064) == 8 * 38 * 8 * 4


def test_compact_quantize_ema_validation(lib):
    c = _fake_cache(cap=100, cap16=65)
    pol = _pol()
    wsb = lib.confk_workspace_size(M._lib.WS_COMPACT, ctypes.byref(c), 2, 0, 0)
    assert wsb == 2 * 3 * (16 + 2 * 100) * 4 + 256  # plans, then one job flag per (layer, sequence) padded to 256 B
    cp = lambda cc, p, stride=0, ws=FAKE, n=wsb: lib.confk_compact(  # noqa: E731
        ctypes.byref(cc), 0, 2, FAKE, stride, FAKE, ctypes.byref(p), FAKE, FAKE, None, ws, n, None)
    assert cp(c, _pol(), ws=None) == M.ERR_WORKSPACE
    assert cp(c, _pol(), n=wsb - 1) == M.ERR_WORKSPACE
    assert cp(c, _pol(protect=30)) == M.ERR_BUDGET             # P > N_high
    assert cp(c, _pol(n_low=99)) == M.ERR_BUDGET               # no slot for N_low + 1 + new
    assert cp(c, _pol(window=64), stride=5) == M.ERR_INVALID_ARG
    assert cp(c, _pol(window=80)) == M.ERR_BUDGET              # FP16 ring too small
    assert cp(c, _pol(lam=1.5)) == M.ERR_INVALID_ARG
    assert cp(c, _pol(protect=20, window=16, n_high=24, order=1)) == M.ERR_BUDGET  # P > W, fill order
    assert cp(c, _pol(order=2)) == M.ERR_INVALID_ARG          # unknown survivor order
    assert cp(c, _pol(order=-1)) == M.ERR_INVALID_ARG
    assert cp(c, _pol(block=8)) == M.ERR_INVALID_ARG          # blocks below 16 tokens
    assert cp(c, _pol(block=-16)) == M.ERR_INVALID_ARG
    big = _fake_cache(cap=16 * 513, cap16=65)                 # 513 blocks of 16
    wbig = lib.confk_workspace_size(M._lib.WS_COMPACT, ctypes.byref(big), 2, 0, 0)
    assert cp(big, _pol(block=16), n=wbig) == M.ERR_UNSUPPORTED
    # the fused EMA + compaction call validates like the two calls it replaces
    ec = lambda cc, p, mass=FAKE, t=5, ws=FAKE, n=wsb, flags=0: lib.confk_ema_compact(  # noqa: E731
        ctypes.byref(cc), 0, 2, mass, ctypes.byref(p), t, FAKE, FAKE, 0, FAKE, FAKE, None, flags, ws, n, None)
    assert ec(c, _pol(), mass=None) == M.ERR_INVALID_ARG
    assert ec(c, _pol(), flags=2) == M.ERR_INVALID_ARG      # unknown flag bit
    assert ec(c, _pol(), flags=-1) == M.ERR_INVALID_ARG
    assert ec(c, _pol(), flags=M._lib.FUSE_QUANTIZE, ws=None) == M.ERR_WORKSPACE
    assert ec(c, _pol(), t=-1) == M.ERR_INVALID_ARG
    assert ec(c, _pol(), ws=None) == M.ERR_WORKSPACE
    assert ec(c, _pol(protect=30)) == M.ERR_BUDGET
    assert ec(c, _pol(lam=1.5)) == M.ERR_INVALID_ARG
    q = lambda mode, n_src=10, k=FAKE: lib.confk_quantize(  # noqa: E731
        ctypes.byref(c), 0, 2, 0, ctypes.byref(pol), mode, k, FAKE, n_src, None)
    assert q(7) == M.ERR_INVALID_ARG
    assert q(M.QUANT_PREFILL, n_src=100) == M.ERR_BUDGET
    assert q(M.QUANT_PREFILL, k=None) == M.ERR_INVALID_ARG
    assert q(M.QUANT_PREFILL, n_src=-1) == M.ERR_INVALID_ARG
    assert lib.confk_ema_rank(ctypes.byref(c), 0, 2, FAKE, ctypes.byref(pol), -1, FAKE, None) \
        == M.ERR_INVALID_ARG
    assert lib.confk_ema_rank(ctypes.byref(c), 0, 2, FAKE, ctypes.byref(pol), 3, None, None) \
        == M.ERR_INVALID_ARG  # no score buffer (a NULL mass is allowed: a step without mass)


def test_binding_raises_on_error_code():
    with pytest.raises(M.ConfkError) as e:
        M.check("confk_compact", M.ERR_BUDGET)
    assert e.value.code == M.ERR_BUDGET


def test_read_probe_validation():
    probe = _lib.load_probe()
    addr = FAKE.value
    r = lambda buf=addr, nbytes=65536, sink=FAKE: probe.confk_read_probe(  # noqa: E731
        ctypes.c_void_p(buf), nbytes, sink, None)
    assert r(buf=None) == M.ERR_INVALID_ARG
    assert r(nbytes=0) == M.ERR_INVALID_ARG
    assert r(nbytes=65536 + 16384) == M.ERR_INVALID_ARG  # not a whole number of blocks
    assert r(buf=addr + 4) == M.ERR_INVALID_ARG          # not 16-byte aligned
    assert r(sink=None) == M.ERR_INVALID_ARG
