"""Host-side checks of the C ABI that need no GPU: the library loads, exports every function
include/tfm.h declares, and every argument check returns its status before any launch.
Pointers passed here are never dereferenced (validation fails first), so nothing runs on a
device."""
import ctypes
import os
import re
import subprocess

import pytest

from decoder_only_transformer_rmsnorm_amd import synth, tfm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "tfm.h")

OK, NULL, SHAPE, DTYPE, WS, ALIGN, UNSUP = 0, -1, -2, -3, -4, -5, -6
P = 0x10000  # a 16-byte aligned fake device address (never dereferenced here)
PM = 0x10004  # misaligned


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tfm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return tfm.lib()


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", tfm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(L, n)
    assert set(tfm.EXPORTS) == set(names)


def test_status_strings(L):
    for code in range(0, -9, -1):
        s = L.tfm_status_string(code).decode()
        assert s and s != "unknown status"
    assert L.tfm_status_string(5).decode() == "unknown status"
    assert b"gfx950" in L.tfm_version()


def test_rope_table_validation(L):
    assert L.tfm_rope_table_init(None, 8, 16, 1e4, None) == NULL
    assert L.tfm_rope_table_init(PM, 8, 16, 1e4, None) == ALIGN
    assert L.tfm_rope_table_init(P, 8, 15, 1e4, None) == SHAPE
    assert L.tfm_rope_table_init(P, 0, 16, 1e4, None) == SHAPE
    assert L.tfm_rope_table_init(P, 8, 16, -1.0, None) == SHAPE


def test_rmsnorm_validation(L):
    f = L.tfm_rmsnorm
    assert f(P, 2, P, 1, P + 64, 1, 4, 8, 1e-5, None) == DTYPE
    assert f(P, 0, P, 1, P + 64, 1, 4, 6, 1e-5, None) == SHAPE
    assert f(P, 0, P, 1, P + 64, 1, -1, 8, 1e-5, None) == SHAPE
    assert f(P, 0, P, 1, P + 64, 1, 4, 8, -1.0, None) == SHAPE
    assert f(None, 0, P, 1, P + 64, 1, 4, 8, 1e-5, None) == NULL
    assert f(PM, 0, P, 1, P + 64, 1, 4, 8, 1e-5, None) == ALIGN
    assert f(P, 0, P, 1, P, 1, 4, 8, 1e-5, None) == SHAPE       # y aliases x
    assert f(None, 0, None, 1, None, 1, 0, 8, 1e-5, None) == OK  # empty: nothing launched


def test_embed_and_rope_validation(L):
    assert L.tfm_embed(P, 4, P, 3, 10, 8, P, None, None) == DTYPE
    assert L.tfm_embed(P, 4, P, 1, 10, 6, P, None, None) == SHAPE
    assert L.tfm_embed(None, 4, P, 1, 10, 8, P, None, None) == NULL
    assert L.tfm_embed(P, 0, None, 1, 10, 8, None, None, None) == OK
    assert L.tfm_rope(P, 1, 64, None, 2, 4, 2, 30, P, 8, None) == SHAPE   # d_head % 4
    assert L.tfm_rope(P, 1, 60, None, 2, 4, 2, 32, P, 8, None) == SHAPE   # stride < H*dh
    assert L.tfm_rope(P, 1, 66, None, 2, 4, 2, 32, P, 8, None) == ALIGN   # stride % 4
    assert L.tfm_rope(P, 1, 64, None, 2, 9, 2, 32, P, 8, None) == SHAPE   # S > max_seq, no pos
    assert L.tfm_rope(None, 1, 64, None, 2, 4, 2, 32, P, 8, None) == NULL


def test_linear_validation(L):
    f = L.tfm_linear
    assert f(P, P, 1, None, P, 1, 16, 8, 12, 8, None) == SHAPE      # bf16 K % 8
    assert f(P, P, 0, None, P, 0, 16, 8, 10, 8, None) == SHAPE      # f32 K % 4
    assert f(P, P, 1, P, P, 1, 16, 8, 16, 8, None) == DTYPE         # residual needs f32 out
    assert f(P, P, 1, None, P, 1, 16, 8, 16, 7, None) == SHAPE      # ldy < N
    assert f(P, P, 1, None, None, 1, 16, 8, 16, 8, None) == NULL
    assert f(P, PM, 1, None, P, 1, 16, 8, 16, 8, None) == ALIGN
    assert f(None, None, 1, None, None, 1, 0, 8, 16, 8, None) == OK  # M == 0


def test_qkv_rope_validation(L):
    f = L.tfm_qkv_rope
    ok = dict(xn=P, wq=P, wk=P, wv=P, qkv=P, B=2, S=8, d=64, Hq=4, Hkv=2, dh=16, cs=P, ms=8, dt=0)
    call = lambda **kw: f(*[dict(ok, **kw)[k] for k in ("xn", "wq", "wk", "wv", "qkv")], None,
                          *[dict(ok, **kw)[k] for k in ("B", "S", "d", "Hq", "Hkv", "dh", "cs", "ms", "dt")], None)
    assert call(dt=5) == DTYPE
    assert call(dh=18) == SHAPE
    assert call(d=60, dt=1) == SHAPE
    assert call(S=9) == SHAPE            # S > max_seq with default positions
    assert call(wk=None) == NULL
    assert call(qkv=PM) == ALIGN
    assert call(B=0) == OK


def test_attention_validation(L):
    f = L.tfm_causal_attention
    args = lambda **kw: dict(dict(q=P, qs=256, k=P, v=P, kvs=128, o=P, os=256, B=2, S=8, Hq=4,
                                  Hkv=2, dh=64, dt=1), **kw)
    call = lambda a: f(a["q"], a["qs"], a["k"], a["v"], a["kvs"], a["o"], a["os"], a["B"],
                       a["S"], a["Hq"], a["Hkv"], a["dh"], a["dt"], None)
    assert call(args(Hkv=3)) == SHAPE
    assert call(args(qs=128)) == SHAPE
    assert call(args(dh=16)) == UNSUP            # bf16 supports 32/64/128
    assert call(args(dh=48, qs=192, os=192, kvs=96)) == UNSUP
    # bf16 addresses one sequence's keys with 32-bit byte offsets
    assert call(args(S=(1 << 20), kvs=1024)) == UNSUP
    assert call(args(S=(1 << 20), kvs=1024, dt=0, q=None)) == NULL  # f32 has no such limit
    assert call(args(dt=7)) == DTYPE
    assert call(args(q=None)) == NULL
    assert call(args(qs=260)) == ALIGN
    assert call(args(k=PM)) == ALIGN
    assert call(args(S=0)) == OK


def test_sliding_window_attention_validation(L):
    f = L.tfm_sliding_window_attention
    call = lambda W, q=P, S=8, dt=1, dh=64: f(q, 256, P, P, 128, P, 256, 2, S, 4, 2, dh, W, dt,
                                              None)
    assert call(-1) == SHAPE
    assert call(-1, S=0) == SHAPE                  # the window is checked before the size
    assert call(5, dh=16) == UNSUP
    assert call(5, q=None) == NULL
    assert call(5, S=0) == OK
    assert call(0, S=0) == OK


def _cfg(**kw):
    c = tfm.make_config(synth.SMALL_BF16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes_plan(L):
    c = _cfg()
    B, S = 32, 256
    n = L.tfm_workspace_bytes(ctypes.byref(c), B, S)
    M, D, F, e = B * S, 512, 1344, 2
    # plus the per-row partial sums of squares of the RMSNorm split across products (bf16,
    # d_model <= 3072): 16 floats per row
    expect = 256 + M * D * 4 + M * D * e + M * 3 * D * e + M * D * e + M * F * e + M * 16 * 4
    assert n == expect
    assert L.tfm_workspace_bytes(ctypes.byref(_cfg(n_kv_heads=5)), B, S) == 0
    assert L.tfm_workspace_bytes(ctypes.byref(c), B, 257) == 0    # S > max_seq_len
    assert L.tfm_workspace_bytes(None, B, S) == 0
    assert L.tfm_swiglu_workspace_bytes(100, 704, 1) == -(-100 * 704 * 2 // 256) * 256


def _layer():
    return tfm.LayerWeights(*([P] * 9))


def test_block_and_model_validation(L):
    c = _cfg()
    lw = _layer()
    ws_need = L.tfm_workspace_bytes(ctypes.byref(c), 2, 16)
    blk = lambda cfg=c, w=lw, x=P, B=2, S=16, cs=P, ws=P, nb=ws_need: L.tfm_block_forward(
        ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(w) if w is not None else None,
        x, None, B, S, cs, ws, nb, None)
    assert blk(nb=ws_need - 1) == WS
    assert blk(x=None) == NULL
    assert blk(x=PM) == ALIGN
    assert blk(cfg=_cfg(d_head=30)) == SHAPE
    assert blk(cfg=_cfg(dtype=4)) == DTYPE
    assert blk(cfg=_cfg(d_head=16, n_heads=32)) == UNSUP
    assert blk(S=300) == SHAPE
    assert blk(cfg=_cfg(attn_window=-1)) == SHAPE
    assert blk(cfg=_cfg(attn_full_every=-2)) == SHAPE
    assert blk(w=None) == NULL
    bad = _layer(); bad.w3 = None
    assert blk(w=bad) == NULL
    bad = _layer(); bad.wo = PM
    assert blk(w=bad) == ALIGN

    layers = (tfm.LayerWeights * 4)(*[_layer() for _ in range(4)])
    mw = tfm.ModelWeights(P, layers, P, P)
    mdl = lambda cfg=c, w=mw, ld=10000, nb=ws_need, dtl=1: L.tfm_model_forward(
        ctypes.byref(cfg), ctypes.byref(w) if w is not None else None, P, None, P, dtl, ld, 2, 16,
        P, P, nb, None)
    assert mdl(ld=9999) == SHAPE
    assert mdl(nb=100) == WS
    assert mdl(w=None) == NULL
    assert mdl(dtl=2) == DTYPE
    mw2 = tfm.ModelWeights(P, None, P, P)
    assert mdl(w=mw2) == NULL
    layers[2].g_ffn = None
    assert mdl() == NULL


def test_xent_validation(L):
    """Every call here fails validation (or is empty) before any launch."""
    f = L.tfm_lm_head_xent
    need = L.tfm_xent_workspace_bytes(16, 100)
    parts = -(-100 // 128)
    assert need == 2 * (-(-16 * parts * 4 // 256) * 256) + (-(-16 * 4 // 256) * 256)
    assert L.tfm_xent_workspace_bytes(-1, 100) == 0 and L.tfm_xent_workspace_bytes(16, 0) == 0
    call = lambda x=P, w=P, t=P, loss=P, mean=None, M=16, V=100, K=64, ws=P, nb=need: f(
        x, w, t, loss, mean, M, V, K, ws, nb, None)
    assert call(M=-1) == SHAPE
    assert call(V=0) == SHAPE
    assert call(K=60) == SHAPE
    assert call(M=0) == OK
    assert call(x=None) == NULL
    assert call(t=None) == NULL
    assert call(loss=None) == NULL
    assert call(ws=None) == NULL
    assert call(x=PM) == ALIGN
    assert call(w=PM) == ALIGN
    assert call(nb=need - 1) == WS


def test_model_loss_validation(L):
    c = _cfg()
    layers = (tfm.LayerWeights * 4)(*[_layer() for _ in range(4)])
    mw = tfm.ModelWeights(P, layers, P, P)
    need = L.tfm_loss_workspace_bytes(ctypes.byref(c), 2, 16)
    assert need == L.tfm_workspace_bytes(ctypes.byref(c), 2, 16) + \
        L.tfm_xent_workspace_bytes(32, c.vocab)
    loss = lambda cfg=c, w=mw, t=P, out=P, nb=need, B=2: L.tfm_model_loss(
        ctypes.byref(cfg), ctypes.byref(w) if w is not None else None, P, None, t, out, None, B,
        16, P, P, nb, None)
    assert loss(cfg=_cfg(dtype=0)) == UNSUP      # bf16 models only
    assert loss(t=None) == NULL
    assert loss(out=None) == NULL
    assert loss(nb=need - 1) == WS
    assert loss(w=None) == NULL
    assert loss(B=0) == OK
    layers[1].w1 = None
    assert loss() == NULL


def test_swiglu_validation(L):
    f = L.tfm_swiglu_ffn
    need = L.tfm_swiglu_workspace_bytes(64, 704, 1)
    assert f(P, P, P, P, None, P, 64, 256, 704, 1, P, need - 1, None) == WS
    assert f(P, P, P, P, None, P, 64, 250, 704, 1, P, need, None) == SHAPE
    assert f(P, P, P, None, None, P, 64, 256, 704, 1, P, need, None) == NULL
    assert f(P, P, P, P, PM, P, 64, 256, 704, 1, P, need, None) == ALIGN
    assert f(P, P, P, P, None, P, 64, 256, 704, 9, P, need, None) == DTYPE


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The binding and the library never load the oracle; a missing library raises."""
    src = open(os.path.join(ROOT, "decoder_only_transformer_rmsnorm_amd", "tfm.py")).read()
    assert "oracle" not in src.replace("oracle_", "")
    for f in os.listdir(os.path.join(ROOT, "decoder_only_transformer_rmsnorm_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "decoder_only_transformer_rmsnorm_amd",
                                                 "csrc", f)).read()



def test_missing_library_raises(monkeypatch):
    """Without libtfm.so the binding raises instead of computing anything another way."""
    monkeypatch.setattr(tfm, "_lib", None)
    monkeypatch.setattr(tfm, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libtfm.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        tfm.lib()


def test_host_tensors_are_refused():
    """A host (CPU) tensor is refused before any call reaches the library."""
    import torch
    x = torch.zeros((4, 64))
    g = torch.ones(64)
    with pytest.raises(ValueError, match="GPU"):
        tfm.tfm_rmsnorm(x, g, y=torch.empty_like(x))

def _host_model():
    """A DeviceModel shell on the CPU (no weights uploaded): enough to reach the binding's
    argument checks, which run before anything touches the device or the library."""
    import torch
    cfg = synth.ModelConfig(name="h", dtype="bf16", n_layers=1, d_model=64, n_heads=2,
                            n_kv_heads=2, d_head=32, d_ff=128, vocab=100, batch=2, seq=8)
    dm = object.__new__(tfm.DeviceModel)
    dm.cfg, dm.dtype, dm.device, dm.max_seq = cfg, torch.bfloat16, "cpu", 8
    dm.ccfg = tfm.make_config(cfg, 8)
    dm._ws, dm._ws_shape = None, None
    dm.cos_sin = torch.zeros(8 * 32)
    dm._layer_structs = (tfm.LayerWeights * 1)()
    dm.weights = tfm.ModelWeights(None, dm._layer_structs, None, None)
    return dm


def test_binding_checks_dtype_layout_and_size():
    """The library receives bare pointers, so the binding checks dtype, contiguity and the
    element count a call will touch before the call (int64 ids read as int32, a logits buffer
    smaller than B*S rows of the vocabulary, a non-contiguous tensor or a row view running past
    its storage would otherwise be read or written out of bounds on the GPU)."""
    import torch
    dm = _host_model()
    ids32 = torch.zeros((2, 8), dtype=torch.int32)
    cases = [
        (lambda: dm.forward(ids=ids32.long()), -3, "ids"),                              # int64 ids
        (lambda: dm.forward(ids=ids32, positions=torch.arange(16).view(2, 8)), -3, "positions"),
        (lambda: dm.forward(ids=ids32.t()), -2, "contiguous"),                          # transposed
        (lambda: dm.forward(ids=ids32, logits=torch.empty((15, 100), dtype=torch.bfloat16)), -2, "logits"),
        (lambda: dm.forward(ids=ids32, logits=torch.empty((16, 100), dtype=torch.int32)), -3, "dtype"),
        (lambda: dm.forward(ids=ids32, ld_logits=99), -2, "logits"),                    # ld < V
        (lambda: dm.loss(torch.zeros((2, 8), dtype=torch.int64), ids=ids32), -3, "targets"),
        (lambda: dm.loss(torch.zeros((2, 7), dtype=torch.int32), ids=ids32), -2, "targets"),
        (lambda: dm.decode(torch.zeros(16, dtype=torch.bfloat16), 8, ids32[:, 0].contiguous(),
                           torch.zeros(3, dtype=torch.int32)), -2, "positions"),
        (lambda: tfm.tfm_embed(ids32.long(), torch.zeros((100, 64))), -3, "ids"),
        (lambda: tfm.tfm_lm_head_xent(torch.zeros((4, 64), dtype=torch.bfloat16),
                                      torch.zeros((100, 64), dtype=torch.bfloat16),
                                      torch.zeros(4, dtype=torch.int64)), -3, "targets"),
        (lambda: tfm.tfm_linear(torch.zeros((4, 64)), torch.zeros((100, 64)),
                                y=torch.empty((3, 100))), -2, "y"),
        (lambda: tfm.tfm_causal_attention(torch.zeros((1, 8, 64)), torch.zeros((1, 8, 80))[..., :64],
                                          torch.zeros((1, 8, 80))[..., 32:], 2, 2, 32,
                                          kv_stride=80), -2, "v"),         # last row past the end
        (lambda: tfm.tfm_rmsnorm(torch.zeros((4, 64)), torch.ones(63)), -2, "g"),
    ]
    for fn, status, what in cases:
        with pytest.raises(tfm.TfmError) as e:
            fn()
        assert e.value.status == status, (what, e.value)
        assert what in str(e.value), (what, str(e.value))
    # well-formed host tensors pass the checks and are then refused for living on the host
    with pytest.raises(ValueError, match="GPU"):
        dm.forward(ids=ids32)


def test_kv_cache_and_decode_validation(L):
    """Every call fails validation (or is empty) before any launch."""
    c = _cfg()   # d512 bf16: 4 layers, 16/16 heads of 32
    assert L.tfm_kv_cache_bytes(ctypes.byref(c), 2, 100) == 2 * 4 * 2 * 16 * 100 * 32 * 2
    assert L.tfm_kv_cache_bytes(ctypes.byref(c), -1, 100) == 0
    layers = (tfm.LayerWeights * 4)(*[_layer() for _ in range(4)])
    mw = tfm.ModelWeights(P, layers, P, P)
    need = L.tfm_decode_workspace_bytes(ctypes.byref(c), 2, 100)
    assert need > 0
    assert L.tfm_decode_workspace_bytes(ctypes.byref(_cfg(dtype=0)), 2, 100) == 0
    dec = lambda cfg=c, w=mw, pos=P, lg=P, ld=c.vocab, B=2, cache=P, cs=100, nb=need, dtl=1: \
        L.tfm_model_decode(ctypes.byref(cfg), ctypes.byref(w) if w is not None else None, P, pos,
                           lg, dtl, ld, B, P, cache, cs, P, nb, None)
    assert dec(cfg=_cfg(dtype=0)) == UNSUP
    assert dec(cfg=_cfg(n_kv_heads=1)) == UNSUP          # 16 query heads per kv head
    assert dec(cs=0) == SHAPE
    assert dec(cs=131073) == UNSUP
    assert dec(ld=c.vocab - 1) == SHAPE
    assert dec(dtl=5) == DTYPE
    assert dec(B=0) == OK
    assert dec(pos=None) == NULL
    assert dec(cache=None) == NULL
    assert dec(lg=None) == NULL
    assert dec(w=None) == NULL
    assert dec(cache=PM) == ALIGN
    assert dec(nb=need - 1) == WS
    pre_ws = L.tfm_workspace_bytes(ctypes.byref(c), 2, 16)
    pre = lambda cfg=c, cache=P, cs=100, lg=P, nb=pre_ws, B=2: L.tfm_model_prefill(
        ctypes.byref(cfg), ctypes.byref(mw), P, None, lg, 1, cfg.vocab, B, 16, P, cache, cs, P,
        nb, None)
    assert pre(cfg=_cfg(dtype=0)) == UNSUP
    assert pre(cs=0) == SHAPE
    assert pre(B=0) == OK
    assert pre(cache=None) == NULL
    assert pre(nb=pre_ws - 1) == WS
    assert pre(lg=PM) == ALIGN


def test_decode_attention_validation(L):
    f = L.tfm_decode_attention
    need = L.tfm_decode_attention_workspace_bytes(2, 8, 64, 300)
    assert need == -(-2 * 8 * 5 * 66 * 4 // 256) * 256          # at most one split per 64 keys
    call = lambda q=P, qs=512, o=P, os=512, B=2, Hq=8, Hkv=2, dh=64, cs=300, W=0, ws=P, nb=need: f(
        q, qs, P, P, P, o, os, B, Hq, Hkv, dh, cs, W, ws, nb, None)
    assert call(Hkv=3) == SHAPE
    assert call(cs=0) == SHAPE
    assert call(cs=131073) == UNSUP
    assert call(W=-1) == SHAPE
    assert call(qs=256) == SHAPE
    assert call(dh=48, qs=384, os=384) == UNSUP
    assert call(Hq=16, Hkv=1, qs=1024, os=1024) == UNSUP      # at most 8 query heads per kv head
    assert call(B=0) == OK
    assert call(q=None) == NULL
    assert call(o=PM) == ALIGN
    assert call(nb=need - 1) == WS


def test_decode_attention_noalloc_validation(L):
    """The allocation-free variant checks like tfm_decode_attention and refuses, before any
    device call, a call whose split records exceed its static scratch array."""
    f = L.tfm_decode_attention_noalloc
    cap = L.tfm_decode_attention_noalloc_max_bytes()
    assert cap == 4 << 20
    call = lambda q=P, qs=512, o=P, os=512, B=2, Hq=8, Hkv=2, dh=64, cs=300, W=0: f(
        q, qs, P, P, P, o, os, B, Hq, Hkv, dh, cs, W, None)
    assert call(Hkv=3) == SHAPE
    assert call(cs=0) == SHAPE
    assert call(cs=131073) == UNSUP
    assert call(W=-1) == SHAPE
    assert call(dh=48, qs=384, os=384) == UNSUP
    assert call(B=0) == OK
    assert call(q=None) == NULL
    assert call(o=PM) == ALIGN
    # 64 sequences x 32 heads x 64 chunks of 130 floats: 68 MB of records > 4 MiB
    big = dict(B=64, Hq=32, Hkv=4, dh=128, qs=4096, os=4096, cs=4096)
    assert L.tfm_decode_attention_workspace_bytes(64, 32, 128, 4096) > cap
    assert call(**big) == WS


def test_training_entry_points_validation(L):
    """Every call fails validation (or is empty) before any launch."""
    c = _cfg()
    assert L.tfm_train_workspace_bytes(ctypes.byref(c), 2, 16) > 0
    assert L.tfm_train_workspace_bytes(ctypes.byref(_cfg(d_model=4096, n_heads=128)), 2, 16) == 0
    layers = (tfm.LayerWeights * 4)(*[_layer() for _ in range(4)])
    mw = tfm.ModelWeights(P, layers, P, P + 0x100)
    glayers = (tfm.LayerGrads * 4)(*[tfm.LayerGrads(*([P] * 9)) for _ in range(4)])
    need = L.tfm_train_workspace_bytes(ctypes.byref(c), 2, 16)
    def bwd(cfg=c, w=mw, t=P, loss=P, g=None, B=2, nb=need):
        g = tfm.ModelGrads(P, glayers, P, P + 0x200) if g is None else g
        return L.tfm_model_backward(ctypes.byref(cfg), ctypes.byref(w), P, None, t, loss,
                                    ctypes.byref(g), B, 16, P, P, nb, None)
    assert bwd(B=0) == OK
    assert bwd(t=None) == NULL
    assert bwd(loss=None) == NULL
    assert bwd(nb=need - 1) == WS
    assert bwd(g=tfm.ModelGrads(P, glayers, P, None)) == NULL          # untied head needs a grad
    assert bwd(g=tfm.ModelGrads(PM, glayers, P, P)) == ALIGN
    tied = tfm.ModelWeights(P, layers, P, P)
    assert bwd(w=tied, g=tfm.ModelGrads(P, glayers, P, P + 0x200)) == SHAPE
    bad = (tfm.LayerGrads * 4)(*[tfm.LayerGrads(*([P] * 9)) for _ in range(4)])
    bad[3].w2 = None
    assert bwd(g=tfm.ModelGrads(P, bad, P, P + 0x200)) == NULL

    clip = L.tfm_grad_clip_coef
    nb = L.tfm_clip_workspace_bytes(3)
    ptrs = (ctypes.c_void_p * 3)(P, P, P)
    sizes = (ctypes.c_int64 * 3)(10, 20, 30)
    assert clip(ptrs, sizes, 3, 0.0, P, None, P, nb, None) == SHAPE
    assert clip(ptrs, sizes, -1, 1.0, P, None, P, nb, None) == SHAPE
    assert clip(ptrs, sizes, 3, 1.0, None, None, P, nb, None) == NULL
    assert clip(ptrs, sizes, 3, 1.0, P, None, P, nb - 1, None) == WS
    neg = (ctypes.c_int64 * 3)(10, -1, 30)
    assert clip(ptrs, neg, 3, 1.0, P, None, P, nb, None) == SHAPE

    adam = lambda n=10, lr=1e-3, b1=0.9, b2=0.999, step=1, p=P: L.tfm_adamw_step(
        p, None, P, P, P, n, lr, b1, b2, 1e-8, 0.0, step, None, None)
    assert adam(step=0) == SHAPE
    assert adam(b1=1.0) == SHAPE
    assert adam(lr=-1.0) == SHAPE
    assert adam(n=0) == OK
    assert adam(p=None) == NULL

    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    sz = (ctypes.c_int64 * 2)(10, 0)
    multi = lambda ps=arr(P, None), gs=arr(P, None), n=2, sizes=sz, step=1, b2=0.999: \
        L.tfm_adamw_step_multi(ps, None, gs, arr(P, None), arr(P, None), sizes, n, 1e-3, 0.9, b2,
                               1e-8, 0.0, step, None, None)
    assert multi(n=0) == OK
    assert multi(n=-1) == SHAPE
    assert multi(step=0) == SHAPE
    assert multi(b2=1.0) == SHAPE
    assert multi(ps=None) == NULL
    assert multi(gs=arr(None, None)) == NULL                 # tensor 0 has elements
    assert multi(sizes=(ctypes.c_int64 * 2)(10, -3)) == SHAPE


def test_mfma_rate_validation(L):
    L.tfm_mfma_rate.restype = ctypes.c_int
    L.tfm_mfma_rate.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert L.tfm_mfma_rate(10, 4, None, None) == NULL        # no checksum buffer
    assert L.tfm_mfma_rate(0, 4, P, None) == SHAPE           # no iterations
    assert L.tfm_mfma_rate(10, 0, P, None) == SHAPE          # no workgroups
