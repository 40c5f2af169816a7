"""ctypes binding of the plain fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the HIP library or its binding. Inputs are numpy
arrays; weights are passed as float32 (already bf16-rounded for bf16 models) and every
result comes back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SRC_TRAIN = os.path.join(_HERE, "oracle_train.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

c_int, c_i64, c_double = ctypes.c_int, ctypes.c_int64, ctypes.c_double
_p = ctypes.c_void_p


class OracleCfg(ctypes.Structure):
    _fields_ = [("n_layers", c_int), ("d_model", c_int), ("n_heads", c_int),
                ("n_kv_heads", c_int), ("d_head", c_int), ("d_ff", c_int), ("vocab", c_int),
                ("eps", c_double), ("theta", c_double), ("window", c_int), ("full_every", c_int)]


class OracleLayerD(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("g_attn", "wq", "wk", "wv", "wo", "g_ffn", "w1", "w3", "w2")]


class OracleParamsD(ctypes.Structure):
    _fields_ = [("embed", _p), ("layers", ctypes.POINTER(OracleLayerD)), ("g_final", _p),
                ("lm_head", _p)]


class OracleLayer(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("g_attn", "wq", "wk", "wv", "wo", "g_ffn", "w1", "w3", "w2")]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, -O2, OpenMP, strict IEEE double)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-o", _LIB + ".tmp", _SRC, _SRC_TRAIN, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_embedding.restype = c_int
        L.oracle_embedding.argtypes = [_p, c_i64, _p, c_int, c_int, _p]
        L.oracle_rmsnorm.argtypes = [_p, c_i64, c_int, _p, c_double, _p]
        L.oracle_linear.argtypes = [_p, c_i64, c_int, _p, c_int, _p]
        L.oracle_rope.argtypes = [_p, c_int, c_int, c_int, c_int, c_i64, _p, c_double]
        L.oracle_softmax.argtypes = [_p, c_i64, c_int, _p]
        L.oracle_attention.argtypes = [_p, c_i64, _p, _p, c_i64, c_int, c_int, c_int, c_int,
                                       c_int, _p, _p]
        L.oracle_attention_window.argtypes = [_p, c_i64, _p, _p, c_i64, c_int, c_int, c_int,
                                              c_int, c_int, c_int, _p, _p]
        L.oracle_attention_rows.argtypes = [_p, c_i64, _p, _p, c_i64, c_int, c_int, c_int,
                                            c_int, c_int, c_int, _p, c_i64, _p]
        L.oracle_silu.restype = c_double
        L.oracle_silu.argtypes = [c_double]
        L.oracle_swiglu.argtypes = [_p, c_i64, c_int, c_int, _p, _p, _p, _p, _p]
        L.oracle_block.argtypes = [ctypes.POINTER(OracleCfg), ctypes.POINTER(OracleLayer), _p,
                                   _p, c_int, c_int]
        L.oracle_model.restype = c_int
        L.oracle_cross_entropy.argtypes = [_p, c_i64, c_int, _p, _p]
        L.oracle_cross_entropy.restype = c_double
        L.oracle_model.argtypes = [ctypes.POINTER(OracleCfg), _p, ctypes.POINTER(OracleLayer),
                                   _p, _p, _p, _p, c_int, c_int, _p, _p, c_i64, _p]
        L.oracle_num_threads.restype = c_int
        L.oracle_set_num_threads.argtypes = [c_int]
        L.oracle_set_num_threads.restype = None
        L.oracle_model_grads.argtypes = [ctypes.POINTER(OracleCfg), ctypes.POINTER(OracleParamsD),
                                         _p, _p, _p, c_int, c_int, ctypes.POINTER(OracleParamsD)]
        L.oracle_model_grads.restype = c_double
        L.oracle_adamw.argtypes = [_p, _p, _p, _p, c_i64, c_double, c_double, c_double, c_double,
                                   c_double, c_int]
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a) -> int | None:
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """OpenMP threads of the oracle's parallel loops (from the next call on)."""
    lib().oracle_set_num_threads(int(n))


def embedding(ids, E) -> np.ndarray:
    ids, E = _i32(ids), _f32(E)
    n = ids.size
    x = np.empty((n, E.shape[1]), dtype=np.float64)
    if lib().oracle_embedding(_ptr(ids), n, _ptr(E), E.shape[0], E.shape[1], _ptr(x)) != 0:
        raise IndexError("token id outside the vocabulary")
    return x.reshape(ids.shape + (E.shape[1],))


def rmsnorm(x, g, eps: float = 1e-5) -> np.ndarray:
    x, g = _f64(x), _f64(g)
    d = x.shape[-1]
    y = np.empty_like(x)
    lib().oracle_rmsnorm(_ptr(x), x.size // d, d, _ptr(g), eps, _ptr(y))
    return y


def linear(x, W) -> np.ndarray:
    x, W = _f64(x), _f32(W)
    n_out, n_in = W.shape
    assert x.shape[-1] == n_in
    y = np.empty(x.shape[:-1] + (n_out,), dtype=np.float64)
    lib().oracle_linear(_ptr(x), x.size // n_in, n_in, _ptr(W), n_out, _ptr(y))
    return y


def rope(x, n_heads: int, theta: float = 10000.0, pos=None) -> np.ndarray:
    """RoPE on x of shape (B, S, n_heads*dh); returns a new array."""
    x = _f64(x).copy()
    B, S, F = x.shape
    dh = F // n_heads
    pos = None if pos is None else _i32(np.broadcast_to(pos, (B, S)))
    lib().oracle_rope(_ptr(x), B, S, n_heads, dh, F, _ptr(pos), theta)
    return x


def softmax(s) -> np.ndarray:
    s = _f64(s)
    n = s.shape[-1]
    p = np.empty_like(s)
    lib().oracle_softmax(_ptr(s), s.size // n, n, _ptr(p))
    return p


def attention(q, k, v, n_heads: int, n_kv_heads: int, want_probs: bool = False,
              window: int = 0):
    """Causal attention on q (B, S, Hq*dh), k and v (B, S, Hkv*dh); window > 0 limits each
    query to its `window` most recent keys."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, qd = q.shape
    dh = qd // n_heads
    assert k.shape == v.shape == (B, S, n_kv_heads * dh)
    o = np.empty((B, S, qd), dtype=np.float64)
    probs = np.empty((B, n_heads, S, S), dtype=np.float64) if want_probs else None
    if window > 0:
        lib().oracle_attention_window(_ptr(q), qd, _ptr(k), _ptr(v), n_kv_heads * dh, B, S,
                                      n_heads, n_kv_heads, dh, window, _ptr(o), _ptr(probs))
    else:
        lib().oracle_attention(_ptr(q), qd, _ptr(k), _ptr(v), n_kv_heads * dh, B, S, n_heads,
                               n_kv_heads, dh, _ptr(o), _ptr(probs))
    return (o, probs) if want_probs else o


def attention_rows(q, k, v, n_heads: int, n_kv_heads: int, rows, window: int = 0):
    """Attention output at the listed rows (b*S + s) only: (len(rows), Hq*dh)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, qd = q.shape
    dh = qd // n_heads
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, qd), dtype=np.float64)
    lib().oracle_attention_rows(_ptr(q), qd, _ptr(k), _ptr(v), n_kv_heads * dh, B, S, n_heads,
                                n_kv_heads, dh, window, _ptr(rows), rows.size, _ptr(o))
    return o


def decode_attention(q, k_cache, v_cache, n_heads: int, n_kv_heads: int, lens, window: int = 0):
    """One new query per sequence attending to its cached keys [T4 6.1 KV cache: keys and
    values of earlier steps are kept and the new token's are appended before attending].
    q (B, Hq*dh); k_cache, v_cache (B, T, Hkv*dh) token-major, slot t = position t; sequence b
    sees slots lens[b]-window .. lens[b]-1 (from 0 when window is 0 or larger). Plain fp64:
    scores, max-subtracted softmax, weighted sum of values."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, qd = q.shape
    dh = qd // n_heads
    group = n_heads // n_kv_heads
    o = np.zeros((B, qd), np.float64)
    for b in range(B):
        n = int(lens[b])
        t0 = max(0, n - window) if window > 0 else 0
        for h in range(n_heads):
            g = h // group
            qh = q[b, h * dh:(h + 1) * dh]
            kh = kc[b, t0:n, g * dh:(g + 1) * dh]
            vh = vc[b, t0:n, g * dh:(g + 1) * dh]
            sc = kh @ qh / np.sqrt(dh)
            p = np.exp(sc - sc.max())
            o[b, h * dh:(h + 1) * dh] = (p / p.sum()) @ vh
    return o


def silu(u: float) -> float:
    return lib().oracle_silu(float(u))


def swiglu(h, w1, w3, w2, want_hidden: bool = False):
    h, w1, w3, w2 = _f64(h), _f32(w1), _f32(w3), _f32(w2)
    d_ff, d = w1.shape
    rows = h.size // d
    out = np.empty(h.shape, dtype=np.float64)
    u = np.empty(h.shape[:-1] + (d_ff,), dtype=np.float64) if want_hidden else None
    lib().oracle_swiglu(_ptr(h), rows, d, d_ff, _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out), _ptr(u))
    return (out, u) if want_hidden else out


def _cfg(cfg) -> OracleCfg:
    return OracleCfg(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.d_head,
                     cfg.d_ff, cfg.vocab, cfg.eps, cfg.rope_theta,
                     getattr(cfg, "window", 0), getattr(cfg, "full_every", 0))


def _layer(lw, keep: list) -> OracleLayer:
    arrs = [_f32(getattr(lw, n)) for n in ("g_attn", "wq", "wk", "wv", "wo", "g_ffn", "w1",
                                            "w3", "w2")]
    keep.extend(arrs)
    return OracleLayer(*[a.ctypes.data for a in arrs])


def block(cfg, lw, x, pos=None, window: int = 0) -> np.ndarray:
    """One pre-norm block on the residual x of shape (B, S, D); returns a new array. window > 0
    gives the block sliding-window attention."""
    x = _f64(x).copy()
    B, S, _ = x.shape
    keep: list = []
    L = _layer(lw, keep)
    pos = None if pos is None else _i32(np.broadcast_to(pos, (B, S)))
    c = _cfg(cfg)
    c.window, c.full_every = window, 0
    lib().oracle_block(ctypes.byref(c), ctypes.byref(L), _ptr(x), _ptr(pos), B, S)
    return x


def model(cfg, inputs, ids=None, pos=None, rows=None, want_hidden: bool = False):
    """Forward of the whole model. ``ids`` defaults to ``inputs.ids``; ``rows`` (flat indices
    b*S + s) restricts which logits rows are produced. Returns logits (and x_final)."""
    ids = _i32(inputs.ids if ids is None else ids)
    B, S = ids.shape
    keep: list = []
    arr = (OracleLayer * max(1, cfg.n_layers))(*[_layer(lw, keep) for lw in inputs.layers])
    embed, g_final, lm = _f32(inputs.embed), _f32(inputs.g_final), _f32(inputs.lm_head)
    pos = None if pos is None else _i32(np.broadcast_to(pos, (B, S)))
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = B * S if rows_a is None else rows_a.size
    logits = np.empty((n_rows, cfg.vocab), dtype=np.float64)
    xf = np.empty((B * S, cfg.d_model), dtype=np.float64) if want_hidden else None
    c = _cfg(cfg)
    rc = lib().oracle_model(ctypes.byref(c), _ptr(embed), arr, _ptr(g_final), _ptr(lm),
                            _ptr(ids), _ptr(pos), B, S, _ptr(xf), _ptr(rows_a), n_rows,
                            _ptr(logits))
    if rc != 0:
        raise IndexError("token id outside the vocabulary")
    if rows_a is None:
        logits = logits.reshape(B, S, cfg.vocab)
    return (logits, xf) if want_hidden else logits


def cross_entropy(logits, targets):
    """Per-row next-token cross-entropy (rows with a negative target give 0 and are not
    counted) and the mean over counted rows; logits (rows, V), targets (rows,) int."""
    lg = _f64(logits)
    rows, V = lg.shape
    t = _i32(targets).reshape(rows)
    loss = np.zeros(rows, np.float64)
    mean = lib().oracle_cross_entropy(_ptr(lg), rows, V, _ptr(t), _ptr(loss))
    if np.isnan(mean):
        raise ValueError("target outside [0, V)")
    return loss, float(mean)


def next_token_targets(ids):
    """Targets of next-token prediction for (B, S) ids: row (b, s) predicts ids[b, s + 1];
    the last position of each sequence has no target (-1)  [T2 Optimize / Loss: inputs and
    targets are the same sequence shifted by one]."""
    ids = np.asarray(ids)
    t = np.full(ids.shape, -1, np.int32)
    t[:, :-1] = ids[:, 1:]
    return t


# ---------------------------------------------------------------- training step
LAYER_FIELDS = ("g_attn", "wq", "wk", "wv", "wo", "g_ffn", "w1", "w3", "w2")


def params_of(inputs) -> dict:
    """The parameters of a synth.ModelInputs as a dict of float64 arrays (a tied LM head stays
    the same object as the embedding)."""
    embed = _f64(inputs.embed).copy()
    return {"embed": embed,
            "lm_head": embed if inputs.lm_head is inputs.embed else _f64(inputs.lm_head).copy(),
            "g_final": _f64(inputs.g_final).copy(),
            "layers": [{f: _f64(getattr(lw, f)).copy() for f in LAYER_FIELDS}
                       for lw in inputs.layers]}


def _params_struct(params, keep):
    layers = (OracleLayerD * max(1, len(params["layers"])))(
        *[OracleLayerD(*[_ptr(L[f]) for f in LAYER_FIELDS]) for L in params["layers"]])
    keep.append(layers)
    return OracleParamsD(_ptr(params["embed"]), layers, _ptr(params["g_final"]),
                         _ptr(params["lm_head"]))


def model_grads(cfg, params, ids, targets, pos=None):
    """Mean next-token cross-entropy and its gradient with respect to every parameter
    [T2 Optimize / Loss; chain rule through the forward of oracle.model]. params as
    params_of(); ids, targets (B, S) (targets < 0: no target). Returns (loss, grads) with
    grads shaped like params (a tied LM head's gradient is part of the embedding's)."""
    ids = _i32(ids)
    B, S = ids.shape
    t = _i32(np.broadcast_to(targets, (B, S)))
    pos = None if pos is None else _i32(np.broadcast_to(pos, (B, S)))
    for arr in [params["embed"], params["lm_head"], params["g_final"]] + \
            [L[f] for L in params["layers"] for f in LAYER_FIELDS]:
        assert arr.dtype == np.float64 and arr.flags.c_contiguous
    grads = {"embed": np.zeros_like(params["embed"]), "g_final": np.zeros_like(params["g_final"]),
             "layers": [{f: np.zeros_like(L[f]) for f in LAYER_FIELDS} for L in params["layers"]]}
    grads["lm_head"] = grads["embed"] if params["lm_head"] is params["embed"] else \
        np.zeros_like(params["lm_head"])
    keep: list = []
    ps, gs = _params_struct(params, keep), _params_struct(grads, keep)
    c = _cfg(cfg)
    loss = lib().oracle_model_grads(ctypes.byref(c), ctypes.byref(ps), _ptr(ids), _ptr(pos),
                                    _ptr(t), B, S, ctypes.byref(gs))
    if np.isnan(loss):
        raise IndexError("token id outside the vocabulary")
    return float(loss), grads


def adamw(theta, grad, m, v, lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
          weight_decay: float = 1e-3, t: int = 1):
    """One AdamW step [T2 Optimizer - AdamW]; returns new (theta, m, v) as float64 copies."""
    th, mm, vv = _f64(theta).copy(), _f64(m).copy(), _f64(v).copy()
    g = _f64(grad)
    lib().oracle_adamw(_ptr(th), _ptr(g), _ptr(mm), _ptr(vv), th.size, lr, betas[0], betas[1],
                       eps, weight_decay, t)
    return th, mm, vv


def clip_grad_norm(grads, max_norm: float, delta: float = 1e-6):
    """[T2 Gradient Clip]: the global L2 norm of all gradients (the norm of the per-tensor
    norms); when it exceeds max_norm every gradient is scaled by max_norm / (norm + delta).
    Returns (norm, scaled copies)."""
    gs = [_f64(g) for g in grads]
    total = float(np.sqrt(sum(float(np.sum(g * g)) for g in gs)))
    coef = max_norm / (total + delta) if total > max_norm else 1.0
    return total, [g * coef for g in gs]


def cosine_lr(it: int, warmup_iters: int, cos_cycle_iters: int, lr_min: float, lr_max: float):
    """[T2 Cosine LR Scheduler]: linear warm-up to lr_max, cosine decay to lr_min over
    (warmup_iters, cos_cycle_iters), lr_min after."""
    import math
    if it <= warmup_iters:
        return lr_max * it / warmup_iters
    if it < cos_cycle_iters:
        frac = (it - warmup_iters) / (cos_cycle_iters - warmup_iters)
        return lr_min + 0.5 * (lr_max - lr_min) * (1 + math.cos(math.pi * frac))
    return lr_min
