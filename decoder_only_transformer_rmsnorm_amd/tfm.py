"""Thin ctypes binding of libtfm.so (include/tfm.h).

Argument marshalling only: every function takes torch tensors that already live on the
GPU, checks their dtype/contiguity, and passes raw device pointers plus the current HIP
stream to the library. No computation happens here, and there is no fallback: if the
library is missing or the GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtfm.so")

F32, BF16 = 0, 1
STATUS = {0: "TFM_OK", -1: "TFM_ERR_NULL", -2: "TFM_ERR_SHAPE", -3: "TFM_ERR_DTYPE",
          -4: "TFM_ERR_WORKSPACE", -5: "TFM_ERR_ALIGN", -6: "TFM_ERR_UNSUPPORTED",
          -7: "TFM_ERR_HIP", -8: "TFM_ERR_TOKEN", -9: "TFM_ERR_POSITION"}

EXPORTS = ["tfm_status_string", "tfm_last_hip_error", "tfm_version", "tfm_rope_table_init",
           "tfm_embed", "tfm_rmsnorm", "tfm_rope", "tfm_linear", "tfm_qkv_rope", "tfm_causal_attention",
           "tfm_swiglu_workspace_bytes", "tfm_swiglu_ffn", "tfm_workspace_bytes",
           "tfm_block_forward", "tfm_model_forward", "tfm_xent_workspace_bytes",
           "tfm_lm_head_xent", "tfm_loss_workspace_bytes", "tfm_model_loss",
           "tfm_sliding_window_attention", "tfm_kv_cache_bytes", "tfm_model_prefill",
           "tfm_decode_workspace_bytes", "tfm_model_decode",
           "tfm_decode_attention_workspace_bytes", "tfm_decode_attention",
           "tfm_decode_attention_noalloc_max_bytes", "tfm_decode_attention_noalloc",
           "tfm_train_workspace_bytes", "tfm_model_backward", "tfm_clip_workspace_bytes",
           "tfm_grad_clip_coef", "tfm_adamw_step", "tfm_adamw_step_multi",
           "tfm_check_device_flags", "tfm_mfma_rate", "tfm_trace_begin", "tfm_trace_end",
           "tfm_trace_read", "tfm_trace_free"]


class TfmError(RuntimeError):
    def __init__(self, status: int, where: str, hip: int = 0):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)}"
        if status == -7:
            msg += f" (hipError {hip})"
        super().__init__(msg)


c_int, c_i64, c_size, c_p = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class Config(ctypes.Structure):
    _fields_ = [("n_layers", c_int), ("d_model", c_int), ("n_heads", c_int),
                ("n_kv_heads", c_int), ("d_head", c_int), ("d_ff", c_int), ("vocab", c_int),
                ("max_seq_len", c_int), ("eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", c_int), ("attn_window", c_int), ("attn_full_every", c_int)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, c_p) for n in ("g_attn", "wq", "wk", "wv", "wo", "g_ffn", "w1", "w3", "w2")]


class ModelWeights(ctypes.Structure):
    _fields_ = [("embed", c_p), ("layers", ctypes.POINTER(LayerWeights)), ("g_final", c_p),
                ("lm_head", c_p)]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, c_p) for n in ("g_attn", "wq", "wk", "wv", "wo", "g_ffn", "w1", "w3", "w2")]


class ModelGrads(ctypes.Structure):
    _fields_ = [("embed", c_p), ("layers", ctypes.POINTER(LayerGrads)), ("g_final", c_p),
                ("lm_head", c_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtfm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the HIP path has no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "tfm_status_string": (ctypes.c_char_p, [c_int]),
            "tfm_last_hip_error": (c_int, []),
            "tfm_version": (ctypes.c_char_p, []),
            "tfm_mfma_rate": (c_int, [c_i64, c_int, c_p, c_p]),
            "tfm_rope_table_init": (c_int, [c_p, c_int, c_int, ctypes.c_double, c_p]),
            "tfm_embed": (c_int, [c_p, c_i64, c_p, c_int, c_int, c_int, c_p, c_p, c_p]),
            "tfm_rmsnorm": (c_int, [c_p, c_int, c_p, c_int, c_p, c_int, c_i64, c_int,
                                    ctypes.c_float, c_p]),
            "tfm_rope": (c_int, [c_p, c_int, c_i64, c_p, c_int, c_int, c_int, c_int, c_p, c_int,
                                 c_p]),
            "tfm_linear": (c_int, [c_p, c_p, c_int, c_p, c_p, c_int, c_i64, c_int, c_int, c_i64,
                                   c_p]),
            "tfm_qkv_rope": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_int, c_int, c_int, c_int,
                                     c_int, c_int, c_p, c_int, c_int, c_p]),
            "tfm_causal_attention": (c_int, [c_p, c_i64, c_p, c_p, c_i64, c_p, c_i64, c_int,
                                             c_int, c_int, c_int, c_int, c_int, c_p]),
            "tfm_sliding_window_attention": (c_int, [c_p, c_i64, c_p, c_p, c_i64, c_p, c_i64,
                                                     c_int, c_int, c_int, c_int, c_int, c_int,
                                                     c_int, c_p]),
            "tfm_swiglu_workspace_bytes": (c_size, [c_i64, c_int, c_int]),
            "tfm_swiglu_ffn": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_i64, c_int, c_int, c_int,
                                       c_p, c_size, c_p]),
            "tfm_workspace_bytes": (c_size, [ctypes.POINTER(Config), c_int, c_int]),
            "tfm_block_forward": (c_int, [ctypes.POINTER(Config), ctypes.POINTER(LayerWeights),
                                          c_p, c_p, c_int, c_int, c_p, c_p, c_size, c_p]),
            "tfm_model_forward": (c_int, [ctypes.POINTER(Config), ctypes.POINTER(ModelWeights),
                                          c_p, c_p, c_p, c_int, c_i64, c_int, c_int, c_p, c_p,
                                          c_size, c_p]),
            "tfm_xent_workspace_bytes": (c_size, [c_i64, c_int]),
            "tfm_lm_head_xent": (c_int, [c_p, c_p, c_p, c_p, c_p, c_i64, c_int, c_int, c_p,
                                         c_size, c_p]),
            "tfm_loss_workspace_bytes": (c_size, [ctypes.POINTER(Config), c_int, c_int]),
            "tfm_model_loss": (c_int, [ctypes.POINTER(Config), ctypes.POINTER(ModelWeights),
                                       c_p, c_p, c_p, c_p, c_p, c_int, c_int, c_p, c_p, c_size,
                                       c_p]),
            "tfm_kv_cache_bytes": (c_size, [ctypes.POINTER(Config), c_int, c_int]),
            "tfm_model_prefill": (c_int, [ctypes.POINTER(Config), ctypes.POINTER(ModelWeights),
                                          c_p, c_p, c_p, c_int, c_i64, c_int, c_int, c_p, c_p,
                                          c_int, c_p, c_size, c_p]),
            "tfm_decode_workspace_bytes": (c_size, [ctypes.POINTER(Config), c_int, c_int]),
            "tfm_model_decode": (c_int, [ctypes.POINTER(Config), ctypes.POINTER(ModelWeights),
                                         c_p, c_p, c_p, c_int, c_i64, c_int, c_p, c_p, c_int,
                                         c_p, c_size, c_p]),
            "tfm_decode_attention_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int]),
            "tfm_decode_attention": (c_int, [c_p, c_i64, c_p, c_p, c_p, c_p, c_i64, c_int, c_int,
                                             c_int, c_int, c_int, c_int, c_p, c_size, c_p]),
            "tfm_decode_attention_noalloc_max_bytes": (c_size, []),
            "tfm_decode_attention_noalloc": (c_int, [c_p, c_i64, c_p, c_p, c_p, c_p, c_i64, c_int,
                                                     c_int, c_int, c_int, c_int, c_int, c_p]),
            "tfm_train_workspace_bytes": (c_size, [ctypes.POINTER(Config), c_int, c_int]),
            "tfm_model_backward": (c_int, [ctypes.POINTER(Config), ctypes.POINTER(ModelWeights),
                                           c_p, c_p, c_p, c_p, ctypes.POINTER(ModelGrads), c_int,
                                           c_int, c_p, c_p, c_size, c_p]),
            "tfm_clip_workspace_bytes": (c_size, [c_int]),
            "tfm_grad_clip_coef": (c_int, [ctypes.POINTER(c_p), ctypes.POINTER(c_i64), c_int,
                                           ctypes.c_float, c_p, c_p, c_p, c_size, c_p]),
            "tfm_adamw_step": (c_int, [c_p, c_p, c_p, c_p, c_p, c_i64, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, c_int, c_p, c_p]),
            "tfm_adamw_step_multi": (c_int, [ctypes.POINTER(c_p), ctypes.POINTER(c_p),
                                             ctypes.POINTER(c_p), ctypes.POINTER(c_p),
                                             ctypes.POINTER(c_p), ctypes.POINTER(c_i64), c_int,
                                             ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                             ctypes.c_float, ctypes.c_float, c_int, c_p, c_p]),
            "tfm_check_device_flags": (c_int, [c_p, c_p]),
            "tfm_trace_begin": (c_int, [c_int, c_p]),
            "tfm_trace_end": (c_int, [ctypes.POINTER(c_int)]),
            "tfm_trace_read": (c_int, [ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_char_p), c_int]),
            "tfm_trace_free": (None, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(st: int, where: str) -> None:
    if st != 0:
        raise TfmError(st, where, lib().tfm_last_hip_error())


# ------------------------------------------------------------------ tensor helpers
def _torch():
    import torch
    return torch


def dt_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TfmError(-3, f"tensor has dtype {t.dtype}, expected torch.float32 or torch.bfloat16")


def torch_dtype(code: int):
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


class _Arg:
    """A tensor argument of a library call with the checks it needs. The library receives bare
    pointers and cannot check anything, so `_call` checks every argument's dtype, layout and
    the element count the call touches on the host, then that each lives on the GPU, and only
    then passes the pointers."""

    __slots__ = ("t", "what", "dtype", "numel", "exact", "rows")

    def __init__(self, t, what, dtype=None, numel=None, exact=False, rows=None):
        self.t, self.what, self.dtype, self.numel, self.exact, self.rows = \
            t, what, dtype, numel, exact, rows

    def host_check(self) -> None:
        t, what = self.t, self.what
        if self.dtype is not None:
            allowed = self.dtype if isinstance(self.dtype, tuple) else (self.dtype,)
            if t.dtype not in allowed:
                raise TfmError(-3, f"{what} has dtype {t.dtype}, expected "
                                   f"{' or '.join(map(str, allowed))}")
        if self.rows is not None:
            rows, width, stride = self.rows
            if t.dim() == 0 or t.stride(-1) != 1:
                raise TfmError(-2, f"{what} must have unit stride along its last dimension")
            if stride < width:
                raise TfmError(-2, f"{what}: row stride {stride} below the row width {width}")
            need = (rows - 1) * stride + width if rows > 0 else 0
            avail = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
            if need > avail:
                raise TfmError(-2, f"{what}: {rows} rows of {width} (stride {stride}) exceed "
                                   "its storage")
            return
        if not t.is_contiguous():
            raise TfmError(-2, f"{what} is not contiguous")
        n = self.numel
        if n is not None and (t.numel() != n if self.exact else t.numel() < n):
            raise TfmError(-2, f"{what} has {t.numel()} elements, the call uses "
                               f"{'' if self.exact else 'at least '}{n}")

    def pointer(self) -> int:
        if not self.t.is_cuda:
            raise ValueError(f"{self.what} must live on the GPU")
        return self.t.data_ptr()


def _dev(t, what: str = "tensor", dtype=None, numel: int | None = None, exact: bool = False):
    """A contiguous device tensor argument (None passes through as a null pointer); `numel` is
    the element count the call touches (at least, or exactly)."""
    return None if t is None else _Arg(t, what, dtype, numel, exact)


def _dev_rows(t, what: str, dtype, rows: int, width: int, stride: int):
    """A row-view argument: `rows` rows of `width` elements, `stride` elements apart, which must
    lie inside the tensor's storage."""
    return None if t is None else _Arg(t, what, dtype, rows=(rows, width, stride))


def _call(name: str, *args) -> None:
    """Call library function `name` after checking every tensor argument on the host, then on
    the device; raise TfmError on a non-zero status."""
    tensors = [a for a in args if isinstance(a, _Arg)]
    for a in tensors:
        a.host_check()
    ptrs = [a.pointer() if isinstance(a, (_Arg, _StreamArg)) else a for a in args]
    _check(getattr(lib(), name)(*ptrs), name)


def _int32():
    return _torch().int32


def _float_types():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


class _StreamArg:
    """The HIP stream argument of a library call (torch's current stream by default), looked up
    after the tensor arguments have passed their checks."""

    __slots__ = ("stream",)

    def __init__(self, stream):
        self.stream = stream

    def pointer(self):
        torch = _torch()
        s = torch.cuda.current_stream() if self.stream is None else self.stream
        return ctypes.c_void_p(s.cuda_stream)


def _stream(stream=None):
    return _StreamArg(stream)


# ------------------------------------------------------------------ entry points
def tfm_rope_table_init(max_seq: int, d_head: int, theta: float = 10000.0, device="cuda",
                        stream=None):
    torch = _torch()
    t = torch.empty(max_seq * d_head, dtype=torch.float32, device=device)
    _call("tfm_rope_table_init", _dev(t, "cos_sin"), max_seq, d_head, float(theta),
                                     _stream(stream))
    return t


def tfm_embed(ids, table, x=None, err_flag=None, stream=None):
    torch = _torch()
    n = ids.numel()
    vocab, d = table.shape
    if x is None:
        x = torch.empty(ids.shape + (d,), dtype=torch.float32, device=table.device)
    _call("tfm_embed", _dev(ids, "ids", _int32()), n, _dev(table, "table", _float_types()),
                           dt_code(table), vocab, d, _dev(x, "x", torch.float32, n * d),
                           _dev(err_flag, "err_flag", _int32(), 1), _stream(stream))
    return x


def tfm_rmsnorm(x, g, eps: float = 1e-5, out_dtype=None, y=None, stream=None):
    torch = _torch()
    d = x.shape[-1]
    if y is None:
        y = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    ft = _float_types()
    _call("tfm_rmsnorm", _dev(x, "x", ft), dt_code(x), _dev(g, "g", ft, d, exact=True),
                             dt_code(g), _dev(y, "y", ft, x.numel()), dt_code(y), x.numel() // d,
                             d, float(eps), _stream(stream))
    return y


def tfm_rope(x, n_heads: int, d_head: int, cos_sin, max_seq: int, positions=None,
             row_stride: int | None = None, stream=None):
    """In-place RoPE on x of shape (B, S, row) (heads at offsets h*d_head)."""
    B, S = x.shape[0], x.shape[1]
    rs = x.stride(1) if row_stride is None else row_stride
    _call("tfm_rope", _dev_rows(x, "x", _float_types(), B * S, n_heads * d_head, rs),
                          dt_code(x), rs, _dev(positions, "positions", _int32(), B * S, exact=True),
                          B, S, n_heads, d_head,
                          _dev(cos_sin, "cos_sin", _torch().float32, max_seq * d_head),
                          max_seq, _stream(stream))
    return x


def tfm_linear(x, w, residual=None, out_dtype=None, y=None, ldy: int | None = None, stream=None):
    torch = _torch()
    N, K = w.shape
    M = x.numel() // K
    if y is None:
        y = torch.empty((M, N if ldy is None else ldy), dtype=out_dtype or x.dtype, device=x.device)
    ld = y.shape[-1] if ldy is None else ldy
    ft = _float_types()
    _call("tfm_linear", _dev(x, "x", ft, M * K, exact=True), _dev(w, "w", x.dtype), dt_code(x),
                            _dev(residual, "residual", torch.float32, M * ld),
                            _dev_rows(y, "y", ft, M, N, ld), dt_code(y), M, N, K, ld,
                            _stream(stream))
    return y


def next_token_targets(ids):
    """(B, S) int32 targets for next-token prediction: ids shifted left by one, -1 last."""
    torch = _torch()
    t = torch.full_like(ids, -1)
    t[:, :-1] = ids[:, 1:]
    return t.contiguous()


def tfm_lm_head_xent(x, w, targets, loss=None, mean=None, stream=None):
    """Fused LM head + cross-entropy: x (M, K) bf16, w (V, K) bf16, targets (M,) int32 ->
    (loss (M,) float32, mean (1,) float32)."""
    torch = _torch()
    V, K = w.shape
    M = x.numel() // K
    if loss is None:
        loss = torch.empty(M, dtype=torch.float32, device=x.device)
    if mean is None:
        mean = torch.empty(1, dtype=torch.float32, device=x.device)
    n = lib().tfm_xent_workspace_bytes(M, V)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
    _call("tfm_lm_head_xent", _dev(x, "x", torch.bfloat16), _dev(w, "w", torch.bfloat16),
                                  _dev(targets, "targets", _int32(), M, exact=True),
                                  _dev(loss, "loss", torch.float32, M),
                                  _dev(mean, "mean", torch.float32, 1), M, V, K, _dev(ws), n,
                                  _stream(stream))
    return loss, mean


def tfm_qkv_rope(xn, wq, wk, wv, n_heads: int, n_kv_heads: int, d_head: int, cos_sin,
                 max_seq: int, positions=None, qkv=None, stream=None):
    """xn (B, S, d) -> qkv (B, S, (Hq + 2 Hkv) d_head) with RoPE on the q and k columns."""
    torch = _torch()
    B, S, d = xn.shape
    width = (n_heads + 2 * n_kv_heads) * d_head
    if qkv is None:
        qkv = torch.empty((B, S, width), dtype=xn.dtype, device=xn.device)
    dt = xn.dtype
    _call("tfm_qkv_rope", _dev(xn, "xn", _float_types()),
                              _dev(wq, "wq", dt, n_heads * d_head * d, exact=True),
                              _dev(wk, "wk", dt, n_kv_heads * d_head * d, exact=True),
                              _dev(wv, "wv", dt, n_kv_heads * d_head * d, exact=True),
                              _dev(qkv, "qkv", dt, B * S * width),
                              _dev(positions, "positions", _int32(), B * S, exact=True), B,
                              S, d, n_heads, n_kv_heads, d_head,
                              _dev(cos_sin, "cos_sin", torch.float32, max_seq * d_head), max_seq,
                              dt_code(xn), _stream(stream))
    return qkv


def tfm_causal_attention(q, k, v, n_heads: int, n_kv_heads: int, d_head: int, o=None,
                         q_stride=None, kv_stride=None, o_stride=None, stream=None):
    """q (B, S, >=Hq*dh) rows; k, v (B, S, >=Hkv*dh) rows (may be strided column views)."""
    torch = _torch()
    B, S = q.shape[0], q.shape[1]
    if o is None:
        o = torch.empty((B, S, n_heads * d_head), dtype=q.dtype, device=q.device)
    qs = q.stride(1) if q_stride is None else q_stride
    kvs = k.stride(1) if kv_stride is None else kv_stride
    os_ = o.stride(1) if o_stride is None else o_stride
    ft, n = _float_types(), B * S
    _call("tfm_causal_attention", _dev_rows(q, "q", ft, n, n_heads * d_head, qs), qs,
                                      _dev_rows(k, "k", q.dtype, n, n_kv_heads * d_head, kvs),
                                      _dev_rows(v, "v", q.dtype, n, n_kv_heads * d_head, kvs), kvs,
                                      _dev_rows(o, "o", q.dtype, n, n_heads * d_head, os_), os_, B,
                                      S, n_heads, n_kv_heads, d_head, dt_code(q), _stream(stream))
    return o


def tfm_sliding_window_attention(q, k, v, n_heads: int, n_kv_heads: int, d_head: int,
                                 window: int, o=None, q_stride=None, kv_stride=None,
                                 o_stride=None, stream=None):
    """Causal attention over the last `window` keys of each query (window >= S is causal)."""
    torch = _torch()
    B, S = q.shape[0], q.shape[1]
    if o is None:
        o = torch.empty((B, S, n_heads * d_head), dtype=q.dtype, device=q.device)
    qs = q.stride(1) if q_stride is None else q_stride
    kvs = k.stride(1) if kv_stride is None else kv_stride
    os_ = o.stride(1) if o_stride is None else o_stride
    ft, n = _float_types(), B * S
    _call("tfm_sliding_window_attention", _dev_rows(q, "q", ft, n, n_heads * d_head, qs), qs,
                                              _dev_rows(k, "k", q.dtype, n, n_kv_heads * d_head, kvs),
                                              _dev_rows(v, "v", q.dtype, n, n_kv_heads * d_head, kvs),
                                              kvs, _dev_rows(o, "o", q.dtype, n, n_heads * d_head, os_),
                                              os_, B, S, n_heads, n_kv_heads, d_head, window,
                                              dt_code(q), _stream(stream))
    return o


def tfm_swiglu_ffn(xn, w1, w3, w2, residual=None, out=None, stream=None):
    torch = _torch()
    d_ff, d = w1.shape
    rows = xn.numel() // d
    dt = dt_code(xn)
    if out is None:
        out = torch.empty((rows, d), dtype=torch.float32, device=xn.device)
    nbytes = lib().tfm_swiglu_workspace_bytes(rows, d_ff, dt)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=xn.device)
    wt = xn.dtype
    _call("tfm_swiglu_ffn", _dev(xn, "xn", _float_types()), _dev(w1, "w1", wt, d_ff * d, exact=True),
                                _dev(w3, "w3", wt, d_ff * d, exact=True),
                                _dev(w2, "w2", wt, d * d_ff, exact=True),
                                _dev(residual, "residual", torch.float32, rows * d),
                                _dev(out, "out", torch.float32, rows * d),
                                rows, d, d_ff, dt, _dev(ws), nbytes, _stream(stream))
    return out


def make_config(cfg, max_seq: int | None = None) -> Config:
    return Config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.d_head, cfg.d_ff,
                  cfg.vocab, max_seq or cfg.seq, cfg.eps, cfg.rope_theta,
                  BF16 if cfg.dtype == "bf16" else F32, getattr(cfg, "window", 0),
                  getattr(cfg, "full_every", 0))


def tfm_workspace_bytes(ccfg: Config, B: int, S: int) -> int:
    return lib().tfm_workspace_bytes(ctypes.byref(ccfg), B, S)


class DeviceModel:
    """Model weights resident in GPU memory plus the RoPE table and a workspace.

    Holds torch tensors (device memory only); every forward runs through the C ABI.
    """

    LAYER_FIELDS = ("g_attn", "wq", "wk", "wv", "wo", "g_ffn", "w1", "w3", "w2")

    def __init__(self, inputs, device="cuda", max_seq: int | None = None, batch: int | None = None,
                 seq: int | None = None):
        torch = _torch()
        cfg = inputs.cfg
        self.cfg = cfg
        self.dtype = torch_dtype(BF16 if cfg.dtype == "bf16" else F32)
        self.max_seq = max_seq or cfg.seq
        self.ccfg = make_config(cfg, self.max_seq)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=self.dtype)
        self.embed = up(inputs.embed)
        self.lm_head = self.embed if inputs.lm_head is inputs.embed else up(inputs.lm_head)
        self.g_final = up(inputs.g_final)
        self.layers = [{f: up(getattr(lw, f)) for f in self.LAYER_FIELDS} for lw in inputs.layers]
        self._layer_structs = (LayerWeights * max(1, len(self.layers)))(
            *[LayerWeights(*[t.data_ptr() for t in (L[f] for f in self.LAYER_FIELDS)])
              for L in self.layers])
        self.weights = ModelWeights(self.embed.data_ptr(), self._layer_structs,
                                    self.g_final.data_ptr(), self.lm_head.data_ptr())
        self.cos_sin = tfm_rope_table_init(self.max_seq, cfg.d_head, cfg.rope_theta, device)
        self.ids = torch.from_numpy(inputs.ids).to(device)
        self._ws = None
        self._ws_shape = None
        self.device = device

    def workspace(self, B: int, S: int):
        """One workspace per (B, S), large enough for the forward and for the fused loss."""
        torch = _torch()
        if self._ws_shape != (B, S):
            n = max(tfm_workspace_bytes(self.ccfg, B, S),
                    lib().tfm_loss_workspace_bytes(ctypes.byref(self.ccfg), B, S))
            if n == 0:
                raise TfmError(-2, "tfm_workspace_bytes")
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
            self._ws_shape = (B, S)
        return self._ws

    def layer_struct(self, i: int) -> LayerWeights:
        return self._layer_structs[i]

    def forward(self, ids=None, positions=None, logits=None, logits_dtype=None, ld_logits=None,
                stream=None):
        torch = _torch()
        ids = self.ids if ids is None else ids
        B, S = ids.shape
        V = self.cfg.vocab
        ld = V if ld_logits is None else ld_logits
        if logits is None:
            logits = torch.empty((B * S, ld), dtype=logits_dtype or self.dtype, device=self.device)
        ws = self.workspace(B, S)
        _call("tfm_model_forward", ctypes.byref(self.ccfg), ctypes.byref(self.weights),
                                       _dev(ids, "ids", _int32(), B * S, exact=True),
                                       _dev(positions, "positions", _int32(), B * S, exact=True),
                                       _dev_rows(logits, "logits", _float_types(), B * S, V, ld),
                                       dt_code(logits), ld, B, S, _dev(self.cos_sin), _dev(ws),
                                       ws.numel(), _stream(stream))
        return logits

    def loss(self, targets, ids=None, positions=None, loss=None, mean=None, stream=None):
        """Forward ending in the fused LM-head cross-entropy: per-token loss (B*S,) float32 and
        the mean over tokens with a target (1,) float32; targets (B, S) int32, -1 = none."""
        torch = _torch()
        ids = self.ids if ids is None else ids
        B, S = ids.shape
        if loss is None:
            loss = torch.empty(B * S, dtype=torch.float32, device=self.device)
        if mean is None:
            mean = torch.empty(1, dtype=torch.float32, device=self.device)
        ws = self.workspace(B, S)
        i32, f32, n = _int32(), torch.float32, B * S
        _call("tfm_model_loss", ctypes.byref(self.ccfg), ctypes.byref(self.weights),
                                    _dev(ids, "ids", i32, n, exact=True),
                                    _dev(positions, "positions", i32, n, exact=True),
                                    _dev(targets, "targets", i32, n, exact=True),
                                    _dev(loss, "loss", f32, n), _dev(mean, "mean", f32, 1), B, S,
                                    _dev(self.cos_sin), _dev(ws), ws.numel(), _stream(stream))
        return loss, mean

    def check_flags(self, stream=None) -> None:
        _call("tfm_check_device_flags", _dev(self._ws), _stream(stream))

    # ---- KV-cache decoding
    def kv_cache(self, B: int, cache_seq: int):
        """A zeroed KV cache for B sequences of up to cache_seq positions (all layers)."""
        torch = _torch()
        n = lib().tfm_kv_cache_bytes(ctypes.byref(self.ccfg), B, cache_seq)
        return torch.zeros(n // 2, dtype=torch.bfloat16, device=self.device)

    def prefill(self, cache, cache_seq: int, ids=None, positions=None, logits=True,
                logits_dtype=None, stream=None):
        """Forward over ids (B, S) that also fills the cache; returns the logits (or None)."""
        torch = _torch()
        ids = self.ids if ids is None else ids
        B, S = ids.shape
        V = self.cfg.vocab
        out = torch.empty((B * S, V), dtype=logits_dtype or self.dtype,
                          device=self.device) if logits else None
        ws = self.workspace(B, S)
        need = lib().tfm_kv_cache_bytes(ctypes.byref(self.ccfg), B, cache_seq)
        _call("tfm_model_prefill", ctypes.byref(self.ccfg), ctypes.byref(self.weights),
                                       _dev(ids, "ids", _int32(), B * S, exact=True),
                                       _dev(positions, "positions", _int32(), B * S, exact=True),
                                       _dev(out, "logits"),
                                       dt_code(out) if out is not None else BF16, V, B, S,
                                       _dev(self.cos_sin),
                                       _dev(cache, "kv_cache", torch.bfloat16, need // 2),
                                       cache_seq, _dev(ws), ws.numel(), _stream(stream))
        return out

    def decode_workspace(self, B: int, cache_seq: int):
        torch = _torch()
        key = ("decode", B, cache_seq)
        if getattr(self, "_dws_key", None) != key:
            n = lib().tfm_decode_workspace_bytes(ctypes.byref(self.ccfg), B, cache_seq)
            if n == 0:
                raise TfmError(-6, "tfm_decode_workspace_bytes")
            self._dws = torch.empty(n, dtype=torch.uint8, device=self.device)
            self._dws_key = key
        return self._dws

    def decode(self, cache, cache_seq: int, ids, positions, logits=None, logits_dtype=None,
               stream=None):
        """One decode step: ids (B,) int32 at positions (B,) int32 -> logits (B, V)."""
        torch = _torch()
        B = ids.shape[0]
        V = self.cfg.vocab
        if logits is None:
            logits = torch.empty((B, V), dtype=logits_dtype or self.dtype, device=self.device)
        ws = self.decode_workspace(B, cache_seq)
        need = lib().tfm_kv_cache_bytes(ctypes.byref(self.ccfg), B, cache_seq)
        ld = logits.shape[-1]
        _call("tfm_model_decode", ctypes.byref(self.ccfg), ctypes.byref(self.weights),
                                      _dev(ids, "ids", _int32(), B, exact=True),
                                      _dev(positions, "positions", _int32(), B, exact=True),
                                      _dev_rows(logits, "logits", _float_types(), B, V, ld),
                                      dt_code(logits), ld, B, _dev(self.cos_sin),
                                      _dev(cache, "kv_cache", torch.bfloat16, need // 2),
                                      cache_seq, _dev(ws), ws.numel(), _stream(stream))
        return logits

    def check_decode_flags(self, stream=None) -> None:
        _call("tfm_check_device_flags", _dev(self._dws), _stream(stream))


def tfm_decode_attention(q, k_cache, v_cache, positions, n_heads: int, n_kv_heads: int,
                         d_head: int, window: int = 0, o=None, stream=None):
    """q (B, Hq*dh) bf16; caches (B, Hkv, cache_seq, dh) bf16; positions (B,) int32."""
    torch = _torch()
    B, cache_seq = q.shape[0], k_cache.shape[2]
    if o is None:
        o = torch.empty((B, n_heads * d_head), dtype=q.dtype, device=q.device)
    n = lib().tfm_decode_attention_workspace_bytes(B, n_heads, d_head, cache_seq)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    bf, cache_n = torch.bfloat16, B * n_kv_heads * cache_seq * d_head
    _call("tfm_decode_attention", _dev_rows(q, "q", bf, B, n_heads * d_head, q.stride(0)),
                                      q.stride(0), _dev(k_cache, "k_cache", bf, cache_n, exact=True),
                                      _dev(v_cache, "v_cache", bf, cache_n, exact=True),
                                      _dev(positions, "positions", _int32(), B, exact=True),
                                      _dev_rows(o, "o", bf, B, n_heads * d_head, o.stride(0)),
                                      o.stride(0), B, n_heads,
                                      n_kv_heads, d_head, cache_seq, window, _dev(ws), ws.numel(),
                                      _stream(stream))
    return o


def tfm_decode_attention_noalloc(q, k_cache, v_cache, positions, n_heads: int, n_kv_heads: int,
                                 d_head: int, window: int = 0, o=None, stream=None):
    """tfm_decode_attention with its split records in the library's static device scratch
    (no workspace, nothing allocated by the library). Concurrent calls on one GPU race."""
    torch = _torch()
    B, cache_seq = q.shape[0], k_cache.shape[2]
    if o is None:
        o = torch.empty((B, n_heads * d_head), dtype=q.dtype, device=q.device)
    bf, cache_n = torch.bfloat16, B * n_kv_heads * cache_seq * d_head
    _call("tfm_decode_attention_noalloc",
          _dev_rows(q, "q", bf, B, n_heads * d_head, q.stride(0)), q.stride(0),
          _dev(k_cache, "k_cache", bf, cache_n, exact=True),
          _dev(v_cache, "v_cache", bf, cache_n, exact=True),
          _dev(positions, "positions", _int32(), B, exact=True),
          _dev_rows(o, "o", bf, B, n_heads * d_head, o.stride(0)), o.stride(0), B, n_heads,
          n_kv_heads, d_head, cache_seq, window, _stream(stream))
    return o


class LaunchTrace:
    """Times every kernel launch of the forward path inside real steps (tfm_trace_begin /
    tfm_trace_end / tfm_trace_read): inside the `with` block each launch records a HIP event
    on its stream; afterwards `records` lists (label, milliseconds) in launch order."""

    def __init__(self, capacity: int, stream=None):
        self.capacity, self.stream, self.records = capacity, stream, []

    def __enter__(self):
        _call("tfm_trace_begin", self.capacity, _stream(self.stream))
        return self

    def __exit__(self, *exc):
        L = lib()
        n = c_int(0)
        L.tfm_trace_end(ctypes.byref(n))
        try:
            if exc[0] is None and n.value > 0:
                ms = (ctypes.c_float * n.value)()
                labels = (ctypes.c_char_p * n.value)()
                _check(L.tfm_trace_read(ms, labels, n.value), "tfm_trace_read")
                self.records = [(labels[i].decode(), float(ms[i])) for i in range(n.value)]
        finally:
            L.tfm_trace_free()
        return False


def tfm_block_forward(dm: DeviceModel, layer: int, x, positions=None, stream=None):
    """One block of ``dm`` on the fp32 residual x (B, S, D), in place."""
    B, S = x.shape[0], x.shape[1]
    ws = dm.workspace(B, S)
    n = B * S
    _call("tfm_block_forward", ctypes.byref(dm.ccfg), ctypes.byref(dm.layer_struct(layer)),
                                   _dev(x, "x", _torch().float32, n * dm.cfg.d_model, exact=True),
                                   _dev(positions, "positions", _int32(), n, exact=True), B, S,
                                   _dev(dm.cos_sin), _dev(ws),
                                   ws.numel(), _stream(stream))
    return x


def tfm_model_forward(dm: DeviceModel, ids=None, positions=None, **kw):
    return dm.forward(ids=ids, positions=positions, **kw)


class Trainer:
    """One training step on the GPU for a DeviceModel [T2 Optimize; T3 12]: forward and
    backward of the mean next-token cross-entropy (tfm_model_backward), global-norm gradient
    clipping (tfm_grad_clip_coef) and AdamW (tfm_adamw_step_multi). Keeps fp32 master weights, fp32
    gradients and the two AdamW moments; for bf16 models the DeviceModel's bf16 weights are
    rewritten from the masters after every step."""

    def __init__(self, dm: "DeviceModel", lr: float = 1e-3, betas=(0.9, 0.95), eps: float = 1e-8,
                 weight_decay: float = 0.1, max_norm: float | None = 1.0):
        torch = _torch()
        self.dm, self.lr, self.betas, self.eps, self.wd, self.max_norm = dm, lr, betas, eps, \
            weight_decay, max_norm
        self.t = 0
        self.tied = dm.lm_head is dm.embed
        names = ["embed"] + ([] if self.tied else ["lm_head"]) + ["g_final"]
        self.params = [(n, getattr(dm, n)) for n in names]
        for l, L in enumerate(dm.layers):
            self.params += [(f"layers.{l}.{f}", L[f]) for f in DeviceModel.LAYER_FIELDS]
        f32 = torch.float32
        self.master = {n: (w if w.dtype == f32 else w.float()) for n, w in self.params}
        self.grad = {n: torch.zeros_like(self.master[n], dtype=f32) for n, _ in self.params}
        self.m = {n: torch.zeros_like(self.grad[n]) for n, _ in self.params}
        self.v = {n: torch.zeros_like(self.grad[n]) for n, _ in self.params}
        G = self.grad
        self._lg = (LayerGrads * max(1, len(dm.layers)))(
            *[LayerGrads(*[G[f"layers.{l}.{f}"].data_ptr() for f in DeviceModel.LAYER_FIELDS])
              for l in range(len(dm.layers))])
        self.cgrads = ModelGrads(G["embed"].data_ptr(), self._lg, G["g_final"].data_ptr(),
                                 G["embed"].data_ptr() if self.tied else G["lm_head"].data_ptr())
        self.loss = torch.zeros(1, dtype=f32, device=dm.device)
        self.coef = torch.ones(1, dtype=f32, device=dm.device)
        self.norm = torch.zeros(1, dtype=f32, device=dm.device)
        n = len(self.params)
        self._gptrs = (c_p * n)(*[G[k].data_ptr() for k, _ in self.params])
        self._gsizes = (c_i64 * n)(*[G[k].numel() for k, _ in self.params])
        self._cws = torch.empty(lib().tfm_clip_workspace_bytes(n), dtype=torch.uint8,
                                device=dm.device)
        # pointer tables of the batched AdamW step
        pm = [self.master[k] for k, _ in self.params]
        self._pptrs = (c_p * n)(*[t.data_ptr() for t in pm])
        self._pbptrs = (c_p * n)(*[None if w is self.master[k] else w.data_ptr()
                                   for k, w in self.params])
        self._mptrs = (c_p * n)(*[self.m[k].data_ptr() for k, _ in self.params])
        self._vptrs = (c_p * n)(*[self.v[k].data_ptr() for k, _ in self.params])
        self._ws = None
        self._ws_shape = None

    def workspace(self, B: int, S: int):
        torch = _torch()
        if self._ws_shape != (B, S):
            nb = lib().tfm_train_workspace_bytes(ctypes.byref(self.dm.ccfg), B, S)
            if nb == 0:
                raise TfmError(-6, "tfm_train_workspace_bytes")
            self._ws = None
            self._ws = torch.empty(nb, dtype=torch.uint8, device=self.dm.device)
            self._ws_shape = (B, S)
        return self._ws

    def backward(self, ids, targets, positions=None, stream=None):
        """Fills self.grad; returns the mean loss (device tensor of 1)."""
        B, S = ids.shape
        ws = self.workspace(B, S)
        dm = self.dm
        i32 = _int32()
        _call("tfm_model_backward", ctypes.byref(dm.ccfg), ctypes.byref(dm.weights),
                                        _dev(ids, "ids", i32, B * S, exact=True),
                                        _dev(positions, "positions", i32, B * S, exact=True),
                                        _dev(targets, "targets", i32, B * S, exact=True),
                                        _dev(self.loss),
                                        ctypes.byref(self.cgrads), B, S, _dev(dm.cos_sin), _dev(ws),
                                        ws.numel(), _stream(stream))
        return self.loss

    def clip(self, stream=None):
        _call("tfm_grad_clip_coef", self._gptrs, self._gsizes, len(self.params),
                                        self.max_norm, _dev(self.coef), _dev(self.norm),
                                        _dev(self._cws), self._cws.numel(), _stream(stream))

    def optimizer_step(self, lr: float | None = None, stream=None):
        self.t += 1
        lr = self.lr if lr is None else lr
        coef = self.coef if self.max_norm is not None else None
        _call("tfm_adamw_step_multi", self._pptrs, self._pbptrs, self._gptrs, self._mptrs,
                                          self._vptrs, self._gsizes, len(self.params), lr,
                                          self.betas[0], self.betas[1], self.eps, self.wd, self.t,
                                          _dev(coef), _stream(stream))

    def step(self, ids, targets, positions=None, lr: float | None = None, stream=None):
        """Forward + backward, clipping (if max_norm) and one AdamW step; returns the loss."""
        loss = self.backward(ids, targets, positions, stream)
        if self.max_norm is not None:
            self.clip(stream)
        self.optimizer_step(lr, stream)
        return loss
