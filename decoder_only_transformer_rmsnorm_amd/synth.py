"""Seeded synthetic inputs for the decoder forward: configurations, token ids and weights.

This module is shared by the HIP path's tests and bench and by the CPU oracle's tests.
It holds none of the model's arithmetic: it only draws random numbers, scales them to the
requested standard deviation, optionally truncates them, and rounds them to bfloat16 when a
configuration runs in bf16. Both sides receive exactly the same values.

Draw order (one ``numpy.random.Generator(PCG64(seed))`` per call of :func:`make_inputs`):
token ids, then the embedding table, then per layer W_Q, W_K, W_V, W_O, W1, W3, W2, then the
LM-head matrix when it is not tied to the embedding. RMSNorm gains are 1 unless ``gamma_std``
is given, in which case they are drawn last (after everything above) as 1 + N(0, gamma_std).

Weight layout is (out_features, in_features), row-major, as the pages store Linear weights
("Transformer 篇" page, section 5.3 Linear: y = x @ W.T).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    dtype: str            # "f32" or "bf16": storage type of weights and GEMM operands
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    d_head: int
    d_ff: int
    vocab: int
    batch: int
    seq: int
    tied: bool = False
    eps: float = 1e-5
    rope_theta: float = 10000.0
    init_std: float = 0.02
    trunc_sigma: float | None = None   # resample draws with |z| > trunc_sigma
    out_proj_scale: float = 1.0        # multiplies the std of W_O and W2
    window: int = 0                    # > 0: sliding-window attention of this many keys
    full_every: int = 0                # > 0: every full_every-th layer keeps full attention

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.d_head

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.d_head

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 model, then bf16 models from small to long-context GQA.
TINY_F32 = ModelConfig("tiny_f32_L2_d64", F32, 2, 64, 4, 4, 16, 176, 65, 4, 64, tied=True)
SMALL_BF16 = ModelConfig("bf16_L4_d512_s256", BF16, 4, 512, 16, 16, 32, 1344, 10000, 32, 256,
                         trunc_sigma=2.0)
GPT2S_BF16 = ModelConfig("bf16_L12_d768_s1024", BF16, 12, 768, 12, 12, 64, 2048, 50257, 8, 1024,
                         out_proj_scale=1.0 / math.sqrt(2 * 12))
XL_BF16 = ModelConfig("bf16_L48_d1600_s1024", BF16, 48, 1600, 25, 25, 64, 4288, 50257, 4, 1024)
LONG_GQA_BF16 = ModelConfig("bf16_gqa_L4_d2048_s8192", BF16, 4, 2048, 16, 4, 128, 5504, 32000, 1, 8192)

CONFIGS = [TINY_F32, SMALL_BF16, GPT2S_BF16, XL_BF16, LONG_GQA_BF16]
BY_NAME = {c.name: c for c in CONFIGS}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out.reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, std: float, trunc: float | None) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if trunc is not None:
        bad = np.abs(z) > trunc
        while bad.any():
            z[bad] = rng.standard_normal(size=int(bad.sum()), dtype=np.float32)
            bad = np.abs(z) > trunc
    z *= np.float32(std)
    return z


@dataclasses.dataclass
class LayerWeights:
    g_attn: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    g_ffn: np.ndarray
    w1: np.ndarray
    w3: np.ndarray
    w2: np.ndarray


@dataclasses.dataclass
class ModelInputs:
    cfg: ModelConfig
    ids: np.ndarray            # int32 (B, S)
    embed: np.ndarray          # float32 (V, D), bf16-representable for bf16 configs
    layers: list[LayerWeights]
    g_final: np.ndarray
    lm_head: np.ndarray        # the same array object as ``embed`` when tied

    def n_params(self) -> int:
        n = self.embed.size + self.g_final.size
        if self.lm_head is not self.embed:
            n += self.lm_head.size
        for lw in self.layers:
            n += sum(getattr(lw, f.name).size for f in dataclasses.fields(lw))
        return n


def make_inputs(cfg: ModelConfig, seed: int = 0, gamma_std: float | None = None,
                qk_gain: float = 1.0, zero_blocks: bool = False) -> ModelInputs:
    """Draw ids and weights for ``cfg``.

    ``qk_gain`` multiplies W_Q and W_K after drawing (a stress variant whose attention
    probabilities are peaked). ``zero_blocks`` sets every projection weight to zero.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq), dtype=np.int64).astype(np.int32)
    std, tr = cfg.init_std, cfg.trunc_sigma
    D = cfg.d_model
    embed = _normal(rng, (cfg.vocab, D), std, tr)
    raw_layers = []
    for _ in range(cfg.n_layers):
        wq = _normal(rng, (cfg.q_dim, D), std, tr)
        wk = _normal(rng, (cfg.kv_dim, D), std, tr)
        wv = _normal(rng, (cfg.kv_dim, D), std, tr)
        wo = _normal(rng, (D, cfg.q_dim), std * cfg.out_proj_scale, tr)
        w1 = _normal(rng, (cfg.d_ff, D), std, tr)
        w3 = _normal(rng, (cfg.d_ff, D), std, tr)
        w2 = _normal(rng, (D, cfg.d_ff), std * cfg.out_proj_scale, tr)
        raw_layers.append([wq, wk, wv, wo, w1, w3, w2])
    lm_head = embed if cfg.tied else _normal(rng, (cfg.vocab, D), std, tr)
    gains = []
    for _ in range(2 * cfg.n_layers + 1):
        if gamma_std is None:
            gains.append(np.ones(D, dtype=np.float32))
        else:
            gains.append((1.0 + _normal(rng, (D,), gamma_std, None)).astype(np.float32))

    def fin(a: np.ndarray) -> np.ndarray:
        return round_to_bf16(a) if cfg.dtype == BF16 else a

    layers = []
    for i, (wq, wk, wv, wo, w1, w3, w2) in enumerate(raw_layers):
        if zero_blocks:
            wq, wk, wv, wo, w1, w3, w2 = (np.zeros_like(w) for w in (wq, wk, wv, wo, w1, w3, w2))
        if qk_gain != 1.0:
            wq = wq * np.float32(qk_gain)
            wk = wk * np.float32(qk_gain)
        layers.append(LayerWeights(fin(gains[2 * i]), fin(wq), fin(wk), fin(wv), fin(wo),
                                   fin(gains[2 * i + 1]), fin(w1), fin(w3), fin(w2)))
    embed_f = fin(embed)
    lm_f = embed_f if cfg.tied else fin(lm_head)
    return ModelInputs(cfg, ids, embed_f, layers, fin(gains[-1]), lm_f)


def random_array(shape, seed: int, std: float = 1.0, dtype: str = F32) -> np.ndarray:
    """A seeded N(0, std) float32 array, rounded to bf16 values when ``dtype`` is bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = _normal(rng, shape, std, None)
    return round_to_bf16(a) if dtype == BF16 else a


def param_count(vocab: int, d_model: int, n_layers: int, d_ff: int, n_heads: int | None = None,
                n_kv_heads: int | None = None, d_head: int | None = None, tied: bool = False) -> int:
    """Number of weights the inputs above hold: embedding, LM head (unless tied), per-layer
    projections and two gains, and the final gain."""
    if n_heads is None:
        qd = kvd = d_model
    else:
        qd, kvd = n_heads * d_head, n_kv_heads * d_head
    per_layer = d_model * qd * 2 + d_model * kvd * 2 + 3 * d_model * d_ff + 2 * d_model
    return vocab * d_model * (1 if tied else 2) + n_layers * per_layer + d_model
