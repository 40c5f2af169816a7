"""Work accounting for the decoder forward: FLOPs per GEMM family and HBM bytes per kernel.

Matmul FLOPs follow the rule on "从零实现一个完整的 LLM（CS336）——Transformer 篇" (dujian.net),
parameter and FLOP accounting section: an (m x n) by (n x p) product costs 2mnp. That page
counts attention as two full T x T products per head; the causal path only needs the visible
(query, key) pairs, so ``attention="causal"`` counts 4 * d_head per visible pair, i.e.
4 * d_head * Hq * B * S(S+1)/2, and ``attention="full"`` reproduces the page's convention.
"""
from __future__ import annotations


def visible_pairs(seq: int, window: int = 0) -> int:
    """(query, key) pairs one head of one sequence scores: query s sees keys
    max(0, s - window + 1) .. s (all s + 1 of them when window is 0 or >= seq)."""
    if window <= 0 or window >= seq:
        return seq * (seq + 1) // 2
    return window * (window + 1) // 2 + (seq - window) * window


def attention_flops(batch: int, seq: int, n_heads: int, d_head: int, window: int = 0) -> int:
    """Two products (Q.K^T and P.V) of 2 * d_head flops per visible pair and head."""
    return 4 * d_head * n_heads * batch * visible_pairs(seq, window)


def forward_flops(cfg, batch: int | None = None, seq: int | None = None,
                  attention: str = "causal") -> dict:
    B = cfg.batch if batch is None else batch
    S = cfg.seq if seq is None else seq
    M = B * S
    D, F, V, L = cfg.d_model, cfg.d_ff, cfg.vocab, cfg.n_layers
    qd, kvd = cfg.n_heads * cfg.d_head, cfg.n_kv_heads * cfg.d_head
    qkv = 2 * M * D * (qd + 2 * kvd)
    out = 2 * M * qd * D
    ffn = 2 * M * D * 2 * F + 2 * M * F * D
    if attention == "causal":
        att = attention_flops(B, S, cfg.n_heads, cfg.d_head)
    elif attention == "full":
        att = 4 * cfg.d_head * cfg.n_heads * B * S * S
    else:
        raise ValueError(attention)
    lm = 2 * M * D * V
    per = {"qkv": qkv * L, "out": out * L, "proj": (qkv + out) * L, "ffn": ffn * L,
           "attn": att * L, "lm_head": lm}
    per["total"] = per["proj"] + per["ffn"] + per["attn"] + lm
    per["gemm"] = per["proj"] + per["ffn"] + lm
    return per


def rmsnorm_bytes(rows: int, d: int, in_bytes: int = 4, out_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one RMSNorm call: read each input element once, write each
    output element once (the gain vector is negligible and counted too)."""
    return rows * d * (in_bytes + out_bytes) + d * out_bytes


def model_rmsnorm_bytes(cfg) -> int:
    w = 4 if cfg.dtype == "f32" else 2
    return (2 * cfg.n_layers + 1) * rmsnorm_bytes(cfg.tokens, cfg.d_model, 4, w)


def decode_bytes(cfg, batch: int, context: int, elt: int = 2) -> dict:
    """Algorithmic HBM bytes of one KV-cache decode step (one new token per sequence, each
    attending to `context` cached positions including its own): every weight matrix read
    once (the LM head included; B embedding rows), every layer's K and V cache read over the
    context and one slot of each written. Activations (B rows) are negligible and omitted."""
    D, F, V, L = cfg.d_model, cfg.d_ff, cfg.vocab, cfg.n_layers
    qd, kvd = cfg.n_heads * cfg.d_head, cfg.n_kv_heads * cfg.d_head
    weights = (L * ((qd + 2 * kvd) * D + qd * D + 3 * F * D + 2 * D) + V * D + D) * elt
    embed = batch * D * elt
    cache_read = L * 2 * batch * kvd * context * elt
    cache_write = L * 2 * batch * kvd * elt
    total = weights + embed + cache_read + cache_write
    return {"weights": weights, "kv_cache_read": cache_read, "total": total}


RIDGE_BF16 = 2.5e15 / 8.0e12   # flop per HBM byte where the bf16 MFMA and HBM rooflines meet


def norm_split(cfg) -> bool:
    """Whether the forward splits each block's RMSNorms across the products that write and read
    the residual (bf16 models with d_model <= 3072: at most 16 column tiles of 192, the row
    partials one row of the partials buffer holds)."""
    return cfg.dtype == "bf16" and cfg.d_model <= 3072


def step_kernels(cfg, batch: int | None = None, seq: int | None = None,
                 logits_bytes: int | None = None) -> dict:
    """Algorithmic work of each kernel of one forward, per launch: {label: {"launches",
    "flops", "bytes"}}, the labels those of the library's launch trace. Bytes read every input
    element once and write every output element once (weights included, the residual read and
    written by the residual products); FLOPs follow forward_flops. Where launches of one label
    differ (the last down projection writes no split RMSNorm), the figures are the mean over
    its launches."""
    B = cfg.batch if batch is None else batch
    S = cfg.seq if seq is None else seq
    M = B * S
    D, F, V, L = cfg.d_model, cfg.d_ff, cfg.vocab, cfg.n_layers
    e = 2 if cfg.dtype == "bf16" else 4
    lb = e if logits_bytes is None else logits_bytes
    qd, kvd = cfg.n_heads * cfg.d_head, cfg.n_kv_heads * cfg.d_head
    W = qd + 2 * kvd
    split = norm_split(cfg)
    parts = -(-D // 192)                  # row partials of the split RMSNorm per row
    part_b = M * parts * 4
    rms = rmsnorm_bytes(M, D, 4, e)
    window = getattr(cfg, "window", 0)
    k = {}
    k["fill_flags"] = {"launches": 1, "flops": 0, "bytes": 8}
    # the embedding pass also writes the first block's normalised input (when there is a block)
    k["embed"] = {"launches": 1, "flops": 0,
                  "bytes": M * 4 + M * D * e + M * D * 4 + (M * D * e + D * e if L else 0)}
    k["rmsnorm"] = {"launches": (1 if split else 2 * L) if L else 1, "flops": 0,
                    "bytes": rms + D * e}
    rope_table = S * cfg.d_head * 4       # (cos, sin) of every position 0..S-1
    k["gemm_qkv_rope"] = {"launches": L, "flops": 2 * M * D * W,
                          "bytes": M * D * e + W * D * e + M * W * e + rope_table
                          + (part_b * (L - 1) / L if split else 0)}
    full_layers = L
    if window:
        fe = getattr(cfg, "full_every", 0)
        full_layers = sum(1 for l in range(L) if fe > 0 and l % fe == fe - 1)
    att_bytes = M * qd * e + 2 * M * kvd * e + M * qd * e
    if full_layers:
        k["attention"] = {"launches": full_layers,
                          "flops": attention_flops(B, S, cfg.n_heads, cfg.d_head),
                          "bytes": att_bytes}
    if full_layers < L:
        k["attention_window"] = {"launches": L - full_layers,
                                 "flops": attention_flops(B, S, cfg.n_heads, cfg.d_head, window),
                                 "bytes": att_bytes}
    res_rw = 2 * M * D * 4
    k["gemm_out_residual"] = {"launches": L, "flops": 2 * M * qd * D,
                              "bytes": M * qd * e + qd * D * e + res_rw
                              + ((M * D * e + part_b) if split else 0)}
    k["gemm_swiglu"] = {"launches": L, "flops": 2 * M * D * 2 * F,
                        "bytes": M * D * e + 2 * F * D * e + M * F * e + (part_b if split else 0)}
    k["gemm_down_residual"] = {"launches": L, "flops": 2 * M * F * D,
                               "bytes": M * F * e + F * D * e + res_rw
                               + ((M * D * e + part_b) * (L - 1) / L if split else 0)}
    k["gemm_lm_head"] = {"launches": 1, "flops": 2 * M * D * V,
                         "bytes": M * D * e + V * D * e + M * V * lb}
    for v in k.values():
        v["bytes"] = int(round(v["bytes"]))
        v["bound"] = "mfma" if v["flops"] > RIDGE_BF16 * v["bytes"] else "hbm"
    return k
