"""Host checks of the work accounting that bench.py divides by: attention pair counts against
brute force over the band mask, and the GEMM FLOPs against the 2mnp rule summed over the
model's weight shapes."""
import numpy as np
import pytest

from decoder_only_transformer_rmsnorm_amd import accounting, synth


@pytest.mark.parametrize("S,W", [(1, 0), (7, 0), (7, 3), (7, 7), (7, 50), (64, 1), (300, 48)])
def test_visible_pairs_match_the_band_mask(S, W):
    s = np.arange(S)[:, None]
    t = np.arange(S)[None, :]
    mask = t <= s
    if 0 < W:
        mask &= t > s - W
    assert accounting.visible_pairs(S, W) == int(mask.sum())


def test_forward_flops_follow_the_weight_shapes():
    cfg = synth.GPT2S_BF16
    inp = synth.make_inputs(cfg.replace(n_layers=1, batch=1, seq=4), seed=0)
    L0 = inp.layers[0]
    per_token_layer = 2 * sum(getattr(L0, f).size for f in ("wq", "wk", "wv", "wo", "w1", "w3", "w2"))
    f = accounting.forward_flops(cfg)
    M = cfg.batch * cfg.seq
    assert f["proj"] + f["ffn"] == cfg.n_layers * M * per_token_layer
    assert f["lm_head"] == 2 * M * inp.lm_head.size
    assert f["attn"] == cfg.n_layers * accounting.attention_flops(cfg.batch, cfg.seq, cfg.n_heads,
                                                                   cfg.d_head)


@pytest.mark.parametrize("name", ["TINY_F32", "SMALL_BF16", "GPT2S_BF16", "XL_BF16", "LONG_GQA_BF16"])
def test_step_kernels_add_up_to_the_forward(name):
    """The per-kernel work the benchmark rates each launch by sums, over the launches of one
    forward, to the whole forward's FLOPs; the RMSNorm launches and their bytes follow whether
    the norms are split across the products."""
    cfg = getattr(synth, name)
    k = accounting.step_kernels(cfg)
    total = sum(v["flops"] * v["launches"] for v in k.values())
    assert total == accounting.forward_flops(cfg)["total"]
    split = accounting.norm_split(cfg)
    # the first block's RMSNorm runs inside the embedding pass
    assert k["rmsnorm"]["launches"] == (1 if split else 2 * cfg.n_layers)
    M, D = cfg.tokens, cfg.d_model
    e = 2 if cfg.dtype == "bf16" else 4
    assert k["gemm_lm_head"]["bytes"] == M * D * e + cfg.vocab * D * e + M * cfg.vocab * e
    for v in k.values():
        assert v["bound"] == ("mfma" if v["flops"] > accounting.RIDGE_BF16 * v["bytes"] else "hbm")
