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
