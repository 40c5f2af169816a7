"""GPU parity of the fused LM-head cross-entropy (tfm_lm_head_xent, tfm_model_loss) against the
fp64 oracle ("LLM 2" Optimize / Loss: loss = logsumexp(logits) - logits[target]).

Tolerances
  * Standalone: the GPU forms each logit from bf16 inputs with fp32 accumulation over K terms,
    so |dz| <= K 2^-23 sum_k |x_k w_k|; the log-sum-exp moves by at most max |dz| and the
    target logit by the same, plus fp32 rounding of the exp sums (well under 1e-4 absolute at
    these sizes): tol = 2 K 2^-23 max_j sum_k |x_k w_jk| + 1e-4 (1 + |loss|).
  * Against the GPU's own float32 logits (same products, different summation order only):
    1e-4 absolute.
  * Whole model: the loss is 1-Lipschitz in each of logsumexp and the target logit, so the
    logits bar max|dL| <= 2e-2 max|L| gives |d loss| <= 4e-2 max|L|.
"""
import numpy as np
import pytest

import oracle
from decoder_only_transformer_rmsnorm_amd import synth
from helpers import F32_EPS, say, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoder_only_transformer_rmsnorm_amd import tfm
    tfm.lib()
    yield


def tfm_mod():
    from decoder_only_transformer_rmsnorm_amd import tfm
    return tfm


def _problem(M, V, K, seed, x_std=1.0, w_std=0.05):
    g = np.random.Generator(np.random.PCG64(seed))
    x = synth.round_to_bf16(g.normal(0, x_std, (M, K)).astype(np.float32))
    w = synth.round_to_bf16(g.normal(0, w_std, (V, K)).astype(np.float32))
    t = g.integers(-1, V, M).astype(np.int32)
    t[0] = 0
    if M > 1:
        t[1] = V - 1
    return x, w, t


def _tol(x, w, loss_ref, rows=None):
    K = x.shape[1]
    xs = np.abs(x if rows is None else x[rows]).astype(np.float64)
    bound = (xs @ np.abs(w).T.astype(np.float64)).max(axis=1)
    return 2 * K * F32_EPS * bound + 1e-4 * (1 + np.abs(loss_ref))


@pytest.mark.parametrize("M,V,K", [(300, 1000, 256), (192, 128, 64), (5, 7, 64), (777, 3001, 512)])
def test_lm_head_xent_matches_oracle(M, V, K):
    tfm = tfm_mod()
    say(f"xent M={M} V={V} K={K}")
    x, w, t = _problem(M, V, K, seed=M + V)
    loss, mean = tfm.tfm_lm_head_xent(to_dev(x, "bf16"), to_dev(w, "bf16"),
                                      torch.from_numpy(t).cuda())
    torch.cuda.synchronize()
    ref, ref_mean = oracle.cross_entropy(oracle.linear(x, w), t)
    got = to_np(loss)
    err = np.abs(got - ref)
    tol = _tol(x, w, ref)
    say(f"  max err {err.max():.3e}, worst err/tol {(err / tol).max():.3f}")
    assert np.isfinite(got).all()
    assert (err <= tol).all()
    assert (got[t < 0] == 0).all()
    assert abs(float(mean.item()) - ref_mean) <= float(tol.max())


def test_lm_head_xent_matches_its_own_unfused_logits():
    """Same inputs through tfm_linear (float32 logits) and the CPU logsumexp: only the order of
    the fp32 sums differs, so the two agree far inside the oracle tolerance."""
    tfm = tfm_mod()
    M, V, K = 400, 5000, 384
    x, w, t = _problem(M, V, K, seed=7)
    xd, wd, td = to_dev(x, "bf16"), to_dev(w, "bf16"), torch.from_numpy(t).cuda()
    loss, _ = tfm.tfm_lm_head_xent(xd, wd, td)
    logits = tfm.tfm_linear(xd, wd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.cross_entropy(to_np(logits), t)
    err = float(np.abs(to_np(loss) - ref).max())
    say(f"  fused vs unfused max err {err:.3e}")
    assert err <= 1e-4


def test_lm_head_xent_ignored_rows_mean_and_bad_target():
    tfm = tfm_mod()
    M, V, K = 130, 300, 64
    x, w, _ = _problem(M, V, K, seed=9)
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")
    none = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    loss, mean = tfm.tfm_lm_head_xent(xd, wd, none)
    torch.cuda.synchronize()
    assert float(loss.abs().max()) == 0.0 and float(mean.item()) == 0.0
    t = np.random.Generator(np.random.PCG64(10)).integers(0, V, M).astype(np.int32)
    t[17] = V                          # out of range: that row's loss is NaN
    loss, _ = tfm.tfm_lm_head_xent(xd, wd, torch.from_numpy(t).cuda())
    torch.cuda.synchronize()
    got = to_np(loss)
    assert np.isnan(got[17]) and np.isfinite(np.delete(got, 17)).all()


def test_lm_head_xent_full_size_sampled():
    """The d768 LM-head shape (8192 x 50257 x 768) in one launch; the oracle recomputes a
    sample of rows (each a full 50257-wide logsumexp)."""
    tfm = tfm_mod()
    M, V, K = 8192, 50257, 768
    g = np.random.Generator(np.random.PCG64(21))
    x = synth.round_to_bf16(g.normal(0, 1.0, (M, K)).astype(np.float32))
    w = synth.round_to_bf16(g.normal(0, 0.02, (V, K)).astype(np.float32))
    t = g.integers(0, V, M).astype(np.int32)
    loss, mean = tfm.tfm_lm_head_xent(to_dev(x, "bf16"), to_dev(w, "bf16"),
                                      torch.from_numpy(t).cuda())
    torch.cuda.synchronize()
    rows = np.array([0, 1, 191, 192, 4095, 5000, 8190, 8191])
    ref, _ = oracle.cross_entropy(oracle.linear(x[rows], w), t[rows])
    got = to_np(loss)[rows]
    err = np.abs(got - ref)
    tol = _tol(x, w, ref, rows)
    say(f"  sampled max err {err.max():.3e}, worst err/tol {(err / tol).max():.3f}")
    assert (err <= tol).all()
    assert np.isfinite(to_np(loss)).all()


def _model_case(cfg, seqs, prefix=None, gamma_std=None):
    tfm = tfm_mod()
    inp = synth.make_inputs(cfg, seed=0, gamma_std=gamma_std)
    dm = tfm.DeviceModel(inp)
    ids = dm.ids
    targets = tfm.next_token_targets(ids)
    loss, mean = dm.loss(targets)
    dm.check_flags()
    torch.cuda.synchronize()
    got = to_np(loss).reshape(cfg.batch, cfg.seq)
    t_np = oracle.next_token_targets(inp.ids)
    S = cfg.seq if prefix is None else prefix
    worst = 0.0
    for b in seqs:
        logits = oracle.model(cfg, inp, ids=inp.ids[b:b + 1, :S])
        tb = t_np[b, :S].copy()
        ref, _ = oracle.cross_entropy(logits.reshape(S, cfg.vocab), tb)
        bar = 4e-2 * float(np.abs(logits).max())
        err = float(np.abs(got[b, :S] - ref).max())
        worst = max(worst, err / bar)
        say(f"  seq {b}: max |d loss| {err:.3e} (bar {bar:.3e})")
        assert err <= bar
    return dm, loss, mean, worst


def test_model_loss_small_full_size():
    """The d512 / 4-layer workload at batch 32 x 256: fused loss of 3 sequences against the
    oracle's logits, the mean over all tokens, and run-to-run bitwise determinism."""
    cfg = synth.SMALL_BF16
    dm, loss, mean, _ = _model_case(cfg, [0, 13, 31])
    got = to_np(loss).reshape(cfg.batch, cfg.seq)
    assert (got[:, -1] == 0).all()                    # last position has no target
    expect = float(got[:, :-1].astype(np.float64).mean())
    assert abs(float(mean.item()) - expect) <= 1e-5 * abs(expect)
    tfm = tfm_mod()
    again, _ = dm.loss(tfm.next_token_targets(dm.ids))
    assert torch.equal(loss, again)


def test_model_loss_split_norm_nonunit_gains():
    """A 3-layer d256 bf16 model with RMSNorm gains 1 + N(0, 0.1): the fused loss runs the same
    trunk as the forward, with each block's RMSNorms split across the products that write and
    read the residual ("Transformer 篇" (dujian.net) 5.6), so every row's loss is compared with
    the oracle's."""
    cfg = synth.ModelConfig(name="loss_gain", dtype="bf16", n_layers=3, d_model=256, n_heads=8,
                            n_kv_heads=2, d_head=32, d_ff=704, vocab=1000, batch=3, seq=96)
    _model_case(cfg, [0, 1, 2], gamma_std=0.1)


def test_model_loss_d768_full_size_sampled():
    """The benchmark workload (d768, 12 layers, 8 x 1024): one whole sequence against the
    oracle; and the fused loss against the logsumexp of the same model's float32 logits."""
    cfg = synth.GPT2S_BF16
    dm, loss, _, _ = _model_case(cfg, [5])
    lg = dm.forward(logits_dtype=torch.float32)
    torch.cuda.synchronize()
    t = oracle.next_token_targets(synth.make_inputs(cfg, seed=0).ids).reshape(-1)
    rows = np.arange(0, cfg.batch * cfg.seq, 97)
    ref, _ = oracle.cross_entropy(to_np(lg[torch.from_numpy(rows).cuda()]), t[rows])
    err = float(np.abs(to_np(loss)[rows] - ref).max())
    say(f"  fused vs model float32 logits: max err {err:.3e}")
    assert err <= 1e-3
