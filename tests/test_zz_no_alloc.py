"""GPU check of tfm_decode_attention_noalloc, the decode attention entry point for callers that
cannot allocate: its split records live in the library's static device scratch instead of a
workspace. Through the C ABI it must give exactly what tfm_decode_attention gives on the same
inputs (the same kernels run), on consecutive calls where the second is smaller than the first
(the scratch keeps the previous call's records), and both match the fp64 oracle to the bar of
the decode attention parity tests ("LLMs-from-scratch" (deepseek.csdn.net) 6.1 KV cache)."""
import numpy as np
import pytest

import oracle
from decoder_only_transformer_rmsnorm_amd import synth
from helpers import BF16_ULP, assert_within, say, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoder_only_transformer_rmsnorm_amd import tfm
    tfm.lib()
    yield


def _case(B, Hq, Hkv, dh, T, pos, W, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    q = synth.round_to_bf16(g.normal(size=(B, Hq * dh)).astype(np.float32))
    k = synth.round_to_bf16(g.normal(size=(B, T, Hkv * dh)).astype(np.float32))
    v = synth.round_to_bf16(g.normal(size=(B, T, Hkv * dh)).astype(np.float32))
    hm = lambda c: np.ascontiguousarray(c.reshape(B, T, Hkv, dh).transpose(0, 2, 1, 3))
    return q, k, v, hm(k), hm(v), np.asarray(pos, np.int32)


def test_decode_attention_noalloc_matches_workspace_entry_point():
    from decoder_only_transformer_rmsnorm_amd import tfm
    L = tfm.lib()
    cap = L.tfm_decode_attention_noalloc_max_bytes()
    # first a long grouped-query cache (many split records), then a smaller one
    cases = [(1, 16, 4, 128, 8192, [8000], 0, 1), (2, 8, 2, 64, 2048, [1500, 77], 300, 2),
             (1, 16, 4, 128, 8192, [8000], 0, 1)]
    outs = []
    for B, Hq, Hkv, dh, T, pos, W, seed in cases:
        need = L.tfm_decode_attention_workspace_bytes(B, Hq, dh, T)
        say(f"noalloc decode attention B={B} Hq={Hq} Hkv={Hkv} dh={dh} cache={T} pos={pos} "
            f"window={W}: records {need} B of {cap}")
        assert 0 < need <= cap
        q, k, v, kh, vh, p = _case(B, Hq, Hkv, dh, T, pos, W, seed)
        qd, kd, vd = to_dev(q, "bf16"), to_dev(kh, "bf16"), to_dev(vh, "bf16")
        pd = torch.from_numpy(p).cuda()
        got = tfm.tfm_decode_attention_noalloc(qd, kd, vd, pd, Hq, Hkv, dh, window=W)
        want = tfm.tfm_decode_attention(qd, kd, vd, pd, Hq, Hkv, dh, window=W)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "differs from tfm_decode_attention"
        ref = oracle.decode_attention(q, k, v, Hq, Hkv, p + 1, window=W)
        tol = 2 * BF16_ULP * np.abs(ref) + 1e-5 * float(np.abs(v).max())
        assert_within(to_np(got), ref, tol, "noalloc decode attention")
        outs.append(got.clone())
    assert torch.equal(outs[0], outs[2])   # the same inputs again after a smaller call


def test_decode_attention_noalloc_refuses_oversized_calls():
    from decoder_only_transformer_rmsnorm_amd import tfm
    L = tfm.lib()
    B, Hq, Hkv, dh, T = 64, 32, 4, 128, 4096
    assert L.tfm_decode_attention_workspace_bytes(B, Hq, dh, T) > L.tfm_decode_attention_noalloc_max_bytes()
    q = torch.zeros((B, Hq * dh), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, T, dh), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(tfm.TfmError) as e:
        tfm.tfm_decode_attention_noalloc(q, kc, kc, pos, Hq, Hkv, dh)
    assert e.value.status == -4
