"""Pin of the oracle's fp64 LM-head logits against numpy's fp64 matmul (an independent library
routine) on small shapes, with and without the LoRA delta ([lanes] "헤드냐, LoRA냐": the draft path
adds a low-rank delta to the frozen AR weights)."""
import numpy as np
import pytest

from refdist import bf16_round, bf16_value


@pytest.mark.parametrize("M,H,V,r", [(3, 16, 40, 2), (5, 64, 129, 4), (1, 1, 7, 1)])
def test_lmhead_logits_match_numpy(orc, M, H, V, r):
    rng = np.random.default_rng(M * 100 + H + V)
    h = bf16_round(rng.standard_normal((M, H)))
    W = bf16_round(rng.standard_normal((H, V)) * 0.02)
    A = bf16_round(rng.standard_normal((H, r)) * 0.01)
    Bl = bf16_round(rng.standard_normal((r, V)) * 0.01)
    hv, Wv, Av, Bv = (bf16_value(x) for x in (h, W, A, Bl))
    base = orc.lmhead_logits(h, W)
    assert np.allclose(base, hv @ Wv, rtol=1e-13, atol=1e-15)
    lora = orc.lmhead_logits(h, W, A, Bl, scale=1.0)
    assert np.allclose(lora, hv @ Wv + (hv @ Av) @ Bv, rtol=1e-13, atol=1e-15)
    half = orc.lmhead_logits(h, W, A, Bl, scale=0.5)
    assert np.allclose(half - base, 0.5 * (lora - base), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("M,H,V,r", [(4, 96, 53, 3), (3, 1024, 40, 16), (2, 4096, 24, 16)])
def test_lmhead_rows_helper_matches_plain_oracle(orc, M, H, V, r):
    """The numpy-product helper used at full size agrees with the plain loops, also at a
    contraction length that matters (H up to 4096) with a rank-16 LoRA delta, so the helper's
    operand layout (W[H][V], A[H][r], B[r][V]) is checked where a transposed index would show."""
    rng = np.random.default_rng(7 + H)
    h = bf16_round(rng.standard_normal((M, H)))
    W = bf16_round(rng.standard_normal((H, V)) * 0.02)
    A = bf16_round(rng.standard_normal((H, r)) * 0.01)
    Bl = bf16_round(rng.standard_normal((r, V)) * 0.01)
    plain = orc.lmhead_logits(h, W, A, Bl, scale=1.0)
    helper = orc.lmhead_logits_rows(h, W, A, Bl, 1.0)
    assert np.allclose(plain, helper, rtol=1e-12, atol=1e-14)
    wide = orc.lmhead_logits_rows(h, orc.widen_bf16(W), orc.widen_bf16(A), orc.widen_bf16(Bl), 1.0)
    assert np.array_equal(wide, helper)
    # the check can fail: W with its columns reversed does not agree
    if V >= 2 and H >= 2:
        assert not np.allclose(plain, orc.lmhead_logits_rows(h, W[:, ::-1].copy(), A, Bl, 1.0))
