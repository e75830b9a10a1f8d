"""The host packer (comet_pack_weights) against the oracle, bit for bit, after
decoding its fragment-ordered output with the documented layout."""
import numpy as np
import pytest

import w4ax_mixed_precision_amd as comet
from gen import synth
from tests.layout import decode_wq


@pytest.mark.parametrize("name", ["tiny", "q_proj_7b", "down_7b", "decode_70b_n8192_m1"])
def test_pack_matches_oracle(orc, name):
    cfg = synth.CONFIGS[name]
    W = synth.make_w(cfg)
    score = synth.make_scores(cfg)
    if cfg.N * cfg.K > 40e6:                  # bound host time: a slice of output channels
        W = W[:1024]
    N, K = W.shape
    pk = comet.comet_pack_weights(W, score, cfg.nb8)
    perm, flags = orc.channel_order(score, cfg.nb8)
    qw, sw16, wsum = orc.quantize_weights(W, perm)
    assert np.array_equal(pk["perm"], perm)
    assert np.array_equal(pk["flags"], flags)
    assert np.array_equal(pk["w_scale"].T, sw16)
    assert np.array_equal(pk["w_sum"].T.astype(np.int32), wsum)
    assert np.array_equal(decode_wq(pk["Wq"], N, K), qw)


def test_pack_edge_values(orc):
    """All-zero groups, subnormal scales, clamping, ties in the scores."""
    N, K = 128, 384
    rng = np.random.default_rng(4)
    W = synth.to_fp16(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    W[0] = 0
    W[1, :128] = 0
    W[1, 5] = 0x800A           # -10 * 2^-24: scale rounds to the smallest subnormal, code clamps
    W[2, 200] = 0x3C00          # a lone 1.0
    score = np.repeat(np.arange(K // 4, dtype=np.float32), 4)[rng.permutation(K)]
    for nb8 in (0, 1, 3):
        pk = comet.comet_pack_weights(W, score, nb8)
        perm, flags = orc.channel_order(score, nb8)
        qw, sw16, wsum = orc.quantize_weights(W, perm)
        assert np.array_equal(pk["perm"], perm) and np.array_equal(pk["flags"], flags)
        assert np.array_equal(pk["w_scale"].T, sw16)
        assert np.array_equal(pk["w_sum"].T.astype(np.int32), wsum)
        assert np.array_equal(decode_wq(pk["Wq"], N, K), qw)
