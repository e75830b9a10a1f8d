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


def test_e2m3_codes_of_the_header():
    """The header's E2M3 codes of |q| = 0..7 decode, by the format's definition,
    to exactly 0..7, and their sign-bit twins to -0..-7."""
    from tests.layout import e2m3_value
    codes = np.array([0, 8, 16, 20, 24, 26, 28, 30])
    assert np.array_equal(e2m3_value(codes), np.arange(8.0))
    assert np.array_equal(e2m3_value(codes | 32), -np.arange(8.0))
    # every other code is not an integer in [-7, 7] or is a duplicate zero
    other = np.setdiff1d(np.arange(64), np.concatenate([codes, codes | 32]))
    v = e2m3_value(other)
    assert not np.any((v == np.round(v)) & (np.abs(v) <= 7) & (v != 0))


@pytest.mark.parametrize("name,nb8", [("tiny", 1), ("q_proj_7b", 4), ("down_7b", 22), ("tiny", 0),
                                      ("tiny", 4)])
def test_repack_fp6_matches_oracle(orc, name, nb8):
    from tests.layout import decode_wq_fp6
    cfg = synth.CONFIGS[name]
    W = synth.make_w(cfg)
    score = synth.make_scores(cfg)
    if cfg.N * cfg.K > 20e6:
        W = W[:512]
    N, K = W.shape
    pk = comet.comet_repack_weights_fp6(comet.comet_pack_weights(W, score, nb8))
    assert pk["WqF"].size == comet.wq_fp6_bytes(N, K, nb8)
    perm, _ = orc.channel_order(score, nb8)
    qw, _, _ = orc.quantize_weights(W, perm)
    assert np.array_equal(decode_wq_fp6(pk["WqF"], N, K, nb8), qw)


@pytest.mark.parametrize("name", ["tiny", "q_proj_7b"])
def test_qoq_pack_matches_oracle(name):
    """The library's QoQ pack (perm, s1, s2, z, unsigned codes in fragment order)
    equals the oracle's progressive group quantization bit for bit."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    from tests.layout import decode_wu
    cfg = synth.CONFIGS[name]
    W, score = synth.make_w(cfg), synth.make_scores(cfg)
    pk = comet.comet_pack_weights_qoq(W, score)
    perm, _ = O.channel_order(score, 0)
    s1, w8, s2, z, u = O.qoq_quantize_weights(W, perm)
    assert np.array_equal(pk["perm"], perm)
    assert np.array_equal(pk["s1"], s1)
    assert np.array_equal((pk["s2z"] & 0xFF).T, s2)
    assert np.array_equal((pk["s2z"] >> 8).T, z)
    assert np.array_equal(decode_wu(pk["Wu"], cfg.N, cfg.K), u)


@pytest.mark.parametrize("nb8,nf", [(0, 128), (1, 256), (2, 0)])
def test_pack_quik_matches_oracle(orc, nb8, nf):
    """QUIK's split pack: the perm, the quantized part (decoded) and the fp16
    outlier fragments (decoded) against the oracle's step 10 arrays."""
    from tests.layout import decode_wf, decode_wq_fp6
    cfg = synth.CONFIGS["q_proj_7b"]
    W = synth.make_w(cfg)[:256]
    score = synth.make_scores(cfg)
    N, K = W.shape
    pk = comet.comet_pack_weights_quik(W, score, nb8, nf)
    perm, flags = orc.quik_split(score, nb8, nf)
    kq = K - nf
    qw, sw16, wsum = orc.quantize_weights(np.ascontiguousarray(W[:, perm[:kq]]), np.arange(kq, dtype=np.int32))
    assert np.array_equal(pk["perm"], perm)
    assert np.array_equal(pk["w_scale"].T, sw16)
    assert np.array_equal(pk["w_sum"].T.astype(np.int32), wsum)
    assert np.array_equal(decode_wq(pk["Wq"], N, kq), qw)
    assert np.array_equal(decode_wq_fp6(pk["WqF"], N, kq, nb8), qw)
    if nf:
        assert np.array_equal(decode_wf(pk["Wf"], N, nf), W[:, perm[kq:]])


def test_fp6_activation_tile_covers_every_byte_once():
    """The FP6 activation tile (the quantizer writes it, the GEMM and the test
    decoder read it): every byte of a 1536-byte tile belongs to exactly one
    (row, group, byte), a row's heads form one 64-byte run and its tails one
    32-byte run, and the 8-bit tile's two 1 KB halves use the heads' map."""
    from tests.layout import _tile_rows_index
    head, tail = _tile_rows_index()
    seen = np.zeros(1536, np.int32)
    np.add.at(seen, head.ravel(), 1)
    np.add.at(seen, tail.ravel(), 1)
    assert (seen == 1).all()
    for r in range(16):
        assert sorted(head[r].ravel()) == list(range(64 * r, 64 * r + 64))
        assert sorted(tail[r].ravel()) == list(range(1024 + 32 * r, 1024 + 32 * r + 32))
    # a lane's 16-byte head and 8-byte tail stay aligned for the 128- and 64-bit LDS reads
    assert (head[:, :, 0] % 16 == 0).all() and (tail[:, :, 0] % 8 == 0).all()
