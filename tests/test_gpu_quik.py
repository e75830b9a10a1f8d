"""QUIK's fp16 outlier columns on the GPU (FP6 layout) against the oracle's
step 10 (QUIK blog, deep-paper.org/paper/2310.09259, section "第二步: 前向传播
(在线)": the quantized part and the fp16 outlier part on their own paths, the
results added): the quantized codes and scales and the fp16 outlier tiles bit
for bit, Y within the gates, over the small-grid split plans, the 128 x 256
tile, ragged rows and one row."""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import decode_xf, decode_xq_fp6

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()
    return t


def _layer(seed, M, N, K):
    rng = np.random.default_rng(seed)
    X = rng.normal(0, 1, (M, K)).astype(np.float32)
    X[:, rng.permutation(K)[: K // 10]] *= 50.0
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    calib = rng.normal(0, 1, (64, K)).astype(np.float32)
    calib[:, np.argsort(-np.abs(X).max(0))[: K // 10]] *= 50.0
    return synth.to_fp16(X), synth.to_fp16(W), np.abs(calib).max(0).astype(np.float32)


def _run(torch, M, K, N, nb8, nf, seed):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    G.log(f"[quik] M={M} K={K} N={N} nb8={nb8} nf={nf}")
    X, W, score = _layer(seed, M, N, K)
    pk = comet.comet_pack_weights_quik(W, score, nb8, nf)
    w = comet.upload_weights(pk)
    perm, flags = O.quik_split(score, nb8, nf)
    assert np.array_equal(pk["perm"], perm)
    kq = K - nf
    pq = np.ascontiguousarray(perm[:kq])
    qw, sw16, _ = O.quantize_weights(np.ascontiguousarray(W[:, pq]), np.arange(kq, dtype=np.int32))
    qa, sa = O.quantize_activations(np.ascontiguousarray(X[:, pq]), np.arange(kq, dtype=np.int32), flags)
    Xd = torch.from_numpy(X.view(np.float16)).cuda()
    Xq, xs, Xf = comet.comet_quant_act_quik_fp6(Xd, w["perm"], nb8, nf)
    Y = comet.comet_w4ax_gemm_quik_fp6(Xq, xs, Xf, w, M)
    Y2 = comet.comet_w4ax_gemm_quik_fp6(Xq, xs, Xf, w, M)
    torch.cuda.synchronize()
    # the quantized part's codes and scales, and the fp16 outlier tiles
    assert np.array_equal(decode_xq_fp6(Xq.cpu().numpy(), M, kq, nb8), qa)
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), sa.view(np.uint32))
    Xf_h = Xf.cpu().numpy().view(np.uint16)
    assert np.array_equal(decode_xf(Xf_h, M, nf), X[:, perm[kq:]]) if nf else True
    if nf:                                               # padded rows are zero
        mp = (M + 15) // 16 * 16
        pad = decode_xf(np.concatenate([Xf_h, np.zeros(0, np.uint16)]), mp, nf)[M:]
        assert not pad.any()
    yb = Y.cpu().numpy().view(np.uint16)
    assert np.array_equal(yb, Y2.cpu().numpy().view(np.uint16)), "determinism"
    rows = G.sample_rows(M)
    P = O.block_partials(qa[rows], qw)
    y32, _, ye = O.epilogue(P, sa[rows], sw16)
    Xf_o = np.ascontiguousarray(X[rows][:, perm[kq:]])
    Wf_o = np.ascontiguousarray(W[:, perm[kq:]])
    y32, Y16, ye = O.quik_outlier_add(Xf_o, Wf_o, y32, ye)
    tabs = (np.abs(sa[rows].astype(np.float64)[:, None, :] * G.f16(sw16)[None, :, :] * P)).sum(-1)
    tabs += np.abs(G.f16(Xf_o)) @ np.abs(G.f16(Wf_o)).T
    y1, y2_ok, y2r = G.gate_y(G.f16(yb[rows]), ye, tabs, kq // 128 + nf)
    G.log(f"[quik] gates: Y1 {y1:.2e}, Y2 {y2r:.3f}")
    assert y1 <= 1e-3 and y2_ok, (y1, y2r)
    return Y


# (M, K, N, nb8, nf): one 16-row tile; a split plan with the work queue
# (q_proj_7b-like); ragged rows; one row; the 128 x 256 tile over 1024 tiles;
# rows wider than the LDS staging (the quantizer's and the gather's global
# paths)
SHAPES = [(16, 512, 512, 0, 128), (128, 4096, 4096, 4, 256), (100, 1024, 512, 1, 256), (1, 8192, 1024, 2, 128),
          (4096, 2048, 8192, 2, 256), (5, 33280, 256, 3, 256)]


@pytest.mark.parametrize("M,K,N,nb8,nf", SHAPES)
def test_quik_parity(torch, M, K, N, nb8, nf):
    _run(torch, M, K, N, nb8, nf, seed=M + K + nf)


def test_quik_nf0_is_the_plain_fp6_gemm(torch):
    """With no outlier channels the QUIK calls are the plain FP6 calls, bit for bit."""
    import w4ax_mixed_precision_amd as comet
    M, K, N, nb8 = 64, 1024, 1024, 1
    X, W, score = _layer(11, M, N, K)
    pq = comet.upload_weights(comet.comet_pack_weights_quik(W, score, nb8, 0))
    pp = comet.upload_weights(comet.comet_repack_weights_fp6(comet.comet_pack_weights(W, score, nb8)))
    Xd = torch.from_numpy(X.view(np.float16)).cuda()
    Xq, xs, Xf = comet.comet_quant_act_quik_fp6(Xd, pq["perm"], nb8, 0)
    Yq = comet.comet_w4ax_gemm_quik_fp6(Xq, xs, Xf, pq, M)
    Xq2, xs2 = comet.comet_quant_act_fp6(Xd, pp["perm"], nb8)
    Yp = comet.comet_w4ax_gemm_fp6(Xq2, xs2, pp, M)
    torch.cuda.synchronize()
    assert np.array_equal(Yq.cpu().numpy().view(np.uint16), Yp.cpu().numpy().view(np.uint16))
