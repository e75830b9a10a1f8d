"""GPU parity of the asymmetric 4-bit activation variant (QUIK blog, section
"反量化背后的数学": activations with a scale and a zero point, weights with a
scale only, the zero-point term from the offline weight sum) through the C ABI
against the oracle's step 3b.

Bit-exact: stored codes u, 8-bit codes, steps and zero points
(comet_quant_act_asym) and every INT32 block partial sum((u - z) q_w)
(comet_w4ax_gemm_asym_partials). Y (comet_w4ax_gemm_asym) within gates Y1 and
Y2, in the launch configuration of each row count (streaming kernels up to 64
rows, the tiled kernel above).
"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import decode_xq

pytestmark = pytest.mark.gpu

LAYERS = ["tiny", "q_proj_7b", "down_7b", "decode_70b_n8192_m1", "decode_70b_n10240_m16",
          "decode_70b_n8192_m64", "decode_70b_n10240_m64", "decode_70b_n28672_m64", "prefill_up_70b"]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()
    return t


def check(torch, X, W_side, M, K, N, nb8, rows=None, label=""):
    """Quantize X on the GPU and the CPU, then compare codes, partials and Y."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    perm, flags, qw, sw16, pk = (W_side[k] for k in ("perm", "flags", "qw", "sw16", "pk"))
    qa, u4, sa, za = O.quantize_activations_asym(X, perm, flags)
    w = comet.upload_weights(pk)
    Xd = torch.from_numpy(X.view(np.float16)).cuda()
    Xq, xs, xz = comet.comet_quant_act_asym(Xd, w["perm"], nb8)
    Y = comet.comet_w4ax_gemm_asym(Xq, xs, xz, w, M)
    torch.cuda.synchronize()
    nb = K // 128
    nb4 = nb - nb8
    q = decode_xq(Xq.cpu().numpy(), M, K, nb8).astype(np.int16)
    assert np.array_equal(q[:, : nb4 * 128] + 8, u4[:, : nb4 * 128].astype(np.int16)), f"{label}: 4-bit codes"
    assert np.array_equal(q[:, nb4 * 128:], qa[:, nb4 * 128:].astype(np.int16)), f"{label}: 8-bit codes"
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), sa.view(np.uint32)), f"{label}: steps"
    assert np.array_equal(xz.cpu().numpy()[:, :M].T, za), f"{label}: zero points"
    rows = G.sample_rows(M) if rows is None else rows
    d = {"qa": qa, "sa": sa, "qw": qw, "sw16": sw16}
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, rows)
    runs = np.split(rows, np.where(np.diff(rows) != 1)[0] + 1)
    for run in runs:
        P = comet.comet_w4ax_gemm_asym_partials(Xq, xs, xz, w, M, int(run[0]), len(run))
        idx = np.searchsorted(rows, run)
        assert np.array_equal(P.cpu().numpy(), P_o[idx]), f"{label}: partials differ on rows {run[0]}.."
    yhat = G.f16(Y.cpu().numpy().view(np.uint16)[rows])
    y1, y2_ok, y2r = G.gate_y(yhat, ye, tabs, nb)
    G.log(f"[asym] {label}: Y1 max rel err {y1:.3e}, Y2 worst err/bound {y2r:.3f}")
    assert y1 <= 1e-3 and y2_ok
    return Y, yhat, ye


@pytest.mark.parametrize("name", LAYERS)
def test_asym_layer_parity(torch, name):
    cfg = synth.CONFIGS[name]
    G.log(f"[asym] {name}")
    wd = G._weights(cfg)
    X = synth.make_x(cfg)
    check(torch, X, wd, cfg.M, cfg.K, cfg.N, cfg.nb8, label=name)


@pytest.mark.parametrize("M,K,N,nb8", [
    (1, 128, 128, 0), (3, 256, 256, 1), (16, 8192, 1152, 7), (17, 512, 384, 0),
    (24, 8192, 1152, 7), (33, 384, 640, 3), (40, 8192, 10240, 0), (64, 8192, 640, 64),
    (48, 2048, 1024, 2), (100, 1024, 512, 1), (130, 640, 256, 2), (5, 33024, 128, 4),
    (2, 8192, 14336, 3),
])
def test_asym_edge_shapes(torch, M, K, N, nb8):
    """Every kernel path (one- and multi-group streaming, LDS ring and register
    forms, the tiled kernel, the global gather of K > 32768), all-4-bit and
    all-8-bit layers, ragged M, and blocks whose range needs no negative part
    (z = 0), no positive part (z = 15) or nothing (all zero)."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    G.log(f"[asym edge] M={M} K={K} N={N} nb8={nb8}")
    cfg = synth.LayerConfig("edge", M, K, N, 7 * M + K + nb8)
    X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
    if M > 2:
        X[0] = 0                                                     # all-zero token
        X[1] = np.abs(X[1].view(np.float16)).view(np.uint16)         # all positive: z = 0
        X[2] = (-np.abs(X[2].view(np.float16))).view(np.uint16)      # all negative: z = 15
    perm, flags = O.channel_order(score, nb8)
    qw, sw16, wsum = O.quantize_weights(W, perm)
    pk = comet.comet_pack_weights(W, score, nb8)
    wd = {"perm": perm, "flags": flags, "qw": qw, "sw16": sw16, "pk": pk}
    Y, yhat, ye = check(torch, X, wd, M, K, N, nb8, rows=np.arange(M), label=f"M={M} K={K} N={N}")
    if M > 2:
        assert np.all(yhat[0] == 0)


def test_asym_determinism(torch):
    import w4ax_mixed_precision_amd as comet
    cfg = synth.CONFIGS["decode_70b_n8192_m64"]
    wd = G._weights(cfg)
    w = comet.upload_weights(wd["pk"])
    X = torch.from_numpy(synth.make_x(cfg).view(np.float16)).cuda()
    Xq, xs, xz = comet.comet_quant_act_asym(X, w["perm"], cfg.nb8)
    Y1 = comet.comet_w4ax_gemm_asym(Xq, xs, xz, w, cfg.M)
    Y2 = comet.comet_w4ax_gemm_asym(Xq, xs, xz, w, cfg.M)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
