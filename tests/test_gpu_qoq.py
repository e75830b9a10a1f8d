"""GPU parity of the QoQ W4A8 variant (progressive group quantization; QoQ/QServe
article, sections "渐进式分组量化" and "W4A8 GEMM的核心设计") through the C ABI
against the oracle's step 8: per-token INT8 codes and scales, the exact INT32
products P (weights dequantized to 8 bits in registers before the matrix
instruction) and Y, all bit for bit: Y = fp16(fl(s_x s1) float(P)) is the same
three roundings on both sides.
"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import decode_xq_token_i8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()
    return t


def check(torch, X, W, score, label, rows=None):
    """rows: None for every row, else contiguous row ranges the oracle's product
    is compared on (codes and scales are compared on every row)."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    M, K = X.shape
    N = W.shape[0]
    if rows is None:
        d = O.qoq_layer(X, W, score)
    else:
        d = O.qoq_layer(X, W, score, rows[0])
        for r in rows[1:]:
            P2, y2, Y2, e2 = O.qoq_gemm(d["qa"], d["sa"], d["u"], d["s2"], d["z"], d["s1"], r)
            d["P"] = np.concatenate([d["P"], P2])
            d["Y16"] = np.concatenate([d["Y16"], Y2])
            d["yexact"] = np.concatenate([d["yexact"], e2])
    sel = np.arange(M) if rows is None else np.concatenate([np.arange(a, b) for a, b in rows])
    w = comet.upload_qoq(comet.comet_pack_weights_qoq(W, score))
    Xd = torch.from_numpy(X.view(np.float16)).cuda()
    Xq, xs = comet.comet_quant_act_token_i8(Xd, w["perm"])
    Y = comet.comet_w4a8_qoq_gemm(Xq, xs, w, M)
    P = comet.comet_w4a8_qoq_gemm_products(Xq, xs, w, M)
    torch.cuda.synchronize()
    assert np.array_equal(decode_xq_token_i8(Xq.cpu().numpy(), M, K), d["qa"]), f"{label}: codes"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), d["sa"].view(np.uint32)), f"{label}: scales"
    assert np.array_equal(P.cpu().numpy()[sel], d["P"]), f"{label}: products"
    yg = Y.cpu().numpy().view(np.uint16)[sel]
    assert np.array_equal(yg, d["Y16"]), f"{label}: Y"
    rms = float(np.sqrt(np.mean(d["yexact"] ** 2)))
    rel = np.abs(G.f16(yg) - d["yexact"]) / np.maximum(np.abs(d["yexact"]), 1e-2 * rms + 1e-300)
    G.log(f"[qoq] {label}: codes, scales, products and Y bit-exact; Y1 {float(rel.max()):.3e}")
    assert float(rel.max()) <= 1e-3


@pytest.mark.parametrize("name", ["tiny", "decode_70b_n8192_m1", "decode_70b_n28672_m16",
                                  "decode_70b_n10240_m64"])
def test_qoq_layer_parity(torch, name):
    cfg = synth.CONFIGS[name]
    G.log(f"[qoq] {name}")
    check(torch, synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg), name)


@pytest.mark.parametrize("M,K,N", [(1, 128, 128), (3, 256, 256), (17, 4096, 384), (33, 11008, 256),
                                   (64, 512, 1280), (48, 32768, 128)])
def test_qoq_edge_shapes(torch, M, K, N):
    """Ragged M over one to four row tiles, one block, the 7B down-projection width,
    the widest K, an all-zero token and an all-zero weight row."""
    G.log(f"[qoq edge] M={M} K={K} N={N}")
    cfg = synth.LayerConfig("qoq_edge", M, K, N, 3 * M + K)
    X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
    if M > 2:
        X[1] = 0
    W[5] = 0
    check(torch, X, W, score, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("name", ["q_proj_7b", "up_gate_7b", "prefill_up_70b"])
def test_qoq_prefill_parity(torch, name):
    """The tiled kernel (M > 64), in the launch configuration the benchmark
    times; full-size layers compared on their first and last 16 rows."""
    cfg = synth.CONFIGS[name]
    G.log(f"[qoq prefill] {name}")
    rows = None if cfg.M <= 128 else [(0, 16), (cfg.M - 16, cfg.M)]
    check(torch, synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg), name, rows)


@pytest.mark.parametrize("M,K,N", [(65, 256, 128), (100, 1024, 256), (130, 384, 384), (257, 2048, 128)])
def test_qoq_prefill_edge_shapes(torch, M, K, N):
    G.log(f"[qoq prefill edge] M={M} K={K} N={N}")
    cfg = synth.LayerConfig("qoq_pedge", M, K, N, 5 * M + K)
    X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
    X[M - 1] = 0
    check(torch, X, W, score, f"M={M} K={K} N={N}")
