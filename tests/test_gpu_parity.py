"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: activation codes and scales (comet_quant_act) and every INT32 block
partial (comet_w4ax_gemm_partials). Y (comet_w4ax_gemm) within gate Y1
(max relative error 1e-3, floored at 1e-2 rms) and gate Y2 (a rigorous
per-element FP32 bound). Full-size layers are checked on sampled rows, in the
launch configuration the benchmark times.
"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import decode_xq, zero_extended_codes_valid

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "q_proj_7b"]
MEDIUM = ["up_gate_7b", "down_7b"]
DECODE = [f"decode_70b_n{n}_m{m}" for n in (10240, 8192, 28672) for m in (1, 4, 16, 64)]
PREFILL = ["prefill_down_70b", "prefill_up_70b"]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()        # the HIP library must load: no fallback
    return t


def run_layer(torch, name):
    import w4ax_mixed_precision_amd as comet
    d = G.host_layer(name)
    pk = d["pk"]
    cfg = d["cfg"]
    X, w = G.device_layer(d, pk)
    Xq, xs = comet.comet_quant_act(X, w["perm"], cfg.nb8)
    Y = comet.comet_w4ax_gemm(Xq, xs, w, cfg.M)
    torch.cuda.synchronize()
    return d, pk, w, Xq, xs, Y


@pytest.mark.parametrize("name", SMALL + MEDIUM + DECODE + PREFILL)
def test_layer_parity(torch, name):
    import w4ax_mixed_precision_amd as comet
    G.log(f"[parity] {name}")
    d, pk, w, Xq, xs, Y = run_layer(torch, name)
    cfg = d["cfg"]
    # comet_quant_act: codes and scales bit-exact
    xq_h = Xq.cpu().numpy()
    assert zero_extended_codes_valid(xq_h, cfg.M, cfg.K, cfg.nb8)
    qa = decode_xq(xq_h, cfg.M, cfg.K, cfg.nb8)
    assert np.array_equal(qa, d["qa"]), "activation codes differ"
    sa = xs.cpu().numpy().T
    assert np.array_equal(sa.view(np.uint32), d["sa"].view(np.uint32)), "activation scales differ"
    # partials bit-exact on the sampled rows
    rows = G.sample_rows(cfg.M)
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, rows)
    runs = np.split(rows, np.where(np.diff(rows) != 1)[0] + 1)
    for run in runs:
        P = comet.comet_w4ax_gemm_partials(Xq, xs, w, cfg.M, int(run[0]), len(run))
        idx = np.searchsorted(rows, run)
        assert np.array_equal(P.cpu().numpy(), P_o[idx]), f"partials differ on rows {run[0]}.."
    # Y gates
    yhat = G.f16(Y.cpu().numpy().view(np.uint16)[rows])
    y1, y2_ok, y2_ratio = G.gate_y(yhat, ye, tabs, cfg.nb)
    G.log(f"[parity] {name}: Y1 max rel err {y1:.3e}, Y2 worst err/bound {y2_ratio:.3f}")
    assert y1 <= 1e-3
    assert y2_ok


def _custom_layer(M, K, N, nb8, seed, zero_rows=(), zero_block_rows=(), ldx=None):
    cfg = synth.LayerConfig("edge", M, K, N, seed)
    X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
    for r in zero_rows:
        X[r] = 0
    from oracle import oracle as O
    d = O.quantize_layer(X, W, score, nb8)
    for r, b in zero_block_rows:        # zero one permuted block of a row
        X[r, d["perm"][128 * b:128 * (b + 1)]] = 0
    d = O.quantize_layer(X, W, score, nb8)
    d.update({"X": X, "W": W, "score": score,
              "cfg": synth.LayerConfig("edge", M, K, N, seed, int8_frac=None)})
    if ldx is not None:
        Xp = np.zeros((M, ldx), np.uint16)
        Xp[:, :K] = X
        d["Xpad"] = Xp
    return d


@pytest.mark.parametrize("M,K,N,nb8", [
    (1, 128, 128, 0), (1, 128, 128, 1), (3, 256, 256, 2), (17, 512, 384, 0),
    (33, 384, 640, 3), (100, 1024, 512, 1), (5, 33024, 128, 4),   # K > 32768: global gather path
    # decode kernels with the LDS weight ring (8, 4 and 16 blocks per wave)
    (2, 4096, 384, 3), (16, 8192, 1152, 7), (9, 16384, 128, 20),
    # decode kernels for 17..64 rows, several channel groups per wave: the
    # LDS-ring form at 64 blocks (narrow: two groups, eight waves; wide: four
    # groups, four waves; wide with eight waves on grids below one
    # workgroup per CU) and the register form at other block counts
    (24, 8192, 1152, 7), (64, 8192, 640, 0), (40, 8192, 10240, 64), (57, 8192, 12288, 5),
    (20, 1024, 24576, 1), (48, 2048, 1024, 16),
    # half-group units (N = 2048 H): H = 5 at one to four row tiles, H = 7 at one
    (16, 8192, 10240, 64), (25, 8192, 10240, 0), (3, 8192, 14336, 7), (64, 8192, 10240, 9),
])
def test_edge_shapes(torch, M, K, N, nb8):
    import w4ax_mixed_precision_amd as comet
    G.log(f"[edge] M={M} K={K} N={N} nb8={nb8}")
    d = _custom_layer(M, K, N, nb8, seed=M * 7 + K + nb8,
                      zero_rows=(0,) if M > 2 else (), zero_block_rows=((M - 1, 0),))
    pk = comet.comet_pack_weights(d["W"], d["score"], nb8)
    w = comet.upload_weights(pk)
    X = torch.from_numpy(d["X"].view(np.float16)).cuda()
    Xq, xs = comet.comet_quant_act(X, w["perm"], nb8)
    Y = comet.comet_w4ax_gemm(Xq, xs, w, M)
    P = comet.comet_w4ax_gemm_partials(Xq, xs, w, M)
    torch.cuda.synchronize()
    assert np.array_equal(decode_xq(Xq.cpu().numpy(), M, K, nb8), d["qa"])
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), d["sa"].view(np.uint32))
    rows = np.arange(M)
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, rows)
    assert np.array_equal(P.cpu().numpy(), P_o)
    yhat = G.f16(Y.cpu().numpy().view(np.uint16))
    y1, y2_ok, _ = G.gate_y(yhat, ye, tabs, K // 128)
    assert y1 <= 1e-3 and y2_ok
    if M > 2:
        assert np.all(yhat[0] == 0)          # an all-zero token row gives exact zeros


def test_strided_x_and_y(torch):
    """ldx > K and ldy > N: only the leading columns are read or written."""
    import w4ax_mixed_precision_amd as comet
    M, K, N, nb8 = 20, 512, 256, 1
    d = _custom_layer(M, K, N, nb8, seed=77, ldx=K + 40)
    pk = comet.comet_pack_weights(d["W"], d["score"], nb8)
    w = comet.upload_weights(pk)
    Xpad = torch.from_numpy(d["Xpad"].view(np.float16)).cuda()
    Xpad[:, K:] = float("nan")               # must never be read
    Xq, xs = comet.comet_quant_act(Xpad, w["perm"], nb8)
    Ybig = torch.full((M, N + 72), 7.0, dtype=torch.float16, device="cuda")
    comet.comet_w4ax_gemm(Xq, xs, w, M, Y=Ybig)
    torch.cuda.synchronize()
    assert np.array_equal(decode_xq(Xq.cpu().numpy(), M, K, nb8), d["qa"])
    yb = Ybig.cpu().numpy()
    assert np.all(yb[:, N:] == 7.0)
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, np.arange(M))
    y1, y2_ok, _ = G.gate_y(yb[:, :N].astype(np.float64), ye, tabs, K // 128)
    assert y1 <= 1e-3 and y2_ok


def test_guard_canaries(torch):
    """Outputs written exactly inside their extents: guard bytes around Xq, x_scale and Y."""
    import w4ax_mixed_precision_amd as comet
    M, K, N, nb8 = 37, 640, 384, 2
    d = _custom_layer(M, K, N, nb8, seed=91)
    pk = comet.comet_pack_weights(d["W"], d["score"], nb8)
    w = comet.upload_weights(pk)
    X = torch.from_numpy(d["X"].view(np.float16)).cuda()
    pad = 256
    nxq = comet.xq_bytes(M, K, nb8)
    xq_buf = torch.full((nxq + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    xs_buf = torch.full(((K // 128) * M + 2 * pad,), -3.0, dtype=torch.float32, device="cuda")
    y_buf = torch.full((M * N + 2 * pad,), 5.0, dtype=torch.float16, device="cuda")
    Xq = xq_buf[pad:pad + nxq]
    xs = xs_buf[pad:pad + (K // 128) * M].view(K // 128, M)
    Y = y_buf[pad:pad + M * N].view(M, N)
    comet.comet_quant_act(X, w["perm"], nb8, Xq=Xq, x_scale=xs)
    comet.comet_w4ax_gemm(Xq, xs, w, M, Y=Y)
    torch.cuda.synchronize()
    xb, sb, yb = xq_buf.cpu().numpy(), xs_buf.cpu().numpy(), y_buf.cpu().numpy()
    assert np.all(xb[:pad] == 0xA5) and np.all(xb[pad + nxq:] == 0xA5)
    assert np.all(sb[:pad] == -3.0) and np.all(sb[-pad:] == -3.0)
    assert np.all(yb[:pad] == 5.0) and np.all(yb[-pad:] == 5.0)
    assert np.array_equal(decode_xq(xb[pad:pad + nxq], M, K, nb8), d["qa"])


def test_determinism_and_streams(torch):
    """Bit-identical Y across runs, and on a side stream."""
    import w4ax_mixed_precision_amd as comet
    d, pk, w, Xq, xs, Y = run_layer(torch, "q_proj_7b")
    cfg = d["cfg"]
    Y2 = comet.comet_w4ax_gemm(Xq, xs, w, cfg.M)
    s = torch.cuda.Stream()
    X = torch.from_numpy(d["X"].view(np.float16)).cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        Xq3, xs3 = comet.comet_quant_act(X, w["perm"], cfg.nb8)
        Y3 = comet.comet_w4ax_gemm(Xq3, xs3, w, cfg.M)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2) and torch.equal(Y, Y3)
    assert torch.equal(Xq, Xq3) and torch.equal(xs, xs3)


@pytest.mark.parametrize("name", ["decode_70b_n8192_m1", "decode_70b_n28672_m16", "decode_70b_n10240_m64"])
def test_decode_determinism_and_streams(torch, name):
    """The streaming kernels (split-K inside the workgroup, summed in wave order):
    bit-identical Y across runs and on a side stream."""
    import w4ax_mixed_precision_amd as comet
    d, pk, w, Xq, xs, Y = run_layer(torch, name)
    cfg = d["cfg"]
    Y2 = comet.comet_w4ax_gemm(Xq, xs, w, cfg.M)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        Y3 = comet.comet_w4ax_gemm(Xq, xs, w, cfg.M)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2) and torch.equal(Y, Y3)
