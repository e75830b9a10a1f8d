"""GPU parity of the FP6-layout path (comet_quant_act_fp6, comet_w4ax_gemm_fp6)
through the C ABI against the CPU oracle: the same bars as the INT4 layout.

Bit-exact activation codes (decoded from FP6 E2M3) and scales, bit-exact INT32
block partials, Y within gates Y1 and Y2. Full-size layers on sampled rows in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import decode_xq_fp6
from tests.test_gpu_parity import _custom_layer

pytestmark = pytest.mark.gpu

LAYERS = ["tiny", "q_proj_7b", "up_gate_7b", "down_7b", "decode_70b_n8192_m1",
          "decode_70b_n10240_m64", "prefill_down_70b", "prefill_up_70b"]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()        # the HIP library must load: no fallback
    return t


def check(torch, d, w, X, M, K, N, nb8, rows):
    import w4ax_mixed_precision_amd as comet
    Xq, xs = comet.comet_quant_act_fp6(X, w["perm"], nb8)
    Y = comet.comet_w4ax_gemm_fp6(Xq, xs, w, M)
    torch.cuda.synchronize()
    assert np.array_equal(decode_xq_fp6(Xq.cpu().numpy(), M, K, nb8), d["qa"]), "activation codes differ"
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), d["sa"].view(np.uint32)), "scales differ"
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, rows)
    runs = np.split(rows, np.where(np.diff(rows) != 1)[0] + 1)
    for run in runs:
        P = comet.comet_w4ax_gemm_fp6_partials(Xq, xs, w, M, int(run[0]), len(run))
        idx = np.searchsorted(rows, run)
        assert np.array_equal(P.cpu().numpy(), P_o[idx]), f"partials differ on rows {run[0]}.."
    yhat = G.f16(Y.cpu().numpy().view(np.uint16)[rows])
    y1, y2_ok, y2_ratio = G.gate_y(yhat, ye, tabs, K // 128)
    G.log(f"[fp6] Y1 max rel err {y1:.3e}, Y2 worst err/bound {y2_ratio:.3f}")
    assert y1 <= 1e-3
    assert y2_ok
    return Xq, xs, Y, yhat


@pytest.mark.parametrize("name", LAYERS)
def test_layer_parity_fp6(torch, name):
    G.log(f"[fp6 parity] {name}")
    d = G.host_layer(name)
    cfg = d["cfg"]
    X, w = G.device_layer(d, d["pk"])
    check(torch, d, w, X, cfg.M, cfg.K, cfg.N, cfg.nb8, G.sample_rows(cfg.M))


@pytest.mark.parametrize("M,K,N,nb8", [
    (1, 128, 128, 0), (1, 128, 128, 1), (3, 256, 256, 2), (17, 512, 384, 0),
    (33, 384, 640, 3), (100, 1024, 512, 1), (130, 640, 256, 5), (257, 896, 384, 2),
    (5, 33024, 128, 4),   # K > 32768: global gather path of the quantizer
    # grids below a wave that the cost model keeps whole (short K)
    (384, 1024, 12800, 2), (128, 1280, 14080, 3),
    # split grids: 80 tiles x 6 runs (8-bit blocks inside and across runs),
    # 40 tiles x 6 runs with a ragged row tile, and 130 tiles x 7 runs: more
    # runs than the resident grid, so the work queue deals the rest
    (64, 8192, 10240, 7), (100, 4096, 5120, 3), (64, 6144, 16640, 12),
])
def test_edge_shapes_fp6(torch, M, K, N, nb8):
    import w4ax_mixed_precision_amd as comet
    G.log(f"[fp6 edge] M={M} K={K} N={N} nb8={nb8}")
    d = _custom_layer(M, K, N, nb8, seed=M * 7 + K + nb8 + 1,
                      zero_rows=(0,) if M > 2 else (), zero_block_rows=((M - 1, 0),))
    pk = comet.comet_repack_weights_fp6(comet.comet_pack_weights(d["W"], d["score"], nb8))
    w = comet.upload_weights(pk)
    X = torch.from_numpy(d["X"].view(np.float16)).cuda()
    _, _, _, yhat = check(torch, d, w, X, M, K, N, nb8, np.arange(M))
    if M > 2:
        assert np.all(yhat[0] == 0)          # an all-zero token row gives exact zeros


def test_strided_and_guards_fp6(torch):
    """ldx > K, ldy > N, and guard bytes around every output buffer."""
    import w4ax_mixed_precision_amd as comet
    M, K, N, nb8 = 37, 640, 384, 2
    d = _custom_layer(M, K, N, nb8, seed=93, ldx=K + 24)
    pk = comet.comet_repack_weights_fp6(comet.comet_pack_weights(d["W"], d["score"], nb8))
    w = comet.upload_weights(pk)
    Xpad = torch.from_numpy(d["Xpad"].view(np.float16)).cuda()
    Xpad[:, K:] = float("nan")               # must never be read
    pad = 256
    nxq = comet.xq_fp6_bytes(M, K, nb8)
    xq_buf = torch.full((nxq + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    xs_buf = torch.full(((K // 128) * M + 2 * pad,), -3.0, dtype=torch.float32, device="cuda")
    Ybig = torch.full((M + 2, N + 40), 7.0, dtype=torch.float16, device="cuda")
    Xq = xq_buf[pad:pad + nxq]
    xs = xs_buf[pad:pad + (K // 128) * M].view(K // 128, M)
    comet.comet_quant_act_fp6(Xpad, w["perm"], nb8, Xq=Xq, x_scale=xs)
    comet.comet_w4ax_gemm_fp6(Xq, xs, w, M, Y=Ybig[1:M + 1])
    torch.cuda.synchronize()
    xb, sb, yb = xq_buf.cpu().numpy(), xs_buf.cpu().numpy(), Ybig.cpu().numpy()
    assert np.all(xb[:pad] == 0xA5) and np.all(xb[pad + nxq:] == 0xA5)
    assert np.all(sb[:pad] == -3.0) and np.all(sb[-pad:] == -3.0)
    assert np.all(yb[0] == 7.0) and np.all(yb[M + 1] == 7.0) and np.all(yb[:, N:] == 7.0)
    assert np.array_equal(decode_xq_fp6(xb[pad:pad + nxq], M, K, nb8), d["qa"])
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, np.arange(M))
    y1, y2_ok, _ = G.gate_y(yb[1:M + 1, :N].astype(np.float64), ye, tabs, K // 128)
    assert y1 <= 1e-3 and y2_ok


def test_fp6_matches_int4_layout(torch):
    """Both layouts give bit-identical partials; Y agrees up to the epilogue's
    summation order (the FP6 path splits this small grid's blocks into runs,
    the INT4 tiled kernel does not), so both are held to the gates."""
    import w4ax_mixed_precision_amd as comet
    d = G.host_layer("q_proj_7b")
    cfg = d["cfg"]
    X, w = G.device_layer(d, d["pk"])
    Xq4, xs4 = comet.comet_quant_act(X, w["perm"], cfg.nb8)
    Xq6, xs6 = comet.comet_quant_act_fp6(X, w["perm"], cfg.nb8)
    P4 = comet.comet_w4ax_gemm_partials(Xq4, xs4, w, cfg.M)
    P6 = comet.comet_w4ax_gemm_fp6_partials(Xq6, xs6, w, cfg.M)
    Y4 = comet.comet_w4ax_gemm(Xq4, xs4, w, cfg.M)
    Y6 = comet.comet_w4ax_gemm_fp6(Xq6, xs6, w, cfg.M)
    torch.cuda.synchronize()
    assert torch.equal(xs4, xs6)
    assert torch.equal(P4, P6)
    rows = np.arange(cfg.M)
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, rows)
    for Y in (Y4, Y6):
        y1, y2_ok, _ = G.gate_y(G.f16(Y.cpu().numpy().view(np.uint16)), ye, tabs, cfg.nb)
        assert y1 <= 1e-3 and y2_ok


@pytest.mark.parametrize("name", ["q_proj_7b", "decode_70b_n10240_m64"])
def test_fp6_work_queue(torch, name):
    """The work queue dealing most of a split plan's runs: the partials call
    capped at 8 workgroups (one per XCD: each takes its first run directly
    and the rest from its XCD's counter) gives the oracle's partials bit for
    bit, the same as the uncapped call, and leaves the counters at zero."""
    import w4ax_mixed_precision_amd as comet
    G.log(f"[fp6 queue] {name}")
    d = G.host_layer(name)
    cfg = d["cfg"]
    need = comet.fp6_workspace_bytes(cfg.M, cfg.N, cfg.K, cfg.nb8)
    assert need > 0, "a split plan"
    X, w = G.device_layer(d, d["pk"])
    Xq, xs = comet.comet_quant_act_fp6(X, w["perm"], cfg.nb8)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    P8 = comet.comet_w4ax_gemm_fp6_partials(Xq, xs, w, cfg.M, workspace=ws, max_workgroups=8)
    torch.cuda.synchronize()
    assert int(ws[:256].count_nonzero()) == 0
    P = comet.comet_w4ax_gemm_fp6_partials(Xq, xs, w, cfg.M, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(P8, P)
    rows = np.arange(cfg.M)
    P_o = G.oracle_rows(d, rows)[0]
    assert np.array_equal(P8.cpu().numpy(), P_o)


def test_fp6_workspace_shared_across_shapes(torch):
    """One workspace serves split grids of different shapes in turn: only its
    queue counters must start at zero (each call leaves them zero); the
    partial tiles one shape leaves behind must not disturb the next. The
    partial region starts poisoned (NaN bytes)."""
    import w4ax_mixed_precision_amd as comet
    shapes = ["down_7b", "decode_70b_n8192_m1", "decode_70b_n10240_m64", "q_proj_7b", "tiny"]
    need = max(comet.fp6_workspace_bytes(synth.CONFIGS[n].M, synth.CONFIGS[n].N, synth.CONFIGS[n].K,
                                         synth.CONFIGS[n].nb8) for n in shapes)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    ws[:256] = 0
    for name in shapes:
        G.log(f"[fp6 shared ws] {name}")
        d = G.host_layer(name)
        cfg = d["cfg"]
        X, w = G.device_layer(d, d["pk"])
        Xq, xs = comet.comet_quant_act_fp6(X, w["perm"], cfg.nb8)
        Y = torch.full((cfg.M, cfg.N), float("nan"), dtype=torch.float16, device="cuda")
        comet.comet_w4ax_gemm_fp6(Xq, xs, w, cfg.M, Y=Y, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:256].count_nonzero()) == 0, f"{name}: counters not returned to zero"
        rows = G.sample_rows(cfg.M)
        P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, rows)
        yhat = G.f16(Y.cpu().numpy().view(np.uint16)[rows])
        y1, y2_ok, _ = G.gate_y(yhat, ye, tabs, cfg.nb)
        assert y1 <= 1e-3 and y2_ok, name


def test_determinism_fp6(torch):
    import w4ax_mixed_precision_amd as comet
    d = G.host_layer("up_gate_7b")
    cfg = d["cfg"]
    X, w = G.device_layer(d, d["pk"])
    Xq, xs = comet.comet_quant_act_fp6(X, w["perm"], cfg.nb8)
    Y1 = comet.comet_w4ax_gemm_fp6(Xq, xs, w, cfg.M)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        Y2 = comet.comet_w4ax_gemm_fp6(Xq, xs, w, cfg.M)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_wide_tile_fp6(torch):
    """A grid large enough for the 128 x 256 workgroup tile, with a ragged last
    row tile: sampled rows (the tail included) against the oracle, and every Y
    bit-identical to the INT4-layout kernel (same per-output summation order)."""
    import w4ax_mixed_precision_amd as comet
    M, K, N, nb8 = 4000, 1024, 8192, 2
    G.log(f"[fp6 wide] M={M} K={K} N={N} nb8={nb8}")
    d = _custom_layer(M, K, N, nb8, seed=4242)
    pk = comet.comet_pack_weights(d["W"], d["score"], nb8)
    w = comet.upload_weights(comet.comet_repack_weights_fp6(pk))
    X = torch.from_numpy(d["X"].view(np.float16)).cuda()
    rows = np.unique(np.concatenate([G.sample_rows(M), np.arange(M - 40, M)]))
    _, _, Y6, _ = check(torch, d, w, X, M, K, N, nb8, rows)
    Xq4, xs4 = comet.comet_quant_act(X, w["perm"], nb8)
    Y4 = comet.comet_w4ax_gemm(Xq4, xs4, w, M)
    torch.cuda.synchronize()
    assert torch.equal(Y4, Y6)
