"""The allocation-free FP6 GEMM (comet_w4ax_gemm_fp6_noalloc) through the C ABI:
the same Y, bit for bit, as comet_w4ax_gemm_fp6 with a workspace of its own,
on two calls in a row (the second with a smaller input, so the fixed scratch
holds the first call's partial tiles), and within the gates against the
oracle. (That every split plan fits the fixed scratch is checked on the CPU,
in test_boundary.py.)"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()        # the HIP library must load: no fallback
    return t


def _run(torch, name):
    import w4ax_mixed_precision_amd as comet
    d = G.host_layer(name)
    cfg = d["cfg"]
    need = comet.fp6_workspace_bytes(cfg.M, cfg.N, cfg.K, cfg.nb8)
    G.log(f"[no-alloc] {name}: workspace {need} bytes (scratch {comet.NOALLOC_SCRATCH_BYTES})")
    assert 0 < need <= comet.NOALLOC_SCRATCH_BYTES
    X, w = G.device_layer(d, d["pk"])
    Xq, xs = comet.comet_quant_act_fp6(X, w["perm"], cfg.nb8)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    Y_ref = comet.comet_w4ax_gemm_fp6(Xq, xs, w, cfg.M, workspace=ws)
    Y = torch.full((cfg.M, cfg.N), float("nan"), dtype=torch.float16, device="cuda")
    comet.comet_w4ax_gemm_fp6_noalloc(Xq, xs, w, cfg.M, Y=Y)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref), f"{name}: Y differs from comet_w4ax_gemm_fp6"
    rows = G.sample_rows(cfg.M)
    P_o, y32, Y16_o, ye, tabs = G.oracle_rows(d, rows)
    y1, y2_ok, _ = G.gate_y(G.f16(Y.cpu().numpy().view(np.uint16)[rows]), ye, tabs, cfg.nb)
    assert y1 <= 1e-3 and y2_ok, name


def test_no_alloc_two_calls(torch):
    """down_7b (256 tiles x 2 runs, 32 MiB of partial tiles), then the smaller
    q_proj_7b (32 tiles x 8 runs) on the scratch the first call left behind."""
    _run(torch, "down_7b")
    _run(torch, "q_proj_7b")
