"""Every positive finite fp16 value as the absmax of a 4-bit and of an 8-bit
block, on the GPU, against the CPU oracle.

Row m (31,743 rows, K = 256, block 0 4-bit, block 1 8-bit, identity channel
order) holds the m-th positive finite fp16 value a (0x0001 .. 0x7BFF) at one
position of each block and fp16 fractions of it elsewhere, so every scale
s = a / qmax and reciprocal qmax / a the quantizer can meet is formed once per
block width. Scales (bit patterns) and codes must equal the oracle's for
comet_quant_act and comet_quant_act_fp6. The fused RMSNorm and SwiGLU
quantizers run on the same rows (gamma = 1; SwiGLU with the row as the gate
and up = 1) and must equal the oracle's normalize-then-quantize and
silu-then-quantize, which sweeps their scale path over the same span of
magnitudes (QUIK blog, deep-paper.org/paper/2310.09259, section 核融合: the
statistics and the quantization happen in one kernel, so its division must be
the oracle's).
"""
import numpy as np
import pytest

from tests import gpu_common as G
from tests.layout import decode_xq, decode_xq_fp6

pytestmark = pytest.mark.gpu

K = 256
NB8 = 1


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()        # the HIP library must load: no fallback
    return t


@pytest.fixture(scope="module")
def rows():
    """[31743, 256] fp16 bit patterns; row m has absmax a_m in both blocks."""
    a = np.arange(1, 0x7C00, dtype=np.uint16)                  # every positive finite fp16
    M = a.size
    av = a.view(np.float16).astype(np.float64)
    rng = np.random.default_rng(31743)
    frac = rng.uniform(-1.0, 1.0, (M, K))
    X = (frac * av[:, None]).astype(np.float16)                # |x| <= a (rounding is monotone)
    pos = rng.integers(0, 128, (M, 2))
    sign = np.where(rng.random((M, 2)) < 0.5, -1.0, 1.0)
    X[np.arange(M), pos[:, 0]] = (sign[:, 0] * av).astype(np.float16)
    X[np.arange(M), 128 + pos[:, 1]] = (sign[:, 1] * av).astype(np.float16)
    X = X.view(np.uint16)
    assert np.array_equal(np.abs(X[:, :128].view(np.float16)).max(1).view(np.uint16), a)
    assert np.array_equal(np.abs(X[:, 128:].view(np.float16)).max(1).view(np.uint16), a)
    return X


def _identity():
    from oracle import oracle as O
    perm, flags = O.channel_order(np.arange(K, dtype=np.float32), NB8)
    assert np.array_equal(perm, np.arange(K))
    return perm, flags


def _compare(torch, Xq, xs, qa_o, sa_o, fp6, label):
    M = sa_o.shape[0]
    dec = decode_xq_fp6 if fp6 else decode_xq
    qa = dec(Xq.cpu().numpy(), M, K, NB8)
    sa = xs.cpu().numpy().T
    bad = np.nonzero(sa.view(np.uint32) != sa_o.view(np.uint32))
    assert bad[0].size == 0, f"{label}: scales differ at rows {bad[0][:5]}, blocks {bad[1][:5]}"
    badq = np.nonzero((qa != qa_o).any(1))[0]
    assert badq.size == 0, f"{label}: codes differ on rows {badq[:5]}"


@pytest.mark.parametrize("fp6", [False, True])
def test_every_absmax_plain(torch, rows, fp6):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    G.log(f"[scales] plain quantizer, fp6={fp6}, {rows.shape[0]} rows")
    perm, flags = _identity()
    qa_o, sa_o = O.quantize_activations(rows, perm, flags)
    # the closed forms the oracle itself is pinned to: s = a / qmax in binary32
    a32 = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    assert np.array_equal(sa_o[:, 0], a32 / np.float32(7))
    assert np.array_equal(sa_o[:, 1], a32 / np.float32(127))
    X = torch.from_numpy(rows.view(np.float16)).cuda()
    pd = torch.from_numpy(perm).cuda()
    q = comet.comet_quant_act_fp6 if fp6 else comet.comet_quant_act
    Xq, xs = q(X, pd, NB8)
    torch.cuda.synchronize()
    _compare(torch, Xq, xs, qa_o, sa_o, fp6, "quant_act" + ("_fp6" if fp6 else ""))


@pytest.mark.parametrize("fp6", [False, True])
def test_every_absmax_rmsnorm_fused(torch, rows, fp6):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    G.log(f"[scales] RMSNorm-fused quantizer, fp6={fp6}")
    perm, flags = _identity()
    gamma = np.full(K, 0x3C00, np.uint16)                       # 1.0
    Xn = O.rmsnorm(rows, gamma, 1e-5)
    qa_o, sa_o = O.quantize_activations(Xn, perm, flags)
    X = torch.from_numpy(rows.view(np.float16)).cuda()
    g = torch.from_numpy(gamma.view(np.float16)).cuda()
    Xq, xs = comet.comet_rmsnorm_quant_act(X, g, 1e-5, torch.from_numpy(perm).cuda(), NB8, fp6=fp6)
    torch.cuda.synchronize()
    _compare(torch, Xq, xs, qa_o, sa_o, fp6, "rmsnorm_quant_act")


@pytest.mark.parametrize("fp6", [False, True])
def test_every_absmax_swiglu_fused(torch, rows, fp6):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    G.log(f"[scales] SwiGLU-fused quantizer, fp6={fp6}")
    perm, flags = _identity()
    up = np.full(rows.shape, 0x3C00, np.uint16)                 # 1.0: h = fp16(silu(g))
    H = O.swiglu(rows, up)
    qa_o, sa_o = O.quantize_activations(H, perm, flags)
    gate = torch.from_numpy(rows.view(np.float16)).cuda()
    u = torch.from_numpy(up.view(np.float16)).cuda()
    Xq, xs = comet.comet_swiglu_quant_act(gate, u, torch.from_numpy(perm).cuda(), NB8, fp6=fp6)
    torch.cuda.synchronize()
    _compare(torch, Xq, xs, qa_o, sa_o, fp6, "swiglu_quant_act")
