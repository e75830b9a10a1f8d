"""GPU parity of the RMS normalization fused into the quantizer
(comet_rmsnorm_quant_act[_fp6]) and of the normalization on its own
(comet_rmsnorm), through the C ABI against the CPU oracle.

Bit-exact: the normalized fp16 rows, and the codes and scales of the fused
calls against the oracle's quantization of its own normalized rows, on every
kernel path of the quantizer (per-row kernel with the row in LDS or in global
memory, the element-wise staging of an unaligned ldx, the persistent row
kernel), both layouts; and the fused calls against normalize-then-quantize on
the GPU, byte for byte.
"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import decode_xq, decode_xq_fp6

pytestmark = pytest.mark.gpu

EPS = 1e-5


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()        # the HIP library must load: no fallback
    return t


def _inputs(M, K, seed, kind="planted", zero_rows=()):
    cfg = synth.LayerConfig("norm", M, K, 128, seed, x_kind=kind)
    X = synth.make_x(cfg)
    for r in zero_rows:
        X[r] = 0
    rng = np.random.default_rng(seed)
    gamma = synth.to_fp16(1.0 + 0.25 * rng.standard_normal(K))
    score = synth.make_scores(cfg)
    return X, gamma, score


def _oracle(X, gamma, score, nb8):
    from oracle import oracle as O
    Xn = O.rmsnorm(X, gamma, EPS)
    perm, flags = O.channel_order(score, nb8)
    qa, sa = O.quantize_activations(Xn, perm, flags)
    return Xn, perm, qa, sa


def _device(torch, a, ld=None):
    a = np.asarray(a)
    if ld is not None and ld != a.shape[-1]:
        pad = np.zeros(a.shape[:-1] + (ld,), a.dtype)
        pad[..., :a.shape[-1]] = a
        a = pad
    return torch.from_numpy(a.view(np.float16).copy()).cuda()


@pytest.mark.parametrize("M,K,ldx", [(1, 128, 128), (3, 1000, 1000), (37, 4096, 4100), (1000, 8192, 8192),
                                     (5, 33024, 33024)])
def test_rmsnorm_parity(torch, M, K, ldx):
    import w4ax_mixed_precision_amd as comet
    G.log(f"[rmsnorm] M={M} K={K} ldx={ldx}")
    X, gamma, _ = _inputs(M, K, seed=M + K, zero_rows=(0,) if M > 2 else ())
    from oracle import oracle as O
    want = O.rmsnorm(X, gamma, EPS)
    Xd = _device(torch, X, ldx)
    out = torch.full((M, K + 8), 3.0, dtype=torch.float16, device="cuda")
    comet.comet_rmsnorm(Xd, _device(torch, gamma), EPS, K=K, Xn=out[:, :K])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[:, :K].view(np.uint16), want)
    assert np.all(got[:, K:] == 3.0)                  # columns past K untouched


# (M, K, ldx, nb8): per-row kernel with the row in LDS (M < 256), element-wise
# staging (ldx not a multiple of 8), row in global memory (K > 32768), and the
# persistent row kernel (M >= 256), including the 70B hidden size
CASES = [(1, 128, 128, 0), (1, 128, 128, 1), (17, 1024, 1024, 2), (100, 4096, 4100, 3), (100, 4096, 4096, 32),
         (5, 33024, 33024, 4), (300, 2048, 2048, 1), (1000, 8192, 8192, 7)]


@pytest.mark.parametrize("fp6", [False, True])
@pytest.mark.parametrize("M,K,ldx,nb8", CASES)
def test_fused_quant_parity(torch, M, K, ldx, nb8, fp6):
    import w4ax_mixed_precision_amd as comet
    G.log(f"[rmsnorm quant] M={M} K={K} ldx={ldx} nb8={nb8} fp6={fp6}")
    X, gamma, score = _inputs(M, K, seed=3 * M + K + nb8, zero_rows=(M - 1,) if M > 1 else ())
    _, perm, qa, sa = _oracle(X, gamma, score, nb8)
    gp = comet.comet_permute_channels(gamma, perm)
    Xq, xs = comet.comet_rmsnorm_quant_act(_device(torch, X, ldx), _device(torch, gp), EPS,
                                           torch.from_numpy(perm).cuda(), nb8, fp6=fp6)
    torch.cuda.synchronize()
    dec = decode_xq_fp6 if fp6 else decode_xq
    assert np.array_equal(dec(Xq.cpu().numpy(), M, K, nb8), qa), "codes differ"
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), sa.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("fp6", [False, True])
def test_fused_equals_unfused(torch, fp6):
    """comet_rmsnorm then comet_quant_act[_fp6] gives the same bytes as the
    fused call (the 70B up/gate input: 4096 tokens x 8192 channels)."""
    import w4ax_mixed_precision_amd as comet
    M, K, nb8 = 4096, 8192, 7
    X, gamma, score = _inputs(M, K, seed=77)
    from oracle import oracle as O
    perm, _ = O.channel_order(score, nb8)
    pd = torch.from_numpy(perm).cuda()
    Xd, gd = _device(torch, X), _device(torch, gamma)
    gp = _device(torch, comet.comet_permute_channels(gamma, perm))
    Xn = comet.comet_rmsnorm(Xd, gd, EPS)
    q = comet.comet_quant_act_fp6 if fp6 else comet.comet_quant_act
    Xq_u, xs_u = q(Xn, pd, nb8)
    Xq_f, xs_f = comet.comet_rmsnorm_quant_act(Xd, gp, EPS, pd, nb8, fp6=fp6)
    torch.cuda.synchronize()
    assert torch.equal(xs_u, xs_f)
    if fp6:          # padding rows of the last 16-row tile are not written: compare the rows
        a = decode_xq_fp6(Xq_u.cpu().numpy(), M, K, nb8)
        b = decode_xq_fp6(Xq_f.cpu().numpy(), M, K, nb8)
        assert np.array_equal(a, b)
    else:
        assert torch.equal(Xq_u, Xq_f)
