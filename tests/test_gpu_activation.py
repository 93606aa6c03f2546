"""The device GeLU forms of the GEMM epilogues (pblock_activation) against the oracle, at the
error bounds of the published methods they use, on a dense grid through both tails.

Each bound is the method's stated error in exact arithmetic plus the fp32 evaluation of it:
  * bf16 path, erfc from Abramowitz and Stegun 7.1.26: |erf error| < 1.5e-7, so GeLU = z Phi(z)
    is off by at most 7.5e-8 |z|; fp32 Horner steps and the exponential add about 1e-6 of
    h = erfc(|z|/sqrt 2)/2 and a few ulp of the result;
  * fp32 path, erfc from Numerical Recipes' erfcc: fractional error of erfc < 1.2e-7; the fp32
    argument of the exponential (about z^2/2 in magnitude) adds about 2^-22 z^2/2 relative;
  * the tanh form (Hendrycks and Gimpel) evaluated as z sigmoid(2y): a few ulp plus the
    rounding of the exponential's argument (2y log2 e in magnitude);
  * the derivative Phi(z) + z phi(z) of the backward pass: A&S for Phi, the same exponential
    for phi.
The fp64 references lose relative accuracy in the far negative tail (1 + erf cancels), so every
bound has an absolute floor of 1e-15; the fp32 path's tail is also checked relatively against
z erfc(-z/sqrt 2)/2 from scipy's erfc.
"""
import math

import numpy as np
import pytest

import oracle
from gpu_helpers import log

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import transformer_block_fwd_amd as tb  # noqa: E402

FLOOR = 1e-15
U = 2.0 ** -22  # two fp32 units of roundoff


def _grid():
    dense = np.linspace(-12.0, 12.0, (1 << 20) + 1, dtype=np.float32)
    special = np.array([0.0, 1e-30, -1e-30, 1e-8, -1e-8, 0.5, -0.5, 1.0, -1.0, 2.70, -2.70], np.float32)
    return np.concatenate([dense, special])


def _device(z, form):
    zt = torch.from_numpy(z).cuda()
    out = torch.empty_like(zt)
    tb.pblock_activation(zt, out, form)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _h(z):
    from scipy.special import erfc

    return 0.5 * erfc(np.abs(z) / math.sqrt(2.0))


def _check(name, got, ref, bound, z):
    err = np.abs(got - ref)
    ratio = err / bound
    i = int(ratio.argmax())
    log(f"[gelu] {name}: max abs err {err.max():.3e}, worst err/bound {ratio[i]:.3f} at z = {z[i]:.5f}")
    assert np.isfinite(got).all()
    assert (err <= bound).all(), f"{name}: error {err[i]:.3e} > bound {bound[i]:.3e} at z = {z[i]}"


def test_gelu_erf_bf16_path():
    z = _grid()
    zd = z.astype(np.float64)
    ref = oracle.gelu(zd)
    bound = np.abs(zd) * (7.5e-8 + 1e-6 * _h(zd)) + U * np.abs(ref) + FLOOR
    _check("erf (A&S 7.1.26, bf16 path)", _device(z, "gelu_erf_bf16"), ref, bound, zd)


def test_gelu_erf_f32_path():
    from scipy.special import erfc

    z = _grid()
    zd = z.astype(np.float64)
    got = _device(z, "gelu_erf_f32")
    ref = oracle.gelu(zd)
    h = _h(zd)
    bound = np.abs(zd) * h * (1.2e-7 + 2 * U * (2 + zd * zd / 2)) + U * np.abs(ref) + FLOOR
    _check("erf (NR erfcc, fp32 path)", got, ref, bound, zd)
    # relative accuracy in the negative tail, against an erfc-based reference without cancellation
    neg = zd < -1e-6
    ref_tail = zd[neg] * 0.5 * erfc(-zd[neg] / math.sqrt(2.0))
    rel = np.abs(got[neg] - ref_tail) / np.abs(ref_tail)
    rel_bound = 1.2e-7 + 2 * U * (2 + zd[neg] ** 2 / 2)
    log(f"[gelu] erf fp32 path, negative tail: max relative error {rel.max():.3e}, "
        f"worst ratio {(rel / rel_bound).max():.3f}")
    assert (rel <= rel_bound).all()


def test_gelu_tanh_form():
    z = _grid()
    zd = z.astype(np.float64)
    ref = oracle.gelu_tanh(zd)
    a = 2.8853900817779268 * np.abs(0.7978845608028654 * (zd + 0.044715 * zd ** 3))
    bound = U * (4 + a) * np.abs(ref) + FLOOR
    _check("tanh form", _device(z, "gelu_tanh"), ref, bound, zd)


def test_gelu_erf_derivative():
    z = _grid()
    zd = z.astype(np.float64)
    ref = oracle.gelu_grad(zd)
    phi = np.exp(-zd * zd / 2) / math.sqrt(2 * math.pi)
    bound = 7.5e-8 + 1e-6 * _h(zd) + np.abs(zd) * phi * U * (2 + zd * zd) + U * np.abs(ref) + FLOOR
    _check("derivative Phi + z phi (A&S 7.1.26)", _device(z, "gelu_erf_grad"), ref, bound, zd)


@pytest.mark.parametrize("form", sorted(tb.ACTIVATION_FORMS))
def test_extreme_arguments_reach_their_limits(form):
    """Far outside the grid every form returns its limit, finite: GeLU(z) -> z for z >> 0 and
    -> 0 for z << 0; the derivative -> 1 and 0.  Exponentials overflow or underflow there and
    must not leave an inf or a NaN."""
    big = np.array([20.0, 50.0, 1e4, 3e38], np.float32)
    z = np.concatenate([big, -big])
    got = _device(z, form)
    assert np.isfinite(got).all(), got
    if form == "gelu_erf_grad":
        want = np.concatenate([np.ones(4), np.zeros(4)])
        assert np.abs(got - want).max() <= 1e-7
    else:
        want = np.concatenate([big.astype(np.float64), np.zeros(4)])
        assert (np.abs(got - want) <= 2 ** -23 * np.abs(want) + 1e-30).all(), got


def test_activation_rejections():
    z = torch.zeros(16, device="cuda")
    out = torch.zeros(16, device="cuda")
    lib = tb._abi.lib()
    assert lib.pblock_activation(z.data_ptr(), out.data_ptr(), 16, 9, None) == tb._abi.PBLOCK_ERR_ARG
    assert lib.pblock_activation(0, out.data_ptr(), 16, 0, None) == tb._abi.PBLOCK_ERR_NULL
    assert lib.pblock_activation(z.data_ptr(), out.data_ptr(), -1, 0, None) == tb._abi.PBLOCK_ERR_SHAPE
    assert lib.pblock_activation(z.data_ptr(), z.data_ptr() + 4, 8, 0, None) == tb._abi.PBLOCK_ERR_ALIAS
    # in place is allowed
    assert lib.pblock_activation(z.data_ptr(), z.data_ptr(), 16, 0, None) == tb._abi.PBLOCK_OK
    torch.cuda.synchronize()
    assert bool((z == 0).all())
