"""gfx950 builtin behaviour the layer kernels rely on (needs an MI355X):
MFMA operand/result lane layouts, the fp4 conversions (exact with scale 1;
the f32 scale operand contributes only its exponent), OCP E4M3 decode and
float -> bf16 round-to-nearest-even. Probe kernels live in tests/gpu_probe."""
import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_helpers import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "gpu_probe", "libprobe.so")
E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] + [-0.0, -.5, -1, -1.5, -2, -3, -4, -6])


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_mfma_layouts(probe):
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(0)
    say("[case] mfma 32x32x16 / 16x16x32 lane layouts")
    A = torch.randn(32, 16, generator=g).to(torch.bfloat16)
    B = torch.randn(16, 32, generator=g).to(torch.bfloat16)
    C = torch.zeros(32, 32, device=dev)
    Ad, Bd = A.to(dev), B.to(dev)  # keep the device copies alive during the call
    probe.probe_mfma32(_p(Ad), _p(Bd), _p(C))
    torch.cuda.synchronize()
    assert torch.allclose(C.cpu(), A.float() @ B.float(), atol=1e-5, rtol=1e-5)
    A = torch.randn(16, 32, generator=g).to(torch.bfloat16)
    B = torch.randn(32, 16, generator=g).to(torch.bfloat16)
    C = torch.zeros(16, 16, device=dev)
    Ad, Bd = A.to(dev), B.to(dev)
    probe.probe_mfma16(_p(Ad), _p(Bd), _p(C))
    torch.cuda.synchronize()
    assert torch.allclose(C.cpu(), A.float() @ B.float(), atol=1e-5, rtol=1e-5)


def test_fp4_conversions(probe):
    dev = torch.device("cuda:0")
    say("[case] fp4 scaled conversions")
    n = 512
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    nib = np.stack([(codes >> (4 * j)) & 0xF for j in range(8)], 1)
    cd = torch.from_numpy(codes.view(np.int32)).to(dev)
    ob = torch.zeros(8 * n, dtype=torch.bfloat16, device=dev)
    of = torch.zeros(8 * n, device=dev)
    # scale 1: plain e2m1 values, element order low nibble first
    ones = torch.ones(n, device=dev)
    probe.probe_cvt_fp4(_p(cd), _p(ones), _p(ob), _p(of), n)
    torch.cuda.synchronize()
    assert np.array_equal(ob.float().cpu().numpy().reshape(n, 8), E2M1[nib])
    assert np.array_equal(of.cpu().numpy().reshape(n, 8), E2M1[nib])
    # the scale operand acts through its exponent only (1.75 acts as 1, 448 as 256)
    sc = np.array([1.75, 448.0, 0.8125, 2.0 ** -9] * (n // 4), dtype=np.float32)
    scd = torch.from_numpy(sc).to(dev)
    probe.probe_cvt_fp4(_p(cd), _p(scd), _p(ob), _p(of), n)
    torch.cuda.synchronize()
    pow2 = np.exp2(np.floor(np.log2(sc.astype(np.float64))))
    assert np.array_equal(of.cpu().numpy().reshape(n, 8), E2M1[nib] * pow2[:, None])


def test_e4m3_decode(probe):
    dev = torch.device("cuda:0")
    say("[case] OCP E4M3 decode")
    b = torch.arange(256, dtype=torch.uint8)
    out = torch.zeros(256, device=dev)
    bd = b.view(torch.int32).to(dev)
    probe.probe_cvt_fp8(_p(bd), _p(out))
    torch.cuda.synchronize()
    want = b.view(torch.float8_e4m3fn).float().numpy()
    got = out.cpu().numpy()
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]) and np.isnan(got[~ok]).all()


def test_bf16_rounding(probe):
    dev = torch.device("cuda:0")
    say("[case] float -> bf16 rounding")
    g = torch.Generator().manual_seed(1)
    v = torch.cat([torch.randn(100000, generator=g) * 3,
                   torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(2 + 2 ** -7)])])
    o = torch.zeros(v.numel(), dtype=torch.bfloat16, device=dev)
    vd = v.to(dev)
    probe.probe_f32_to_bf16(_p(vd), _p(o), v.numel())
    torch.cuda.synchronize()
    assert torch.equal(o.cpu().view(torch.int16), v.to(torch.bfloat16).view(torch.int16))
