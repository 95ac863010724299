"""The inspection probes against the published peaks their rooflines use, on an MI355X.

The roofline peaks must be upper bounds: the library's plain fp32 FMA loop
and its streaming read stay below the fp32 vector peak (157.3 TFLOP/s) and
the HBM peak (8 TB/s), and reach a fair share of them, so that the peaks are
neither too low (the bench once priced fp32 arithmetic at 78.6 TFLOP/s,
which plain FMAs exceed) nor unreachable.  Every call goes through the C ABI.
"""

import errno

import pytest

from full_reference_video_amd import vqm

pytestmark = pytest.mark.gpu

FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_valu_probe_is_below_the_fp32_peak_and_above_half_of_it(torch_cuda):
    rates = {w: vqm.vqm_debug_valu_probe(waves_per_simd=w, iters=4000, reps=2) for w in (1, 8)}
    print(rates, flush=True)
    assert all(0.0 < t < FP32_PEAK_TFLOPS for t in rates.values())
    assert rates[8] > 78.6  # more than 16 lanes per clock per SIMD would allow
    assert rates[8] > rates[1]  # more resident waves, more of the rate


def test_read_probe_is_below_the_hbm_peak(torch_cuda):
    torch = torch_cuda
    n = 512 << 20
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    ms = vqm.vqm_debug_read_probe(buf, reps=3)
    gbps = n / (ms * 1e-3) / 1e9
    print(f"{gbps:.1f} GB/s", flush=True)
    assert 0.5 * HBM_PEAK_GBS < gbps < HBM_PEAK_GBS


def test_valu_probe_refuses_bad_arguments(torch_cuda):
    for args in ((0, 10, 1), (33, 10, 1), (4, 0, 1), (4, 10, 0)):
        with pytest.raises(vqm.VqmError) as e:
            vqm.vqm_debug_valu_probe(*args)
        assert e.value.rc == -errno.EINVAL
