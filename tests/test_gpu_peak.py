"""The matrix-core throughput microbenchmark used for the roofline context."""

import ctypes

import pytest

from helpers import log

pytestmark = pytest.mark.gpu


def test_mfma_peak_plausible_and_errors():
    import torch
    import matrix_inverse_roots_amd as m
    # datasheet dense peaks (TFLOP/s); a register-only MFMA chain reaches a large
    # fraction of them and cannot exceed them by more than the boost clock allows
    sheet = {"f32": 157.3, "f64": 78.6, "f16": 2516.6, "bf16": 2516.6}
    for d, peak in sheet.items():
        t = m.shampoo_mfma_peak(d)
        log(f"{d}: {t:.1f} TFLOP/s ({t / peak:.1%} of the datasheet)")
        assert 0.5 * peak < t < 1.1 * peak
    sink = torch.zeros(16, device="cuda")
    out = ctypes.c_double(0.0)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert m.lib.shampoo_mfma_peak(99, ctypes.c_void_p(sink.data_ptr()), st, ctypes.byref(out)) == m.E_UNSUPPORTED
    assert m.lib.shampoo_mfma_peak(m.F32, None, st, ctypes.byref(out)) == m.E_INVALID
