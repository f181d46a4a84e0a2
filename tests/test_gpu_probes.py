"""The measurement probes: the copy probe copies, the issue probes run and count."""
import ctypes

import pytest
import torch

import selective_state_space_72_amd as ms
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def test_copy_probe_copies_exactly():
    lib = ms.load_library()
    n = (1 << 20) + 16  # not a multiple of the grid's stride
    src = torch.randn(n // 4 * 4, device=DEV)
    dst = torch.zeros_like(src)
    st = lib.mamba_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                              src.numel() * 4, 37, None)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(src, dst)


@pytest.mark.parametrize("kind, per_wave_iter", [(0, 8), (1, 8), (2, 8), (3, 16)])
def test_issue_probes_run_and_count(kind, per_wave_iter):
    lib = ms.load_library()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 2 * 256, device=DEV)
    n = ctypes.c_uint64(0)
    st = lib.mamba_probe_issue(kind, 2, 16, cus, ctypes.c_void_p(sink.data_ptr()),
                               ctypes.byref(n), None)
    torch.cuda.synchronize()
    assert st == 0
    assert n.value == cus * 2 * 4 * 16 * per_wave_iter
