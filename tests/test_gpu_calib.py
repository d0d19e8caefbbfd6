"""The measurement helpers of libdsa_calib.so do what their counters and
context figures assume: the copy copies, the fill writes every word, and the
read stream runs (sizes that are not a whole number of 16 KiB items, so the
clamped last item is exercised)."""
import ctypes

import pytest
import torch

from sparse_attention_kv_dsa_amd import build as dsa_build

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
vp = ctypes.c_void_p


def _lib():
    L = ctypes.CDLL(dsa_build.lib_path("libdsa_calib.so"))
    L.dsa_calib_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    L.dsa_calib_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    L.dsa_calib_fill.argtypes = [vp, ctypes.c_size_t, ctypes.c_uint32, vp]
    return L


@pytest.mark.parametrize("words", [4, 4096, 4100, 1 << 20, (1 << 20) + 12])
def test_copy_fill_read(words):
    L = _lib()
    sp = vp(torch.cuda.current_stream().cuda_stream)
    src = torch.arange(words + 8, dtype=torch.int32, device=DEV)
    dst = torch.full((words + 8,), -7, dtype=torch.int32, device=DEV)
    assert L.dsa_calib_copy(src.data_ptr(), dst.data_ptr(), words * 4, sp) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:words], src[:words])
    assert (dst[words:] == -7).all()                      # nothing past the end
    assert L.dsa_calib_fill(dst.data_ptr(), words * 4, 0xFF800000, sp) == 0
    torch.cuda.synchronize()
    f = dst.view(torch.float32)
    assert torch.isinf(f[:words]).all() and (f[:words] < 0).all()
    assert (dst[words:] == -7).all()
    sink = torch.zeros(L.dsa_calib_read_sink_words(), dtype=torch.int32, device=DEV)
    assert L.dsa_calib_read(src.data_ptr(), words * 4, sink.data_ptr(), sp) == 0
    torch.cuda.synchronize()
