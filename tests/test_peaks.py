"""The measured-peaks library (include/tsa_peaks.h): exports and argument
checks on the host; on the GPU, that its kernels do the work they are timed
for (the MFMA chains' sums, an exact copy, the xor of what was read)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsa_peaks.h")
LIB = os.path.join(ROOT, "top_selected_attention_amd", "peaks", "libtsa_peaks.so")


def _lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} missing: build first (top_selected_attention_amd/build.py)")
    return ctypes.CDLL(LIB)


def test_exports_match_header():
    names = re.findall(r"^int (tsa_\w+)\(", open(HEADER).read(), re.M)
    assert sorted(names) == ["tsa_fill_registers", "tsa_peak_copy", "tsa_peak_mfma",
                             "tsa_peak_read", "tsa_peak_read_cached"]
    L = _lib()
    for n in names:
        assert hasattr(L, n), n


def test_invalid_arguments_rejected_before_launch():
    L = _lib()
    L.tsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    L.tsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                ctypes.c_void_p]
    L.tsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p]
    L.tsa_peak_read_cached.argtypes = L.tsa_peak_read.argtypes
    fl = ctypes.c_double()
    fake = ctypes.c_void_p(0x1000)
    assert L.tsa_peak_mfma(2, 1, 1, 1.0, fake, ctypes.byref(fl), None) == -1    # dtype
    assert L.tsa_peak_mfma(0, 0, 1, 1.0, fake, ctypes.byref(fl), None) == -1    # no blocks
    assert L.tsa_peak_mfma(0, 1, 0, 1.0, fake, ctypes.byref(fl), None) == -1    # no iterations
    assert L.tsa_peak_mfma(0, 1, 1, 1.0, None, ctypes.byref(fl), None) == -1    # null out
    assert L.tsa_peak_copy(fake, ctypes.c_void_p(0x2000), 24, 1, None) == -1    # not 16-byte sized
    assert L.tsa_peak_copy(fake, ctypes.c_void_p(0x1008), 16, 1, None) == -1    # misaligned dst
    assert L.tsa_peak_copy(fake, ctypes.c_void_p(0x1010), 64, 1, None) == -1    # overlap
    assert L.tsa_peak_read(fake, 16, 0, fake, None) == -1                       # no blocks
    assert L.tsa_peak_read(None, 16, 1, fake, None) == -1                       # null src
    assert L.tsa_peak_read_cached(fake, 16, 0, fake, None) == -1                # no blocks
    assert L.tsa_peak_read_cached(fake, 24, 1, fake, None) == -1                # not 16-byte sized


@pytest.mark.gpu
def test_mfma_chain_sum_and_flops():
    import torch
    from top_selected_attention_amd import peaks
    for dt in ("bf16", "fp16"):
        out, fl = peaks.mfma(dt, n_blocks=8, iters=100, a=0.5)
        torch.cuda.synchronize()
        # each chain's element 0 sums 16 products a*a per MFMA, 4 chains
        assert torch.equal(out.cpu(), torch.full((8,), 64 * 100 * 0.25)), dt
        assert fl == 8 * 4 * 4 * 100 * 2 * 32 * 32 * 16


@pytest.mark.gpu
def test_copy_and_read_are_exact():
    import torch
    from top_selected_attention_amd import peaks
    g = torch.Generator().manual_seed(7)
    n = (3 << 20) + 4 * 37            # 16-byte multiple with a ragged tail past the unrolled loop
    x = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, generator=g)
    xd = x.cuda()
    yd = torch.zeros_like(xd)
    peaks.copy(xd, yd, n_blocks=64)
    o = torch.zeros(64, dtype=torch.int32, device="cuda")
    peaks.read(xd, o, n_blocks=64)
    oc = torch.zeros(64, dtype=torch.int32, device="cuda")
    peaks.read(xd, oc, n_blocks=64, cached=True)
    torch.cuda.synchronize()
    assert torch.equal(yd.cpu(), x)
    want = np.bitwise_xor.reduce(x.numpy().view(np.uint32))
    for out in (o, oc):
        assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == want
