"""What this chip sustains, measured with the kernels of libtsa_peaks.so
(declared in include/tsa_peaks.h): dense bf16 / fp16 MFMA issue rate, HBM
copy / read bandwidth, and the read bandwidth of data that misses the L2s
but stays in the 256 MB memory-side cache (MALL).  Launches go to torch's current stream and are timed
with events on it."""

import ctypes
import os

import torch

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsa_peaks.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built (run top_selected_attention_amd/build.py)")
        L = ctypes.CDLL(_LIB)
        L.tsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                    ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                    ctypes.c_void_p]
        L.tsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_void_p]
        L.tsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
        L.tsa_peak_read_cached.argtypes = L.tsa_peak_read.argtypes
        L.tsa_fill_registers.argtypes = [ctypes.c_uint, ctypes.c_void_p]
        for f in (L.tsa_peak_mfma, L.tsa_peak_copy, L.tsa_peak_read, L.tsa_peak_read_cached,
                  L.tsa_fill_registers):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def mfma(dtype="bf16", n_blocks=2048, iters=2000, a=1.0):
    """One launch of the MFMA issue kernel: returns (out tensor [n_blocks],
    dense FLOPs of the launch)."""
    out = torch.empty(n_blocks, dtype=torch.float32, device="cuda")
    fl = ctypes.c_double()
    _check(lib().tsa_peak_mfma({"bf16": 0, "fp16": 1}[dtype], n_blocks, iters, a,
                               ctypes.c_void_p(out.data_ptr()), ctypes.byref(fl), _stream()),
           "tsa_peak_mfma")
    return out, fl.value


def copy(src, dst, n_blocks=8192):
    if dst.numel() * dst.element_size() < src.numel() * src.element_size():
        raise ValueError("dst smaller than src")
    _check(lib().tsa_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                               src.numel() * src.element_size(), n_blocks, _stream()),
           "tsa_peak_copy")


def read(src, out, n_blocks=8192, cached=False):
    """Reads all of src (nontemporal loads, or plain ones with cached=True);
    out[b] = xor of the words workgroup b read."""
    if out.numel() * out.element_size() < 4 * n_blocks:
        raise ValueError("out holds fewer than n_blocks words")
    f = lib().tsa_peak_read_cached if cached else lib().tsa_peak_read
    _check(f(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(), n_blocks,
             ctypes.c_void_p(out.data_ptr()), _stream()),
           "tsa_peak_read_cached" if cached else "tsa_peak_read")


def fill_registers(pattern):
    """Writes ``pattern`` (32 bits) into every SIMD's registers (test aid)."""
    _check(lib().tsa_fill_registers(pattern & 0xffffffff, _stream()), "tsa_fill_registers")


def _timed(f, n):
    for _ in range(3):
        f()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def measure(n_bytes=1 << 30):
    """Sustained MFMA TFLOP/s (bf16, fp16) and HBM GB/s (copy counts read +
    write) on this device."""
    res = {}
    for dt in ("bf16", "fp16"):
        holder = {}

        def run():
            holder["out"], holder["fl"] = mfma(dt)
        ms = _timed(run, 10)
        res[f"mfma_{dt}_tflops"] = round(holder["fl"] / (ms * 1e-3) / 1e12, 1)
    x = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1.0)
    o = torch.empty(8192, dtype=torch.int32, device="cuda")
    ms = _timed(lambda: copy(x, y), 20)
    res["hbm_copy_gbs"] = round(2 * n_bytes / (ms * 1e-3) / 1e9, 1)
    ms = _timed(lambda: read(x, o), 20)
    res["hbm_read_gbs"] = round(n_bytes / (ms * 1e-3) / 1e9, 1)
    # 160 MiB with plain loads: far past the eight 4 MB L2s, inside the MALL
    # once read (the warm-up reads of _timed bring it in)
    m_bytes = 160 << 20
    xm = x[: m_bytes // 4]
    ms = _timed(lambda: read(xm, o, cached=True), 50)
    res["mall_read_gbs"] = round(m_bytes / (ms * 1e-3) / 1e9, 1)
    return res
