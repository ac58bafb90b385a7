"""Python binding of the top-selected-attention HIP library (libtsa.so).

Argument marshalling only: every function checks tensor dtypes, shapes and
devices, sizes and allocates the workspace and outputs with torch, and calls
the C ABI declared in ``include/top_selected_attention.h`` on torch's current
stream.  All arithmetic runs in the library's HIP kernels; there is no other
execution path, and importing this package raises if the library is missing.

Entry points (names as in the C ABI):
  bsa_fwd, bsa_bwd, bsa_compact             block-sparse attention (BNSD or
                                             TND, optional atten_mask)
  nsa_select_fwd, nsa_select_bwd, nsa_compact   NSA selected attention (TND)
  sfa_paged_fwd                              sparse flash attention decode
  sfa_sharedkv_fwd                           shared-KV decode: band over the
                                             original cache + compressed top-k
  floyd_fwd, floyd_bwd                       FloydAttention (two score products
                                             batched over the query's two
                                             sequence axes, one softmax)
The ``*Plan`` classes (BsaPlan, NsaPlan, SfaPlan, SfaSharedkvPlan, FloydPlan)
pre-allocate outputs and workspace for repeated calls.
"""

import ctypes
import math
import os

import torch

from . import _abi
from ._abi import TsaError, BF16, FP16, LAYOUT_BNSD, LAYOUT_TND, LAYOUT_BSND  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python top_selected_attention_amd/build.py` "
        "(there is no fallback implementation)")

lib = _abi.load(LIB_PATH)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return FP16
    raise TypeError(f"expected bfloat16 or float16, got {t.dtype}")


def _check(t, name, dtype=None, shape=None, align16=None):
    """align16 (default: for 16-bit float tensors): the kernels move the
    tensor in 16-byte pieces, so its address must be a multiple of 16."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if align16 is None:
        align16 = t.dtype in (torch.bfloat16, torch.float16)
    if align16 and t.data_ptr() % 16:
        raise ValueError(f"{name} must start at a 16-byte aligned address (a view at an "
                         f"element offset is not): {t.data_ptr():#x}")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _ceil(a, b):
    return -(-a // b)


# ----------------------------------------------------------------------------
# Block-sparse attention
# ----------------------------------------------------------------------------

class BsaPlan:
    """Forward and backward of block-sparse attention for fixed tensors.

    BNSD: q [B, N1, Sq, 128], k/v [B, N2, Skv, 128]; TND (varlen, when
    cu_seqlens_q / cu_seqlens_kv are given as host B+1 prefix sums):
    q [T, N1, 128], k/v [Tk, N2, 128], with Sq / Skv the longest sequences.
    bf16 or fp16; block_mask u8 [B, N1, ceil(Sq/block_q), ceil(Skv/block_kv)].
    atten_mask (optional): u8 or bool, [Sq, Skv] or [B|1, N1|1, Sq, Skv]
    (size-1 or stride-0 axes shared), rows contiguous; non-zero / True = that
    score is excluded.  ``fwd()`` writes ``self.out`` / ``self.lse`` (LSE [B, N1, Sq] or
    [T, N1]); ``bwd(dout)`` writes ``self.dq`` / ``self.dk`` / ``self.dv``.
    """

    def __init__(self, q, k, v, block_mask, block_q, block_kv, scale=None, sparse_mode=0,
                 backward=True, cu_seqlens_q=None, cu_seqlens_kv=None, atten_mask=None):
        _check(q, "q"), _check(k, "k", q.dtype), _check(v, "v", q.dtype)
        tnd = cu_seqlens_q is not None or cu_seqlens_kv is not None
        if tnd:
            if cu_seqlens_q is None or cu_seqlens_kv is None:
                raise ValueError("TND needs both cu_seqlens_q and cu_seqlens_kv")
            if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
                raise ValueError("q, k, v must be TND with k and v of one shape")
            self.cu_q, self.cu_kv = _host_i32(cu_seqlens_q), _host_i32(cu_seqlens_kv)
            B = self.cu_q.numel() - 1
            if self.cu_kv.numel() != B + 1:
                raise ValueError("cu_seqlens_q and cu_seqlens_kv differ in length")
            T, N1, D = q.shape
            Tk, N2, _ = k.shape
            if int(self.cu_q[-1]) != T or int(self.cu_kv[-1]) != Tk or k.shape[2] != D:
                raise ValueError("cu_seqlens do not match q / k")
            Sq = int((self.cu_q[1:] - self.cu_q[:-1]).max()) if B > 0 else 0
            Skv = int((self.cu_kv[1:] - self.cu_kv[:-1]).max()) if B > 0 else 0
            lse_shape, layout = (T, N1), LAYOUT_TND
            seq = dict(cu_seqlens_q=ctypes.cast(self.cu_q.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
                       cu_seqlens_kv=ctypes.cast(self.cu_kv.data_ptr(), ctypes.POINTER(ctypes.c_int32)))
        else:
            if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
                raise ValueError("q, k, v must be BNSD with k and v of one shape")
            B, N1, Sq, D = q.shape
            _, N2, Skv, _ = k.shape
            if k.shape[0] != B or k.shape[3] != D:
                raise ValueError("q and k disagree in B or D")
            lse_shape, layout, seq = (B, N1, Sq), LAYOUT_BNSD, {}
        QB, KB = _ceil(Sq, block_q), _ceil(Skv, block_kv)
        _check(block_mask, "block_mask", torch.uint8, (B, N1, QB, KB), align16=True)
        seq.update(_atten_mask_fields(atten_mask, B, N1, Sq, Skv))
        self.atten_mask = atten_mask
        self.q, self.k, self.v, self.mask = q, k, v, block_mask
        self.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        dev = q.device
        self.out = torch.empty_like(q)
        self.lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
        self.fa = _abi.BsaFwdArgs(
            dtype=_dtype_code(q), q_layout=layout, kv_layout=layout,
            B=B, N1=N1, N2=N2, Sq=Sq, Skv=Skv, D=D, block_q=block_q, block_kv=block_kv,
            sparse_mode=sparse_mode, scale=self.scale, validate=0,
            block_mask=block_mask.data_ptr(), q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(),
            out=self.out.data_ptr(), lse=self.lse.data_ptr(), **seq)
        nb = ctypes.c_size_t()
        _abi.call(lib.bsa_fwd_workspace_size, ctypes.byref(self.fa), ctypes.byref(nb))
        self.ws_fwd = _workspace(nb.value, dev)
        # fwd() builds the block lists (both directions) in the workspace; the
        # backward then shares that workspace and reuses them
        self._lists = False
        self.backward = backward
        if backward:
            self.dout = None
            self.dq = torch.empty_like(q)
            self.dk = torch.empty_like(k)
            self.dv = torch.empty_like(v)
            self.ba = _abi.BsaBwdArgs(
                dtype=_dtype_code(q), q_layout=layout, kv_layout=layout,
                B=B, N1=N1, N2=N2, Sq=Sq, Skv=Skv, D=D, block_q=block_q, block_kv=block_kv,
                sparse_mode=sparse_mode, scale=self.scale, validate=0,
                block_mask=block_mask.data_ptr(), q=q.data_ptr(), k=k.data_ptr(),
                v=v.data_ptr(), out=self.out.data_ptr(), dout=0, lse=self.lse.data_ptr(),
                dq=self.dq.data_ptr(), dk=self.dk.data_ptr(), dv=self.dv.data_ptr(), **seq)

    def fwd(self):
        self.fa.reuse_lists = 0
        _abi.call(lib.bsa_fwd, ctypes.byref(self.fa), _ptr(self.ws_fwd),
                  ctypes.c_size_t(self.ws_fwd.numel()), _stream())
        self._lists = True
        return self.out, self.lse

    def set_dout(self, dout):
        _check(dout, "dout", self.q.dtype, self.q.shape)
        self.dout = dout
        self.ba.dout = dout.data_ptr()
        nb = ctypes.c_size_t()
        _abi.call(lib.bsa_bwd_workspace_size, ctypes.byref(self.ba), ctypes.byref(nb))
        if nb.value > self.ws_fwd.numel():
            self.ws_fwd = _workspace(nb.value, self.q.device)
            self._lists = False
        self.ws_bwd = self.ws_fwd

    def set_out(self, out, lse):
        """Use an externally produced forward output / LSE in the backward."""
        _check(out, "out", self.q.dtype, self.q.shape)
        _check(lse, "lse", torch.float32, self.lse.shape)
        self.ba.out, self.ba.lse = out.data_ptr(), lse.data_ptr()
        self._ext = (out, lse)

    def bwd(self, dout=None):
        if dout is not None and dout is not self.dout:
            self.set_dout(dout)
        if self.dout is None:
            raise ValueError("bwd needs dout")
        self.ba.reuse_lists = 1 if self._lists else 0
        _abi.call(lib.bsa_bwd, ctypes.byref(self.ba), _ptr(self.ws_bwd),
                  ctypes.c_size_t(self.ws_bwd.numel()), _stream())
        self._lists = True
        return self.dq, self.dk, self.dv


def _atten_mask_fields(am, B, N1, Sq, Skv):
    """Pointer and plane strides of an atten_mask tensor (see BsaPlan)."""
    if am is None:
        return {}
    if not isinstance(am, torch.Tensor) or not am.is_cuda:
        raise ValueError("atten_mask must be a device tensor")
    if am.dtype not in (torch.uint8, torch.bool):
        raise TypeError(f"atten_mask must be uint8 or bool, got {am.dtype}")
    if am.dim() == 2:
        am = am[None, None]
    if am.dim() != 4 or tuple(am.shape[2:]) != (Sq, Skv) or am.shape[0] not in (1, B) \
            or am.shape[1] not in (1, N1):
        raise ValueError(f"atten_mask must be [Sq, Skv] or [B|1, N1|1, Sq, Skv] with "
                         f"Sq={Sq}, Skv={Skv}, got {tuple(am.shape)}")
    if Sq * Skv > 0 and ((Skv > 1 and am.stride(3) != 1) or (Sq > 1 and am.stride(2) != Skv)):
        raise ValueError("atten_mask rows must be contiguous, Skv elements apart")
    sb = am.stride(0) if am.shape[0] > 1 else 0
    sn = am.stride(1) if am.shape[1] > 1 else 0
    return dict(atten_mask=am.data_ptr(), atten_mask_stride_b=sb, atten_mask_stride_n=sn)


def bsa_fwd(q, k, v, block_mask, block_q, block_kv, scale=None, sparse_mode=0,
            cu_seqlens_q=None, cu_seqlens_kv=None, atten_mask=None):
    """Block-sparse attention forward (BNSD, or TND with cu_seqlens): returns (out, lse)."""
    plan = BsaPlan(q, k, v, block_mask, block_q, block_kv, scale, sparse_mode, backward=False,
                   cu_seqlens_q=cu_seqlens_q, cu_seqlens_kv=cu_seqlens_kv, atten_mask=atten_mask)
    return plan.fwd()


def bsa_bwd(q, k, v, out, dout, lse, block_mask, block_q, block_kv, scale=None, sparse_mode=0,
            cu_seqlens_q=None, cu_seqlens_kv=None, atten_mask=None):
    """Block-sparse attention backward (BNSD, or TND with cu_seqlens): returns (dq, dk, dv)."""
    plan = BsaPlan(q, k, v, block_mask, block_q, block_kv, scale, sparse_mode, backward=True,
                   cu_seqlens_q=cu_seqlens_q, cu_seqlens_kv=cu_seqlens_kv, atten_mask=atten_mask)
    plan.set_out(out, lse)
    return plan.bwd(dout)


def bsa_compact(block_mask, N2, Sq, Skv, block_q, block_kv):
    """The forward / reverse CSR lists of a BlockSparseMask (int32 device tensors,
    entry arrays trimmed to their used length)."""
    B, N1, QB, KB = block_mask.shape
    _check(block_mask, "block_mask", torch.uint8, (B, N1, _ceil(Sq, block_q), _ceil(Skv, block_kv)),
           align16=True)
    dev = block_mask.device
    a = _abi.BsaFwdArgs(dtype=BF16, q_layout=LAYOUT_BNSD, kv_layout=LAYOUT_BNSD, B=B, N1=N1,
                        N2=N2, Sq=Sq, Skv=Skv, D=128, block_q=block_q, block_kv=block_kv,
                        sparse_mode=0, scale=1.0, validate=0, block_mask=block_mask.data_ptr())
    nb = ctypes.c_size_t()
    _abi.call(lib.bsa_compact_workspace_size, ctypes.byref(a), ctypes.byref(nb))
    ws = _workspace(nb.value, dev)
    R, C = B * N1 * QB, B * N2 * KB
    i32 = dict(dtype=torch.int32, device=dev)
    row_ptr, col = torch.empty(R + 1, **i32), torch.empty(max(R * KB, 1), **i32)
    rev_ptr, rev = torch.empty(C + 1, **i32), torch.empty(max(R * KB, 1), **i32)
    _abi.call(lib.bsa_compact, ctypes.byref(a), _ptr(row_ptr), _ptr(col), _ptr(rev_ptr),
              _ptr(rev), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream())
    nnz = int(row_ptr[-1].item())
    return row_ptr, col[:nnz], rev_ptr, rev[:nnz]


# ----------------------------------------------------------------------------
# NSA selected attention
# ----------------------------------------------------------------------------

def _host_i32(x):
    t = torch.as_tensor(x, dtype=torch.int32, device="cpu").contiguous()
    return t


class NsaPlan:
    """Forward and backward of NSA selected attention for fixed tensors.

    q [T, N1, D], k [Tk, N2, D], v [Tk, N2, 128] (TND) with D = 128 or 192,
    topk int32 [T, N2, sbc] device,
    cu_seqlens_q / cu_seqlens_kv: B+1 prefix sums (host sequences or tensors).
    """

    def __init__(self, q, k, v, topk, cu_seqlens_q, cu_seqlens_kv, sbs, scale=None,
                 sparse_mode=2, validate=False, backward=True):
        _check(q, "q"), _check(k, "k", q.dtype), _check(v, "v", q.dtype)
        T, N1, D = q.shape
        Tk, N2, _ = k.shape
        sbc = topk.shape[-1]
        _check(topk, "topk", torch.int32, (T, N2, sbc))
        self.cu_q, self.cu_kv = _host_i32(cu_seqlens_q), _host_i32(cu_seqlens_kv)
        B = self.cu_q.numel() - 1
        self.q, self.k, self.v, self.topk = q, k, v, topk
        self.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        dev = q.device
        self.out = torch.empty((T, N1, v.shape[2]), dtype=q.dtype, device=dev)
        self.lse = torch.empty((T, N1), dtype=torch.float32, device=dev)
        common = dict(dtype=_dtype_code(q), layout=LAYOUT_TND, B=B, T=T, Tk=Tk, N1=N1, N2=N2,
                      D=D, Dv=v.shape[2],
                      cu_seqlens_q=ctypes.cast(self.cu_q.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
                      cu_seqlens_kv=ctypes.cast(self.cu_kv.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
                      sbs=sbs, sbc=sbc, sparse_mode=sparse_mode, scale=self.scale,
                      validate=int(bool(validate)), topk=topk.data_ptr(), q=q.data_ptr(),
                      k=k.data_ptr(), v=v.data_ptr())
        self.common = common
        self.fa = _abi.NsaFwdArgs(out=self.out.data_ptr(), lse=self.lse.data_ptr(), **common)
        nb = ctypes.c_size_t()
        _abi.call(lib.nsa_select_fwd_workspace_size, ctypes.byref(self.fa), ctypes.byref(nb))
        self.ws_fwd = _workspace(nb.value, dev)
        # fwd() builds the per-row lists in the workspace; the backward shares
        # it and adds only the reverse lists
        self._lists = False
        if backward:
            self.dout = None
            self.dq = torch.empty_like(q)
            self.dk = torch.empty_like(k)
            self.dv = torch.empty_like(v)
            self.ba = _abi.NsaBwdArgs(out=self.out.data_ptr(), dout=0, lse=self.lse.data_ptr(),
                                      dq=self.dq.data_ptr(), dk=self.dk.data_ptr(),
                                      dv=self.dv.data_ptr(), **common)

    def fwd(self):
        self.fa.reuse_lists = 0
        _abi.call(lib.nsa_select_fwd, ctypes.byref(self.fa), _ptr(self.ws_fwd),
                  ctypes.c_size_t(self.ws_fwd.numel()), _stream())
        self._lists = True
        return self.out, self.lse

    def set_dout(self, dout):
        _check(dout, "dout", self.q.dtype, self.out.shape)
        self.dout = dout
        self.ba.dout = dout.data_ptr()
        nb = ctypes.c_size_t()
        _abi.call(lib.nsa_select_bwd_workspace_size, ctypes.byref(self.ba), ctypes.byref(nb))
        if nb.value > self.ws_fwd.numel():
            self.ws_fwd = _workspace(nb.value, self.q.device)
            self._lists = False
        self.ws_bwd = self.ws_fwd

    def set_out(self, out, lse):
        _check(out, "out", self.q.dtype, self.out.shape)
        _check(lse, "lse", torch.float32, self.lse.shape)
        self.ba.out, self.ba.lse = out.data_ptr(), lse.data_ptr()
        self._ext = (out, lse)

    def bwd(self, dout=None):
        if dout is not None and dout is not self.dout:
            self.set_dout(dout)
        if self.dout is None:
            raise ValueError("bwd needs dout")
        self.ba.reuse_lists = 2 if self._lists else 0
        _abi.call(lib.nsa_select_bwd, ctypes.byref(self.ba), _ptr(self.ws_bwd),
                  ctypes.c_size_t(self.ws_bwd.numel()), _stream())
        return self.dq, self.dk, self.dv


def nsa_select_fwd(q, k, v, topk, cu_seqlens_q, cu_seqlens_kv, sbs, scale=None, sparse_mode=2,
                   validate=False):
    """NSA selected attention forward: returns (out, lse)."""
    return NsaPlan(q, k, v, topk, cu_seqlens_q, cu_seqlens_kv, sbs, scale, sparse_mode,
                   validate, backward=False).fwd()


def nsa_select_bwd(q, k, v, out, dout, lse, topk, cu_seqlens_q, cu_seqlens_kv, sbs, scale=None,
                   sparse_mode=2, validate=False):
    """NSA selected attention backward: returns (dq, dk, dv)."""
    plan = NsaPlan(q, k, v, topk, cu_seqlens_q, cu_seqlens_kv, sbs, scale, sparse_mode, validate)
    plan.set_out(out, lse)
    return plan.bwd(dout)


def nsa_compact(topk, cu_seqlens_q, cu_seqlens_kv, N1, sbs, sparse_mode=2, validate=False):
    """The forward / reverse CSR lists of NSA topk_indices:
    (row_ptr, col, rev_ptr, rev, blocks_total), device int32 tensors."""
    T, N2, sbc = topk.shape
    _check(topk, "topk", torch.int32)
    cu_q, cu_kv = _host_i32(cu_seqlens_q), _host_i32(cu_seqlens_kv)
    a = _abi.NsaFwdArgs(dtype=BF16, layout=LAYOUT_TND, B=cu_q.numel() - 1, T=T,
                        Tk=int(cu_kv[-1]), N1=N1, N2=N2, D=128, Dv=128,
                        cu_seqlens_q=ctypes.cast(cu_q.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
                        cu_seqlens_kv=ctypes.cast(cu_kv.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
                        sbs=sbs, sbc=sbc, sparse_mode=sparse_mode, scale=1.0,
                        validate=int(bool(validate)), topk=topk.data_ptr())
    nb = ctypes.c_size_t()
    _abi.call(lib.nsa_compact_workspace_size, ctypes.byref(a), ctypes.byref(nb))
    NB = ctypes.c_int32()
    _abi.call(lib.nsa_compact_blocks_total, ctypes.byref(a), ctypes.byref(NB))
    dev = topk.device
    ws = _workspace(nb.value, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    R = T * N2
    row_ptr, col = torch.empty(R + 1, **i32), torch.empty(max(R * sbc, 1), **i32)
    rev_ptr, rev = torch.empty(N2 * NB.value + 1, **i32), torch.empty(max(R * sbc, 1), **i32)
    _abi.call(lib.nsa_compact, ctypes.byref(a), _ptr(row_ptr), _ptr(col), _ptr(rev_ptr),
              _ptr(rev), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream())
    nnz = int(row_ptr[-1].item())
    return row_ptr, col[:nnz], rev_ptr, rev[:nnz], NB.value


# ----------------------------------------------------------------------------
# Sparse flash attention (paged decode)
# ----------------------------------------------------------------------------

class SfaPlan:
    """Paged sparse flash attention decode for fixed tensors.

    q [B, Sq, N1, 512], q_rope [B, Sq, N1, 64] (BSND); key_cache [P, page, 1, 512],
    key_rope_cache [P, page, 1, 64], value_cache [P, page, 1, 512] (may be key_cache);
    block_table int32 [B, max_pages]; kv_lens int32 [B]; topk_indices int32
    [B, Sq, 1, K] (-1 = empty).  With cu_seqlens_q (host B+1 prefix sums) the
    queries are TND: q [T, N1, 512], q_rope [T, N1, 64], topk_indices
    [T, 1, K], out [T, N1, 512], lse [T, N1].
    """

    def __init__(self, q, q_rope, key_cache, key_rope_cache, value_cache, block_table, kv_lens,
                 topk_indices, scale=None, sparse_mode=3, sparse_block_size=1, validate=False,
                 cu_seqlens_q=None):
        for t, n in ((q, "q"), (q_rope, "q_rope"), (key_cache, "key_cache"),
                     (key_rope_cache, "key_rope_cache"), (value_cache, "value_cache")):
            _check(t, n, q.dtype)
        P, page, N2, _ = key_cache.shape
        Dv = value_cache.shape[3]
        K = topk_indices.shape[-1]
        extra = {}
        if cu_seqlens_q is not None:
            self.cu_q = _host_i32(cu_seqlens_q)
            B = self.cu_q.numel() - 1
            T, N1, D = q.shape
            Sq, Dr = 0, q_rope.shape[2]
            if int(self.cu_q[-1]) != T:
                raise ValueError("cu_seqlens_q does not match q")
            tok_shape, layout = (T,), LAYOUT_TND
            extra = dict(T=T, cu_seqlens_q=ctypes.cast(self.cu_q.data_ptr(),
                                                       ctypes.POINTER(ctypes.c_int32)))
        else:
            B, Sq, N1, D = q.shape
            Dr = q_rope.shape[3]
            tok_shape, layout = (B, Sq), LAYOUT_BSND
        _check(block_table, "block_table", torch.int32)
        _check(kv_lens, "kv_lens", torch.int32, (B,))
        _check(topk_indices, "topk_indices", torch.int32, tok_shape + (N2, K))
        self.keep = (q, q_rope, key_cache, key_rope_cache, value_cache, block_table, kv_lens,
                     topk_indices)
        self.scale = 1.0 / math.sqrt(D + Dr) if scale is None else float(scale)
        dev = q.device
        self.out = torch.empty(tok_shape + (N1, Dv), dtype=q.dtype, device=dev)
        self.lse = torch.empty(tok_shape + (N1,), dtype=torch.float32, device=dev)
        self.a = _abi.SfaArgs(
            dtype=_dtype_code(q), q_layout=layout, B=B, Sq=Sq, N1=N1, N2=N2, D=D, Dr=Dr,
            Dv=Dv, num_pages=P, page_size=page, max_pages=block_table.shape[1], topk=K,
            sparse_block_size=sparse_block_size, sparse_mode=sparse_mode, scale=self.scale,
            validate=int(bool(validate)), q=q.data_ptr(), q_rope=q_rope.data_ptr(),
            key_cache=key_cache.data_ptr(), key_rope_cache=key_rope_cache.data_ptr(),
            value_cache=value_cache.data_ptr(), block_table=block_table.data_ptr(),
            kv_lens=kv_lens.data_ptr(), topk_indices=topk_indices.data_ptr(),
            out=self.out.data_ptr(), lse=self.lse.data_ptr(), **extra)
        nb = ctypes.c_size_t()
        _abi.call(lib.sfa_paged_fwd_workspace_size, ctypes.byref(self.a), ctypes.byref(nb))
        self.ws = _workspace(nb.value, dev)

    def fwd(self):
        _abi.call(lib.sfa_paged_fwd, ctypes.byref(self.a), _ptr(self.ws),
                  ctypes.c_size_t(self.ws.numel()), _stream())
        return self.out, self.lse

    def fwd_noalloc(self):
        """The same forward through sfa_paged_fwd_noalloc: the library's fixed
        per-GPU scratch instead of this plan's workspace (for callers that
        cannot allocate; overlapping calls on one GPU race)."""
        _abi.call(lib.sfa_paged_fwd_noalloc, ctypes.byref(self.a), _stream())
        return self.out, self.lse


def sfa_paged_fwd(q, q_rope, key_cache, key_rope_cache, value_cache, block_table, kv_lens,
                  topk_indices, scale=None, sparse_mode=3, sparse_block_size=1, validate=False,
                  cu_seqlens_q=None):
    """Paged sparse flash attention forward (BSND, or TND queries with
    cu_seqlens_q): returns (out, lse)."""
    return SfaPlan(q, q_rope, key_cache, key_rope_cache, value_cache, block_table, kv_lens,
                   topk_indices, scale, sparse_mode, sparse_block_size, validate,
                   cu_seqlens_q).fwd()


class SfaSharedkvPlan:
    """Shared-KV two-branch sparse decode for fixed tensors: a band of
    win_left past / win_right future tokens over the original paged KV plus
    cmp_topk selected entries of a compressed paged KV, in one softmax.

    q [B, Sq, N1, 512] / q_rope [B, Sq, N1, 64] (BSND), or [T, N1, ...] with
    host cu_seqlens_q (TND); seqused_kv int32 [B]; ori = (key_cache [P, page,
    1, 512], key_rope_cache [P, page, 1, 64], block_table int32 [B, max_pages])
    or None; cmp = (key_cache, key_rope_cache, block_table, topk int32
    [tokens, 1, K]) or None.  ``fwd()`` returns (out, lse).  ``metadata()``
    makes the task list once (``self.tasks``); later ``fwd()`` calls use it
    and skip the list kernel, as every layer of a decode step may.
    """

    def __init__(self, q, q_rope, seqused_kv, ori=None, cmp=None, scale=None, win_left=127,
                 win_right=0, cmp_ratio=4, cu_seqlens_q=None):
        _check(q, "q"), _check(q_rope, "q_rope", q.dtype)
        extra = {}
        if cu_seqlens_q is not None:
            self.cu_q = _host_i32(cu_seqlens_q)
            B = self.cu_q.numel() - 1
            T, N1, D = q.shape
            Sq, Dr = 0, q_rope.shape[2]
            if int(self.cu_q[-1]) != T:
                raise ValueError("cu_seqlens_q does not match q")
            tok_shape, layout = (T,), LAYOUT_TND
            extra = dict(T=T, cu_seqlens_q=ctypes.cast(self.cu_q.data_ptr(),
                                                       ctypes.POINTER(ctypes.c_int32)))
        else:
            B, Sq, N1, D = q.shape
            Dr = q_rope.shape[3]
            tok_shape, layout = (B, Sq), LAYOUT_BSND
        _check(seqused_kv, "seqused_kv", torch.int32, (B,))
        if ori is not None:
            okc, okrc, obt = ori
            _check(okc, "ori key_cache", q.dtype), _check(okrc, "ori key_rope_cache", q.dtype)
            _check(obt, "ori block_table", torch.int32)
            extra.update(has_ori_kv=1, ori_win_left=win_left, ori_win_right=win_right,
                         ori_num_pages=okc.shape[0], ori_page_size=okc.shape[1],
                         ori_max_pages=obt.shape[1], ori_key_cache=okc.data_ptr(),
                         ori_key_rope_cache=okrc.data_ptr(), ori_block_table=obt.data_ptr())
        if cmp is not None:
            ckc, ckrc, cbt, idx = cmp
            _check(ckc, "cmp key_cache", q.dtype), _check(ckrc, "cmp key_rope_cache", q.dtype)
            _check(cbt, "cmp block_table", torch.int32)
            K = idx.shape[-1]
            _check(idx, "cmp topk", torch.int32, tok_shape + (1, K))
            extra.update(has_cmp_kv=1, cmp_ratio=cmp_ratio, cmp_topk=K,
                         cmp_num_pages=ckc.shape[0], cmp_page_size=ckc.shape[1],
                         cmp_max_pages=cbt.shape[1], cmp_key_cache=ckc.data_ptr(),
                         cmp_key_rope_cache=ckrc.data_ptr(), cmp_block_table=cbt.data_ptr(),
                         cmp_topk_indices=idx.data_ptr())
        self.keep = (q, q_rope, seqused_kv, ori, cmp)
        self.scale = 1.0 / math.sqrt(D + Dr) if scale is None else float(scale)
        dev = self.q_device = q.device
        self.out = torch.empty(tok_shape + (N1, D), dtype=q.dtype, device=dev)
        self.lse = torch.empty(tok_shape + (N1,), dtype=torch.float32, device=dev)
        self.a = _abi.SfaSharedkvArgs(
            dtype=_dtype_code(q), q_layout=layout, B=B, Sq=Sq, N1=N1, N2=1, D=D, Dr=Dr,
            scale=self.scale, q=q.data_ptr(), q_rope=q_rope.data_ptr(),
            seqused_kv=seqused_kv.data_ptr(), out=self.out.data_ptr(), lse=self.lse.data_ptr(),
            **extra)
        nb = ctypes.c_size_t()
        _abi.call(lib.sfa_sharedkv_fwd_workspace_size, ctypes.byref(self.a), ctypes.byref(nb))
        self.ws = _workspace(nb.value, dev)
        self.tasks = None

    def metadata(self):
        """Makes the task list (device) that later fwd() calls use."""
        nb = ctypes.c_size_t()
        _abi.call(lib.sfa_sharedkv_metadata_size, ctypes.byref(self.a), ctypes.byref(nb))
        if self.tasks is None or self.tasks.numel() < nb.value:
            self.tasks = _workspace(nb.value, self.q_device)
        self.a.tasks = None
        _abi.call(lib.sfa_sharedkv_metadata, ctypes.byref(self.a), _ptr(self.tasks),
                  ctypes.c_size_t(self.tasks.numel()), _stream())
        self.a.tasks = self.tasks.data_ptr()
        return self.tasks

    def fwd(self):
        _abi.call(lib.sfa_sharedkv_fwd, ctypes.byref(self.a), _ptr(self.ws),
                  ctypes.c_size_t(self.ws.numel()), _stream())
        return self.out, self.lse


def sfa_sharedkv_fwd(q, q_rope, seqused_kv, ori=None, cmp=None, scale=None, win_left=127,
                     win_right=0, cmp_ratio=4, cu_seqlens_q=None):
    """Shared-KV two-branch sparse decode: returns (out, lse)."""
    return SfaSharedkvPlan(q, q_rope, seqused_kv, ori, cmp, scale, win_left, win_right,
                           cmp_ratio, cu_seqlens_q).fwd()



# ----------------------------------------------------------------------------
# FloydAttention
# ----------------------------------------------------------------------------

class FloydPlan:
    """Forward and backward of FloydAttention for fixed tensors.

    q [B, H, N, M, D]; k1, v1 [B, H, N, K, D]; k2, v2 [B, H, M, K, D] (bf16 or
    fp16).  ``fwd()`` returns (out [B, H, N, M, D], lse [B, H, N, M]);
    ``bwd(dout)`` returns (dq, dk1, dv1, dk2, dv2).
    """

    def __init__(self, q, k1, v1, k2, v2, scale=None, backward=True):
        _check(q, "q")
        for t, n in ((k1, "k1"), (v1, "v1"), (k2, "k2"), (v2, "v2")):
            _check(t, n, q.dtype)
        if q.dim() != 5:
            raise ValueError("q must be [B, H, N, M, D]")
        B, H, N, M, D = q.shape
        K = k1.shape[3]
        if tuple(k1.shape) != (B, H, N, K, D) or v1.shape != k1.shape:
            raise ValueError(f"k1 / v1 must be {(B, H, N, K, D)}")
        if tuple(k2.shape) != (B, H, M, K, D) or v2.shape != k2.shape:
            raise ValueError(f"k2 / v2 must be {(B, H, M, K, D)}")
        self.q, self.k1, self.v1, self.k2, self.v2 = q, k1, v1, k2, v2
        self.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        dev = q.device
        self.out = torch.empty_like(q)
        self.lse = torch.empty((B, H, N, M), dtype=torch.float32, device=dev)
        common = dict(dtype=_dtype_code(q), B=B, H=H, N=N, M=M, K=K, D=D, scale=self.scale,
                      q=q.data_ptr(), k1=k1.data_ptr(), v1=v1.data_ptr(), k2=k2.data_ptr(),
                      v2=v2.data_ptr())
        self.fa = _abi.FloydFwdArgs(out=self.out.data_ptr(), lse=self.lse.data_ptr(), **common)
        nb = ctypes.c_size_t()
        _abi.call(lib.floyd_fwd_workspace_size, ctypes.byref(self.fa), ctypes.byref(nb))
        size = nb.value
        if backward:
            self.dq = torch.empty_like(q)
            self.dk1, self.dv1 = torch.empty_like(k1), torch.empty_like(v1)
            self.dk2, self.dv2 = torch.empty_like(k2), torch.empty_like(v2)
            self.ba = _abi.FloydBwdArgs(out=self.out.data_ptr(), dout=0, lse=self.lse.data_ptr(),
                                        dq=self.dq.data_ptr(), dk1=self.dk1.data_ptr(),
                                        dv1=self.dv1.data_ptr(), dk2=self.dk2.data_ptr(),
                                        dv2=self.dv2.data_ptr(), **common)
            self.ba.dout = self.out.data_ptr()          # a placeholder for the size query
            _abi.call(lib.floyd_bwd_workspace_size, ctypes.byref(self.ba), ctypes.byref(nb))
            size = max(size, nb.value)
            self.dout = None
        # one workspace serves both directions
        self.ws = _workspace(size, dev)

    def fwd(self):
        _abi.call(lib.floyd_fwd, ctypes.byref(self.fa), _ptr(self.ws),
                  ctypes.c_size_t(self.ws.numel()), _stream())
        return self.out, self.lse

    def set_out(self, out, lse):
        """Use an externally produced forward output / LSE in the backward."""
        _check(out, "out", self.q.dtype, self.q.shape)
        _check(lse, "lse", torch.float32, self.lse.shape)
        self.ba.out, self.ba.lse = out.data_ptr(), lse.data_ptr()
        self._ext = (out, lse)

    def set_dout(self, dout):
        _check(dout, "dout", self.q.dtype, self.q.shape)
        self.dout = dout
        self.ba.dout = dout.data_ptr()

    def bwd(self, dout=None):
        if dout is not None and dout is not self.dout:
            self.set_dout(dout)
        if self.dout is None:
            raise ValueError("bwd needs dout")
        _abi.call(lib.floyd_bwd, ctypes.byref(self.ba), _ptr(self.ws),
                  ctypes.c_size_t(self.ws.numel()), _stream())
        return self.dq, self.dk1, self.dv1, self.dk2, self.dv2


def floyd_fwd(q, k1, v1, k2, v2, scale=None):
    """FloydAttention forward: returns (out, lse)."""
    return FloydPlan(q, k1, v1, k2, v2, scale, backward=False).fwd()


def floyd_bwd(q, k1, v1, k2, v2, out, dout, lse, scale=None):
    """FloydAttention backward: returns (dq, dk1, dv1, dk2, dv2)."""
    plan = FloydPlan(q, k1, v1, k2, v2, scale, backward=True)
    plan.set_out(out, lse)
    return plan.bwd(dout)
