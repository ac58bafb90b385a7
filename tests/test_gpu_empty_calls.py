"""Calls with no query rows or tokens, through the C ABI on the GPU.

A forward with no query rows must leave lists that a backward reusing the
workspace can read (here the workspace starts filled with 0xFF bytes, so a
list the forward did not write would send the dK/dV kernels to garbage
rows), and a backward with no rows must not trust lists it never wrote.
Every call with no work records the stage events it was asked for.
"""

import ctypes

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _tsa():
    import top_selected_attention_amd as tsa
    return tsa


def _ws(lib, size_fn, args):
    nb = ctypes.c_size_t()
    _tsa()._abi.call(size_fn, ctypes.byref(args), ctypes.byref(nb))
    return torch.full((max(nb.value, 1),), 0xFF, dtype=torch.uint8, device="cuda")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    return evs, (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])


def _all_recorded(evs):
    torch.cuda.synchronize()
    for i in range(0, len(evs), 2):
        assert evs[i].elapsed_time(evs[i + 1]) >= 0.0


@pytest.mark.parametrize("layout", ["bnsd", "tnd"])
def test_bsa_zero_query_rows_then_reusing_backward_gives_zero_dk_dv(layout):
    tsa = _tsa()
    A = tsa._abi
    B, N1, N2, Skv, bq, bkv = 2, 4, 2, 256, 64, 64
    dev = "cuda"
    if layout == "bnsd":
        Sq = 0
        q = torch.empty((B, N1, 0, 128), dtype=torch.bfloat16, device=dev)
        k = W.normal((B, N2, Skv, 128), 11, "bf16").to(dev)
        v = W.normal((B, N2, Skv, 128), 12, "bf16").to(dev)
        seq, lay = {}, A.LAYOUT_BNSD
    else:
        # every query sequence is empty, the longest-length arguments are not
        Sq = 128
        cu_q = torch.zeros(B + 1, dtype=torch.int32)
        cu_k = torch.tensor([0, Skv, 2 * Skv], dtype=torch.int32)
        q = torch.empty((0, N1, 128), dtype=torch.bfloat16, device=dev)
        k = W.normal((2 * Skv, N2, 128), 11, "bf16").to(dev)
        v = W.normal((2 * Skv, N2, 128), 12, "bf16").to(dev)
        P = ctypes.POINTER(ctypes.c_int32)
        seq = dict(cu_seqlens_q=ctypes.cast(cu_q.data_ptr(), P),
                   cu_seqlens_kv=ctypes.cast(cu_k.data_ptr(), P))
        lay = A.LAYOUT_TND
    QB, KB = -(-Sq // bq), -(-Skv // bkv)
    mask = torch.ones((B, N1, QB, KB), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1] if layout == "tnd" else (B, N1, Sq), dtype=torch.float32,
                      device=dev)
    dk, dv = torch.full_like(k, 7.0), torch.full_like(v, 7.0)
    dq, dout = torch.empty_like(q), torch.empty_like(q)
    common = dict(dtype=0, q_layout=lay, kv_layout=lay, B=B, N1=N1, N2=N2, Sq=Sq, Skv=Skv, D=128,
                  block_q=bq, block_kv=bkv, sparse_mode=0, scale=0.088, validate=0,
                  block_mask=mask.data_ptr(), q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(),
                  **seq)
    ba = A.BsaBwdArgs(out=out.data_ptr(), dout=dout.data_ptr(), lse=lse.data_ptr(),
                      dq=dq.data_ptr(), dk=dk.data_ptr(), dv=dv.data_ptr(), **common)
    ws = _ws(tsa.lib, tsa.lib.bsa_bwd_workspace_size, ba)
    evs, arr = _events(2)
    fa = A.BsaFwdArgs(out=out.data_ptr(), lse=lse.data_ptr(), **common)
    fa.n_events, fa.events = 2, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    A.call(tsa.lib.bsa_fwd, ctypes.byref(fa), ctypes.c_void_p(ws.data_ptr()),
           ctypes.c_size_t(ws.numel()), _stream())
    _all_recorded(evs)
    ba.reuse_lists = 1
    A.call(tsa.lib.bsa_bwd, ctypes.byref(ba), ctypes.c_void_p(ws.data_ptr()),
           ctypes.c_size_t(ws.numel()), _stream())
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


def test_bsa_backward_with_zero_rows_ignores_stale_lists():
    """A reusing backward on a workspace that no forward touched: with no
    query rows it writes its own empty lists."""
    tsa = _tsa()
    A = tsa._abi
    B, N1, N2, Skv = 1, 2, 1, 192
    q = torch.empty((B, N1, 0, 128), dtype=torch.float16, device="cuda")
    k = W.normal((B, N2, Skv, 128), 21, "fp16").cuda()
    v = W.normal((B, N2, Skv, 128), 22, "fp16").cuda()
    dk, dv = torch.full_like(k, 3.0), torch.full_like(v, 3.0)
    lse = torch.empty((B, N1, 0), dtype=torch.float32, device="cuda")
    ba = A.BsaBwdArgs(dtype=1, q_layout=0, kv_layout=0, B=B, N1=N1, N2=N2, Sq=0, Skv=Skv, D=128,
                      block_q=128, block_kv=64, sparse_mode=2, scale=0.088, validate=0,
                      block_mask=0, q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(),
                      out=q.data_ptr(), dout=q.data_ptr(), lse=lse.data_ptr(), dq=q.data_ptr(),
                      dk=dk.data_ptr(), dv=dv.data_ptr())
    ws = _ws(tsa.lib, tsa.lib.bsa_bwd_workspace_size, ba)
    evs, arr = _events(4)
    ba.reuse_lists, ba.n_events, ba.events = 1, 4, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    A.call(tsa.lib.bsa_bwd, ctypes.byref(ba), ctypes.c_void_p(ws.data_ptr()),
           ctypes.c_size_t(ws.numel()), _stream())
    _all_recorded(evs)
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


def test_nsa_zero_tokens_then_reusing_backward_gives_zero_dk_dv():
    tsa = _tsa()
    A = tsa._abi
    N1, N2, sbs, sbc = 4, 2, 64, 16
    cu_q = torch.zeros(3, dtype=torch.int32)
    cu_k = torch.tensor([0, 1024, 3072], dtype=torch.int32)
    Tk = 3072
    q = torch.empty((0, N1, 128), dtype=torch.bfloat16, device="cuda")
    k = W.normal((Tk, N2, 128), 31, "bf16").cuda()
    v = W.normal((Tk, N2, 128), 32, "bf16").cuda()
    topk = torch.empty((0, N2, sbc), dtype=torch.int32, device="cuda")
    lse = torch.empty((0, N1), dtype=torch.float32, device="cuda")
    dk, dv = torch.full_like(k, 5.0), torch.full_like(v, 5.0)
    P = ctypes.POINTER(ctypes.c_int32)
    common = dict(dtype=0, layout=1, B=2, T=0, Tk=Tk, N1=N1, N2=N2, D=128, Dv=128,
                  cu_seqlens_q=ctypes.cast(cu_q.data_ptr(), P),
                  cu_seqlens_kv=ctypes.cast(cu_k.data_ptr(), P), sbs=sbs, sbc=sbc,
                  sparse_mode=2, scale=0.088, validate=0, topk=topk.data_ptr(), q=q.data_ptr(),
                  k=k.data_ptr(), v=v.data_ptr())
    ba = A.NsaBwdArgs(out=q.data_ptr(), dout=q.data_ptr(), lse=lse.data_ptr(), dq=q.data_ptr(),
                      dk=dk.data_ptr(), dv=dv.data_ptr(), **common)
    ws = _ws(tsa.lib, tsa.lib.nsa_select_bwd_workspace_size, ba)
    evs, arr = _events(2)
    fa = A.NsaFwdArgs(out=q.data_ptr(), lse=lse.data_ptr(), **common)
    fa.n_events, fa.events = 2, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    A.call(tsa.lib.nsa_select_fwd, ctypes.byref(fa), ctypes.c_void_p(ws.data_ptr()),
           ctypes.c_size_t(ws.numel()), _stream())
    _all_recorded(evs)
    for reuse in (2, 1):
        ws.fill_(0xFF)
        dk.fill_(5.0), dv.fill_(5.0)
        ba.reuse_lists = reuse
        A.call(tsa.lib.nsa_select_bwd, ctypes.byref(ba), ctypes.c_void_p(ws.data_ptr()),
               ctypes.c_size_t(ws.numel()), _stream())
        torch.cuda.synchronize()
        assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


def test_sfa_zero_tokens_records_its_events():
    tsa = _tsa()
    A = tsa._abi
    z = torch.empty((0, 4, 1, 512), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((2, 16, 1, 512), dtype=torch.bfloat16, device="cuda")
    krc = torch.zeros((2, 16, 1, 64), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    a = A.SfaArgs(dtype=0, q_layout=2, B=0, Sq=4, N1=4, N2=1, D=512, Dr=64, Dv=512,
                  num_pages=2, page_size=16, max_pages=2, topk=8, sparse_block_size=1,
                  sparse_mode=3, scale=0.04, validate=0, q=z.data_ptr(), q_rope=z.data_ptr(),
                  key_cache=kc.data_ptr(), key_rope_cache=krc.data_ptr(),
                  value_cache=kc.data_ptr(), block_table=bt.data_ptr(), kv_lens=bt.data_ptr(),
                  topk_indices=bt.data_ptr(), out=z.data_ptr(), lse=0)
    ws = _ws(tsa.lib, tsa.lib.sfa_paged_fwd_workspace_size, a)
    evs, arr = _events(2)
    a.n_events, a.events = 2, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    A.call(tsa.lib.sfa_paged_fwd, ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()),
           ctypes.c_size_t(ws.numel()), _stream())
    _all_recorded(evs)


def test_sfa_sharedkv_zero_tokens_records_its_events():
    tsa = _tsa()
    x = W.sfa_sharedkv_inputs(lens=[0, 0], kv_lens=[256, 128], N1=4, page=16, cmp_topk=8,
                              seed_base=170)
    cu, q, qr, kvl, ori, cmp = x
    plan = tsa.SfaSharedkvPlan(q.cuda(), qr.cuda(), torch.as_tensor(kvl).cuda(),
                               ori=tuple(torch.as_tensor(t).cuda() for t in ori),
                               cmp=tuple(torch.as_tensor(t).cuda() for t in cmp),
                               cu_seqlens_q=cu)
    evs, arr = _events(3)
    plan.a.n_events, plan.a.events = 3, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    plan.fwd()
    _all_recorded(evs)
    assert plan.out.numel() == 0
