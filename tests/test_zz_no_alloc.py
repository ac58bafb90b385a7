"""sfa_paged_fwd_noalloc: the paged sparse decode with the library's fixed
per-GPU scratch instead of a caller workspace, checked through the C ABI
against sfa_paged_fwd on the same inputs (two calls in a row, the second
with a smaller input), and its size limit (on the CPU: the check runs before
any launch)."""

import ctypes

import pytest
import torch

import workloads as W


def _tsa():
    import top_selected_attention_amd as tsa
    return tsa


def _plan(B, Sq, N1, kv_len, topk, page, seed):
    tsa = _tsa()
    q, qr, kc, krc, bt, kvl, idx = W.sfa_inputs(B=B, Sq=Sq, N1=N1, page=page, kv_len=kv_len,
                                                topk=topk, seed_base=seed)
    d = torch.device("cuda", 0)
    kcd = kc.to(d)
    return tsa.SfaPlan(q.to(d), qr.to(d), kcd, krc.to(d), kcd, torch.from_numpy(bt).to(d),
                       torch.from_numpy(kvl).to(d), torch.from_numpy(idx).to(d), None, 3)


def _noalloc_equals_workspace_call(plan):
    tsa = _tsa()
    ref_out, ref_lse = (t.clone() for t in plan.fwd())
    out, lse = torch.full_like(plan.out, float("nan")), torch.full_like(plan.lse, float("nan"))
    a = tsa._abi.SfaArgs.from_buffer_copy(plan.a)
    a.out, a.lse = out.data_ptr(), lse.data_ptr()
    tsa._abi.call(tsa.lib.sfa_paged_fwd_noalloc, ctypes.byref(a),
                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(lse, ref_lse)


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    tsa = _tsa()
    # 32 decode tokens of 64 heads over 8 splits: 33.6 MB of scratch
    big = _plan(B=8, Sq=4, N1=64, kv_len=8192, topk=2048, page=128, seed=190)
    nb = ctypes.c_size_t()
    tsa._abi.call(tsa.lib.sfa_paged_fwd_workspace_size, ctypes.byref(big.a), ctypes.byref(nb))
    assert 32 << 20 < nb.value <= tsa.lib.sfa_paged_fwd_noalloc_max_bytes()
    _noalloc_equals_workspace_call(big)
    # then a smaller call: the scratch still holds the first call's partials
    small = _plan(B=2, Sq=2, N1=16, kv_len=1000, topk=300, page=64, seed=200)
    _noalloc_equals_workspace_call(small)
    # and the first shape again, through the plan's own method
    o1 = big.fwd()[0].clone()
    o2 = big.fwd_noalloc()[0]
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_noalloc_refuses_a_call_beyond_its_scratch():
    """256 decode tokens of 128 heads (one split each) need 64 MiB of partial
    outputs plus their LSEs: more than the fixed scratch, refused before any
    launch (so the device pointers are never touched)."""
    tsa = _tsa()
    A = tsa._abi
    fake = 1 << 20
    a = A.SfaArgs(dtype=0, q_layout=2, B=64, Sq=4, N1=128, N2=1, D=512, Dr=64, Dv=512,
                  num_pages=32768, page_size=128, max_pages=512, topk=2048, sparse_block_size=1,
                  sparse_mode=3, scale=0.04, validate=0, q=fake, q_rope=fake, key_cache=fake,
                  key_rope_cache=fake, value_cache=fake, block_table=fake, kv_lens=fake,
                  topk_indices=fake, out=fake, lse=fake)
    nb = ctypes.c_size_t()
    A.call(tsa.lib.sfa_paged_fwd_workspace_size, ctypes.byref(a), ctypes.byref(nb))
    assert nb.value > tsa.lib.sfa_paged_fwd_noalloc_max_bytes() == 64 << 20
    assert tsa.lib.sfa_paged_fwd_noalloc(ctypes.byref(a), None) == 7
    assert tsa.lib.tsa_status_string(7).decode().startswith("the call needs more scratch")
