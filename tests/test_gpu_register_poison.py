"""Every attention kernel launched right after every SIMD's registers were
filled with +inf or NaN bits (the peaks library's tsa_fill_registers): a
kernel that reads a register it never wrote would turn such leftovers into
wrong results, which the oracle comparison shows.  Where a call first builds
lists, the lists are built beforehand and the call reuses them, so that the
attention kernel is the first launch after the fill."""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

PATTERNS = [0x7F800000, 0xFFC00000]   # +inf, a quiet NaN
OUT_TOL, GRAD_TOL = 2e-2, 3e-2


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _close(gpu, ref, tol, what):
    g = _np(gpu) if isinstance(gpu, torch.Tensor) else gpu
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    err, sc = np.abs(g - ref).max(), np.abs(ref).max()
    assert err <= tol * max(sc, 1e-30), f"{what}: max err {err:.3e} vs {tol} * {sc:.3e}"


def _fill(pattern):
    from top_selected_attention_amd import peaks
    peaks.fill_registers(pattern)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("pattern", PATTERNS)
def test_bsa_after_register_fill(pattern):
    import top_selected_attention_amd as tsa
    rng = np.random.default_rng(700)
    B, N1, N2, S, bq = 1, 4, 2, 384, 64
    q, k, v, do = (W.normal((B, n, S, 128), 701 + i, "bf16")
                   for i, n in enumerate((N1, N2, N2, N1)))
    mask = W.mask_random(rng, B, N1, S // bq, S // bq, 0.5, causal=True)
    am = (rng.random((S, S)) < 0.2).astype(np.uint8)
    np.fill_diagonal(am, 0)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    plan = tsa.BsaPlan(qd, kd, vd, torch.from_numpy(mask).cuda(), bq, bq, 0.088, 2,
                       atten_mask=torch.from_numpy(am).cuda())
    plan.set_dout(dod)                # sizes the shared workspace for the backward first
    plan.fwd()                        # lists into that workspace
    _fill(pattern)
    plan.fa.reuse_lists = 1
    tsa._abi.call(tsa.lib.bsa_fwd, ctypes.byref(plan.fa), ctypes.c_void_p(plan.ws_fwd.data_ptr()),
                  ctypes.c_size_t(plan.ws_fwd.numel()), _stream())
    torch.cuda.synchronize()
    qn, kn, vn, don = _np(q), _np(k), _np(v), _np(do)
    ro, rl = oracle.bsa_fwd(qn, kn, vn, mask, bq, bq, 0.088, 2, atten_mask=am)
    _close(plan.out, ro, OUT_TOL, "out")
    _fill(pattern)
    dq, dk, dv = plan.bwd()
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.bsa_bwd(qn, kn, vn, _np(plan.out), don, mask, bq, bq, 0.088, 2,
                                   atten_mask=am)
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        _close(g, r, GRAD_TOL, name)


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("N1,N2", [(32, 2), (64, 2)])        # the 16- and 32-head kernels
def test_nsa_after_register_fill(pattern, N1, N2):
    import top_selected_attention_amd as tsa
    cu, q, k, v, do, topk = W.nsa_inputs([256, 320], N1=N1, N2=N2, sbs=64, sbc=4, seed_base=710)
    dev = torch.device("cuda")
    plan = tsa.NsaPlan(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(topk).to(dev), cu, cu,
                       64, 0.088, 2)
    plan.fwd()
    plan.bwd(do.to(dev))              # builds the reverse lists too
    _fill(pattern)
    plan.fa.reuse_lists = 1
    tsa._abi.call(tsa.lib.nsa_select_fwd, ctypes.byref(plan.fa),
                  ctypes.c_void_p(plan.ws_fwd.data_ptr()), ctypes.c_size_t(plan.ws_fwd.numel()),
                  _stream())
    torch.cuda.synchronize()
    qn, kn, vn, don = _np(q), _np(k), _np(v), _np(do)
    ro, _ = oracle.nsa_fwd(qn, kn, vn, topk, cu, cu, 64, 0.088, 2)
    _close(plan.out, ro, OUT_TOL, "out")
    _fill(pattern)
    plan.ba.reuse_lists = 1
    tsa._abi.call(tsa.lib.nsa_select_bwd, ctypes.byref(plan.ba),
                  ctypes.c_void_p(plan.ws_bwd.data_ptr()), ctypes.c_size_t(plan.ws_bwd.numel()),
                  _stream())
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.nsa_bwd(qn, kn, vn, _np(plan.out), don, topk, cu, cu, 64, 0.088, 2)
    for name, g, r in (("dq", plan.dq, rdq), ("dk", plan.dk, rdk), ("dv", plan.dv, rdv)):
        _close(g, r, GRAD_TOL, name)


@pytest.mark.parametrize("pattern", PATTERNS)
def test_sfa_after_register_fill(pattern):
    import top_selected_attention_amd as tsa
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs(B=2, Sq=3, N1=64, page=32, kv_len=1000,
                                                    topk=300, seed_base=50, extra_pages=3)
    scale = 1 / math.sqrt(576)
    d = torch.device("cuda")
    kcd = kc.to(d)
    plan = tsa.SfaPlan(q.to(d), qr.to(d), kcd, krc.to(d), kcd, torch.from_numpy(bt).to(d),
                       torch.from_numpy(kv_lens).to(d), torch.from_numpy(idx).to(d), scale, 3)
    _fill(pattern)
    out, lse = plan.fwd()
    torch.cuda.synchronize()
    ro, _ = oracle.sfa_fwd(_np(q), _np(qr), _np(kc), _np(krc), _np(kc), bt, kv_lens, idx, scale,
                           sparse_mode=3)
    _close(out, ro, OUT_TOL, "out")


@pytest.mark.parametrize("pattern", PATTERNS)
def test_sfa_sharedkv_after_register_fill(pattern):
    import top_selected_attention_amd as tsa
    cu, q, qr, kvl, ori, cmp = W.sfa_sharedkv_inputs(lens=[3, 1, 2], kv_lens=[700, 2000, 300],
                                                     N1=64, page=64, cmp_ratio=4, cmp_topk=96,
                                                     seed_base=720)
    dev = lambda t: torch.as_tensor(t).cuda()  # noqa: E731
    plan = tsa.SfaSharedkvPlan(dev(q), dev(qr), dev(kvl), tuple(dev(t) for t in ori),
                               tuple(dev(t) for t in cmp), 0.04, cu_seqlens_q=cu)
    plan.metadata()
    _fill(pattern)
    out, _ = plan.fwd()
    torch.cuda.synchronize()
    f = lambda t: t.float().numpy() if isinstance(t, torch.Tensor) else t  # noqa: E731
    ro, _ = oracle.sfa_sharedkv_fwd(_np(q), _np(qr), cu, kvl, 0.04, ori=tuple(f(t) for t in ori),
                                    cmp=tuple(f(t) for t in cmp))
    _close(out, ro, OUT_TOL, "out")
