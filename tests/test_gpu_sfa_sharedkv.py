"""Shared-KV two-branch sparse decode on the GPU against the float64 oracle:
a band over the original paged KV plus compressed top-k, one softmax.

Tolerances: output 2e-2 relative to the oracle's max magnitude, LSE
2e-3 * max(1, max|ref|).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-2, 2e-3


def _tsa():
    import top_selected_attention_amd as tsa
    return tsa


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _dev(x):
    return torch.as_tensor(x).cuda()


def _run_case(lens, kv_lens, N1, page, cmp_ratio, K, seed, win_left=127, win_right=0,
              use_ori=True, use_cmp=True, dtype="bf16", tnd=True, rows=None):
    tsa = _tsa()
    cu, q, qr, kvl, ori, cmp = W.sfa_sharedkv_inputs(lens=lens, kv_lens=kv_lens, N1=N1,
                                                     page=page, cmp_ratio=cmp_ratio, cmp_topk=K,
                                                     seed_base=seed, dtype=dtype, extra_pages=2)
    ori_d = tuple(_dev(t) for t in ori) if use_ori else None
    cmp_d = tuple(_dev(t) for t in cmp) if use_cmp else None
    scale = 1 / math.sqrt(576)
    if tnd:
        out, lse = tsa.sfa_sharedkv_fwd(_dev(q), _dev(qr), _dev(kvl), ori_d, cmp_d, scale,
                                        win_left, win_right, cmp_ratio, cu_seqlens_q=cu)
    else:                                    # equal lengths as BSND [B, Sq, ...]
        B, Sq = len(lens), lens[0]
        cmp_b = None
        if use_cmp:
            cmp_b = cmp_d[:3] + (cmp_d[3].reshape(B, Sq, 1, K),)
        out, lse = tsa.sfa_sharedkv_fwd(_dev(q).reshape(B, Sq, N1, 512),
                                        _dev(qr).reshape(B, Sq, N1, 64), _dev(kvl), ori_d, cmp_b,
                                        scale, win_left, win_right, cmp_ratio)
        out, lse = out.reshape(-1, N1, 512), lse.reshape(-1, N1)
    torch.cuda.synchronize()
    # caches as float32 (exact for 16-bit values); the oracle widens the rows it gathers
    f = lambda t: t.float().numpy() if isinstance(t, torch.Tensor) else t  # noqa: E731
    ro, rl = oracle.sfa_sharedkv_fwd(_np(q), _np(qr), cu, kvl, scale,
                                     ori=tuple(f(t) for t in ori) if use_ori else None,
                                     cmp=tuple(f(t) for t in cmp) if use_cmp else None,
                                     win_left=win_left, win_right=win_right, cmp_ratio=cmp_ratio,
                                     tokens=rows)
    o, l = _np(out), _np(lse)
    if rows is not None:
        o, l, ro, rl = o[rows], l[rows], ro[rows], rl[rows]
    assert np.isfinite(o).all()
    err, sc = np.abs(o - ro).max(), np.abs(ro).max()
    assert err <= OUT_TOL * sc, f"out: {err:.3e} vs {OUT_TOL} * {sc:.3e}"
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l)), "LSE: -inf pattern differs"
    if fin.any():
        assert np.abs(l[fin] - rl[fin]).max() <= LSE_TOL * max(1.0, np.abs(rl[fin]).max())
    return out, lse


def test_bsnd_both_branches():
    _run_case([3, 3], [300, 1000], 64, 32, 4, 64, 130, tnd=False)


def test_tnd_ragged_short_sequences():
    # an empty entry; a sequence shorter than the band; one whose compressed
    # length is below its query count (its first tokens see no compressed id)
    _run_case([1, 4, 0, 2, 3], [50, 900, 100, 513, 6], 64, 32, 4, 96, 140)


def test_band_only():
    _run_case([2, 3], [200, 700], 64, 64, 4, 32, 150, use_cmp=False)


def test_compressed_only_ratio_128():
    _run_case([2, 2], [70000, 33000], 64, 128, 128, 512, 160, use_ori=False)


def test_band_with_future_tokens_fp16_16_heads():
    # win_right > 0: keys past the token's position, up to the sequence end
    _run_case([4, 1], [300, 90], 16, 16, 4, 40, 170, win_left=31, win_right=8, dtype="fp16")


def test_deterministic_bitwise():
    a = _run_case([4, 4], [4000, 2500], 64, 64, 4, 512, 180)
    b = _run_case([4, 4], [4000, 2500], 64, 64, 4, 512, 180)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_workload_full_size_sampled():
    """The full decode batch (32 entries x 4 tokens, 64 heads, KV 65536 with
    a 128-token band, compressed 4x with 512 selected entries) in the timed
    configuration; a sample of tokens is checked."""
    w = W.sfa_sharedkv_workload()
    rows = [0, 3, 29, 64, 101, 127]
    _run_case([w["Sq"]] * w["B"], [w["kv_len"]] * w["B"], w["N1"], w["page"], w["cmp_ratio"],
              w["cmp_topk"], 120, rows=rows)


def test_task_list_made_once_serves_other_ids():
    """A task list made by the metadata call for one set of compressed ids
    serves a forward over other ids (another layer of the decode step): the
    result matches the oracle for the new ids, and a fresh list gives the
    same bits as the list made inside the forward."""
    tsa = _tsa()
    lens, kv_lens, N1, K = [1, 4, 0, 3], [900, 4000, 70, 2600], 64, 128
    cu, q, qr, kvl, ori, cmp = W.sfa_sharedkv_inputs(lens=lens, kv_lens=kv_lens, N1=N1, page=64,
                                                     cmp_ratio=4, cmp_topk=K, seed_base=190)
    _, _, _, _, _, cmp2 = W.sfa_sharedkv_inputs(lens=lens, kv_lens=kv_lens, N1=N1, page=64,
                                                cmp_ratio=4, cmp_topk=K, seed_base=200)
    ori_d = tuple(_dev(t) for t in ori)
    cmp_d = tuple(_dev(t) for t in cmp)
    plan = tsa.SfaSharedkvPlan(_dev(q), _dev(qr), _dev(kvl), ori_d, cmp_d, 0.04,
                               cu_seqlens_q=cu)
    inline, _ = plan.fwd()
    inline = inline.clone()
    plan.metadata()
    listed, _ = plan.fwd()
    torch.cuda.synchronize()
    assert torch.equal(inline, listed)
    # the other layer's ids, copied into the same id tensor the plan points at
    cmp_d[3].copy_(_dev(cmp2[3]))
    out, lse = plan.fwd()
    torch.cuda.synchronize()
    f = lambda t: t.float().numpy() if isinstance(t, torch.Tensor) else t  # noqa: E731
    ro, rl = oracle.sfa_sharedkv_fwd(_np(q), _np(qr), cu, kvl, 0.04, ori=tuple(f(t) for t in ori),
                                     cmp=tuple(f(t) for t in cmp[:3]) + (cmp2[3],))
    err, sc = np.abs(_np(out) - ro).max(), np.abs(ro).max()
    assert err <= OUT_TOL * sc, f"out: {err:.3e} vs {OUT_TOL} * {sc:.3e}"
    assert np.abs(_np(lse) - rl).max() <= LSE_TOL * max(1.0, np.abs(rl).max())


def test_tokens_before_the_sequence_start_see_nothing():
    """More decode tokens than original KV rows: tokens whose position
    kv_len - Sq_b + s is negative have no band rows and no compressed ids, and
    get Out = 0 and LSE = -inf; the later ones see their short band."""
    out, lse = _run_case([5, 2], [3, 300], 64, 16, 4, 8, 210)
    assert torch.all(out[:2] == 0) and torch.all(torch.isneginf(lse[:2]))
    assert torch.isfinite(lse[2:]).all()


@pytest.mark.parametrize("N1", [1, 2, 128])
def test_head_count_limits(N1):
    """N1 from 1 (one partly used head group) to 128 (two head groups)."""
    _run_case([2, 3], [500, 2000], N1, 64, 4, 64, 220 + N1)


def test_no_tokens_at_all():
    """Every entry without decode tokens: the calls launch nothing and return
    empty outputs."""
    tsa = _tsa()
    cu, q, qr, kvl, ori, cmp = W.sfa_sharedkv_inputs(lens=[0, 0], kv_lens=[100, 300], N1=64,
                                                     page=32, cmp_ratio=4, cmp_topk=16,
                                                     seed_base=260)
    out, lse = tsa.sfa_sharedkv_fwd(_dev(q), _dev(qr), _dev(kvl), tuple(_dev(t) for t in ori),
                                    tuple(_dev(t) for t in cmp), 0.04, cu_seqlens_q=cu)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 64, 512) and tuple(lse.shape) == (0, 64)
