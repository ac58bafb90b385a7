"""Paged sparse flash attention (decode) on the GPU against the float64 oracle.

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


def _run(q, qr, kc, krc, bt, kv_lens, idx, scale, mode, sbs=1, validate=False):
    tsa = _tsa()
    d = torch.device("cuda")
    kcd = kc.to(d)
    out, lse = tsa.sfa_paged_fwd(q.to(d), qr.to(d), kcd, krc.to(d), kcd,
                                 torch.from_numpy(bt).to(d), torch.from_numpy(kv_lens).to(d),
                                 torch.from_numpy(idx).to(d), scale, mode, sbs, validate)
    torch.cuda.synchronize()
    return out, lse


def _check(out, lse, ro, rl, rows=None):
    o, l = _np(out), _np(lse)
    if rows is not None:
        o = np.stack([o[b, s] for b, s in rows])
        l = np.stack([l[b, s] for b, s in rows])
        ro = np.stack([ro[b, s] for b, s in rows])
        rl = np.stack([rl[b, s] for b, s in rows])
    assert np.isfinite(o).all()
    err, sc = np.abs(o - ro).max(), np.abs(ro).max()
    assert err <= OUT_TOL * sc, f"out: {err:.3e} vs {OUT_TOL} * {sc:.3e}"
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.abs(l[fin] - rl[fin]).max() <= LSE_TOL * max(1.0, np.abs(rl[fin]).max())


@pytest.mark.parametrize("N1,page,kv_len,K,mode", [
    (64, 16, 200, 40, 3),        # one split, K not a multiple of 32
    (64, 32, 1000, 300, 3),      # several splits
    (16, 16, 64, 64, 0),         # 16 heads (idle waves), no mask, every key selected
    (128, 64, 700, 100, 3),      # two head groups
])
def test_sfa_small(N1, page, kv_len, K, mode):
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs(B=2, Sq=3, N1=N1, page=page, kv_len=kv_len,
                                                    topk=K, seed_base=50, extra_pages=3)
    kv_lens[1] = kv_len - 5                      # a shorter sequence
    idx[0, 1, 0, -7:] = -1                       # empty slots
    idx[1] = np.where(idx[1] >= kv_lens[1], -1, idx[1])
    scale = 1 / math.sqrt(576)
    out, lse = _run(q, qr, kc, krc, bt, kv_lens, idx, scale, mode)
    ro, rl = oracle.sfa_fwd(_np(q), _np(qr), _np(kc), _np(krc), _np(kc), bt, kv_lens, idx, scale,
                            sparse_mode=mode)
    _check(out, lse, ro, rl)


def test_sfa_sparse_blocks_and_fp16():
    rng = np.random.default_rng(5)
    B, Sq, N1, page, kv_len, sbs = 2, 2, 64, 32, 512, 8
    q, qr, kc, krc, bt, kv_lens, _ = W.sfa_inputs(B=B, Sq=Sq, N1=N1, page=page, kv_len=kv_len,
                                                  topk=8, seed_base=60, dtype="fp16")
    nblk = kv_len // sbs
    idx = np.stack([np.stack([np.sort(rng.choice(nblk, 20, replace=False))
                              for _ in range(Sq)]) for _ in range(B)])[:, :, None, :]
    idx = idx.astype(np.int32)
    out, lse = _run(q, qr, kc, krc, bt, kv_lens, idx, 0.05, 3, sbs=sbs)
    ro, rl = oracle.sfa_fwd(_np(q), _np(qr), _np(kc), _np(krc), _np(kc), bt, kv_lens, idx, 0.05,
                            sparse_mode=3, sparse_block_size=sbs)
    _check(out, lse, ro, rl)


def test_sfa_decode_full_size_sampled():
    """The full 32 x 4 decode batch (64 heads, 2048 of 65536 keys, page 128)
    in the timed configuration; a sample of decode tokens is checked."""
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs()
    scale = 1 / math.sqrt(576)
    out, lse = _run(q, qr, kc, krc, bt, kv_lens, idx, scale, 3)
    rows = [(0, 0), (0, 3), (7, 1), (15, 2), (31, 3), (20, 0)]
    ro, rl = oracle.sfa_fwd(_np(q), _np(qr), kc.float().numpy(), krc.float().numpy(),
                            kc.float().numpy(), bt, kv_lens, idx, scale, sparse_mode=3,
                            tokens=rows)
    _check(out, lse, ro, rl, rows=rows)


def test_sfa_validate_reports_bad_ids():
    tsa = _tsa()
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs(B=1, Sq=2, N1=64, page=16, kv_len=128,
                                                    topk=16, seed_base=70)
    idx[0, 1, 0, 3] = 500
    with pytest.raises(tsa.TsaError) as ei:
        _run(q, qr, kc, krc, bt, kv_lens, idx, 0.04, 3, validate=True)
    assert ei.value.status == 6
