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


def _tnd_inputs(lens, kv_lens, N1, page, K, seed, dtype="bf16"):
    """TND decode queries: entry b has lens[b] tokens; each selects up to K
    distinct positions of [0, kv_len - lens[b] + s] (rightDownCausal), -1 in
    the slots left over; pages are a random permutation."""
    rng = np.random.default_rng(seed)
    B, T = len(lens), int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pages = [-(-int(n) // page) for n in kv_lens]
    P = sum(pages) + 2
    perm = rng.permutation(P)
    bt = np.zeros((B, max(pages)), np.int32)
    off = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    idx = np.full((T, 1, K), -1, np.int32)
    for b in range(B):
        for s in range(lens[b]):
            hi = int(kv_lens[b]) - lens[b] + s + 1
            n = min(K, hi)
            idx[cu[b] + s, 0, :n] = np.sort(rng.choice(hi, size=n, replace=False))
    q = W.normal((T, N1, 512), seed + 1, dtype)
    qr = W.normal((T, N1, 64), seed + 2, dtype)
    kc = W.normal((P, page, 1, 512), seed + 3, dtype)
    krc = W.normal((P, page, 1, 64), seed + 4, dtype)
    return cu, q, qr, kc, krc, bt, np.asarray(kv_lens, np.int32), idx


@pytest.mark.parametrize("lens,kv_lens,N1,page,K", [
    ([1, 4, 0, 2, 3], [300, 900, 200, 513, 640], 64, 32, 256),   # ragged, an empty entry
    ([2, 1], [130, 4100], 16, 128, 2048),                          # many splits, 16 heads
])
def test_sfa_tnd_ragged_queries(lens, kv_lens, N1, page, K):
    tsa = _tsa()
    cu, q, qr, kc, krc, bt, kvl, idx = _tnd_inputs(lens, kv_lens, N1, page, K, 90)
    scale = 1 / math.sqrt(576)
    d = torch.device("cuda")
    kcd = kc.to(d)
    out, lse = tsa.sfa_paged_fwd(q.to(d), qr.to(d), kcd, krc.to(d), kcd, torch.from_numpy(bt).to(d),
                                 torch.from_numpy(kvl).to(d), torch.from_numpy(idx).to(d), scale,
                                 3, cu_seqlens_q=cu)
    torch.cuda.synchronize()
    ro, rl = oracle.sfa_fwd_tnd(_np(q), _np(qr), _np(kc), _np(krc), _np(kc), bt, kvl, idx, cu,
                                scale, 3)
    o, l = _np(out), _np(lse)
    assert np.isfinite(o).all()
    err, sc = np.abs(o - ro).max(), np.abs(ro).max()
    assert err <= OUT_TOL * sc, f"out: {err:.3e} vs {OUT_TOL} * {sc:.3e}"
    assert np.abs(l - rl).max() <= LSE_TOL * max(1.0, np.abs(rl).max())


def test_sfa_tnd_equal_lengths_is_bsnd_bitwise():
    tsa = _tsa()
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs(B=3, Sq=2, N1=64, page=64, kv_len=1500,
                                                    topk=512, seed_base=95)
    d = torch.device("cuda")
    kcd, krcd = kc.to(d), krc.to(d)
    btd, kvd = torch.from_numpy(bt).to(d), torch.from_numpy(kv_lens).to(d)
    o1, l1 = tsa.sfa_paged_fwd(q.to(d), qr.to(d), kcd, krcd, kcd, btd, kvd,
                               torch.from_numpy(idx).to(d), 0.04, 3)
    cu = np.arange(4, dtype=np.int32) * 2
    o2, l2 = tsa.sfa_paged_fwd(q.reshape(6, 64, 512).to(d), qr.reshape(6, 64, 64).to(d), kcd, krcd,
                               kcd, btd, kvd, torch.from_numpy(idx.reshape(6, 1, -1)).to(d), 0.04,
                               3, cu_seqlens_q=cu)
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(6, 64, 512), o2) and torch.equal(l1.reshape(6, 64), l2)


def test_sfa_unselected_rows_are_never_read():
    """Noise in cache rows that no decode token selects (and in unused pages)
    leaves O and LSE bit-identical."""
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs(B=2, Sq=2, N1=64, page=32, kv_len=640,
                                                    topk=96, seed_base=85, extra_pages=4)
    scale = 1 / math.sqrt(576)
    o1, l1 = _run(q, qr, kc, krc, bt, kv_lens, idx, scale, 3)
    sel = np.zeros(kc.shape[0] * kc.shape[1], bool)
    for b in range(idx.shape[0]):
        ids = idx[b].reshape(-1)
        ids = ids[ids >= 0]
        sel[bt[b][ids // 32] * 32 + ids % 32] = True
    kc2, krc2 = kc.clone(), krc.clone()
    noise = ~torch.from_numpy(sel).reshape(kc.shape[0], kc.shape[1])
    kc2[noise] = (W.normal(tuple(kc.shape), 95) * 50)[noise]
    krc2[noise] = (W.normal(tuple(krc.shape), 94) * 50)[noise]
    o2, l2 = _run(q, qr, kc2, krc2, bt, kv_lens, idx, scale, 3)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------
# A value cache of its own (not the key cache)
# ----------------------------------------------------------------------------

def _run_sepv(q, qr, kc, krc, vc, bt, kv_lens, idx, scale, mode, sbs=1):
    tsa = _tsa()
    d = torch.device("cuda")
    out, lse = tsa.sfa_paged_fwd(q.to(d), qr.to(d), kc.to(d), krc.to(d), vc.to(d),
                                 torch.from_numpy(bt).to(d), torch.from_numpy(kv_lens).to(d),
                                 torch.from_numpy(idx).to(d), scale, mode, sbs)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("N1,page,kv_len,K,mode,sbs,dtype", [
    (64, 16, 200, 40, 3, 1, "bf16"),     # one split, K not a multiple of 32
    (64, 32, 1000, 300, 3, 1, "bf16"),   # several splits
    (16, 16, 64, 64, 0, 1, "fp16"),      # 16 heads (idle waves), no mask
    (128, 64, 700, 100, 3, 1, "bf16"),   # two head groups
    (32, 32, 512, 12, 3, 8, "bf16"),     # sparse blocks of 8 positions
])
def test_sfa_separate_value_cache(N1, page, kv_len, K, mode, sbs, dtype):
    """"aclnnSparseFlashAttention", constraints section: value rows of
    D = 512 of their own; the oracle gathers them from value_cache."""
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs(B=2, Sq=3, N1=N1, page=page, kv_len=kv_len,
                                                    topk=K, seed_base=55, extra_pages=3,
                                                    dtype=dtype)
    vc = W.normal(tuple(kc.shape), 59, dtype)
    if sbs > 1:
        rng = np.random.default_rng(57)
        nblk = kv_len // sbs
        idx = np.stack([np.stack([np.sort(rng.choice(nblk, K, replace=False)) for _ in range(3)])
                        for _ in range(2)])[:, :, None, :].astype(np.int32)
    kv_lens[1] = kv_len - 5
    idx[0, 1, 0, -3:] = -1
    idx[1] = np.where(idx[1] * sbs >= kv_lens[1], -1, idx[1])
    scale = 1 / math.sqrt(576)
    out, lse = _run_sepv(q, qr, kc, krc, vc, bt, kv_lens, idx, scale, mode, sbs)
    ro, rl = oracle.sfa_fwd(_np(q), _np(qr), _np(kc), _np(krc), _np(vc), bt, kv_lens, idx, scale,
                            sparse_mode=mode, sparse_block_size=sbs)
    _check(out, lse, ro, rl)


def test_sfa_separate_value_cache_equal_to_keys_matches_shared():
    """A value cache that holds the key rows (a copy, not the same pointer)
    gives the shared-KV result within rounding of the summation order."""
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs(B=2, Sq=2, N1=64, page=32, kv_len=800,
                                                    topk=200, seed_base=65)
    scale = 1 / math.sqrt(576)
    o1, l1 = _run(q, qr, kc, krc, bt, kv_lens, idx, scale, 3)
    o2, l2 = _run_sepv(q, qr, kc, krc, kc.clone(), bt, kv_lens, idx, scale, 3)
    assert torch.allclose(o1.float(), o2.float(), atol=2e-2, rtol=0)
    assert torch.allclose(l1, l2, atol=1e-4, rtol=0)
