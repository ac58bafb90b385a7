"""Pins of the CPU oracle against facts fixed independently of it.

Every test here runs on the CPU.  None re-types the oracle's formulas: each
compares it with an independent computation (PyTorch autograd through a dense
attention, central finite differences, brute-force loops, closed forms) or
checks an invariant the mathematics fixes.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _dense_torch(q, k, v, scale, causal, G):
    """Independent dense attention: torch CPU float64 with autograd.
    q [N1, S, D], k/v [N2, S, D] (one batch)."""
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    kr = kt.repeat_interleave(G, dim=0)
    vr = vt.repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kr[None], vr[None], is_causal=causal, scale=scale)[0]
    return qt, kt, vt, out


# ----------------------------------------------------------------------------
# Dense special case: every block selected == textbook attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N1,N2", [(2, 2), (4, 2)])
def test_bsa_all_blocks_equals_dense_attention(causal, N1, N2):
    r = _rng(1)
    S, D, bq, bkv = 40, 16, 8, 8          # ragged: 40 = 5 blocks of 8
    q = r.standard_normal((1, N1, S, D))
    k = r.standard_normal((1, N2, S, D))
    v = r.standard_normal((1, N2, S, D))
    do = r.standard_normal((1, N1, S, D))
    scale = 1 / math.sqrt(D)
    mask = np.ones((1, N1, 5, 5), np.uint8)
    out, lse = oracle.bsa_fwd(q, k, v, mask, bq, bkv, scale, 2 if causal else 0)
    qt, kt, vt, ref = _dense_torch(q[0], k[0], v[0], scale, causal, N1 // N2)
    np.testing.assert_allclose(out[0], ref.detach().numpy(), rtol=0, atol=1e-12)
    # LSE against torch.logsumexp over the dense scores
    s = scale * torch.tensor(q[0]) @ torch.tensor(k[0]).repeat_interleave(N1 // N2, 0).transpose(1, 2)
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse[0], torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)
    # gradients against autograd
    ref.backward(torch.tensor(do[0]))
    dq, dk, dv = oracle.bsa_bwd(q, k, v, out, do, mask, bq, bkv, scale, 2 if causal else 0)
    for mine, theirs in ((dq[0], qt.grad), (dk[0], kt.grad), (dv[0], vt.grad)):
        t = theirs.numpy()
        assert np.abs(mine - t).max() <= 1e-10 * np.abs(t).max()


@pytest.mark.parametrize("D,Dv", [(8, 8), (12, 8)])
def test_nsa_all_blocks_equals_dense_attention(D, Dv):
    """Every block selected is dense causal attention (torch, autograd),
    with value heads as wide as or narrower than the query/key heads."""
    r = _rng(2)
    seqlens, N1, N2, sbs = [16, 24], 4, 2, 4
    cu = np.array([0, 16, 40])
    T = 40
    q, k, v = r.standard_normal((T, N1, D)), r.standard_normal((T, N2, D)), r.standard_normal((T, N2, Dv))
    do = r.standard_normal((T, N1, Dv))
    scale = 0.3
    # every token selects every block of its sequence (sbc = blocks of the longest; the
    # shorter sequence lists its 4 blocks; use one topk width per call -> two calls)
    for b, S in enumerate(seqlens):
        sl = slice(cu[b], cu[b + 1])
        nb = S // sbs
        topk = np.tile(r.permutation(nb), (S, N2, 1)).astype(np.int32)
        cu1 = np.array([0, S])
        out, lse = oracle.nsa_fwd(q[sl], k[sl], v[sl], topk, cu1, cu1, sbs, scale, 2)
        qt, kt, vt, ref = _dense_torch(q[sl].transpose(1, 0, 2), k[sl].transpose(1, 0, 2),
                                       v[sl].transpose(1, 0, 2), scale, True, N1 // N2)
        np.testing.assert_allclose(out, ref.detach().numpy().transpose(1, 0, 2), atol=1e-12, rtol=0)
        ref.backward(torch.tensor(do[sl].transpose(1, 0, 2)))
        dq, dk, dv = oracle.nsa_bwd(q[sl], k[sl], v[sl], out, do[sl], topk, cu1, cu1, sbs, scale, 2)
        for mine, theirs in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
            t = theirs.numpy().transpose(1, 0, 2)
            assert np.abs(mine - t).max() <= 1e-10 * np.abs(t).max()


def test_sfa_identity_pages_all_tokens_equals_dense_mqa():
    r = _rng(3)
    B, Sq, N1, D, Dr, page, kv_len = 2, 3, 4, 16, 8, 8, 24
    q, qr = r.standard_normal((B, Sq, N1, D)), r.standard_normal((B, Sq, N1, Dr))
    P = B * kv_len // page
    kc, krc = r.standard_normal((P, page, 1, D)), r.standard_normal((P, page, 1, Dr))
    bt = np.arange(P).reshape(B, kv_len // page)
    kv_lens = np.full(B, kv_len)
    topk = np.tile(np.arange(kv_len), (B, Sq, 1, 1))
    scale = 1 / math.sqrt(D + Dr)
    out, lse = oracle.sfa_fwd(q, qr, kc, krc, kc, bt, kv_lens, topk, scale, sparse_mode=3)
    for b in range(B):
        keys = kc[bt[b]].reshape(kv_len, D)
        kro = krc[bt[b]].reshape(kv_len, Dr)
        qcat = torch.tensor(np.concatenate([q[b], qr[b]], -1)).transpose(0, 1)   # [N1, Sq, D+Dr]
        kcat = torch.tensor(np.concatenate([keys, kro], -1))[None].expand(N1, -1, -1)
        vals = torch.tensor(keys)[None].expand(N1, -1, -1)
        # rightDownCausal: query s at position kv_len - Sq + s
        allowed = torch.arange(kv_len)[None, :] <= (kv_len - Sq + torch.arange(Sq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qcat, kcat, vals, attn_mask=allowed,
                                                               scale=scale)
        np.testing.assert_allclose(out[b], ref.numpy().transpose(1, 0, 2), atol=1e-12, rtol=0)


def test_sfa_tnd_ragged_queries_equal_dense_mqa_per_sequence():
    """TND queries (1, 3 and 2 decode tokens per sequence), every position
    selected: each sequence is dense MQA with its own rightDownCausal offset
    kv_len - Sq_b (torch, float64)."""
    r = _rng(31)
    lens, N1, D, Dr, page = [1, 3, 2], 4, 16, 8, 8
    kv_lens = np.array([24, 16, 20])
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, qr = r.standard_normal((T, N1, D)), r.standard_normal((T, N1, Dr))
    pages = [-(-int(n) // page) for n in kv_lens]
    P = sum(pages)
    kc, krc = r.standard_normal((P, page, 1, D)), r.standard_normal((P, page, 1, Dr))
    bt = np.zeros((B, max(pages)), np.int64)
    perm = r.permutation(P)
    off = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    K = int(kv_lens.max())
    topk = np.full((T, 1, K), -1)
    for b in range(B):
        topk[cu[b]:cu[b + 1], 0, :kv_lens[b]] = np.arange(kv_lens[b])
    scale = 1 / math.sqrt(D + Dr)
    out, lse = oracle.sfa_fwd_tnd(q, qr, kc, krc, kc, bt, kv_lens, topk, cu, scale, 3)
    for b in range(B):
        n, sq = int(kv_lens[b]), lens[b]
        keys = kc[bt[b, :pages[b]]].reshape(-1, D)[:n]
        kro = krc[bt[b, :pages[b]]].reshape(-1, Dr)[:n]
        sl = slice(cu[b], cu[b + 1])
        qcat = torch.tensor(np.concatenate([q[sl], qr[sl]], -1)).transpose(0, 1)  # [N1, sq, .]
        kcat = torch.tensor(np.concatenate([keys, kro], -1))[None].expand(N1, -1, -1)
        vals = torch.tensor(keys)[None].expand(N1, -1, -1)
        allowed = torch.arange(n)[None, :] <= (n - sq + torch.arange(sq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qcat, kcat, vals, attn_mask=allowed,
                                                               scale=scale)
        np.testing.assert_allclose(out[sl], ref.numpy().transpose(1, 0, 2), atol=1e-12, rtol=0)
    assert np.all(np.isfinite(lse))


def test_sfa_tnd_equal_lengths_equals_bsnd():
    r = _rng(32)
    B, Sq, N1, D, Dr, page, kv_len = 3, 2, 2, 8, 4, 4, 16
    q, qr = r.standard_normal((B, Sq, N1, D)), r.standard_normal((B, Sq, N1, Dr))
    P = B * kv_len // page
    kc, krc = r.standard_normal((P, page, 1, D)), r.standard_normal((P, page, 1, Dr))
    bt = r.permutation(P).reshape(B, kv_len // page)
    kv_lens = np.array([16, 11, 14])
    topk = np.stack([np.stack([np.sort(r.choice(kv_lens[b] - 1, 5, replace=False))
                               for s in range(Sq)]) for b in range(B)])[:, :, None, :]
    o, l = oracle.sfa_fwd(q, qr, kc, krc, kc, bt, kv_lens, topk, 0.3, 3)
    cu = np.arange(B + 1) * Sq
    ot, lt = oracle.sfa_fwd_tnd(q.reshape(B * Sq, N1, D), qr.reshape(B * Sq, N1, Dr), kc, krc,
                                kc, bt, kv_lens, topk.reshape(B * Sq, 1, -1), cu, 0.3, 3)
    assert np.array_equal(o.reshape(B * Sq, N1, D), ot)
    assert np.array_equal(l.reshape(B * Sq, N1), lt)


def test_sfa_page_table_permutation_is_invisible():
    """Moving pages around the physical cache (and the table with them) changes nothing."""
    r = _rng(4)
    B, Sq, N1, D, Dr, page, kv_len = 2, 2, 2, 8, 4, 4, 16
    P = 10
    q, qr = r.standard_normal((B, Sq, N1, D)), r.standard_normal((B, Sq, N1, Dr))
    kc, krc = r.standard_normal((P, page, 1, D)), r.standard_normal((P, page, 1, Dr))
    bt = r.permutation(P)[:8].reshape(B, 4)
    kv_lens = np.array([16, 13])
    topk = np.stack([np.stack([np.sort(r.choice(kv_lens[b] - Sq + s + 1, 6, replace=False))
                               for s in range(Sq)]) for b in range(B)])[:, :, None, :]
    o1, l1 = oracle.sfa_fwd(q, qr, kc, krc, kc, bt, kv_lens, topk, 0.25)
    perm = r.permutation(P)                       # physical page p moves to perm[p]
    kc2, krc2 = np.empty_like(kc), np.empty_like(krc)
    kc2[perm], krc2[perm] = kc, krc
    o2, l2 = oracle.sfa_fwd(q, qr, kc2, krc2, kc2, perm[bt], kv_lens, topk, 0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _sdpa_over_positions(q_tok, qr_tok, kc, krc, bt_row, selected, scale):
    """torch float64 attention of one decode token's heads over the cache
    rows at the positions where ``selected`` (bool over positions) is true;
    the value is the 512-wide key row (shared KV)."""
    pos = np.nonzero(selected)[0]
    page = kc.shape[1]
    keys = np.concatenate([kc[bt_row[pos // page], pos % page, 0],
                           krc[bt_row[pos // page], pos % page, 0]], -1)
    vals = kc[bt_row[pos // page], pos % page, 0]
    qq = torch.tensor(np.concatenate([q_tok, qr_tok], -1))             # [N1, D+Dr]
    H = qq.shape[0]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qq[:, None], torch.tensor(keys)[None].expand(H, -1, -1),
        torch.tensor(vals)[None].expand(H, -1, -1), scale=scale)[:, 0]
    return ref.numpy(), torch.logsumexp(scale * qq @ torch.tensor(keys).T, -1).numpy()


@pytest.mark.parametrize("mode", [0, 3])
def test_sfa_sparse_blocks_equal_attention_over_the_blocks_positions(mode):
    """"aclnnSparseFlashAttention", constraints section: an id selects a
    sparse block of sparse_block_size consecutive positions.  Position p
    belongs to the block p // sbs; the positions are marked from that
    membership test (not by expanding ids), and torch attends over them:
    the sequence's last block is partial (kv_len 30, sbs 4) and, under
    rightDownCausal, the cut falls inside a selected block."""
    r = _rng(33)
    B, Sq, N1, D, Dr, page, sbs = 2, 3, 4, 16, 8, 8, 4
    kv_lens = np.array([30, 21])
    P = 12
    q, qr = r.standard_normal((B, Sq, N1, D)), r.standard_normal((B, Sq, N1, Dr))
    kc, krc = r.standard_normal((P, page, 1, D)), r.standard_normal((P, page, 1, Dr))
    bt = r.permutation(P).reshape(B, 6)[:, :4]
    K = 4
    topk = np.full((B, Sq, 1, K), -1)
    for b in range(B):
        nblk = -(-int(kv_lens[b]) // sbs)
        for s in range(Sq):
            ids = r.choice(nblk - 1, 2, replace=False)
            # the last (partial / causally cut) block first; slot 3 stays empty (-1)
            topk[b, s, 0, :3] = [nblk - 1, ids[0], ids[1]]
    scale = 1 / math.sqrt(D + Dr)
    out, lse = oracle.sfa_fwd(q, qr, kc, krc, kc, bt, kv_lens, topk, scale, sparse_mode=mode,
                              sparse_block_size=sbs)
    for b in range(B):
        n = int(kv_lens[b])
        positions = np.arange(n)
        for s in range(Sq):
            chosen = set(int(i) for i in topk[b, s, 0] if i >= 0)
            selected = np.array([(p // sbs) in chosen for p in positions])
            if mode == 3:
                selected &= positions <= n - Sq + s
            ref, ref_lse = _sdpa_over_positions(q[b, s], qr[b, s], kc, krc, bt[b], selected, scale)
            np.testing.assert_allclose(out[b, s], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, s], ref_lse, rtol=0, atol=1e-12)


def test_sfa_mode0_all_tokens_is_dense_mqa_without_a_mask():
    """sparse_mode 0 masks nothing: with every position selected, each decode
    token (even the earlier ones of Sq = 3, which rightDownCausal would cut)
    is dense MQA over the whole sequence (torch, no attn_mask)."""
    r = _rng(34)
    B, Sq, N1, D, Dr, page, kv_len = 2, 3, 4, 16, 8, 8, 24
    q, qr = r.standard_normal((B, Sq, N1, D)), r.standard_normal((B, Sq, N1, Dr))
    P = B * kv_len // page
    kc, krc = r.standard_normal((P, page, 1, D)), r.standard_normal((P, page, 1, Dr))
    bt = r.permutation(P).reshape(B, kv_len // page)
    kv_lens = np.full(B, kv_len)
    topk = np.tile(np.arange(kv_len), (B, Sq, 1, 1))
    scale = 1 / math.sqrt(D + Dr)
    out, lse = oracle.sfa_fwd(q, qr, kc, krc, kc, bt, kv_lens, topk, scale, sparse_mode=0)
    for b in range(B):
        keys = kc[bt[b]].reshape(kv_len, D)
        kro = krc[bt[b]].reshape(kv_len, Dr)
        qcat = torch.tensor(np.concatenate([q[b], qr[b]], -1)).transpose(0, 1)   # [N1, Sq, D+Dr]
        kcat = torch.tensor(np.concatenate([keys, kro], -1))[None].expand(N1, -1, -1)
        vals = torch.tensor(keys)[None].expand(N1, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(qcat, kcat, vals, scale=scale)
        np.testing.assert_allclose(out[b], ref.numpy().transpose(1, 0, 2), atol=1e-12, rtol=0)
        full = torch.logsumexp(scale * qcat @ kcat.transpose(1, 2), -1).numpy().T
        np.testing.assert_allclose(lse[b], full, atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------
# Shared-KV two-branch decode (band over the original KV + compressed top-k)
# ----------------------------------------------------------------------------

def _skv_small(seed=40, lens=(1, 3, 2), kv_lens=(40, 70, 9), cmp_ratio=4, K=6):
    x = W.sfa_sharedkv_inputs(lens=lens, kv_lens=kv_lens, N1=4, D=16, Dr=8, page=8,
                              cmp_ratio=cmp_ratio, cmp_topk=K, seed_base=seed, dtype="fp32")
    cu, q, qr, kvl, ori, cmp = x
    f = lambda t: t.double().numpy() if isinstance(t, torch.Tensor) else t  # noqa: E731
    return (cu, f(q), f(qr), kvl, tuple(f(t) for t in ori), tuple(f(t) for t in cmp))


def _rows(kc, krc, bt, pos):
    page = kc.shape[1]
    phys, row = bt[pos // page], pos % page
    return np.concatenate([kc[phys, row, 0], krc[phys, row, 0]], 1), kc[phys, row, 0]


def test_sfa_sharedkv_equals_dense_attention_over_the_union():
    """Each token's keys gathered straight from the caches (band rows, then
    the compressed rows it may see) and run through torch's attention equal
    the oracle; with win_left = 3 the band is shorter than most sequences."""
    cu, q, qr, kvl, ori, cmp = _skv_small()
    scale = 0.21
    out, lse = oracle.sfa_sharedkv_fwd(q, qr, cu, kvl, scale, ori=ori, cmp=cmp, win_left=3,
                                       cmp_ratio=4)
    for b in range(len(kvl)):
        sq, n = int(cu[b + 1] - cu[b]), int(kvl[b])
        for s in range(sq):
            t = int(cu[b]) + s
            p = n - sq + s
            band = np.arange(max(0, p - 3), p + 1)
            ids = cmp[3][t, 0]
            ids = ids[(ids >= 0) & (ids <= n // 4 - sq + s)]
            k1, v1 = _rows(ori[0], ori[1], ori[2][b], band)
            k2, v2 = _rows(cmp[0], cmp[1], cmp[2][b], ids)
            kk, vv = torch.tensor(np.concatenate([k1, k2])), torch.tensor(np.concatenate([v1, v2]))
            qq = torch.tensor(np.concatenate([q[t], qr[t]], 1))
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq[:, None], kk[None].expand(4, -1, -1), vv[None].expand(4, -1, -1),
                scale=scale)[:, 0]
            np.testing.assert_allclose(out[t], ref.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[t], torch.logsumexp(scale * qq @ kk.T, -1).numpy(),
                                       rtol=0, atol=1e-12)


@pytest.mark.parametrize("wl,wr", [(3, 2), (0, 5), (127, 1)])
def test_sfa_sharedkv_band_with_future_tokens_equals_attention_over_it(wl, wr):
    """"SparseAttnSharedkvMetadata", parameter list: mask mode 4 keeps
    ori_win_left past and ori_win_right future original tokens around the
    query's position p.  The band is marked per position by the offset test
    -wl <= j - p <= wr (and 0 <= j < kv_len), not by a range; torch attends
    over the marked rows.  Later decode tokens' bands reach past kv_len and
    are clipped there."""
    cu, q, qr, kvl, ori, cmp = _skv_small(44, lens=(1, 3, 2), kv_lens=(40, 70, 9))
    scale = 0.23
    out, lse = oracle.sfa_sharedkv_fwd(q, qr, cu, kvl, scale, ori=ori, cmp=None, win_left=wl,
                                       win_right=wr)
    for b in range(len(kvl)):
        sq, n = int(cu[b + 1] - cu[b]), int(kvl[b])
        j = np.arange(n)
        for s in range(sq):
            t = int(cu[b]) + s
            p = n - sq + s
            selected = (j - p >= -wl) & (j - p <= wr)
            ref, ref_lse = _sdpa_over_positions(q[t], qr[t], ori[0], ori[1], ori[2][b], selected,
                                                scale)
            np.testing.assert_allclose(out[t], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[t], ref_lse, rtol=0, atol=1e-12)
    # the future half matters: entry 1's first token (p = kv_len - 3) has two
    # future tokens, and a band without them differs
    o0, _ = oracle.sfa_sharedkv_fwd(q, qr, cu, kvl, scale, ori=ori, cmp=None, win_left=wl,
                                    win_right=0)
    t1 = int(cu[1])
    assert not np.allclose(o0[t1], out[t1])


def test_sfa_sharedkv_band_alone_is_sfa_over_the_window():
    """Without the compressed branch the decode is the pinned SFA path with
    the window positions as its selection (rightDownCausal)."""
    cu, q, qr, kvl, ori, cmp = _skv_small(41)
    o1, l1 = oracle.sfa_sharedkv_fwd(q, qr, cu, kvl, 0.3, ori=ori, cmp=None, win_left=127)
    T = q.shape[0]
    idx = np.full((T, 1, 128), -1)
    for b in range(len(kvl)):
        sq, n = int(cu[b + 1] - cu[b]), int(kvl[b])
        for s in range(sq):
            p = n - sq + s
            pos = np.arange(max(0, p - 127), p + 1)
            idx[cu[b] + s, 0, :len(pos)] = pos
    o2, l2 = oracle.sfa_fwd_tnd(q, qr, ori[0], ori[1], ori[0], ori[2], kvl, idx, cu, 0.3, 3)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_sfa_sharedkv_branches_merge_by_lse():
    """One softmax over both key sets is the LSE-weighted merge of the two
    single-branch results: LSE = logaddexp(LSE_ori, LSE_cmp) and
    O = exp(LSE_ori - LSE) O_ori + exp(LSE_cmp - LSE) O_cmp."""
    cu, q, qr, kvl, ori, cmp = _skv_small(42, kv_lens=(64, 128, 40), cmp_ratio=4, K=10)
    ob, lb = oracle.sfa_sharedkv_fwd(q, qr, cu, kvl, 0.25, ori=ori, cmp=cmp, win_left=7)
    oo, lo = oracle.sfa_sharedkv_fwd(q, qr, cu, kvl, 0.25, ori=ori, cmp=None, win_left=7)
    oc, lc = oracle.sfa_sharedkv_fwd(q, qr, cu, kvl, 0.25, ori=None, cmp=cmp, win_left=7)
    lse = np.logaddexp(lo, lc)
    np.testing.assert_allclose(lb, lse, rtol=0, atol=1e-12)
    merged = np.exp(lo - lse)[..., None] * oo + np.exp(lc - lse)[..., None] * oc
    np.testing.assert_allclose(ob, merged, rtol=0, atol=1e-12)


def test_sfa_sharedkv_compressed_alone_all_ids_is_dense_causal_mqa():
    """Without the band, selecting every compressed id is dense MQA over the
    compressed sequence with the rightDownCausal offset cmp_len - Sq_b."""
    lens, kvl = (2, 3), (48, 64)
    cu, q, qr, kv, ori, cmp = _skv_small(43, lens=lens, kv_lens=kvl, cmp_ratio=4, K=16)
    kc, krc, bt, _ = cmp
    T = q.shape[0]
    idx = np.full((T, 1, 16), -1)
    for b in range(2):
        idx[cu[b]:cu[b + 1], 0, :kvl[b] // 4] = np.arange(kvl[b] // 4)
    out, _ = oracle.sfa_sharedkv_fwd(q, qr, cu, kv, 0.2, ori=None, cmp=(kc, krc, bt, idx))
    for b in range(2):
        n, sq = kvl[b] // 4, lens[b]
        k, v = _rows(kc, krc, bt[b], np.arange(n))
        sl = slice(cu[b], cu[b + 1])
        qq = torch.tensor(np.concatenate([q[sl], qr[sl]], -1)).transpose(0, 1)   # [N1, sq, .]
        allowed = torch.arange(n)[None, :] <= (n - sq + torch.arange(sq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, torch.tensor(k)[None].expand(4, -1, -1), torch.tensor(v)[None].expand(4, -1, -1),
            attn_mask=allowed, scale=0.2)
        np.testing.assert_allclose(out[sl], ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# atten_mask (element mask inside the selected blocks; non-zero = excluded)
# ----------------------------------------------------------------------------

def _atten_mask(r, shape, p=0.35):
    """Random exclusions that keep the diagonal, so no row is empty."""
    am = (r.random(shape) < p).astype(np.uint8)
    S = min(shape[-2], shape[-1])
    idx = np.arange(S)
    am[..., idx, idx] = 0
    return am


@pytest.mark.parametrize("causal", [False, True])
def test_bsa_atten_mask_all_blocks_equals_dense_masked_attention(causal):
    """Every block selected, a per-head atten_mask: torch's dense attention
    with the same (inverted: True = take part) boolean mask, float64 autograd."""
    r = _rng(21)
    N1, N2, S, D, bq, bkv = 4, 2, 36, 16, 8, 8     # ragged: 36 = 4.5 blocks
    G = N1 // N2
    q = r.standard_normal((1, N1, S, D))
    k = r.standard_normal((1, N2, S, D))
    v = r.standard_normal((1, N2, S, D))
    do = r.standard_normal((1, N1, S, D))
    am = _atten_mask(r, (1, N1, S, S))
    scale = 1 / math.sqrt(D)
    mask = np.ones((1, N1, 5, 5), np.uint8)
    mode = 2 if causal else 0
    out, lse = oracle.bsa_fwd(q, k, v, mask, bq, bkv, scale, mode, atten_mask=am)
    keep = torch.tensor(am[0] == 0)
    if causal:
        keep &= torch.ones(S, S, dtype=torch.bool).tril()
    qt = torch.tensor(q[0], requires_grad=True)
    kt = torch.tensor(k[0], requires_grad=True)
    vt = torch.tensor(v[0], requires_grad=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kt.repeat_interleave(G, 0)[None], vt.repeat_interleave(G, 0)[None],
        attn_mask=keep[None], scale=scale)[0]
    np.testing.assert_allclose(out[0], ref.detach().numpy(), rtol=0, atol=1e-12)
    sc = scale * torch.tensor(q[0]) @ torch.tensor(k[0]).repeat_interleave(G, 0).transpose(1, 2)
    np.testing.assert_allclose(lse[0], torch.logsumexp(sc.masked_fill(~keep, -math.inf), -1).numpy(),
                               rtol=0, atol=1e-12)
    ref.backward(torch.tensor(do[0]))
    dq, dk, dv = oracle.bsa_bwd(q, k, v, out, do, mask, bq, bkv, scale, mode, atten_mask=am)
    for mine, theirs in ((dq[0], qt.grad), (dk[0], kt.grad), (dv[0], vt.grad)):
        t = theirs.numpy()
        assert np.abs(mine - t).max() <= 1e-10 * np.abs(t).max()


def test_bsa_atten_mask_upper_triangle_is_causal_mode():
    """atten_mask = the strict upper triangle under sparse_mode 0 is
    sparse_mode 2 (top-left causal), bit for bit."""
    r = _rng(22)
    B, N1, N2, S, D, bq, bkv = 2, 2, 1, 20, 8, 8, 4
    q = r.standard_normal((B, N1, S, D))
    k = r.standard_normal((B, N2, S, D))
    v = r.standard_normal((B, N2, S, D))
    do = r.standard_normal((B, N1, S, D))
    mask = W.mask_random(r, B, N1, 3, 5, 0.6)
    tri = np.triu(np.ones((S, S), np.uint8), 1)
    o0, l0 = oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.3, 0, atten_mask=tri)
    o2, l2 = oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.3, 2)
    assert np.array_equal(o0, o2, equal_nan=True) and np.array_equal(l0, l2, equal_nan=True)
    g0 = oracle.bsa_bwd(q, k, v, o0, do, mask, bq, bkv, 0.3, 0, atten_mask=tri)
    g2 = oracle.bsa_bwd(q, k, v, o2, do, mask, bq, bkv, 0.3, 2)
    for a, b_ in zip(g0, g2):
        assert np.array_equal(a, b_, equal_nan=True)


def test_bsa_atten_mask_over_a_whole_block_deselects_it():
    """Excluding every entry of one (Q block, KV block) pair with atten_mask
    gives the result of clearing that pair in the block mask."""
    r = _rng(23)
    B, N1, N2, S, D, bq, bkv = 1, 2, 2, 24, 8, 8, 8
    q = r.standard_normal((B, N1, S, D))
    k = r.standard_normal((B, N2, S, D))
    v = r.standard_normal((B, N2, S, D))
    do = r.standard_normal((B, N1, S, D))
    mask = np.ones((B, N1, 3, 3), np.uint8)
    am = np.zeros((B, N1, S, S), np.uint8)
    am[0, 1, 8:16, 16:24] = 1          # head 1, Q block 1, KV block 2
    cleared = mask.copy()
    cleared[0, 1, 1, 2] = 0
    oa, la = oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.35, 0, atten_mask=am)
    ob, lb = oracle.bsa_fwd(q, k, v, cleared, bq, bkv, 0.35, 0)
    np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)
    ga = oracle.bsa_bwd(q, k, v, oa, do, mask, bq, bkv, 0.35, 0, atten_mask=am)
    gb = oracle.bsa_bwd(q, k, v, ob, do, cleared, bq, bkv, 0.35, 0)
    for a, b_ in zip(ga, gb):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)


def test_bsa_atten_mask_broadcast_forms_agree():
    """[Sq, Skv], [1, 1, Sq, Skv] and its expansion to [B, N1, Sq, Skv] are
    the same mask."""
    r = _rng(24)
    B, N1, N2, S, D, bq, bkv = 2, 2, 2, 16, 8, 8, 8
    q = r.standard_normal((B, N1, S, D))
    k = r.standard_normal((B, N2, S, D))
    v = r.standard_normal((B, N2, S, D))
    mask = W.mask_random(r, B, N1, 2, 2, 0.7)
    am2 = _atten_mask(r, (S, S))
    outs = [oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.3, 0, atten_mask=a)
            for a in (am2, am2[None, None], np.broadcast_to(am2, (B, N1, S, S)).copy())]
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0], equal_nan=True)
        assert np.array_equal(l, outs[0][1], equal_nan=True)


@pytest.mark.parametrize("mode", [0, 2])
def test_bsa_atten_mask_finite_differences(mode):
    r = _rng(25)
    B, N1, N2, S, D, bq, bkv = 1, 2, 1, 16, 8, 4, 4
    a = dict(q=r.standard_normal((B, N1, S, D)), k=r.standard_normal((B, N2, S, D)),
             v=r.standard_normal((B, N2, S, D)))
    do = r.standard_normal((B, N1, S, D))
    mask = W.mask_random(r, B, N1, 4, 4, 0.6)
    am = _atten_mask(r, (B, N1, S, S), 0.5)
    scale = 0.37

    def loss():
        o, _ = oracle.bsa_fwd(a["q"], a["k"], a["v"], mask, bq, bkv, scale, mode, atten_mask=am)
        return float(np.nansum(do * o))

    o, _ = oracle.bsa_fwd(a["q"], a["k"], a["v"], mask, bq, bkv, scale, mode, atten_mask=am)
    g = oracle.bsa_bwd(a["q"], a["k"], a["v"], o, do, mask, bq, bkv, scale, mode, atten_mask=am)
    _fd_check(loss, a, ["q", "k", "v"], list(g))


def test_bsa_tnd_atten_mask_equal_lengths_equals_bnsd():
    """TND with equal lengths and a per-(b, n1) atten_mask is the BNSD
    problem: element positions count from each sequence's start."""
    r = _rng(26)
    B, N1, N2, S, D, bq, bkv = 3, 2, 1, 16, 8, 8, 4
    q = r.standard_normal((B, N1, S, D))
    k = r.standard_normal((B, N2, S, D))
    v = r.standard_normal((B, N2, S, D))
    do = r.standard_normal((B, N1, S, D))
    mask = W.mask_random(r, B, N1, 2, 4, 0.6)
    am = _atten_mask(r, (B, N1, S, S))
    cu = np.arange(B + 1) * S
    tnd = lambda x: x.transpose(0, 2, 1, 3).reshape(B * S, x.shape[1], D)  # noqa: E731
    o, l = oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.4, 0, atten_mask=am)
    ot, lt = oracle.bsa_fwd_tnd(tnd(q), tnd(k), tnd(v), mask, cu, cu, bq, bkv, 0.4, 0,
                                atten_mask=am)
    assert np.array_equal(tnd(o), ot) and np.array_equal(l.transpose(0, 2, 1).reshape(B * S, N1), lt)
    g = oracle.bsa_bwd(q, k, v, o, do, mask, bq, bkv, 0.4, 0, atten_mask=am)
    gt = oracle.bsa_bwd_tnd(tnd(q), tnd(k), tnd(v), ot, tnd(do), mask, cu, cu, bq, bkv, 0.4, 0,
                            atten_mask=am)
    for a_, b_ in zip(g, gt):
        assert np.array_equal(tnd(a_), b_)


# ----------------------------------------------------------------------------
# Finite differences of L = sum(dO * O)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_bsa_tnd_all_blocks_equals_dense_attention_per_sequence(causal):
    """TND varlen with every mask entry set (also past each sequence's end,
    which must be ignored): each sequence equals dense attention over its own
    rows, with causality counted from the sequence start."""
    r = _rng(2)
    lens, N1, N2, D, bq, bkv = [13, 40, 27], 4, 2, 16, 8, 8
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q = r.standard_normal((T, N1, D))
    k = r.standard_normal((T, N2, D))
    v = r.standard_normal((T, N2, D))
    do = r.standard_normal((T, N1, D))
    scale = 1 / math.sqrt(D)
    mask = np.ones((3, N1, 5, 5), np.uint8)
    mode = 2 if causal else 0
    out, lse = oracle.bsa_fwd_tnd(q, k, v, mask, cu, cu, bq, bkv, scale, mode)
    dq, dk, dv = oracle.bsa_bwd_tnd(q, k, v, out, do, mask, cu, cu, bq, bkv, scale, mode)
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        qt, kt, vt, ref = _dense_torch(q[sl].transpose(1, 0, 2), k[sl].transpose(1, 0, 2),
                                       v[sl].transpose(1, 0, 2), scale, causal, N1 // N2)
        np.testing.assert_allclose(out[sl], ref.detach().numpy().transpose(1, 0, 2), rtol=0,
                                   atol=1e-12)
        ref.backward(torch.tensor(do[sl].transpose(1, 0, 2)))
        for mine, theirs in ((dq[sl], qt.grad), (dk[sl], kt.grad), (dv[sl], vt.grad)):
            t = theirs.numpy().transpose(1, 0, 2)
            assert np.abs(mine - t).max() <= 1e-10 * np.abs(t).max()
    assert np.all(np.isfinite(lse))


@pytest.mark.parametrize("mode", [0, 2])
def test_bsa_tnd_equal_lengths_equals_bnsd(mode):
    """TND with B equal-length sequences is the BNSD problem with its axes
    moved: the same numbers, bit for bit."""
    r = _rng(3)
    B, N1, N2, S, D, bq, bkv = 3, 4, 2, 24, 8, 8, 4
    q = r.standard_normal((B, N1, S, D))
    k = r.standard_normal((B, N2, S, D))
    v = r.standard_normal((B, N2, S, D))
    do = r.standard_normal((B, N1, S, D))
    mask = W.mask_random(r, B, N1, 3, 6, 0.5)
    cu = np.arange(B + 1) * S
    tnd = lambda x: x.transpose(0, 2, 1, 3).reshape(B * S, x.shape[1], D)  # noqa: E731
    o, l = oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.4, mode)
    ot, lt = oracle.bsa_fwd_tnd(tnd(q), tnd(k), tnd(v), mask, cu, cu, bq, bkv, 0.4, mode)
    assert np.array_equal(tnd(o), ot) and np.array_equal(l.transpose(0, 2, 1).reshape(B * S, N1), lt)
    g = oracle.bsa_bwd(q, k, v, o, do, mask, bq, bkv, 0.4, mode)
    gt = oracle.bsa_bwd_tnd(tnd(q), tnd(k), tnd(v), ot, tnd(do), mask, cu, cu, bq, bkv, 0.4, mode)
    for a, b_ in zip(g, gt):
        assert np.array_equal(tnd(a), b_)


@pytest.mark.parametrize("mode", [0, 2])
def test_bsa_tnd_finite_differences_and_sequence_isolation(mode):
    r = _rng(4)
    lens, N1, N2, D, bq, bkv = [9, 16], 2, 1, 8, 4, 4
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    a = dict(q=r.standard_normal((T, N1, D)), k=r.standard_normal((T, N2, D)),
             v=r.standard_normal((T, N2, D)))
    do = r.standard_normal((T, N1, D))
    mask = W.mask_random(r, 2, N1, 4, 4, 0.5)
    scale = 0.41

    def loss():
        o, _ = oracle.bsa_fwd_tnd(a["q"], a["k"], a["v"], mask, cu, cu, bq, bkv, scale, mode)
        return float((do * o).sum())

    o, _ = oracle.bsa_fwd_tnd(a["q"], a["k"], a["v"], mask, cu, cu, bq, bkv, scale, mode)
    g = oracle.bsa_bwd_tnd(a["q"], a["k"], a["v"], o, do, mask, cu, cu, bq, bkv, scale, mode)
    _fd_check(loss, a, ["q", "k", "v"], list(g))
    # another sequence's K/V never enters sequence 0's results
    k2, v2 = a["k"].copy(), a["v"].copy()
    k2[cu[1]:] += 5.0
    v2[cu[1]:] -= 3.0
    o2, _ = oracle.bsa_fwd_tnd(a["q"], k2, v2, mask, cu, cu, bq, bkv, scale, mode)
    g2 = oracle.bsa_bwd_tnd(a["q"], k2, v2, o2, do, mask, cu, cu, bq, bkv, scale, mode)
    s0 = slice(0, cu[1])
    assert np.array_equal(o[s0], o2[s0])
    for x, y in zip(g, g2):
        assert np.array_equal(x[s0], y[s0])


def _fd_check(f, args, idx_names, grads, n_probe=12, h=1e-6, seed=0):
    r = _rng(seed)
    for name, g in zip(idx_names, grads):
        x = args[name]
        flat = x.reshape(-1)
        for p in r.choice(flat.size, n_probe, replace=False):
            old = flat[p]
            flat[p] = old + h
            lp = f()
            flat[p] = old - h
            lm = f()
            flat[p] = old
            fd = (lp - lm) / (2 * h)
            an = g.reshape(-1)[p]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, p, fd, an)


@pytest.mark.parametrize("mode", [0, 2])
def test_bsa_finite_differences_gqa(mode):
    r = _rng(5)
    B, N1, N2, S, D, bq, bkv = 1, 2, 1, 16, 8, 4, 4
    a = dict(q=r.standard_normal((B, N1, S, D)), k=r.standard_normal((B, N2, S, D)),
             v=r.standard_normal((B, N2, S, D)))
    do = r.standard_normal((B, N1, S, D))
    mask = W.mask_random(r, B, N1, 4, 4, 0.5)
    scale = 0.37

    def loss():
        o, _ = oracle.bsa_fwd(a["q"], a["k"], a["v"], mask, bq, bkv, scale, mode)
        return float((do * o).sum())

    o, _ = oracle.bsa_fwd(a["q"], a["k"], a["v"], mask, bq, bkv, scale, mode)
    dq, dk, dv = oracle.bsa_bwd(a["q"], a["k"], a["v"], o, do, mask, bq, bkv, scale, mode)
    _fd_check(loss, a, ["q", "k", "v"], [dq, dk, dv])


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("Dv", [8, 5])
def test_nsa_finite_differences(mode, Dv):
    r = _rng(6)
    seqlens, N1, N2, D, sbs, sbc = [12, 8], 4, 2, 8, 4, 2
    cu = np.array([0, 12, 20])
    T = 20
    a = dict(q=r.standard_normal((T, N1, D)), k=r.standard_normal((T, N2, D)),
             v=r.standard_normal((T, N2, Dv)))
    do = r.standard_normal((T, N1, Dv))
    topk = W.nsa_topk_causal(r, seqlens, N2, sbs, sbc)

    def loss():
        o, _ = oracle.nsa_fwd(a["q"], a["k"], a["v"], topk, cu, cu, sbs, 0.4, mode)
        return float((do * o).sum())

    o, _ = oracle.nsa_fwd(a["q"], a["k"], a["v"], topk, cu, cu, sbs, 0.4, mode)
    dq, dk, dv = oracle.nsa_bwd(a["q"], a["k"], a["v"], o, do, topk, cu, cu, sbs, 0.4, mode)
    _fd_check(loss, a, ["q", "k", "v"], [dq, dk, dv])


def test_nsa_duplicate_slot_counts_twice():
    """Gather is literal: listing a block twice doubles its weight in the softmax,
    and its keys' gradient is the sum over both gathered copies (checked by FD)."""
    r = _rng(7)
    cu = np.array([0, 8])
    a = dict(q=r.standard_normal((8, 2, 4)), k=r.standard_normal((8, 1, 4)),
             v=r.standard_normal((8, 1, 4)))
    do = r.standard_normal((8, 2, 4))
    topk = np.tile(np.array([0, 0, 1], np.int32), (8, 1, 1))
    o, _ = oracle.nsa_fwd(a["q"], a["k"], a["v"], topk, cu, cu, 4, 0.5, 0)
    # closed form: weights of block 0 keys doubled -> same as attention with
    # log(2) added to their scores
    s = 0.5 * np.einsum("thd,jd->thj", a["q"], a["k"][:, 0])
    s[:, :, :4] += math.log(2)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    np.testing.assert_allclose(o, p @ a["v"][:, 0], atol=1e-12, rtol=0)

    def loss():
        oo, _ = oracle.nsa_fwd(a["q"], a["k"], a["v"], topk, cu, cu, 4, 0.5, 0)
        return float((do * oo).sum())
    dq, dk, dv = oracle.nsa_bwd(a["q"], a["k"], a["v"], o, do, topk, cu, cu, 4, 0.5, 0)
    _fd_check(loss, a, ["q", "k", "v"], [dq, dk, dv], n_probe=8)


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_softmax_grad_identity():
    r = _rng(8)
    q, k, v = r.standard_normal((7, 5)), r.standard_normal((11, 5)), r.standard_normal((11, 3))
    allowed = r.random((7, 11)) < 0.6
    allowed[:, 0] = True
    out, lse, p = oracle.attend_fwd(q, k, v, allowed, 0.8)
    assert np.abs(p.sum(1) - 1).max() <= 1e-12
    assert np.all(p[~allowed] == 0)
    do = r.standard_normal((7, 3))
    # softmaxGrad read as rowsum(dO * O) equals rowsum(P * dP): the identity the
    # softmax Jacobian requires of it
    dp = do @ v.T
    assert np.abs((do * out).sum(1) - (p * dp).sum(1)).max() <= 1e-12
    # LSE is the log of the softmax denominator: exp(S - LSE) == P
    s = np.where(allowed, 0.8 * q @ k.T, -np.inf)
    np.testing.assert_allclose(np.exp(s - lse[:, None]), p, atol=1e-14, rtol=0)


def test_empty_row_convention():
    q, k, v = np.ones((2, 3)), np.ones((4, 3)), np.ones((4, 2))
    allowed = np.array([[True, False, False, False], [False] * 4])
    out, lse, p = oracle.attend_fwd(q, k, v, allowed, 1.0)
    assert np.all(out[1] == 0) and lse[1] == -np.inf and np.all(p[1] == 0)
    dq, dk, dv = oracle.attend_bwd(q, k, v, allowed, out, np.ones((2, 2)), 1.0)
    assert np.all(dq[1] == 0)


@pytest.mark.parametrize("mode", [0, 2])
def test_bsa_unselected_blocks_do_not_matter(mode):
    r = _rng(9)
    B, N1, N2, S, D, bq, bkv = 1, 2, 2, 32, 8, 8, 8
    q, k, v = (r.standard_normal((B, N1, S, D)), r.standard_normal((B, N2, S, D)),
               r.standard_normal((B, N2, S, D)))
    do = r.standard_normal((B, N1, S, D))
    mask = W.mask_random(r, B, N1, 4, 4, 0.4)
    mask[:, :, :, 3] = 0                       # KV block 3 selected by nobody
    o, l = oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.3, mode)
    g = oracle.bsa_bwd(q, k, v, o, do, mask, bq, bkv, 0.3, mode)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 24:] += 10 * r.standard_normal((B, N2, 8, D))
    v2[:, :, 24:] += 10 * r.standard_normal((B, N2, 8, D))
    o2, l2 = oracle.bsa_fwd(q, k2, v2, mask, bq, bkv, 0.3, mode)
    g2 = oracle.bsa_bwd(q, k2, v2, o2, do, mask, bq, bkv, 0.3, mode)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    assert np.array_equal(g[0], g2[0])
    assert np.array_equal(g[1][:, :, :24], g2[1][:, :, :24])
    assert np.array_equal(g[2][:, :, :24], g2[2][:, :, :24])
    assert np.all(g2[1][:, :, 24:] == 0) and np.all(g2[2][:, :, 24:] == 0)


def test_nsa_slot_order_only_changes_rounding():
    r = _rng(10)
    cu = np.array([0, 32])
    q, k, v = r.standard_normal((32, 4, 8)), r.standard_normal((32, 2, 8)), r.standard_normal((32, 2, 8))
    topk = W.nsa_topk_causal(r, [32], 2, 4, 3)
    o1, l1 = oracle.nsa_fwd(q, k, v, topk, cu, cu, 4, 0.3, 2)
    o2, l2 = oracle.nsa_fwd(q, k, v, topk[:, :, ::-1].copy(), cu, cu, 4, 0.3, 2)
    np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-13, rtol=0)


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------

def test_constant_values_closed_form():
    """V rows all equal to c: O = c for every non-empty row, dP - softmax_grad = 0
    so dQ = dK = 0 exactly, and dV_j = sum_i P_ij dO_i."""
    r = _rng(11)
    B, N1, N2, S, D, bq, bkv = 1, 2, 1, 24, 8, 8, 8
    q, k = r.standard_normal((B, N1, S, D)), r.standard_normal((B, N2, S, D))
    c = r.standard_normal(D)
    v = np.broadcast_to(c, (B, N2, S, D)).copy()
    do = r.standard_normal((B, N1, S, D))
    mask = W.mask_random(r, B, N1, 3, 3, 0.5)
    o, _ = oracle.bsa_fwd(q, k, v, mask, bq, bkv, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-13, rtol=0)
    dq, dk, dv = oracle.bsa_bwd(q, k, v, o, do, mask, bq, bkv, 0.5)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    # dV from the explicit probabilities of one tile
    keys = oracle.bsa_keys(mask[0, 1, 2], bkv, S)
    _, _, p = oracle.attend_fwd(q[0, 1, 16:24], k[0, 0, keys], v[0, 0, keys],
                                np.ones((8, len(keys)), bool), 0.5)
    contrib = p.T @ do[0, 1, 16:24]
    # head 1 tile 2's contribution is part of dv; check a KV block only it selects
    only = [kb for kb in range(3) if mask[0, 1, 2, kb] and mask[0, :, :, kb].sum() == 1]
    for kb in only:
        sel = np.searchsorted(keys, np.arange(kb * 8, kb * 8 + 8))
        np.testing.assert_allclose(dv[0, 0, kb * 8:kb * 8 + 8], contrib[sel], atol=1e-13, rtol=0)


def test_zero_query_gives_uniform_average():
    r = _rng(12)
    B, N, S, D = 1, 1, 16, 4
    q = np.zeros((B, N, S, D))
    k, v = r.standard_normal((B, N, S, D)), r.standard_normal((B, N, S, D))
    mask = np.array([[[[1, 0], [1, 1]]]], np.uint8)
    o, lse = oracle.bsa_fwd(q, k, v, mask, 8, 8, 1.0)
    np.testing.assert_allclose(o[0, 0, :8], np.broadcast_to(v[0, 0, :8].mean(0), (8, D)), atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 8:], np.broadcast_to(v[0, 0, :].mean(0), (8, D)), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0, :8], math.log(8), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 8:], math.log(16), atol=1e-14)


# ----------------------------------------------------------------------------
# Cross-path: NSA with G = 1 and block-constant selection is block-sparse attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [0, 2])
def test_nsa_equals_bsa_for_block_constant_selection(mode):
    r = _rng(13)
    S, N, D, sbs, sbc = 32, 2, 8, 4, 3
    nb = S // sbs
    q, k, v = r.standard_normal((S, N, D)), r.standard_normal((S, N, D)), r.standard_normal((S, N, D))
    do = r.standard_normal((S, N, D))
    # one selection per (query block, head): own block + 2 distinct others
    sel = np.zeros((N, nb, sbc), np.int32)
    mask = np.zeros((1, N, nb, nb), np.uint8)
    for n in range(N):
        for qb in range(nb):
            others = r.choice([x for x in range(nb) if x != qb], sbc - 1, replace=False)
            sel[n, qb] = np.concatenate([[qb], others])
            mask[0, n, qb, sel[n, qb]] = 1
    topk = np.stack([sel[:, t // sbs] for t in range(S)])          # [S, N, sbc]
    cu = np.array([0, S])
    on, ln = oracle.nsa_fwd(q, k, v, topk, cu, cu, sbs, 0.35, mode)
    qb_, kb_, vb_ = (x.transpose(1, 0, 2)[None] for x in (q, k, v))
    ob, lb = oracle.bsa_fwd(qb_, kb_, vb_, mask, sbs, sbs, 0.35, mode)
    np.testing.assert_allclose(on, ob[0].transpose(1, 0, 2), atol=1e-13, rtol=0)
    np.testing.assert_allclose(ln, lb[0].T, atol=1e-13, rtol=0)
    gn = oracle.nsa_bwd(q, k, v, on, do, topk, cu, cu, sbs, 0.35, mode)
    gb = oracle.bsa_bwd(qb_, kb_, vb_, ob, do.transpose(1, 0, 2)[None], mask, sbs, sbs, 0.35, mode)
    for a_, b_ in zip(gn, gb):
        np.testing.assert_allclose(a_, b_[0].transpose(1, 0, 2), atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------
# Compaction: brute force and closed-form counts
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape,n2", [((2, 4, 5, 7), 2), ((1, 3, 1, 1), 3), ((1, 2, 6, 4), 1)])
def test_bsa_compact_brute_force(shape, n2):
    r = _rng(14)
    B, N1, QB, KB = shape
    mask = (r.random(shape) < 0.4).astype(np.uint8) * r.integers(1, 5, shape).astype(np.uint8)
    mask[0, 0, 0, :] = 0                                          # an empty row
    rp, col, rvp, rv = oracle.bsa_compact(mask, n2)
    G = N1 // n2
    fwd_rows, rev_rows = [], []
    for b in range(B):
        for n in range(N1):
            for qb in range(QB):
                fwd_rows.append([kb for kb in range(KB) if mask[b, n, qb, kb]])
    for b in range(B):
        for h in range(n2):
            for kb in range(KB):
                rev_rows.append([g * QB + qb for g in range(G) for qb in range(QB)
                                 if mask[b, h * G + g, qb, kb]])
    for ptr, ent, rows in ((rp, col, fwd_rows), (rvp, rv, rev_rows)):
        assert ptr.dtype == np.int32 and ent.dtype == np.int32
        assert len(ptr) == len(rows) + 1 and ptr[0] == 0
        for i, row in enumerate(rows):
            assert ent[ptr[i]:ptr[i + 1]].tolist() == row


def test_nsa_compact_brute_force():
    r = _rng(15)
    seqlens, N2, sbs, sbc = [12, 20, 8], 2, 4, 2
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    topk = W.nsa_topk_causal(r, seqlens, N2, sbs, sbc)
    topk[3, 1] = [2, 2]                                           # a duplicate
    for mode in (0, 2):
        rp, col, rvp, rv, nb = oracle.nsa_compact(topk, cu, cu, sbs, mode)
        assert nb == 3 + 5 + 2
        blk_off = [0, 3, 8]
        T = cu[-1]
        fwd = []
        for t in range(T):
            b = int(np.searchsorted(cu, t, side="right") - 1)
            pos = t - cu[b]
            for h in range(N2):
                ids = sorted(topk[t, h].tolist())
                fwd.append([i for i in ids if mode == 0 or i * sbs <= pos])
        for i, row in enumerate(fwd):
            assert col[rp[i]:rp[i + 1]].tolist() == row
        for h in range(N2):
            for gb in range(nb):
                b = max(j for j in range(3) if blk_off[j] <= gb)
                want = []
                for t in range(T):
                    if cu[b] <= t < cu[b + 1]:
                        want += [t] * fwd[t * N2 + h].count(gb - blk_off[b])
                row = h * nb + gb
                assert rv[rvp[row]:rvp[row + 1]].tolist() == want


def test_workload_closed_form_counts():
    with open(os.path.join(GOLDEN, "workload_counts.json")) as f:
        gold = json.load(f)
    cu, _, _, _, _, topk = W.nsa_inputs()
    rp, _, _, _, _ = oracle.nsa_compact(topk, cu, cu, 64, 2)
    assert int(rp[-1]) == gold["nsa_varlen_effective_triples"]
    mask = W.bsa_mask(W.bsa_workload(5), 1005)
    assert int((mask != 0).sum()) == gold["bsa_window_128k_selected_pairs"]
    # recipe properties of the NSA selection: distinct ids, own block present
    own = (np.arange(topk.shape[0]) - np.repeat(cu[:-1], np.diff(cu))) // 64
    assert np.all(np.sort(topk, -1)[..., 1:] != np.sort(topk, -1)[..., :-1])
    assert np.all((topk == own[:, None, None]).any(-1))


# ----------------------------------------------------------------------------
# FloydAttention (two batched score products, one softmax)
# ----------------------------------------------------------------------------

def _floyd_inputs(seed, B=1, H=2, N=5, M=6, K=7, D=4):
    r = _rng(seed)
    return (r.standard_normal((B, H, N, M, D)), r.standard_normal((B, H, N, K, D)),
            r.standard_normal((B, H, N, K, D)), r.standard_normal((B, H, M, K, D)),
            r.standard_normal((B, H, M, K, D)), r.standard_normal((B, H, N, M, D)))


def _sdpa_grads(q, k, v, do, scale):
    """Dense attention of q [R, D] over k, v [J, D] (torch float64, autograd)."""
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                                           scale=scale)[0]
    out.backward(torch.tensor(do))
    lse = torch.logsumexp(scale * qt.detach() @ kt.detach().T, -1)
    return out.detach().numpy(), lse.numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_floyd_first_branch_alone_is_attention_batched_over_n():
    """With key2 = value2 = 0 every (b, h, n) is dense attention of the M
    query rows q[b,h,n] over key1 / value1 [b,h,n] (torch, autograd)."""
    q, k1, v1, k2, v2, dy = _floyd_inputs(60)
    k2[:] = 0.0
    v2[:] = 0.0
    scale = 0.37
    y, lse = oracle.floyd_fwd(q, k1, v1, k2, v2, scale)
    dq, dk1, dv1, _, _ = oracle.floyd_bwd(q, k1, v1, k2, v2, y, dy, scale)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            for n in range(q.shape[2]):
                o, l_, gq, gk, gv = _sdpa_grads(q[b, h, n], k1[b, h, n], v1[b, h, n],
                                                dy[b, h, n], scale)
                for mine, ref in ((y, o), (lse, l_), (dq, gq), (dk1, gk), (dv1, gv)):
                    np.testing.assert_allclose(mine[b, h, n], ref, rtol=0, atol=1e-12)


def test_floyd_second_branch_alone_is_attention_batched_over_m():
    """With key1 = value1 = 0 every (b, h, m) is dense attention of the N
    query rows q[b,h,:,m] over key2 / value2 [b,h,m] (the second sequence
    axis as the batch axis)."""
    q, k1, v1, k2, v2, dy = _floyd_inputs(61)
    k1[:] = 0.0
    v1[:] = 0.0
    scale = 0.41
    y, lse = oracle.floyd_fwd(q, k1, v1, k2, v2, scale)
    dq, _, _, dk2, dv2 = oracle.floyd_bwd(q, k1, v1, k2, v2, y, dy, scale)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            for m in range(q.shape[3]):
                o, l_, gq, gk, gv = _sdpa_grads(q[b, h, :, m], k2[b, h, m], v2[b, h, m],
                                                dy[b, h, :, m], scale)
                np.testing.assert_allclose(y[b, h, :, m], o, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[b, h, :, m], l_, rtol=0, atol=1e-12)
                np.testing.assert_allclose(dq[b, h, :, m], gq, rtol=0, atol=1e-12)
                np.testing.assert_allclose(dk2[b, h, m], gk, rtol=0, atol=1e-12)
                np.testing.assert_allclose(dv2[b, h, m], gv, rtol=0, atol=1e-12)


def test_floyd_finite_differences():
    """Central differences of L = sum(dY * Y) for all five inputs, both
    branches live, N != M != K."""
    q, k1, v1, k2, v2, dy = _floyd_inputs(62, B=1, H=2, N=3, M=4, K=5, D=3)
    scale = 0.5
    args = dict(q=q, k1=k1, v1=v1, k2=k2, v2=v2)
    y, _ = oracle.floyd_fwd(q, k1, v1, k2, v2, scale)
    grads = oracle.floyd_bwd(q, k1, v1, k2, v2, y, dy, scale)
    f = lambda: float((oracle.floyd_fwd(**args, scale=scale)[0] * dy).sum())  # noqa: E731
    _fd_check(f, args, ["q", "k1", "v1", "k2", "v2"], grads, n_probe=10)


def test_floyd_transpose_symmetry():
    """Swapping the two sequence axes of the query together with the two
    key/value pairs transposes every result (an axis mix-up fails this)."""
    q, k1, v1, k2, v2, dy = _floyd_inputs(63, N=4, M=6, K=5)
    scale = 0.3
    y, lse = oracle.floyd_fwd(q, k1, v1, k2, v2, scale)
    g = oracle.floyd_bwd(q, k1, v1, k2, v2, y, dy, scale)
    qt, dyt = np.swapaxes(q, 2, 3).copy(), np.swapaxes(dy, 2, 3).copy()
    yt, lset = oracle.floyd_fwd(qt, k2, v2, k1, v1, scale)
    gt = oracle.floyd_bwd(qt, k2, v2, k1, v1, yt, dyt, scale)
    np.testing.assert_allclose(yt, np.swapaxes(y, 2, 3), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lset, np.swapaxes(lse, 2, 3), rtol=0, atol=1e-12)
    np.testing.assert_allclose(gt[0], np.swapaxes(g[0], 2, 3), rtol=0, atol=1e-12)
    for a, b_ in ((gt[1], g[3]), (gt[2], g[4]), (gt[3], g[1]), (gt[4], g[2])):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)


def test_floyd_constant_values_and_probability_rows():
    """value1 rows all a and value2 rows all c give Y = a + c and zero dQ,
    dK1, dK2 (dP - softmax_grad vanishes); the recomputed P has unit rows
    (exp(S - LSE) summed over k)."""
    q, k1, v1, k2, v2, dy = _floyd_inputs(64)
    a, c = _rng(65).standard_normal(4), _rng(66).standard_normal(4)
    v1[:] = a
    v2[:] = c
    y, lse = oracle.floyd_fwd(q, k1, v1, k2, v2, 0.6)
    np.testing.assert_allclose(y, np.broadcast_to(a + c, y.shape), rtol=0, atol=1e-12)
    dq, dk1, _, dk2, _ = oracle.floyd_bwd(q, k1, v1, k2, v2, y, dy, 0.6)
    for gr in (dq, dk1, dk2):
        assert np.abs(gr).max() < 1e-12
    s = 0.6 * (np.einsum("bhnmd,bhnkd->bhnmk", q, k1) + np.einsum("bhnmd,bhmkd->bhnmk", q, k2))
    np.testing.assert_allclose(np.exp(s - lse[..., None]).sum(-1), 1.0, rtol=0, atol=1e-12)
