"""NSA selected attention on the GPU against the float64 CPU oracle.

Tolerances as for block-sparse attention: outputs 2e-2 and gradients 3e-2
relative to the oracle's max magnitude, LSE 2e-3 * max(1, max|ref|), lists
bit-exact.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

OUT_TOL, GRAD_TOL, LSE_TOL = 2e-2, 3e-2, 2e-3


def _tsa():
    import top_selected_attention_amd as tsa
    return tsa


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _close(gpu, ref, tol, what, rows=None):
    g = _np(gpu)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite"
    err, scale = np.abs(g - ref).max(), np.abs(ref).max()
    assert err <= tol * scale, f"{what}: max err {err:.3e} vs {tol} * {scale:.3e}"


def _lse_close(gpu, ref, rows=None):
    g = _np(gpu)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.array_equal(np.isfinite(ref), np.isfinite(g))
    fin = np.isfinite(ref)
    err = np.abs(g[fin] - ref[fin]).max()
    assert err <= LSE_TOL * max(1.0, np.abs(ref[fin]).max()), err


def _case(seqlens, N1, N2, sbs, sbc, seed, dtype="bf16"):
    cu, q, k, v, do, topk = W.nsa_inputs(seqlens, N1=N1, N2=N2, sbs=sbs, sbc=sbc,
                                          seed_base=seed, dtype=dtype)
    return cu, q, k, v, do, topk


# ----------------------------------------------------------------------------
# Compaction
# ----------------------------------------------------------------------------

def _compact_check(topk, cu, N1, sbs, mode):
    tsa = _tsa()
    rp, col, rvp, rv, nb = tsa.nsa_compact(torch.from_numpy(topk).cuda(), cu, cu, N1, sbs, mode)
    erp, ecol, ervp, erv, enb = oracle.nsa_compact(topk, cu, cu, sbs, mode)
    assert nb == enb
    assert np.array_equal(rp.cpu().numpy(), erp)
    assert np.array_equal(col.cpu().numpy(), ecol)
    assert np.array_equal(rvp.cpu().numpy(), ervp)
    assert np.array_equal(rv.cpu().numpy(), erv)


@pytest.mark.parametrize("mode", [0, 2])
def test_compact_nsa_varlen_bit_exact(mode):
    cu, q, k, v, do, topk = W.nsa_inputs()
    _compact_check(topk, cu, 32, 64, mode)


def test_compact_edge_cases_bit_exact():
    rng = np.random.default_rng(3)
    seqlens = [64, 192, 128]
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    topk = W.nsa_topk_causal(rng, seqlens, 2, 32, 2)
    topk[5, 0] = [1, 1]                       # a duplicate
    topk[70, 1] = [5, 0]                      # unsorted, includes a future block
    for mode in (0, 2):
        _compact_check(topk, cu, 4, 32, mode)


# ----------------------------------------------------------------------------
# Forward / backward parity
# ----------------------------------------------------------------------------

def _run(cu, q, k, v, do, topk, sbs, scale, mode):
    tsa = _tsa()
    dev = torch.device("cuda")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    plan = tsa.NsaPlan(qd, kd, vd, torch.from_numpy(topk).to(dev), cu, cu, sbs, scale, mode)
    out, lse = plan.fwd()
    dq, dk, dv = plan.bwd(dod)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("seqlens,N1,N2,sbs,sbc", [
    ([256, 512, 320], 32, 2, 64, 4),    # G = 16 (the NSA workload's grouping)
    ([128, 96], 4, 4, 16, 6),           # G = 1, smallest block size
    ([256, 384], 32, 1, 128, 2),        # G = 32, largest block size
    ([160, 480], 12, 2, 32, 5),         # G = 6 (padded query columns)
    ([192, 240], 8, 2, 48, 4),          # block size not a multiple of 32
])
@pytest.mark.parametrize("mode", [0, 2])
def test_fwd_bwd_small(seqlens, N1, N2, sbs, sbc, mode):
    cu, q, k, v, do, topk = _case(seqlens, N1, N2, sbs, sbc, 70)
    scale = 1 / math.sqrt(128)
    out, lse, dq, dk, dv = _run(cu, q, k, v, do, topk, sbs, scale, mode)
    ro, rl = oracle.nsa_fwd(_np(q), _np(k), _np(v), topk, cu, cu, sbs, scale, mode)
    _close(out, ro, OUT_TOL, "out")
    _lse_close(lse, rl)
    rdq, rdk, rdv = oracle.nsa_bwd(_np(q), _np(k), _np(v), _np(out), _np(do), topk, cu, cu, sbs,
                                   scale, mode)
    _close(dq, rdq, GRAD_TOL, "dq")
    _close(dk, rdk, GRAD_TOL, "dk")
    _close(dv, rdv, GRAD_TOL, "dv")


@pytest.mark.parametrize("seqlens,N1,N2,sbs,sbc,dtype", [
    ([256, 512, 320], 32, 2, 64, 4, "bf16"),   # G = 16
    ([128, 96], 4, 4, 16, 6, "bf16"),          # G = 1, smallest block size
    ([256, 384], 32, 1, 128, 2, "fp16"),       # G = 32, largest block size
    ([192, 240], 12, 2, 48, 4, "bf16"),        # G = 6, block size not a multiple of 32
])
@pytest.mark.parametrize("mode", [0, 2])
def test_fwd_bwd_qk192_v128(seqlens, N1, N2, sbs, sbc, dtype, mode):
    """Query/key heads of 192 dims over value heads of 128 (the reading of
    the two distinct head-dim values the constraints section fixes)."""
    cu, q, k, v, do, topk = W.nsa_inputs(seqlens, N1=N1, N2=N2, D=192, Dv=128, sbs=sbs, sbc=sbc,
                                          seed_base=110, dtype=dtype)
    scale = 1 / math.sqrt(192)
    out, lse, dq, dk, dv = _run(cu, q, k, v, do, topk, sbs, scale, mode)
    assert out.shape[-1] == 128 and dq.shape[-1] == 192 and dk.shape[-1] == 192
    ro, rl = oracle.nsa_fwd(_np(q), _np(k), _np(v), topk, cu, cu, sbs, scale, mode)
    _close(out, ro, OUT_TOL, "out")
    _lse_close(lse, rl)
    rdq, rdk, rdv = oracle.nsa_bwd(_np(q), _np(k), _np(v), _np(out), _np(do), topk, cu, cu, sbs,
                                   scale, mode)
    _close(dq, rdq, GRAD_TOL, "dq")
    _close(dk, rdk, GRAD_TOL, "dk")
    _close(dv, rdv, GRAD_TOL, "dv")


def test_qk192_full_size_sampled_and_deterministic():
    """The nsa_varlen workload (4 sequences, 32/2 heads, 64 x 16 selected)
    with 192-dim query/key heads: sampled tokens against the oracle, whole KV
    blocks with every token that selected them, and bit-identical reruns."""
    cu, q, k, v, do, topk = W.nsa_inputs(D=192, Dv=128, seed_base=120)
    sbs, scale = 64, 1 / math.sqrt(192)
    a = _run(cu, q, k, v, do, topk, sbs, scale, 2)
    b = _run(cu, q, k, v, do, topk, sbs, scale, 2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    out, lse, dq, dk, dv = a
    T = int(cu[-1])
    toks = sorted(set([0, 63, 64, 2047, 2048, 6143, 6144, 14335, 14336, T - 1] +
                      list(range(100, T, 1499))))
    qn, kn, vn, don, on = _np(q), _np(k), _np(v), _np(do), _np(out)
    ro, rl = oracle.nsa_fwd(qn, kn, vn, topk, cu, cu, sbs, scale, 2, tokens=toks)
    _close(out, ro, OUT_TOL, "out", rows=toks)
    _lse_close(lse, rl, rows=toks)
    _, _, rvp, rv, nb = oracle.nsa_compact(topk, cu, cu, sbs, 2)
    gb = 32 + 64 + 5                       # block 5 of the 8192-token sequence, KV head 0
    sel = set(toks) | set(rv[rvp[gb]:rvp[gb + 1]].tolist())
    rows = np.zeros(T, bool)
    start = int(cu[2]) + 5 * sbs
    rows[start:start + sbs] = True
    rdq, rdk, rdv = oracle.nsa_bwd(qn, kn, vn, on, don, topk, cu, cu, sbs, scale, 2,
                                   tokens=sorted(sel))
    _close(dq, rdq, GRAD_TOL, "dq", rows=toks)
    _close(dk[:, 0], rdk[:, 0], GRAD_TOL, "dk", rows=rows)
    _close(dv[:, 0], rdv[:, 0], GRAD_TOL, "dv", rows=rows)


def test_fwd_bwd_fp16_duplicates():
    cu, q, k, v, do, topk = _case([256, 128], 16, 2, 32, 4, 80, dtype="fp16")
    topk[10, 0, 1] = topk[10, 0, 0]                # a block listed twice counts twice
    topk[200, 1, 2] = topk[200, 1, 3]
    scale = 0.1
    out, lse, dq, dk, dv = _run(cu, q, k, v, do, topk, 32, scale, 2)
    ro, rl = oracle.nsa_fwd(_np(q), _np(k), _np(v), topk, cu, cu, 32, scale, 2)
    _close(out, ro, OUT_TOL, "out")
    rdq, rdk, rdv = oracle.nsa_bwd(_np(q), _np(k), _np(v), _np(out), _np(do), topk, cu, cu, 32,
                                   scale, 2)
    _close(dq, rdq, GRAD_TOL, "dq")
    _close(dk, rdk, GRAD_TOL, "dk")
    _close(dv, rdv, GRAD_TOL, "dv")


def test_nsa_varlen_full_size_sampled():
    """The full 4-sequence, 32/2-head workload in the timed configuration;
    sampled tokens for out/LSE/dQ; for dK/dV, whole KV blocks with every
    token that selected them."""
    cu, q, k, v, do, topk = W.nsa_inputs()
    w = W.nsa_workload()
    sbs, scale = w["sbs"], 1 / math.sqrt(128)
    out, lse, dq, dk, dv = _run(cu, q, k, v, do, topk, sbs, scale, 2)
    T = int(cu[-1])
    toks = sorted(set([0, 1, 63, 64, 1000, 2047, 2048, 5000, 6143, 6144, 9000, 14335, 14336,
                       T - 1] + list(range(100, T, 997))))
    qn, kn, vn, don, on = _np(q), _np(k), _np(v), _np(do), _np(out)
    ro, rl = oracle.nsa_fwd(qn, kn, vn, topk, cu, cu, sbs, scale, 2, tokens=toks)
    _close(out, ro, OUT_TOL, "out", rows=toks)
    _lse_close(lse, rl, rows=toks)
    # dK/dV of a few blocks: block 0 and block 64 of the 8192-token sequence,
    # the last block of the first sequence, on KV head 1
    _, _, rvp, rv, nb = oracle.nsa_compact(topk, cu, cu, sbs, 2)
    gblocks = [32 + 64 + 0, 32 + 64 + 64, 31]    # global block ids (seqs have 32, 64, 128, 32)
    sel = set(toks)
    rows = np.zeros(T, bool)
    for gb in gblocks:
        r = 1 * nb + gb
        sel.update(rv[rvp[r]:rvp[r + 1]].tolist())
        seq = 0 if gb < 32 else (1 if gb < 96 else 2)
        start = int(cu[seq]) + (gb - [0, 32, 96][seq]) * sbs
        rows[start:start + sbs] = True
    sel = sorted(sel)
    rdq, rdk, rdv = oracle.nsa_bwd(qn, kn, vn, on, don, topk, cu, cu, sbs, scale, 2, tokens=sel)
    _close(dq, rdq, GRAD_TOL, "dq", rows=toks)
    _close(dk[:, 1], rdk[:, 1], GRAD_TOL, "dk", rows=rows)
    _close(dv[:, 1], rdv[:, 1], GRAD_TOL, "dv", rows=rows)


def test_bwd_deterministic_bitwise():
    cu, q, k, v, do, topk = _case([512, 1024], 32, 2, 64, 8, 90)
    a = _run(cu, q, k, v, do, topk, 64, 0.088, 2)
    b = _run(cu, q, k, v, do, topk, 64, 0.088, 2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_validate_reports_out_of_range_ids():
    tsa = _tsa()
    cu, q, k, v, do, topk = _case([128, 128], 4, 2, 32, 2, 95)
    topk[3, 1, 0] = 9                             # sequence of 128 keys has 4 blocks
    dev = torch.device("cuda")
    with pytest.raises(tsa.TsaError) as ei:
        tsa.nsa_select_fwd(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(topk).to(dev),
                           cu, cu, 32, 0.1, 2, validate=True)
    assert ei.value.status == 6


def test_bwd_reusing_forward_lists_matches_fresh_lists():
    """A backward that reuses the forward's per-row lists (building only the
    reverse lists) equals, bit for bit, one that builds every list itself."""
    tsa = _tsa()
    cu, q, k, v, do, topk = _case([512, 1024], 32, 2, 64, 8, 93)
    out, lse, dq, dk, dv = _run(cu, q, k, v, do, topk, 64, 0.088, 2)
    dev = torch.device("cuda")
    plan = tsa.NsaPlan(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(topk).to(dev), cu, cu, 64,
                       0.088, 2)
    plan.set_out(out, lse)
    dq2, dk2, dv2 = plan.bwd(do.to(dev))          # no forward on this plan: builds all lists
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


@pytest.mark.parametrize("seqlens,N1,N2,sbs,sbc", [
    ([8192], 4, 2, 64, 128),          # the largest selection: sbs * sbc = 8K keys per token
    ([2048, 2304], 8, 2, 16, 128),    # the most blocks (128) of the smallest size
    ([2048, 4096], 4, 1, 128, 16),    # the largest block size with many blocks
])
def test_selection_size_limits_sampled(seqlens, N1, N2, sbs, sbc):
    """Block size / count at the operator's limits (block size <= 128, count
    <= 128, product <= 8K): out / LSE / dQ on sampled tokens, dK / dV on the
    last two blocks of each sequence with every token that selected them."""
    cu, q, k, v, do, topk = _case(seqlens, N1, N2, sbs, sbc, 110)
    scale = 1 / math.sqrt(128)
    out, lse, dq, dk, dv = _run(cu, q, k, v, do, topk, sbs, scale, 2)
    T = int(cu[-1])
    toks = sorted(set([0, 1, sbs - 1, sbs, T - 1] + [int(c) for c in cu[1:-1]] +
                      list(range(37, T, 409))))
    qn, kn, vn, don, on = _np(q), _np(k), _np(v), _np(do), _np(out)
    ro, rl = oracle.nsa_fwd(qn, kn, vn, topk, cu, cu, sbs, scale, 2, tokens=toks)
    _close(out, ro, OUT_TOL, "out", rows=toks)
    _lse_close(lse, rl, rows=toks)
    _, _, rvp, rv, nb = oracle.nsa_compact(topk, cu, cu, sbs, 2)
    sel, rows = set(toks), np.zeros(T, bool)
    first = 0                                   # global id of each sequence's first block
    for b, n in enumerate(seqlens):
        nblk = n // sbs
        for blk in (nblk - 2, nblk - 1):
            for n2 in range(N2):
                r = n2 * nb + first + blk
                sel.update(rv[rvp[r]:rvp[r + 1]].tolist())
            rows[int(cu[b]) + blk * sbs:int(cu[b]) + (blk + 1) * sbs] = True
        first += nblk
    rdq, rdk, rdv = oracle.nsa_bwd(qn, kn, vn, on, don, topk, cu, cu, sbs, scale, 2,
                                   tokens=sorted(sel))
    _close(dq, rdq, GRAD_TOL, "dq", rows=toks)
    _close(dk, rdk, GRAD_TOL, "dk", rows=rows)
    _close(dv, rdv, GRAD_TOL, "dv", rows=rows)


def test_unselected_block_is_never_read():
    """Noise in the K/V rows of a block no token selects on one KV head leaves
    O, LSE and dQ bit-identical and that block's dK/dV exactly zero."""
    cu, q, k, v, do, topk = _case([512, 384], 32, 2, 64, 4, 120)
    blk, n2 = 3, 1                               # block 3 of the first sequence, KV head 1
    t = topk[:, n2]
    t[t == blk] = 0 if blk != 0 else 1          # every token that listed it lists block 0 instead
    rows = slice(int(cu[0]) + blk * 64, int(cu[0]) + (blk + 1) * 64)
    r1 = _run(cu, q, k, v, do, topk, 64, 0.088, 2)
    k2, v2 = k.clone(), v.clone()
    k2[rows, n2] = W.normal((64, 128), 97) * 50
    v2[rows, n2] = W.normal((64, 128), 96) * 50
    r2 = _run(cu, q, k2, v2, do, topk, 64, 0.088, 2)
    for i in range(3):
        assert torch.equal(r1[i], r2[i])
    assert torch.equal(r1[3][:, 1 - n2], r2[3][:, 1 - n2])
    assert (r2[3][rows, n2] == 0).all() and (r2[4][rows, n2] == 0).all()


@pytest.mark.parametrize("N1,N2,sbs,sbc", [(32, 2, 32, 3), (8, 2, 16, 4), (4, 4, 48, 2)])
@pytest.mark.parametrize("mode", [0, 2])
def test_ragged_token_groups(N1, N2, sbs, sbc, mode):
    """Query sequences shorter than their key sequences and not a multiple of
    16 tokens (the forward and dQ work on runs of 16 consecutive tokens, so
    these end in partial runs), one query sequence with no tokens, and a
    block listed twice by one token."""
    kvlens = [(sbc + 1) * sbs, (sbc + 3) * sbs, sbc * sbs, (sbc + 2) * sbs]
    qlens = [kvlens[0] - 5, 37, 0, 2 * sbs + 3]
    rng = np.random.default_rng(7)
    full = W.nsa_topk_causal(rng, kvlens, N2, sbs, sbc)
    kcu = np.concatenate([[0], np.cumsum(kvlens)]).astype(np.int32)
    qcu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    topk = np.concatenate([full[kcu[b]:kcu[b] + qlens[b]] for b in range(4)], axis=0)
    topk = np.ascontiguousarray(topk)
    topk[20, 1, 1] = topk[20, 1, 0]
    T, Tk = int(qcu[-1]), int(kcu[-1])
    q = W.normal((T, N1, 128), 131)
    k = W.normal((Tk, N2, 128), 132)
    v = W.normal((Tk, N2, 128), 133)
    do = W.normal((T, N1, 128), 134)
    scale = 1 / math.sqrt(128)
    tsa = _tsa()
    dev = torch.device("cuda")
    plan = tsa.NsaPlan(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(topk).to(dev), qcu, kcu,
                       sbs, scale, mode)
    out, lse = plan.fwd()
    dq, dk, dv = plan.bwd(do.to(dev))
    torch.cuda.synchronize()
    ro, rl = oracle.nsa_fwd(_np(q), _np(k), _np(v), topk, qcu, kcu, sbs, scale, mode)
    _close(out, ro, OUT_TOL, "out")
    _lse_close(lse, rl)
    rdq, rdk, rdv = oracle.nsa_bwd(_np(q), _np(k), _np(v), _np(out), _np(do), topk, qcu, kcu, sbs,
                                   scale, mode)
    _close(dq, rdq, GRAD_TOL, "dq")
    _close(dk, rdk, GRAD_TOL, "dk")
    _close(dv, rdv, GRAD_TOL, "dv")
