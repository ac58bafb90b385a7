"""Block-sparse attention on the GPU against the float64 CPU oracle.

Tolerances: outputs max|gpu - ref| <= 2e-2 * max|ref|, gradients <= 3e-2 *
max|ref| per tensor, LSE <= 2e-3 * max(1, max|ref|); lists bit-exact.
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
    g = _np(gpu) if isinstance(gpu, torch.Tensor) else gpu
    if rows is not None:
        g, ref = g[rows], ref[rows]
    scale = np.abs(ref).max()
    err = np.abs(g - ref).max()
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    assert err <= tol * max(scale, 1e-30), f"{what}: max err {err:.3e} vs {tol} * {scale:.3e}"


def _lse_close(gpu, ref, rows=None):
    g = _np(gpu)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(g)), "LSE: -inf pattern differs"
    err = np.abs(g[fin] - ref[fin]).max() if fin.any() else 0.0
    assert err <= LSE_TOL * max(1.0, np.abs(ref[fin]).max() if fin.any() else 1.0), err


def _inputs(B, N1, N2, Sq, Skv, dtype, seed, mask_fn):
    dt = "bf16" if dtype == torch.bfloat16 else "fp16"
    q = W.normal((B, N1, Sq, 128), seed + 1, dt)
    k = W.normal((B, N2, Skv, 128), seed + 2, dt)
    v = W.normal((B, N2, Skv, 128), seed + 3, dt)
    do = W.normal((B, N1, Sq, 128), seed + 4, dt)
    mask = mask_fn(np.random.default_rng(seed))
    return q, k, v, do, mask


def _dev(*ts):
    return [torch.as_tensor(t).cuda() for t in ts]


# ----------------------------------------------------------------------------
# Compaction: bit-exact
# ----------------------------------------------------------------------------

def _compact_case(mask, N2, Sq, Skv, bq, bkv):
    tsa = _tsa()
    rp, col, rvp, rv = tsa.bsa_compact(torch.from_numpy(mask).cuda(), N2, Sq, Skv, bq, bkv)
    erp, ecol, ervp, erv = oracle.bsa_compact(mask, N2)
    assert np.array_equal(rp.cpu().numpy(), erp)
    assert np.array_equal(col.cpu().numpy(), ecol)
    assert np.array_equal(rvp.cpu().numpy(), ervp)
    assert np.array_equal(rv.cpu().numpy(), erv)


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_compact_named_workloads_bit_exact(cfg):
    w = W.bsa_workload(cfg)
    mask = W.bsa_mask(w, 1000 + cfg)
    _compact_case(mask, w["N2"], w["S"], w["S"], w["bq"], w["bkv"])


@pytest.mark.parametrize("shape,n2,bq,bkv,S", [
    ((1, 1, 1, 1), 1, 64, 64, 64),          # a single block
    ((2, 4, 3, 70), 2, 16, 16, None),        # GQA, columns not a multiple of 64
    ((1, 2, 130, 5), 1, 16, 16, None),       # rows spanning several row tiles
    ((1, 3, 7, 129), 3, 32, 32, None),       # ragged both ways
])
def test_compact_edge_cases_bit_exact(shape, n2, bq, bkv, S):
    rng = np.random.default_rng(7)
    mask = (rng.random(shape) < 0.3).astype(np.uint8)
    mask[0, 0, 0] = 0                         # an empty row
    B, N1, QB, KB = shape
    Sq, Skv = (S, S) if S else (QB * bq - 3 if QB * bq > 3 else QB * bq, KB * bkv - 5)
    _compact_case(mask, n2, Sq, Skv, bq, bkv)
    full = np.ones(shape, np.uint8)           # a full mask
    _compact_case(full, n2, Sq, Skv, bq, bkv)


# ----------------------------------------------------------------------------
# Forward parity
# ----------------------------------------------------------------------------

def _fwd_check(q, k, v, mask, bq, bkv, scale, mode, q_tiles=None):
    tsa = _tsa()
    qd, kd, vd, md = _dev(q, k, v, torch.from_numpy(mask))
    out, lse = tsa.bsa_fwd(qd, kd, vd, md, bq, bkv, scale, mode)
    torch.cuda.synchronize()
    ro, rl = oracle.bsa_fwd(_np(q), _np(k), _np(v), mask, bq, bkv, scale, mode, q_tiles=q_tiles)
    rows = None
    if q_tiles is not None:
        sel = np.zeros(ro.shape[:3], bool)
        for b, n, qb in q_tiles:
            sel[b, n, qb * bq:(qb + 1) * bq] = True
        rows = sel
    _close(out, ro, OUT_TOL, "out", rows)
    _lse_close(lse, rl, rows)
    return out, lse


def test_fwd_bsa_small_fp16_64x64():
    w, q, k, v, do, mask, scale = W.bsa_inputs(1)
    _fwd_check(q, k, v, mask, 64, 64, scale, 0)


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_fwd_causal_shaped_128_several_tiles(mode, dtype):
    # config-2 structure at a size the oracle finishes in seconds
    q, k, v, do, mask = _inputs(1, 2, 2, 1024, 1024, dtype, 200,
                                lambda r: W.mask_random(r, 1, 2, 8, 8, 0.25, causal=True))
    _fwd_check(q, k, v, mask, 128, 128, 1 / math.sqrt(128), mode)


@pytest.mark.parametrize("Sq,Skv,bq,bkv,N1,N2", [
    (1000, 1000, 128, 128, 2, 2),   # ragged tail on both axes
    (300, 520, 64, 96, 4, 2),       # GQA, rectangular, block_kv not a multiple of 64
    (200, 200, 256, 32, 1, 1),      # block_q larger than a workgroup slice, small block_kv
    (77, 150, 48, 80, 2, 1),        # odd block sizes
])
def test_fwd_ragged_and_gqa(Sq, Skv, bq, bkv, N1, N2):
    QB, KB = -(-Sq // bq), -(-Skv // bkv)
    q, k, v, do, mask = _inputs(1, N1, N2, Sq, Skv, torch.bfloat16, 300,
                                lambda r: W.mask_random(r, 1, N1, QB, KB, 0.4, diagonal=False))
    mask[0, 0, 0, :] = 0            # an empty Q block: out 0, lse -inf
    for mode in (0, 2):
        _fwd_check(q, k, v, mask, bq, bkv, 0.09, mode)


def test_fwd_empty_inputs():
    tsa = _tsa()
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((1, 2, 0, 0), dtype=torch.uint8, device="cuda")
    out, lse = tsa.bsa_fwd(q, k, k, m, 64, 64)
    assert out.shape == q.shape and lse.shape == (1, 2, 0)


def test_fwd_bsa_causal_8k_sampled():
    """The full 2x16x8192 workload in the timed launch configuration; every
    16th Q block of each head plus the first and last are checked."""
    w, q, k, v, do, mask, scale = W.bsa_inputs(2)
    QB = w["S"] // w["bq"]
    tiles = [(b, n, qb) for b in range(w["B"]) for n in range(w["N1"])
             for qb in sorted(set(list(range(0, QB, 16)) + [QB - 1]))]
    tiles = tiles[::4]              # a quarter of those keeps the oracle to seconds
    _fwd_check(q, k, v, mask, w["bq"], w["bkv"], scale, 0, q_tiles=tiles)


# ----------------------------------------------------------------------------
# Backward parity, determinism, perturbation
# ----------------------------------------------------------------------------

def _bwd_gpu(q, k, v, do, mask, bq, bkv, scale, mode):
    tsa = _tsa()
    qd, kd, vd, dod, md = _dev(q, k, v, do, torch.from_numpy(mask))
    plan = tsa.BsaPlan(qd, kd, vd, md, bq, bkv, scale, mode)
    out, lse = plan.fwd()
    dq, dk, dv = plan.bwd(dod)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _bwd_check(q, k, v, do, mask, bq, bkv, scale, mode, q_tiles=None, kv_rows=None):
    out, lse, dq, dk, dv = _bwd_gpu(q, k, v, do, mask, bq, bkv, scale, mode)
    rdq, rdk, rdv = oracle.bsa_bwd(_np(q), _np(k), _np(v), _np(out), _np(do), mask, bq, bkv,
                                   scale, mode, q_tiles=q_tiles)
    qrows = None
    if q_tiles is not None:
        qrows = np.zeros(rdq.shape[:3], bool)
        for b, n, qb in q_tiles:
            qrows[b, n, qb * bq:(qb + 1) * bq] = True
    _close(dq, rdq, GRAD_TOL, "dq", qrows)
    _close(dk, rdk, GRAD_TOL, "dk", kv_rows)
    _close(dv, rdv, GRAD_TOL, "dv", kv_rows)


def test_bwd_bsa_small_fp16_64x64():
    w, q, k, v, do, mask, scale = W.bsa_inputs(1)
    _bwd_check(q, k, v, do, mask, 64, 64, scale, 0)


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_bwd_causal_shaped_128_several_tiles(mode, dtype):
    q, k, v, do, mask = _inputs(1, 2, 2, 1024, 1024, dtype, 400,
                                lambda r: W.mask_random(r, 1, 2, 8, 8, 0.25, causal=True))
    _bwd_check(q, k, v, do, mask, 128, 128, 1 / math.sqrt(128), mode)


@pytest.mark.parametrize("Sq,Skv,bq,bkv,N1,N2", [
    (1000, 1000, 128, 128, 2, 2),
    (300, 520, 64, 96, 4, 2),
    (200, 200, 256, 32, 1, 1),
    (77, 150, 48, 80, 2, 1),
    (256, 384, 128, 192, 2, 2),     # block_kv spanning two dK/dV workgroups
])
def test_bwd_ragged_and_gqa(Sq, Skv, bq, bkv, N1, N2):
    QB, KB = -(-Sq // bq), -(-Skv // bkv)
    q, k, v, do, mask = _inputs(1, N1, N2, Sq, Skv, torch.bfloat16, 500,
                                lambda r: W.mask_random(r, 1, N1, QB, KB, 0.4, diagonal=False))
    mask[0, 0, 0, :] = 0
    if KB > 1:
        mask[:, :, :, KB - 1] = 0   # a KV block nobody selects: dK = dV = 0
    for mode in (0, 2):
        _bwd_check(q, k, v, do, mask, bq, bkv, 0.09, mode)


def test_bwd_bsa_causal_8k_sampled():
    """Full 2x16x8192 workload: dQ on sampled Q blocks; dK/dV on sampled KV
    blocks, each with every Q block on its reverse list included."""
    w, q, k, v, do, mask, scale = W.bsa_inputs(2)
    bq = w["bq"]
    QB = w["S"] // bq
    heads = [(0, 0), (1, 7), (1, 15)]
    kv_blocks = [0, 31, QB - 1]
    tiles = set()
    kv_rows = np.zeros((w["B"], w["N2"], w["S"]), bool)
    for b, n in heads:
        for qb in (0, QB // 2, QB - 1):
            tiles.add((b, n, qb))
        for kb in kv_blocks:
            kv_rows[b, n, kb * bq:(kb + 1) * bq] = True
            for qb in np.nonzero(mask[b, n, :, kb])[0]:
                tiles.add((b, n, int(qb)))
    _bwd_check(q, k, v, do, mask, bq, w["bkv"], scale, 0, q_tiles=sorted(tiles), kv_rows=kv_rows)


def test_bsa_window_128k_sampled():
    """The full 1x8x131072 window workload (8-block window + 24 random
    earlier blocks per Q block) in the timed launch configuration: out / LSE
    / dQ on sampled Q blocks; dK / dV on KV blocks 0, 512 and 1023 of two
    heads, each with every Q block on its reverse list."""
    w, q, k, v, do, mask, scale = W.bsa_inputs(5)
    bq = w["bq"]
    QB = w["S"] // bq
    tiles = set()
    kv_rows = np.zeros((w["B"], w["N2"], w["S"]), bool)
    for b, n in [(0, 0), (0, 7)]:
        for qb in (0, 511, QB - 1):
            tiles.add((b, n, qb))
        for kb in (0, 512, QB - 1):
            kv_rows[b, n, kb * bq:(kb + 1) * bq] = True
            for qb in np.nonzero(mask[b, n, :, kb])[0]:
                tiles.add((b, n, int(qb)))
    tiles = sorted(tiles)
    out, lse, dq, dk, dv = _bwd_gpu(q, k, v, do, mask, bq, w["bkv"], scale, 0)
    qn, kn, vn = _np(q), _np(k), _np(v)
    ro, rl = oracle.bsa_fwd(qn, kn, vn, mask, bq, w["bkv"], scale, 0, q_tiles=tiles)
    qrows = np.zeros(ro.shape[:3], bool)
    for b, n, qb in tiles:
        qrows[b, n, qb * bq:(qb + 1) * bq] = True
    _close(out, ro, OUT_TOL, "out", qrows)
    _lse_close(lse, rl, qrows)
    rdq, rdk, rdv = oracle.bsa_bwd(qn, kn, vn, _np(out), _np(do), mask, bq, w["bkv"], scale, 0,
                                   q_tiles=tiles)
    _close(dq, rdq, GRAD_TOL, "dq", qrows)
    _close(dk, rdk, GRAD_TOL, "dk", kv_rows)
    _close(dv, rdv, GRAD_TOL, "dv", kv_rows)


def test_bwd_deterministic_bitwise():
    """Two backward runs give bit-identical gradients (no atomics)."""
    w, q, k, v, do, mask, scale = W.bsa_inputs(2)
    tsa = _tsa()
    qd, kd, vd, dod, md = _dev(q, k, v, do, torch.from_numpy(mask))
    plan = tsa.BsaPlan(qd, kd, vd, md, w["bq"], w["bkv"], scale, 0)
    plan.fwd()
    g1 = [t.clone() for t in plan.bwd(dod)]
    g2 = [t.clone() for t in plan.bwd(dod)]
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode", [0, 2])
def test_unselected_blocks_are_never_read(mode):
    """Noise in KV blocks nobody selects leaves O, LSE and dQ bit-identical and
    their dK/dV exactly zero."""
    B, N, S, bq = 1, 2, 1024, 128
    q, k, v, do, mask = _inputs(B, N, N, S, S, torch.bfloat16, 600,
                                lambda r: W.mask_random(r, B, N, 8, 8, 0.3, causal=True))
    mask[:, :, :, 3] = 0
    mask[:, :, 3, 3] = 0
    r1 = _bwd_gpu(q, k, v, do, mask, bq, bq, 0.088, mode)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 3 * bq:4 * bq] = W.normal((B, N, bq, 128), 99) * 50
    v2[:, :, 3 * bq:4 * bq] = W.normal((B, N, bq, 128), 98) * 50
    r2 = _bwd_gpu(q, k2, v2, do, mask, bq, bq, 0.088, mode)
    for i in range(3):
        assert torch.equal(r1[i], r2[i])
    sel = torch.ones(S, dtype=torch.bool)
    sel[3 * bq:4 * bq] = False
    assert torch.equal(r1[3][:, :, sel], r2[3][:, :, sel])
    assert torch.equal(r1[4][:, :, sel], r2[4][:, :, sel])
    assert (r2[3][:, :, ~sel] == 0).all() and (r2[4][:, :, ~sel] == 0).all()


def test_bwd_reusing_forward_lists_matches_fresh_lists():
    """A backward that reuses the lists the forward built in the shared
    workspace equals, bit for bit, one that builds them itself."""
    w, q, k, v, do, mask, scale = W.bsa_inputs(2)
    tsa = _tsa()
    qd, kd, vd, dod, md = _dev(q, k, v, do, torch.from_numpy(mask))
    plan = tsa.BsaPlan(qd, kd, vd, md, w["bq"], w["bkv"], scale, 0)
    plan.set_dout(dod)
    out, lse = plan.fwd()
    g1 = [t.clone() for t in plan.bwd()]            # reuses the forward's lists
    fresh = tsa.BsaPlan(qd, kd, vd, md, w["bq"], w["bkv"], scale, 0)
    fresh.set_out(out, lse)
    g2 = fresh.bwd(dod)                             # builds its own lists
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------
# TND (variable-length sequences)
# ----------------------------------------------------------------------------

def _tnd_case(lens_q, lens_kv, N1, N2, bq, bkv, mode, dtype, seed, p=0.5):
    """Ragged sequences; the mask is padded to the longest sequence and holds
    random entries past each sequence's end too (they must be ignored)."""
    tsa = _tsa()
    dt = "bf16" if dtype == torch.bfloat16 else "fp16"
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int32)
    T, Tk, B = int(cq[-1]), int(ck[-1]), len(lens_q)
    Sq, Skv = max(lens_q), max(lens_kv)
    q = W.normal((T, N1, 128), seed + 1, dt)
    k = W.normal((Tk, N2, 128), seed + 2, dt)
    v = W.normal((Tk, N2, 128), seed + 3, dt)
    do = W.normal((T, N1, 128), seed + 4, dt)
    QB, KB = -(-Sq // bq), -(-Skv // bkv)
    mask = (np.random.default_rng(seed).random((B, N1, QB, KB)) < p).astype(np.uint8)
    for i in range(min(QB, KB)):
        mask[:, :, i, i] = 1
    scale = 1 / math.sqrt(128)
    qd, kd, vd, dod = _dev(q, k, v, do)
    plan = tsa.BsaPlan(qd, kd, vd, torch.from_numpy(mask).cuda(), bq, bkv, scale, mode,
                       cu_seqlens_q=cq, cu_seqlens_kv=ck)
    out, lse = plan.fwd()
    dq, dk, dv = plan.bwd(dod)
    torch.cuda.synchronize()
    qn, kn, vn, don = _np(q), _np(k), _np(v), _np(do)
    ro, rl = oracle.bsa_fwd_tnd(qn, kn, vn, mask, cq, ck, bq, bkv, scale, mode)
    _close(out, ro, OUT_TOL, "out")
    _lse_close(lse, rl)
    rdq, rdk, rdv = oracle.bsa_bwd_tnd(qn, kn, vn, _np(out), don, mask, cq, ck, bq, bkv, scale,
                                       mode)
    _close(dq, rdq, GRAD_TOL, "dq")
    _close(dk, rdk, GRAD_TOL, "dk")
    _close(dv, rdv, GRAD_TOL, "dv")


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("lens_q,lens_kv,N1,N2,bq,bkv", [
    ([200, 512, 77], [200, 512, 77], 4, 2, 64, 64),      # GQA, tails in every sequence
    ([300, 1000, 129], [300, 1000, 129], 2, 2, 128, 128),
    ([64, 0, 100], [64, 0, 100], 2, 1, 32, 48),          # an empty sequence, odd block size
    ([100, 300], [250, 180], 4, 4, 64, 32),              # query and key lengths differ
])
def test_tnd_varlen_fwd_bwd(lens_q, lens_kv, N1, N2, bq, bkv, mode):
    _tnd_case(lens_q, lens_kv, N1, N2, bq, bkv, mode, torch.bfloat16, 500)


def test_tnd_varlen_fp16():
    _tnd_case([130, 257], [130, 257], 2, 2, 64, 64, 2, torch.float16, 510)


def test_tnd_varlen_workload_sampled():
    """The full TND workload (sequences of 2048, 4096, 8192, 2048 tokens, 16
    query / 4 KV heads, 128x128 blocks) in the timed launch configuration:
    out / LSE / dQ on sampled Q blocks; dK / dV on sampled KV blocks of a KV
    head, with every Q block of its 4 query heads that selected them."""
    tsa = _tsa()
    w = W.bsa_tnd_workload()
    cu, q, k, v, do, mask = W.bsa_tnd_inputs()
    bq, bkv, scale = w["bq"], w["bkv"], 1 / math.sqrt(128)
    qd, kd, vd, dod = _dev(q, k, v, do)
    plan = tsa.BsaPlan(qd, kd, vd, torch.from_numpy(mask).cuda(), bq, bkv, scale, 0,
                       cu_seqlens_q=cu, cu_seqlens_kv=cu)
    out, lse = plan.fwd()
    dq, dk, dv = plan.bwd(dod)
    torch.cuda.synchronize()
    G = w["N1"] // w["N2"]
    tiles = set()
    qrows = np.zeros((int(cu[-1]), w["N1"]), bool)
    kv_rows = np.zeros((int(cu[-1]), w["N2"]), bool)
    for b, n2, kb in [(0, 0, 0), (2, 3, 0), (2, 3, 63), (1, 1, 17)]:
        kv_rows[cu[b] + kb * bkv:cu[b] + (kb + 1) * bkv, n2] = True
        for n1 in range(n2 * G, (n2 + 1) * G):
            for qb in np.nonzero(mask[b, n1, :, kb])[0]:
                tiles.add((b, n1, int(qb)))
    for b, n1, qb in [(0, 0, 0), (2, 15, 63), (3, 5, 15), (1, 9, 31)]:
        tiles.add((b, n1, qb))
    tiles = sorted(tiles)
    for b, n1, qb in tiles:
        qrows[cu[b] + qb * bq:cu[b] + (qb + 1) * bq, n1] = True
    qn, kn, vn, don = _np(q), _np(k), _np(v), _np(do)
    ro, rl = oracle.bsa_fwd_tnd(qn, kn, vn, mask, cu, cu, bq, bkv, scale, 0, q_tiles=tiles)
    _close(out, ro, OUT_TOL, "out", qrows)
    _lse_close(lse, rl, qrows)
    rdq, rdk, rdv = oracle.bsa_bwd_tnd(qn, kn, vn, _np(out), don, mask, cu, cu, bq, bkv, scale, 0,
                                       q_tiles=tiles)
    _close(dq, rdq, GRAD_TOL, "dq", qrows)
    _close(dk, rdk, GRAD_TOL, "dk", kv_rows)
    _close(dv, rdv, GRAD_TOL, "dv", kv_rows)


@pytest.mark.parametrize("mode", [0, 2])
def test_bwd_shared_block_long_reverse_lists(mode):
    """A KV block every Q block of every head selects (an attention-sink
    pattern) under GQA: its reverse list is split into segments whose fp32
    partials are reduced in order; dK/dV match the oracle and reruns are
    bit-identical."""
    B, N1, N2, S, bq = 1, 8, 2, 2048, 128
    QB = S // bq

    def mask_fn(rng):
        m = W.mask_random(rng, B, N1, QB, QB, 0.2, causal=True)
        m[:, :, :, 0] = 1
        return m

    q, k, v, do, mask = _inputs(B, N1, N2, S, S, torch.bfloat16, 520, mask_fn)
    _bwd_check(q, k, v, do, mask, bq, bq, 1 / math.sqrt(128), mode)
    a = _bwd_gpu(q, k, v, do, mask, bq, bq, 1 / math.sqrt(128), mode)
    b = _bwd_gpu(q, k, v, do, mask, bq, bq, 1 / math.sqrt(128), mode)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_misaligned_tensor_is_refused_before_launch():
    """A contiguous view at an odd element offset is not 16-byte aligned: the
    binding refuses it, and so does the C ABI (status 2) if called directly."""
    import ctypes
    tsa = _tsa()
    B, N, S, D, bq = 1, 2, 256, 128, 128
    n = B * N * S * D
    base = torch.zeros(n + 8, dtype=torch.bfloat16, device="cuda")
    q_bad = base[1:n + 1].view(B, N, S, D)                 # 2 bytes past a 16-byte boundary
    k = torch.zeros(B, N, S, D, dtype=torch.bfloat16, device="cuda")
    mask = torch.ones(B, N, S // bq, S // bq, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="16-byte"):
        tsa.bsa_fwd(q_bad, k, k, mask, bq, bq)
    plan = tsa.BsaPlan(k, k, k, mask, bq, bq, 0.088, 0, backward=False)
    plan.fa.q = q_bad.data_ptr()
    n_ws = ctypes.c_size_t()
    assert tsa.lib.bsa_fwd_workspace_size(ctypes.byref(plan.fa), ctypes.byref(n_ws)) == 2
