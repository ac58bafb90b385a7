"""Block-sparse attention with an element mask (atten_mask) on the GPU
against the float64 CPU oracle.

atten_mask: u8, non-zero = the score is excluded, [Sq, Skv] or
[B|1, N1|1, Sq, Skv].  Tolerances as for the other BSA tests: outputs
<= 2e-2 * max|ref|, gradients <= 3e-2 * max|ref|, LSE <= 2e-3 * max(1, |ref|).
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


def _close(gpu, ref, tol, what):
    g = _np(gpu)
    scale = np.abs(ref).max()
    err = np.abs(g - ref).max()
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    assert err <= tol * max(scale, 1e-30), f"{what}: max err {err:.3e} vs {tol} * {scale:.3e}"


def _lse_close(gpu, ref):
    g = _np(gpu)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(g)), "LSE: -inf pattern differs"
    if fin.any():
        err = np.abs(g[fin] - ref[fin]).max()
        assert err <= LSE_TOL * max(1.0, np.abs(ref[fin]).max()), err


def _random_am(rng, shape, p):
    """Exclusions with probability p, stored as assorted non-zero byte values."""
    vals = rng.choice(np.array([1, 7, 128, 255], np.uint8), size=shape)
    return np.where(rng.random(shape) < p, vals, 0).astype(np.uint8)


def _run(q, k, v, do, mask, bq, bkv, scale, mode, am_t, **seq):
    tsa = _tsa()
    qd, kd, vd, dod = (torch.as_tensor(t).cuda() for t in (q, k, v, do))
    plan = tsa.BsaPlan(qd, kd, vd, torch.from_numpy(mask).cuda(), bq, bkv, scale, mode,
                       atten_mask=am_t, **seq)
    out, lse = plan.fwd()
    dq, dk, dv = plan.bwd(dod)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _case(B, N1, N2, Sq, Skv, bq, bkv, mode, dtype, seed, am_shape, p_el=0.3, empty_rows=(),
          expand=False):
    dt = "bf16" if dtype == torch.bfloat16 else "fp16"
    rng = np.random.default_rng(seed)
    q = W.normal((B, N1, Sq, 128), seed + 1, dt)
    k = W.normal((B, N2, Skv, 128), seed + 2, dt)
    v = W.normal((B, N2, Skv, 128), seed + 3, dt)
    do = W.normal((B, N1, Sq, 128), seed + 4, dt)
    QB, KB = -(-Sq // bq), -(-Skv // bkv)
    mask = (rng.random((B, N1, QB, KB)) < 0.5).astype(np.uint8)
    for i in range(min(QB, KB)):
        mask[:, :, i, i] = 1
    am = _random_am(rng, am_shape, p_el)
    for r in empty_rows:                      # rows every key of which is excluded
        am[..., r, :] = 1
    am_t = torch.from_numpy(am).cuda()
    if expand:
        am_t = am_t.expand(B, N1, Sq, Skv)    # stride-0 batch / head axes
    scale = 1 / math.sqrt(128)
    out, lse, dq, dk, dv = _run(q, k, v, do, mask, bq, bkv, scale, mode, am_t)
    qn, kn, vn, don = _np(q), _np(k), _np(v), _np(do)
    ro, rl = oracle.bsa_fwd(qn, kn, vn, mask, bq, bkv, scale, mode, atten_mask=am)
    _close(out, ro, OUT_TOL, "out")
    _lse_close(lse, rl)
    rdq, rdk, rdv = oracle.bsa_bwd(qn, kn, vn, _np(out), don, mask, bq, bkv, scale, mode,
                                   atten_mask=am)
    _close(dq, rdq, GRAD_TOL, "dq")
    _close(dk, rdk, GRAD_TOL, "dk")
    _close(dv, rdv, GRAD_TOL, "dv")
    for r in empty_rows:
        assert torch.all(out[:, :, r] == 0) and torch.all(torch.isneginf(lse[:, :, r]))
        assert torch.all(dq[:, :, r] == 0)


@pytest.mark.parametrize("mode", [0, 2])
def test_per_head_mask_gqa_128(mode):
    _case(1, 4, 2, 512, 512, 128, 128, mode, torch.bfloat16, 600, (1, 4, 512, 512))


@pytest.mark.parametrize("mode", [0, 2])
def test_shared_mask_ragged_unaligned_rows(mode):
    # Skv = 333: mask rows are not 4-byte multiples, entries are read bytewise
    _case(1, 2, 2, 300, 333, 64, 64, mode, torch.bfloat16, 610, (300, 333))


def test_per_batch_mask_block_48():
    # 48-key blocks: chunk starts stay 4-byte aligned, chunks end mid-block
    _case(2, 2, 1, 400, 400, 64, 48, 0, torch.bfloat16, 620, (2, 1, 400, 400))


def test_block_50_fp16_causal():
    # 50-key blocks: chunk starts are not 4-byte aligned
    _case(1, 2, 1, 260, 260, 32, 50, 2, torch.float16, 630, (1, 2, 260, 260))


def test_expanded_stride0_mask():
    _case(2, 4, 4, 256, 256, 128, 128, 0, torch.bfloat16, 640, (1, 1, 256, 256), expand=True)


def test_dense_mask_rows_fully_excluded():
    # rows 3 and 200 lose every key: Out 0, LSE -inf, zero dQ
    _case(1, 2, 1, 256, 256, 64, 64, 0, torch.bfloat16, 650, (1, 2, 256, 256), p_el=0.6,
          empty_rows=(3, 200))


def test_zero_mask_is_bitwise_no_mask():
    """An all-zero atten_mask runs the masked kernels to the same bits as no
    mask at all."""
    rng = np.random.default_rng(660)
    B, N1, N2, S, bq = 1, 4, 2, 512, 128
    q, k, v, do = (W.normal((B, n, S, 128), 661 + i, "bf16")
                   for i, n in enumerate((N1, N2, N2, N1)))
    mask = W.mask_random(rng, B, N1, S // bq, S // bq, 0.5, causal=True)
    zero = torch.zeros(S, S, dtype=torch.uint8, device="cuda")
    a = _run(q, k, v, do, mask, bq, bq, 0.088, 2, zero)
    b = _run(q, k, v, do, mask, bq, bq, 0.088, 2, None)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_upper_triangle_mask_matches_causal_mode():
    rng = np.random.default_rng(670)
    B, N1, N2, S, bq = 1, 2, 2, 384, 64
    q, k, v, do = (W.normal((B, n, S, 128), 671 + i, "bf16")
                   for i, n in enumerate((N1, N2, N2, N1)))
    mask = W.mask_random(rng, B, N1, S // bq, S // bq, 0.6, causal=True)
    tri = torch.ones(S, S, dtype=torch.bool, device="cuda").triu(1)
    a = _run(q, k, v, do, mask, bq, bq, 0.088, 0, tri)
    b = _run(q, k, v, do, mask, bq, bq, 0.088, 2, None)
    for x, y, tol in zip(a, b, (OUT_TOL, None, GRAD_TOL, GRAD_TOL, GRAD_TOL)):
        if tol is None:
            _lse_close(x, _np(y))
        else:
            _close(x, _np(y), tol / 4, "mask vs causal")


def test_bwd_deterministic_with_mask():
    rng = np.random.default_rng(680)
    B, N1, N2, S, bq = 1, 8, 2, 1024, 128
    q, k, v, do = (W.normal((B, n, S, 128), 681 + i, "bf16")
                   for i, n in enumerate((N1, N2, N2, N1)))
    mask = W.mask_random(rng, B, N1, S // bq, S // bq, 0.5, causal=True)
    mask[:, :, :, 0] = 1                      # long reverse lists: split dK/dV
    am = torch.from_numpy(_random_am(rng, (S, S), 0.2)).cuda()
    a = _run(q, k, v, do, mask, bq, bq, 0.088, 0, am)
    b = _run(q, k, v, do, mask, bq, bq, 0.088, 0, am)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("mode", [0, 2])
def test_tnd_varlen_with_mask(mode):
    """TND sequences of different lengths: mask positions count from each
    sequence's start, in [Sq, Skv] planes of the longest lengths."""
    tsa = _tsa()
    lens_q, lens_kv, N1, N2, bq, bkv, seed = [200, 77, 333], [150, 90, 333], 4, 2, 64, 64, 690
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int32)
    T, Tk, B = int(cq[-1]), int(ck[-1]), len(lens_q)
    Sq, Skv = max(lens_q), max(lens_kv)
    rng = np.random.default_rng(seed)
    q = W.normal((T, N1, 128), seed + 1, "bf16")
    k = W.normal((Tk, N2, 128), seed + 2, "bf16")
    v = W.normal((Tk, N2, 128), seed + 3, "bf16")
    do = W.normal((T, N1, 128), seed + 4, "bf16")
    QB, KB = -(-Sq // bq), -(-Skv // bkv)
    mask = (rng.random((B, N1, QB, KB)) < 0.6).astype(np.uint8)
    am = _random_am(rng, (B, N1, Sq, Skv), 0.3)
    scale = 1 / math.sqrt(128)
    qd, kd, vd, dod = (torch.as_tensor(t).cuda() for t in (q, k, v, do))
    plan = tsa.BsaPlan(qd, kd, vd, torch.from_numpy(mask).cuda(), bq, bkv, scale, mode,
                       cu_seqlens_q=cq, cu_seqlens_kv=ck, atten_mask=torch.from_numpy(am).cuda())
    out, lse = plan.fwd()
    dq, dk, dv = plan.bwd(dod)
    torch.cuda.synchronize()
    qn, kn, vn, don = _np(q), _np(k), _np(v), _np(do)
    ro, rl = oracle.bsa_fwd_tnd(qn, kn, vn, mask, cq, ck, bq, bkv, scale, mode, atten_mask=am)
    _close(out, ro, OUT_TOL, "out")
    _lse_close(lse, rl)
    rdq, rdk, rdv = oracle.bsa_bwd_tnd(qn, kn, vn, _np(out), don, mask, cq, ck, bq, bkv, scale,
                                       mode, atten_mask=am)
    _close(dq, rdq, GRAD_TOL, "dq")
    _close(dk, rdk, GRAD_TOL, "dk")
    _close(dv, rdv, GRAD_TOL, "dv")
