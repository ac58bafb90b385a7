"""FloydAttention on the GPU against the float64 CPU oracle (through the C
ABI via the binding).

Tolerances as for the other paths: outputs max|gpu - ref| <= 2e-2 *
max|ref|, gradients <= 3e-2 * max|ref| per tensor, LSE <= 2e-3 *
max(1, max|ref|).
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
    g = _np(gpu) if isinstance(gpu, torch.Tensor) else gpu
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    err, scale = np.abs(g - ref).max(), np.abs(ref).max()
    assert err <= tol * scale, f"{what}: max err {err:.3e} vs {tol} * {scale:.3e}"


def _run(q, k1, v1, k2, v2, do, scale):
    tsa = _tsa()
    d = torch.device("cuda")
    plan = tsa.FloydPlan(*(t.to(d) for t in (q, k1, v1, k2, v2)), scale=scale)
    out, lse = plan.fwd()
    grads = plan.bwd(do.to(d))
    torch.cuda.synchronize()
    return out, lse, grads


def _check(q, k1, v1, k2, v2, do, scale, out, lse, grads, heads=None):
    """Oracle comparison; ``heads`` restricts it to (b, h) pairs (heads are
    independent)."""
    sel = heads if heads is not None else [(b, h) for b in range(q.shape[0])
                                            for h in range(q.shape[1])]
    for b, h in sel:
        s_ = (slice(b, b + 1), slice(h, h + 1))
        args = [_np(t[s_]) for t in (q, k1, v1, k2, v2)]
        ro, rl = oracle.floyd_fwd(*args, scale)
        _close(out[s_], ro, OUT_TOL, f"out[{b},{h}]")
        gl = _np(lse[s_])
        assert np.abs(gl - rl).max() <= LSE_TOL * max(1.0, np.abs(rl).max())
        rg = oracle.floyd_bwd(*args, _np(out[s_]), _np(do[s_]), scale)
        for name, g, r in zip(("dq", "dk1", "dv1", "dk2", "dv2"), grads, rg):
            _close(g[s_], r, GRAD_TOL, f"{name}[{b},{h}]")


@pytest.mark.parametrize("B,H,N,M,K,D,dtype", [
    (1, 2, 16, 128, 128, 32, "bf16"),     # smallest sizes of every axis
    (2, 2, 48, 128, 256, 64, "fp16"),     # N not a multiple of the 64-row tile
    (1, 1, 32, 256, 128, 128, "bf16"),    # widest head
    (1, 3, 80, 128, 384, 64, "bf16"),     # ragged tiles along every product
])
def test_fwd_bwd(B, H, N, M, K, D, dtype):
    q, k1, v1, k2, v2, do = W.floyd_inputs(B, H, N, M, K, D, seed_base=150, dtype=dtype)
    scale = 1 / math.sqrt(D)
    out, lse, grads = _run(q, k1, v1, k2, v2, do, scale)
    _check(q, k1, v1, k2, v2, do, scale, out, lse, grads)


def test_bench_workload_two_heads_and_deterministic():
    """The timed 1 x 8 x 256 x 256 x 256 x 64 workload: heads 0 and 5 in
    full against the oracle (heads are independent), bit-identical reruns."""
    q, k1, v1, k2, v2, do = W.floyd_inputs()
    w = W.floyd_workload()
    scale = 1 / math.sqrt(w["D"])
    a = _run(q, k1, v1, k2, v2, do, scale)
    b = _run(q, k1, v1, k2, v2, do, scale)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x, y)
    _check(q, k1, v1, k2, v2, do, scale, a[0], a[1], a[2], heads=[(0, 0), (0, 5)])


def test_second_pair_zero_is_plain_attention_per_row_block():
    """With key2 = value2 = 0 each (b, h, n) is dense attention of q[b,h,n]
    over key1/value1[b,h,n]: compare with torch's float32 attention."""
    q, k1, v1, k2, v2, do = W.floyd_inputs(1, 2, 16, 128, 128, 64, seed_base=160)
    k2.zero_()
    v2.zero_()
    out, lse, _ = _run(q, k1, v1, k2, v2, do, 0.125)
    qq, kk, vv = (t.float().reshape(-1, t.shape[3], t.shape[4]) for t in (q, k1, v1))
    ref = torch.softmax(0.125 * qq @ kk.transpose(1, 2), -1) @ vv
    _close(out.reshape(ref.shape), ref.double().numpy(), OUT_TOL, "out")
