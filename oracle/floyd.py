"""Plain float64 definition of FloydAttention, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

"aclnnFusedFloydAttentionGrad", function description and formula section:
the query is a 5-D tensor whose two sequence axes are both kept; the scores of
query row (n, m) against key index k are the sum of two batched products,
one batched over the first sequence axis and one over the second ("the
sequence dimension is treated as an additional batch axis ... batch matrix
multiplication"):

    S = Mask(scale * (Q K1^T + Q K2^T)),  P = Softmax(S),  Y = P V1 + P V2

and the backward chain dV1 = P^T dY, dV2 = P^T dY, dQ = (dS K1 + dS K2)
scale, dK1 = dS^T Q scale, dK2 = dS^T Q scale, with dS the softmax backward
of dP = dY V1^T + dY V2^T.

Readings (the page's tensor-shape table is lost):

* query [B, H, N, M, D]; key1 / value1 [B, H, N, K, D]; key2 / value2
  [B, H, M, K, D].  The page fixes that axes 0, 2 and 4 of query and key1
  agree (B, N, D) and that key1/value1 and key2/value2 share shapes; key2's
  batch axis is the query's second sequence axis M.  So
  S[b,h,n,m,k] = scale * (q[b,h,n,m] . k1[b,h,n,k] + q[b,h,n,m] . k2[b,h,m,k]).
* The softmax runs over k; the product Q K1^T is batched over (b, h, n) and
  Q K2^T over (b, h, m).
* The page's backward divides by sqrt(d) where the forward multiplies by
  scale: read as the same scale (1/sqrt(D) by default).
* No atten_mask (the Mask operand's layout is not given; every entry kept).
* The forward keeps one fp32 natural-log LSE per query row (the page keeps
  softmaxMax and softmaxSum; LSE = max + ln(sum) carries the same).
* softmax_grad of a row = sum_d dY * Y (as for block-sparse attention).

Parity status: pinned in tests/test_oracle_pins.py (each branch alone is
dense attention batched over its axis, finite differences of every input,
the N <-> M transpose symmetry, constant values, rows of P summing to 1).
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _scores(q, k1, k2, scale):
    """S [B, H, N, M, K]: Q K1^T batched over (b, h, n) plus Q K2^T batched
    over (b, h, m), times scale."""
    s1 = np.matmul(q, np.swapaxes(k1, -1, -2))                 # [B,H,N,M,D] x [B,H,N,D,K]
    qm = np.swapaxes(q, 2, 3)                                   # [B,H,M,N,D]
    s2 = np.swapaxes(np.matmul(qm, np.swapaxes(k2, -1, -2)), 2, 3)   # [B,H,M,N,K] -> N,M
    return scale * (s1 + s2)


def _softmax(s):
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=-1, keepdims=True)
    return e / den, (mx + np.log(den))[..., 0]


def _pv(p, v1, v2):
    """P V1 (batched over n) + P V2 (batched over m): [B, H, N, M, Dv]."""
    y1 = np.matmul(p, v1)                                       # [B,H,N,M,K] x [B,H,N,K,Dv]
    pm = np.swapaxes(p, 2, 3)                                   # [B,H,M,N,K]
    y2 = np.swapaxes(np.matmul(pm, v2), 2, 3)
    return y1 + y2


def floyd_fwd(q, k1, v1, k2, v2, scale):
    """FloydAttention forward.  q [B,H,N,M,D], k1/v1 [B,H,N,K,D], k2/v2
    [B,H,M,K,D].  Returns (y [B,H,N,M,D], lse [B,H,N,M])."""
    q, k1, v1, k2, v2 = (_f64(t) for t in (q, k1, v1, k2, v2))
    p, lse = _softmax(_scores(q, k1, k2, scale))
    return _pv(p, v1, v2), lse


def floyd_bwd(q, k1, v1, k2, v2, y, dy, scale):
    """FloydAttention backward ("aclnnFusedFloydAttentionGrad", formula
    section).  P is recomputed from q, k1, k2; ``y`` is the forward output
    handed in (it enters softmax_grad).  Returns (dq, dk1, dv1, dk2, dv2)."""
    q, k1, v1, k2, v2, y, dy = (_f64(t) for t in (q, k1, v1, k2, v2, y, dy))
    p, _ = _softmax(_scores(q, k1, k2, scale))
    # dP = dY V1^T (batched over n) + dY V2^T (batched over m)
    dp1 = np.matmul(dy, np.swapaxes(v1, -1, -2))
    dym = np.swapaxes(dy, 2, 3)
    dp2 = np.swapaxes(np.matmul(dym, np.swapaxes(v2, -1, -2)), 2, 3)
    dp = dp1 + dp2
    softmax_grad = (dy * y).sum(axis=-1, keepdims=True)
    ds = p * (dp - softmax_grad)
    # dV1 = P^T dY over each n; dV2 = P^T dY over each m
    dv1 = np.matmul(np.swapaxes(p, -1, -2), dy)
    pm = np.swapaxes(p, 2, 3)                                   # [B,H,M,N,K]
    dv2 = np.matmul(np.swapaxes(pm, -1, -2), dym)
    # dQ = (dS K1 + dS K2) scale
    dq1 = np.matmul(ds, k1)
    dsm = np.swapaxes(ds, 2, 3)                                 # [B,H,M,N,K]
    dq2 = np.swapaxes(np.matmul(dsm, k2), 2, 3)
    dq = (dq1 + dq2) * scale
    # dK1 = dS^T Q scale over each n; dK2 = dS^T Q scale over each m
    dk1 = np.matmul(np.swapaxes(ds, -1, -2), q) * scale
    dk2 = np.matmul(np.swapaxes(dsm, -1, -2), np.swapaxes(q, 2, 3)) * scale
    return dq, dk1, dv1, dk2, dv2
