"""Plain float64 definitions of selected-key attention, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

Every public function materialises, for one group of query rows at a time, the
full score matrix over that group's selected keys, the softmax P of it, and the
products the pages define.  The grouping is the definition's own: a Q block
(block-sparse attention), one token's query heads of one KV head (NSA selected
attention), one decode token's query heads (sparse flash attention).

Conventions that the pages leave open, and the reading taken here:

* ``Mask(.)`` removes an entry exactly (score -inf).  A row with no remaining
  key has O = 0, LSE = -inf and zero gradients (parity unpinned: a convention).
* ``softmaxGrad(dOut, attentionOut)`` is the per-row sum of dOut * attentionOut
  (the only reading under which dS = P * (dP - softmax_grad) is the softmax
  Jacobian applied to dP; the tests pin it against rowsum(P * dP)).
* The ``*`` in the backward chain is a matrix product for dP, dV, dQ and dK and
  an element-wise product for dS.
* Query head n1 reads KV head n1 // G, G = N1 / N2 (contiguous groups).
* sparse_mode 2 (causal) keeps key j for query i iff j <= i, positions counted
  from the start of each sequence; mode 3 (rightDownCausal, sparse flash
  attention) places decode token s of Sq at position kv_len - Sq + s.
* The LSE is the natural log of the softmax denominator plus the row max.
* ``atten_mask`` of block-sparse attention (the Mask operand of the formula
  section; its format is not given): u8, element (b, n1, i, j) non-zero =
  the score of query position i and key position j is excluded, zero = kept;
  shape [Sq, Skv] (every batch entry and head) or [B or 1, N1 or 1, Sq, Skv]
  (size-1 axes broadcast).  It only removes entries of the selected blocks;
  with sparse_mode 2 both exclusions apply.  Positions are within a sequence
  in TND.

Parity status: attend_fwd / attend_bwd, bsa_*, nsa_*, sfa_fwd, sfa_fwd_tnd and
sfa_sharedkv_fwd are pinned by
the tests in ``tests/test_oracle_pins.py`` (dense special cases against an
independent torch autograd attention, finite differences, closed forms,
invariants and cross-path equalities).  The empty-row convention is unpinned.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# The core: masked softmax attention over an explicit key set.
# --------------------------------------------------------------------------

def attend_fwd(q, k, v, allowed, scale):
    """Masked softmax attention of R query rows over J keys.

    "aclnnBlockSparseAttentionGrad", formula section (forward, written with S
    and P): S = Mask(scale * Q K^T), P = SoftMax(S), Out = P V.

    q [R, D], k [J, D], v [J, Dv], allowed [R, J] bool (False = masked out).
    Returns (out [R, Dv], lse [R], p [R, J]), all float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    allowed = np.asarray(allowed, dtype=bool)
    s = scale * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    empty = ~allowed.any(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1, initial=-np.inf))
    e = np.exp(s - m[:, None])                      # exp(-inf) == 0 exactly
    denom = e.sum(axis=1)
    p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, denom)[:, None])
    out = p @ v
    lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, denom)))
    return out, lse, p


def attend_bwd(q, k, v, allowed, out, dout, scale):
    """Gradients of masked softmax attention.

    "aclnnBlockSparseAttentionGrad", formula section (backward):
    softmax_grad = softmaxGrad(dOut, attentionOut); dP = dOut V^T;
    dS = P * (dP - softmax_grad); dV = P^T dOut; dQ = (dS K) scale;
    dK = (dS^T Q) scale.

    P is recomputed from q and k (no stored statistics are used); ``out`` is
    the forward output handed in, as the pages' softmaxGrad takes it.
    Returns (dq [R, D], dk [J, D], dv [J, Dv]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    out, dout = _f64(out), _f64(dout)
    _, _, p = attend_fwd(q, k, v, allowed, scale)
    softmax_grad = (dout * out).sum(axis=1)
    dp = dout @ v.T
    ds = p * (dp - softmax_grad[:, None])
    dv = p.T @ dout
    dq = (ds @ k) * scale
    dk = (ds.T @ q) * scale
    return dq, dk, dv


# --------------------------------------------------------------------------
# Block-sparse attention (BlockSparseMask), BNSD layout.
# --------------------------------------------------------------------------

def bsa_keys(mask_row, block_kv, skv):
    """Key positions a Q block attends to: all keys of every KV block whose
    BlockSparseMask entry is non-zero, in ascending order.

    "aclnnBlockSparseAttentionGrad", function description: the mask names the
    KV blocks each Q block selects; blocks are blockShapeX x blockShapeY.
    """
    kbs = np.nonzero(np.asarray(mask_row))[0]
    parts = [np.arange(kb * block_kv, min((kb + 1) * block_kv, skv)) for kb in kbs]
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def _bsa_tiles(B, N1, QB, q_tiles):
    if q_tiles is None:
        return [(b, n, qb) for b in range(B) for n in range(N1) for qb in range(QB)]
    return [tuple(int(x) for x in t) for t in q_tiles]


def _am_slice(atten_mask, b, n1):
    """The [Sq, Skv] plane of ``atten_mask`` that query head n1 of batch entry
    b reads (None when there is no element mask)."""
    if atten_mask is None:
        return None
    am = np.asarray(atten_mask)
    if am.ndim == 2:
        return am
    if am.ndim != 4:
        raise ValueError("atten_mask must be [Sq, Skv] or [B|1, N1|1, Sq, Skv]")
    return am[b if am.shape[0] > 1 else 0, n1 if am.shape[1] > 1 else 0]


def _bsa_allowed(rows, keys, sparse_mode, am=None):
    """Which (row, key) scores of a Q block's selected keys enter the softmax:
    every one, less the causal exclusions (sparse_mode 2) and the entries
    ``am`` (an [Sq, Skv] plane of atten_mask) marks non-zero."""
    allowed = np.ones((len(rows), len(keys)), dtype=bool)
    if sparse_mode == 2:
        allowed &= keys[None, :] <= rows[:, None]
    if am is not None:
        allowed &= am[np.ix_(rows, keys)] == 0
    return allowed


def bsa_fwd(q, k, v, mask, block_q, block_kv, scale, sparse_mode=0, q_tiles=None,
            atten_mask=None):
    """Block-sparse attention forward, BNSD.

    q [B, N1, Sq, D], k [B, N2, Skv, D], v [B, N2, Skv, Dv],
    mask [B, N1, ceil(Sq/block_q), ceil(Skv/block_kv)] (non-zero = keep),
    atten_mask None or as in the module docstring (non-zero = excluded).
    Returns (out [B, N1, Sq, Dv], lse [B, N1, Sq]); rows of Q blocks outside
    ``q_tiles`` (a list of (b, n1, qb), default all) are NaN.
    """
    B, N1, Sq, _ = q.shape
    N2, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = N1 // N2
    QB = -(-Sq // block_q)
    out = np.full((B, N1, Sq, Dv), np.nan)
    lse = np.full((B, N1, Sq), np.nan)
    for b, n1, qb in _bsa_tiles(B, N1, QB, q_tiles):
        rows = np.arange(qb * block_q, min((qb + 1) * block_q, Sq))
        keys = bsa_keys(mask[b, n1, qb], block_kv, Skv)
        n2 = n1 // G
        o, l, _ = attend_fwd(q[b, n1, rows], k[b, n2, keys], v[b, n2, keys],
                             _bsa_allowed(rows, keys, sparse_mode, _am_slice(atten_mask, b, n1)),
                             scale)
        out[b, n1, rows] = o
        lse[b, n1, rows] = l
    return out, lse


def bsa_bwd(q, k, v, out, dout, mask, block_q, block_kv, scale, sparse_mode=0,
            q_tiles=None, atten_mask=None):
    """Block-sparse attention backward, BNSD.

    Returns (dq, dk, dv).  dq rows of Q blocks outside ``q_tiles`` are NaN;
    dk / dv hold the contributions of the Q blocks in ``q_tiles`` only (all Q
    blocks by default, which gives the full gradient; a KV block's gradient is
    exact when every Q block that selects it is in ``q_tiles``).  KV rows no
    Q block selects get exactly 0.
    """
    B, N1, Sq, D = q.shape
    N2, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = N1 // N2
    QB = -(-Sq // block_q)
    dq = np.full((B, N1, Sq, D), np.nan)
    dk = np.zeros((B, N2, Skv, D))
    dv = np.zeros((B, N2, Skv, Dv))
    for b, n1, qb in _bsa_tiles(B, N1, QB, q_tiles):
        rows = np.arange(qb * block_q, min((qb + 1) * block_q, Sq))
        keys = bsa_keys(mask[b, n1, qb], block_kv, Skv)
        n2 = n1 // G
        g_q, g_k, g_v = attend_bwd(q[b, n1, rows], k[b, n2, keys], v[b, n2, keys],
                                   _bsa_allowed(rows, keys, sparse_mode,
                                                _am_slice(atten_mask, b, n1)),
                                   out[b, n1, rows], dout[b, n1, rows], scale)
        dq[b, n1, rows] = g_q
        np.add.at(dk[b, n2], keys, g_k)
        np.add.at(dv[b, n2], keys, g_v)
    return dq, dk, dv


def _tnd_tiles(cu_q, N1, block_q, q_tiles):
    B = len(cu_q) - 1
    if q_tiles is not None:
        return [tuple(int(x) for x in t) for t in q_tiles]
    return [(b, n, qb) for b in range(B) for n in range(N1)
            for qb in range(-(-(int(cu_q[b + 1]) - int(cu_q[b])) // block_q))]


def bsa_fwd_tnd(q, k, v, mask, cu_seqlens_q, cu_seqlens_kv, block_q, block_kv, scale,
                sparse_mode=0, q_tiles=None, atten_mask=None):
    """Block-sparse attention forward, TND (variable-length sequences).

    "aclnnBlockSparseAttentionGrad", layout section: TND rows are the tokens
    of all sequences back to back, sequence b holding rows cu[b] .. cu[b+1]-1
    (the actual sequence lengths are mandatory with TND).  q [T, N1, D],
    k [Tk, N2, D], v [Tk, N2, Dv]; mask [B, N1, QB, KB] with QB / KB the block
    counts of the longest sequences: sequence b reads the entries of its own
    blocks only.  Block positions, the causal test and atten_mask positions
    ([Sq, Skv] planes of the longest lengths) are within a sequence.
    Returns (out [T, N1, Dv], lse [T, N1]); rows outside ``q_tiles`` (a list
    of (b, n1, qb), default all) are NaN.
    """
    cu_q, cu_k = np.asarray(cu_seqlens_q), np.asarray(cu_seqlens_kv)
    T, N1, _ = q.shape
    N2, Dv = k.shape[1], v.shape[2]
    G = N1 // N2
    out = np.full((T, N1, Dv), np.nan)
    lse = np.full((T, N1), np.nan)
    for b, n1, qb in _tnd_tiles(cu_q, N1, block_q, q_tiles):
        q0, sq = int(cu_q[b]), int(cu_q[b + 1] - cu_q[b])
        k0, skv = int(cu_k[b]), int(cu_k[b + 1] - cu_k[b])
        rows = np.arange(qb * block_q, min((qb + 1) * block_q, sq))
        keys = bsa_keys(mask[b, n1, qb, :-(-skv // block_kv)], block_kv, skv)
        n2 = n1 // G
        o, l, _ = attend_fwd(q[q0 + rows, n1], k[k0 + keys, n2], v[k0 + keys, n2],
                             _bsa_allowed(rows, keys, sparse_mode, _am_slice(atten_mask, b, n1)),
                             scale)
        out[q0 + rows, n1] = o
        lse[q0 + rows, n1] = l
    return out, lse


def bsa_bwd_tnd(q, k, v, out, dout, mask, cu_seqlens_q, cu_seqlens_kv, block_q, block_kv,
                scale, sparse_mode=0, q_tiles=None, atten_mask=None):
    """Block-sparse attention backward, TND: the backward chain of the
    formula section per (sequence, head, Q block), with each selected key's
    gradient added back to its row.  Returns (dq, dk, dv); as ``bsa_bwd`` for
    ``q_tiles`` (dq NaN outside them, dk / dv their contributions only)."""
    cu_q, cu_k = np.asarray(cu_seqlens_q), np.asarray(cu_seqlens_kv)
    T, N1, D = q.shape
    Tk, N2, Dv = v.shape
    G = N1 // N2
    dq = np.full((T, N1, D), np.nan)
    dk = np.zeros((Tk, N2, D))
    dv = np.zeros((Tk, N2, Dv))
    for b, n1, qb in _tnd_tiles(cu_q, N1, block_q, q_tiles):
        q0, sq = int(cu_q[b]), int(cu_q[b + 1] - cu_q[b])
        k0, skv = int(cu_k[b]), int(cu_k[b + 1] - cu_k[b])
        rows = np.arange(qb * block_q, min((qb + 1) * block_q, sq))
        keys = bsa_keys(mask[b, n1, qb, :-(-skv // block_kv)], block_kv, skv)
        n2 = n1 // G
        g_q, g_k, g_v = attend_bwd(q[q0 + rows, n1], k[k0 + keys, n2], v[k0 + keys, n2],
                                   _bsa_allowed(rows, keys, sparse_mode,
                                                _am_slice(atten_mask, b, n1)),
                                   out[q0 + rows, n1], dout[q0 + rows, n1], scale)
        dq[q0 + rows, n1] = g_q
        np.add.at(dk[:, n2], k0 + keys, g_k)
        np.add.at(dv[:, n2], k0 + keys, g_v)
    return dq, dk, dv


# --------------------------------------------------------------------------
# NSA selected attention (topk_indices), TND layout.
# --------------------------------------------------------------------------

def nsa_keys(topk_row, sbs, skv_seq):
    """Gather(key, topk_indices[i]) for 0 <= i < selected_block_count: the sbs
    key positions of each listed block, in slot order, duplicates kept.

    "aclnnNsaSelectedAttention", formulas section.  Block ids count in units
    of selected_block_size from the start of the token's own sequence.
    """
    parts = []
    for idx in np.asarray(topk_row).tolist():
        if idx < 0 or idx * sbs >= skv_seq:
            raise ValueError(f"topk block id {idx} outside a sequence of {skv_seq} keys")
        parts.append(np.arange(idx * sbs, min(idx * sbs + sbs, skv_seq)))
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def _nsa_units(cu_q, N2, tokens):
    seq_of = np.searchsorted(np.asarray(cu_q), np.arange(int(cu_q[-1])), side="right") - 1
    toks = range(int(cu_q[-1])) if tokens is None else [int(t) for t in tokens]
    for t in toks:
        b = int(seq_of[t])
        for n2 in range(N2):
            yield t, b, n2


def nsa_fwd(q, k, v, topk, cu_seqlens_q, cu_seqlens_kv, sbs, scale, sparse_mode=2,
            tokens=None):
    """NSA selected attention forward, TND.

    "aclnnNsaSelectedAttention", formulas section: selected_key/value =
    Gather(key/value, topk_indices); attention_out = Softmax(Mask(scale *
    query @ selected_key^T, atten_mask)) @ selected_value.  Constraints
    section: sparseMode 0 (no mask, all selected tokens computed) or 2
    (causal).

    q [T, N1, D], k [Tk, N2, D], v [Tk, N2, Dv], topk [T, N2, sbc] int.
    Returns (out [T, N1, Dv], lse [T, N1]); tokens outside ``tokens`` are NaN.
    """
    T, N1, _ = q.shape
    N2, Dv = k.shape[1], v.shape[2]
    G = N1 // N2
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_kv = np.asarray(cu_seqlens_kv, dtype=np.int64)
    out = np.full((T, N1, Dv), np.nan)
    lse = np.full((T, N1), np.nan)
    for t, b, n2 in _nsa_units(cu_q, N2, tokens):
        pos = t - cu_q[b]
        kv0, skv = cu_kv[b], cu_kv[b + 1] - cu_kv[b]
        keys = nsa_keys(topk[t, n2], sbs, skv)
        allowed = np.ones((G, len(keys)), dtype=bool)
        if sparse_mode == 2:
            allowed &= (keys <= pos)[None, :]
        heads = slice(n2 * G, (n2 + 1) * G)
        o, l, _ = attend_fwd(q[t, heads], k[kv0 + keys, n2], v[kv0 + keys, n2],
                             allowed, scale)
        out[t, heads] = o
        lse[t, heads] = l
    return out, lse


def nsa_bwd(q, k, v, out, dout, topk, cu_seqlens_q, cu_seqlens_kv, sbs, scale,
            sparse_mode=2, tokens=None):
    """NSA selected attention backward, TND.

    The NSA page is a forward operator "for training"; its gradient is the
    chain of "aclnnBlockSparseAttentionGrad" (formula section) applied to the
    gathered keys, with the Gather's own gradient: each gathered row's dK/dV
    is added back to the row it was gathered from (twice if listed twice).
    Returns (dq, dk, dv); dq of tokens outside ``tokens`` is NaN and dk/dv
    then hold only those tokens' contributions.
    """
    T, N1, D = q.shape
    N2, Tk, Dv = k.shape[1], k.shape[0], v.shape[2]
    G = N1 // N2
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_kv = np.asarray(cu_seqlens_kv, dtype=np.int64)
    dq = np.full((T, N1, D), np.nan)
    dk = np.zeros((Tk, N2, D))
    dv = np.zeros((Tk, N2, Dv))
    for t, b, n2 in _nsa_units(cu_q, N2, tokens):
        pos = t - cu_q[b]
        kv0, skv = cu_kv[b], cu_kv[b + 1] - cu_kv[b]
        keys = nsa_keys(topk[t, n2], sbs, skv)
        allowed = np.ones((G, len(keys)), dtype=bool)
        if sparse_mode == 2:
            allowed &= (keys <= pos)[None, :]
        heads = slice(n2 * G, (n2 + 1) * G)
        g_q, g_k, g_v = attend_bwd(q[t, heads], k[kv0 + keys, n2], v[kv0 + keys, n2],
                                   allowed, out[t, heads], dout[t, heads], scale)
        dq[t, heads] = g_q
        np.add.at(dk[:, n2], kv0 + keys, g_k)
        np.add.at(dv[:, n2], kv0 + keys, g_v)
    return dq, dk, dv


# --------------------------------------------------------------------------
# Sparse flash attention over a paged (PA_ND) shared KV cache, inference.
# --------------------------------------------------------------------------

def _sfa_token(q_t, qr_t, topk_t, block_row, kv_len, qpos, key_cache, key_rope_cache,
               value_cache, scale, sparse_mode, sparse_block_size):
    """One decode token's selected-key attention, all query heads: q_t
    [N1, D], qr_t [N1, Dr], topk_t [N2, K]; block_row the sequence's page
    table row; qpos the token's position (rightDownCausal).  Returns (out
    [N1, Dv], lse [N1])."""
    page, N2 = key_cache.shape[1], key_cache.shape[2]
    N1 = q_t.shape[0]
    G = N1 // N2
    out = np.zeros((N1, value_cache.shape[3]))
    lse = np.zeros(N1)
    for n2 in range(N2):
        ids = np.asarray(topk_t[n2]).astype(np.int64)
        ids = ids[ids >= 0]
        if np.any(ids * sparse_block_size >= kv_len):
            raise ValueError("selected id beyond kv_len")
        pos = (ids[:, None] * sparse_block_size
               + np.arange(sparse_block_size)[None, :]).reshape(-1)
        pos = pos[pos < kv_len]
        phys = np.asarray(block_row)[pos // page]
        row = pos % page
        keys = np.concatenate([_f64(key_cache[phys, row, n2]),
                               _f64(key_rope_cache[phys, row, n2])], axis=1)
        vals = _f64(value_cache[phys, row, n2])
        heads = slice(n2 * G, (n2 + 1) * G)
        qcat = np.concatenate([_f64(q_t[heads]), _f64(qr_t[heads])], axis=1)
        allowed = np.ones((G, len(pos)), dtype=bool)
        if sparse_mode == 3:
            allowed &= (pos <= qpos)[None, :]
        o, l, _ = attend_fwd(qcat, keys, vals, allowed, scale)
        out[heads] = o
        lse[heads] = l
    return out, lse


def sfa_fwd(q, q_rope, key_cache, key_rope_cache, value_cache, block_table, kv_lens,
            topk, scale, sparse_mode=3, sparse_block_size=1, tokens=None):
    """Sparse flash attention forward over selected tokens of a paged cache.

    "aclnnSparseFlashAttention", formulas section: softmax(Q K~^T / sqrt(d_k))
    V~ with K~/V~ the selected keys/values; d_k counts the 512-wide head and
    the 64-wide rope part, so a score is scale * (q.k + q_rope.k_rope), which
    is the dot product of the concatenations [q, q_rope] and [k, k_rope].
    "SparseAttnSharedkvMetadata", parameter list: the KV cache is PageAttention
    (PA_ND) paged, seqused_kv gives the active KV length per batch, mask mode 3
    is rightDownCausal (decode token s of Sq sits at position kv_len - Sq + s).

    q [B, Sq, N1, D], q_rope [B, Sq, N1, Dr]; key_cache [P, page, N2, D],
    key_rope_cache [P, page, N2, Dr], value_cache [P, page, N2, Dv];
    block_table [B, max_pages]; kv_lens [B]; topk [B, Sq, N2, K] selected
    sparse-block ids (token positions when sparse_block_size == 1), -1 = none.
    ``tokens``: optional list of (b, s) to compute; others are NaN.
    Returns (out [B, Sq, N1, Dv], lse [B, Sq, N1]).
    """
    B, Sq, N1, _ = q.shape
    Dv = value_cache.shape[3]
    out = np.full((B, Sq, N1, Dv), np.nan)
    lse = np.full((B, Sq, N1), np.nan)
    units = [(b, s) for b in range(B) for s in range(Sq)] if tokens is None else tokens
    for b, s in units:
        kv_len = int(kv_lens[b])
        out[b, s], lse[b, s] = _sfa_token(q[b, s], q_rope[b, s], topk[b, s], block_table[b],
                                          kv_len, kv_len - Sq + s, key_cache, key_rope_cache,
                                          value_cache, scale, sparse_mode, sparse_block_size)
    return out, lse


def sfa_fwd_tnd(q, q_rope, key_cache, key_rope_cache, value_cache, block_table, kv_lens,
                topk, cu_seqlens_q, scale, sparse_mode=3, sparse_block_size=1, tokens=None):
    """Sparse flash attention forward with TND queries.

    "SparseAttnSharedkvMetadata", parameter list: layout_q may be TND, with
    cu_seqlens_q the B+1 prefix sums of each batch entry's query tokens.
    Sequence b's Sq_b = cu[b+1] - cu[b] decode tokens are rows cu[b] ..
    cu[b+1]-1; under rightDownCausal its token s sits at kv_len - Sq_b + s.
    q [T, N1, D], q_rope [T, N1, Dr], topk [T, N2, K]; caches, block_table and
    kv_lens as in ``sfa_fwd``.  ``tokens``: optional list of global rows t.
    Returns (out [T, N1, Dv], lse [T, N1]); rows not computed are NaN.
    """
    cu = np.asarray(cu_seqlens_q)
    T, N1, _ = q.shape
    Dv = value_cache.shape[3]
    out = np.full((T, N1, Dv), np.nan)
    lse = np.full((T, N1), np.nan)
    rows = range(T) if tokens is None else tokens
    for t in rows:
        b = int(np.searchsorted(cu, t, side="right")) - 1
        sq_b = int(cu[b + 1] - cu[b])
        kv_len = int(kv_lens[b])
        out[t], lse[t] = _sfa_token(q[t], q_rope[t], topk[t], block_table[b], kv_len,
                                    kv_len - sq_b + (t - int(cu[b])), key_cache, key_rope_cache,
                                    value_cache, scale, sparse_mode, sparse_block_size)
    return out, lse


def sfa_sharedkv_fwd(q, q_rope, cu_seqlens_q, kv_lens, scale, ori=None, cmp=None,
                     win_left=127, win_right=0, cmp_ratio=4, tokens=None):
    """Shared-KV sparse decode over two key sets in one softmax.

    "SparseAttnSharedkvMetadata", parameter list: the query attends to the
    original KV (ori_kv) under mask mode 4, a band of ori_win_left past and
    ori_win_right future tokens around its own position, and to cmp_topk
    selected entries of a compressed KV (cmp_kv, ori_kv compressed by
    cmp_ratio) under mask mode 3, rightDownCausal; both caches are PageAttention
    paged with one KV head (has_ori_kv / has_cmp_kv say which are given).  The
    score and value rules are those of "aclnnSparseFlashAttention" (formulas):
    score = scale * (q.k + q_rope.k_rope), value = the key's 512-wide row.

    Readings: the two key sets share one softmax (one normalisation); query
    token s of entry b (Sq_b tokens) sits at p = kv_len_b - Sq_b + s in the
    original sequence; the band is [p - win_left, p + win_right] clipped to
    [0, kv_len_b); the compressed sequence holds cmp_len_b = kv_len_b //
    cmp_ratio entries and rightDownCausal lets compressed id c through iff
    c <= cmp_len_b - Sq_b + s.

    q [T, N1, D], q_rope [T, N1, Dr] (TND rows; cu_seqlens_q [B+1] prefix
    sums); kv_lens [B] (seqused_kv).  ori = (key_cache [P, page, 1, D],
    key_rope_cache [P, page, 1, Dr], block_table [B, max_pages]) or None;
    cmp = (key_cache, key_rope_cache, block_table, topk [T, 1, K] compressed
    ids, -1 = empty) or None.  ``tokens``: optional list of rows t.
    Returns (out [T, N1, D], lse [T, N1]); rows not computed are NaN.
    """
    cu = np.asarray(cu_seqlens_q)
    T, N1, D = q.shape
    out = np.full((T, N1, D), np.nan)
    lse = np.full((T, N1), np.nan)
    for t in (range(T) if tokens is None else tokens):
        b = int(np.searchsorted(cu, t, side="right")) - 1
        sq_b, s = int(cu[b + 1] - cu[b]), t - int(cu[b])
        kv_len = int(kv_lens[b])
        keys, vals = [], []
        if ori is not None:
            kc, krc, bt = ori
            page = kc.shape[1]
            p = kv_len - sq_b + s
            pos = np.arange(max(0, p - win_left), min(kv_len, p + win_right + 1))
            phys, row = np.asarray(bt[b])[pos // page], pos % page
            keys.append(np.concatenate([_f64(kc[phys, row, 0]), _f64(krc[phys, row, 0])], 1))
            vals.append(_f64(kc[phys, row, 0]))
        if cmp is not None:
            kc, krc, bt, topk = cmp
            page = kc.shape[1]
            cmp_len = kv_len // cmp_ratio
            ids = np.asarray(topk[t, 0]).astype(np.int64)
            ids = ids[ids >= 0]
            if np.any(ids >= cmp_len):
                raise ValueError("compressed id beyond cmp_len")
            ids = ids[ids <= cmp_len - sq_b + s]
            phys, row = np.asarray(bt[b])[ids // page], ids % page
            keys.append(np.concatenate([_f64(kc[phys, row, 0]), _f64(krc[phys, row, 0])], 1))
            vals.append(_f64(kc[phys, row, 0]))
        kmat = np.concatenate(keys) if keys else np.zeros((0, D + q_rope.shape[2]))
        vmat = np.concatenate(vals) if vals else np.zeros((0, D))
        qcat = np.concatenate([_f64(q[t]), _f64(q_rope[t])], axis=1)
        o, l, _ = attend_fwd(qcat, kmat, vmat, np.ones((N1, len(kmat)), bool), scale)
        out[t], lse[t] = o, l
    return out, lse
