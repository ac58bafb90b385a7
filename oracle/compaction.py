"""Plain definitions of the selected-block lists (integer, compared bit-exactly).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both functions return CSR pairs (pointer array of length rows + 1 starting at
0, then the entries) in int32.  The order is canonical: entries ascending
within each row, rows in row-major order of their index tuple, so exactly one
output is correct.

Parity status: pinned against brute-force loops on small inputs and against
closed-form counts of the synthetic workloads (tests/test_oracle_pins.py).
"""

import numpy as np


def _csr(counts, entries):
    ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    np.cumsum(counts, out=ptr[1:])
    return ptr.astype(np.int32), np.asarray(entries, dtype=np.int32)


def bsa_compact(mask, n2):
    """Lists of a BlockSparseMask.

    "aclnnBlockSparseAttentionGrad", function description: the mask gives, for
    each Q block, the KV blocks it selects.

    mask [B, N1, QB, KB] (non-zero = selected), n2 = number of KV heads
    (N1 % n2 == 0, G = N1 / n2, query head n1 reads KV head n1 // G).

    Returns (row_ptr, col, rev_ptr, rev):
      forward: row (b, n1, qb) -> ascending kb with mask[b, n1, qb, kb] != 0;
      reverse: row (b, n2, kb) -> ascending ids g * QB + qb of the Q blocks of
               the G query heads n1 = n2 * G + g that selected kb.
    """
    sel = np.asarray(mask) != 0
    B, N1, QB, KB = sel.shape
    G = N1 // n2
    fwd = sel.reshape(B * N1 * QB, KB)
    row_ptr, col = _csr(fwd.sum(axis=1), np.nonzero(fwd)[1])
    rev_rows = sel.reshape(B, n2, G, QB, KB).transpose(0, 1, 4, 2, 3).reshape(B * n2 * KB, G * QB)
    rev_ptr, rev = _csr(rev_rows.sum(axis=1), np.nonzero(rev_rows)[1])
    return row_ptr, col, rev_ptr, rev


def nsa_compact(topk, cu_seqlens_q, cu_seqlens_kv, sbs, sparse_mode):
    """Lists of NSA topk_indices.

    "aclnnNsaSelectedAttention", formulas section (Gather by topk_indices) and
    constraints section (sparseMode 2 = causal).

    topk [T, N2, sbc]: block ids relative to the token's own sequence.
    Forward: row (t, n2) -> the token's block ids sorted ascending (a
      duplicate stays), and under sparse_mode 2 without the blocks whose first
      key lies after the token's position (they are wholly masked).
    Reverse: row (n2, gb) with gb = (blocks of the earlier sequences) + id,
      a sequence holding ceil(Skv_b / sbs) blocks -> ascending token ids t
      whose forward row holds that block (twice if it holds it twice).
    Returns (row_ptr, col, rev_ptr, rev, blocks_total).
    """
    topk = np.asarray(topk)
    T, N2, _ = topk.shape
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_kv = np.asarray(cu_seqlens_kv, dtype=np.int64)
    nseq = len(cu_q) - 1
    nblk = [-(-int(cu_kv[b + 1] - cu_kv[b]) // sbs) for b in range(nseq)]
    blk_off = np.concatenate([[0], np.cumsum(nblk)]).astype(np.int64)
    blocks_total = int(blk_off[-1])

    counts, cols = [], []
    triples = []                         # (n2, global block, t) for the reverse lists
    for b in range(nseq):
        for t in range(int(cu_q[b]), int(cu_q[b + 1])):
            pos = t - int(cu_q[b])
            for n2 in range(N2):
                ids = sorted(int(x) for x in topk[t, n2])
                if sparse_mode == 2:
                    ids = [i for i in ids if i * sbs <= pos]
                counts.append(len(ids))
                cols.extend(ids)
                triples.extend((n2, int(blk_off[b]) + i, t) for i in ids)
    row_ptr, col = _csr(np.array(counts, dtype=np.int64), cols)

    rev_counts = np.zeros(N2 * blocks_total, dtype=np.int64)
    for n2, gb, _ in triples:
        rev_counts[n2 * blocks_total + gb] += 1
    triples.sort()
    rev_ptr, rev = _csr(rev_counts, [t for _, _, t in triples])
    return row_ptr, col, rev_ptr, rev, blocks_total
