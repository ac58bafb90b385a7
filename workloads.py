"""Seeded synthetic inputs for block-sparse / top-k-selected attention.

This module only draws random inputs (masks, index lists, page tables,
normal-distributed tensors).  It holds none of the attention arithmetic and
imports neither the product package nor the oracle, so both sides can take
their inputs from it.

Seeds: ``numpy.random.default_rng(1000 + cfg)`` for masks, indices and page
tables; ``default_rng(cfg * 10 + i)`` (i = 1..4 for Q, K, V, dOut; 5.. for
extra tensors) for values, drawn as float32 standard normals and rounded to
the working dtype with round-to-nearest-even.

The five named workloads:

1. ``bsa_small``: block-sparse attention, BNSD, B=1, N1=N2=2, S=512, D=128,
   fp16, 64x64 blocks, diagonal kept plus each other block kept with p=0.5.
2. ``bsa_causal_8k``: B=2, N1=N2=16, S=8192, D=128, bf16, 128x128 blocks,
   causal block mask (kb <= qb) with the diagonal kept and the rest kept with
   p=0.25.
3. ``nsa_varlen``: NSA selected attention, TND, sequences {2048, 4096, 8192,
   2048}, N1=32, N2=2, D=128, bf16, 64-token blocks, 16 per (token, KV head),
   sparse_mode 2; the token's own block is always selected.
4. ``sfa_decode``: paged sparse flash attention, B=32, Sq=4, N1=64, N2=1,
   D=512 + 64 rope, bf16, page 128, KV length 65536, 2048 selected tokens.
5. ``bsa_window_128k``: B=1, N1=N2=8, S=131072, D=128, bf16, 128x128 blocks,
   8-block sliding window plus 24 random earlier blocks per Q block.
"""

import math

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def normal(shape, seed, dtype="bf16"):
    """float32 standard normals from default_rng(seed), rounded to ``dtype``."""
    x = np.random.default_rng(seed).standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(DTYPES[dtype])


# ----------------------------------------------------------------------------
# Block masks
# ----------------------------------------------------------------------------

def mask_random(rng, B, N, QB, KB, p_keep, causal=False, diagonal=True):
    """u8 [B, N, QB, KB]: each block kept i.i.d. with p_keep; the diagonal
    (kb == qb) kept when ``diagonal``; blocks kb > qb dropped when ``causal``."""
    u = rng.random((B, N, QB, KB))
    keep = u < p_keep
    qb = np.arange(QB)[:, None]
    kb = np.arange(KB)[None, :]
    if causal:
        keep &= kb <= qb
    if diagonal:
        keep |= (kb == qb)
    return keep.astype(np.uint8)


def mask_window_random(rng, B, N, QB, KB, window, n_random):
    """u8 [B, N, QB, KB]: blocks max(0, qb-window+1)..qb plus ``n_random``
    distinct uniform draws from [0, qb-window] (all of them if fewer)."""
    mask = np.zeros((B, N, QB, KB), dtype=np.uint8)
    for b in range(B):
        for n in range(N):
            for qb in range(QB):
                lo = max(0, qb - window + 1)
                mask[b, n, qb, lo:qb + 1] = 1
                if lo > 0:
                    cand = lo                      # blocks 0 .. lo-1
                    pick = rng.choice(cand, size=min(n_random, cand), replace=False)
                    mask[b, n, qb, pick] = 1
    return mask


# ----------------------------------------------------------------------------
# NSA top-k block ids
# ----------------------------------------------------------------------------

def nsa_topk_causal(rng, seqlens, n2, sbs, sbc):
    """int32 [T, n2, sbc] block ids relative to each sequence.

    For a token whose own block is q: if q >= sbc - 1, its own block plus
    sbc - 1 distinct uniform draws from [0, q-1]; otherwise all blocks 0..q
    plus blocks q+1 .. sbc-1 (future blocks, wholly masked under causal mode).
    Slot order is shuffled."""
    out = []
    for S in seqlens:
        pos = np.arange(S)
        own = pos // sbs
        nblocks = -(-S // sbs)
        if nblocks < sbc:
            raise ValueError("sequence shorter than selected_block_size * selected_block_count")
        # distinct draws from [0, q-1] by sorting random keys, invalid candidates last
        keys = rng.random((S, n2, nblocks))
        cand = np.arange(nblocks)[None, None, :]
        # valid candidates (< own block) get random keys; future blocks follow in
        # ascending order; the own block itself goes last (it is prepended below)
        keys = np.where(cand < own[:, None, None], keys,
                        np.where(cand == own[:, None, None], np.inf, 2.0 + cand))
        order = np.argsort(keys, axis=2, kind="stable")[:, :, :sbc - 1]
        ids = np.concatenate([np.broadcast_to(own[:, None, None], (S, n2, 1)), order], axis=2)
        # tokens with q < sbc-1: ids are own + the q earlier blocks (random order) + blocks
        # q+1.. in ascending order, i.e. exactly the set {0..sbc-1}
        perm = np.argsort(rng.random((S, n2, sbc)), axis=2)
        ids = np.take_along_axis(ids, perm, axis=2)
        out.append(ids.astype(np.int32))
    return np.concatenate(out, axis=0)


# ----------------------------------------------------------------------------
# Paged KV decode
# ----------------------------------------------------------------------------

def sfa_paged(rng, B, Sq, kv_len, page, topk):
    """block_table int32 [B, ceil(kv_len/page)] = a random permutation of the
    B*ceil(kv_len/page) physical pages; kv_lens int32 [B]; topk int32
    [B, Sq, 1, topk] distinct sorted positions uniform over [0, kv_len - Sq + s]
    (rightDownCausal), -1 in the slots left when fewer positions exist."""
    pages = -(-kv_len // page)
    block_table = rng.permutation(B * pages).reshape(B, pages).astype(np.int32)
    kv_lens = np.full((B,), kv_len, dtype=np.int32)
    idx = np.full((B, Sq, 1, topk), -1, dtype=np.int32)   # -1 = empty slot
    for b in range(B):
        for s in range(Sq):
            hi = kv_len - Sq + s + 1
            n = min(topk, hi)
            idx[b, s, 0, :n] = np.sort(rng.choice(hi, size=n, replace=False))
    return block_table, kv_lens, idx


# ----------------------------------------------------------------------------
# The named workloads
# ----------------------------------------------------------------------------

def bsa_workload(cfg):
    """Shape/recipe dict of a block-sparse workload (cfg in 1, 2, 5)."""
    if cfg == 1:
        return dict(name="bsa_small", B=1, N1=2, N2=2, S=512, D=128, dtype="fp16",
                    bq=64, bkv=64, kind="random", p=0.5, causal=False)
    if cfg == 2:
        return dict(name="bsa_causal_8k", B=2, N1=16, N2=16, S=8192, D=128, dtype="bf16",
                    bq=128, bkv=128, kind="random", p=0.25, causal=True)
    if cfg == 5:
        return dict(name="bsa_window_128k", B=1, N1=8, N2=8, S=131072, D=128, dtype="bf16",
                    bq=128, bkv=128, kind="window", window=8, n_random=24)
    raise ValueError(cfg)


def bsa_mask(w, seed):
    rng = np.random.default_rng(seed)
    QB = -(-w["S"] // w["bq"])
    KB = -(-w["S"] // w["bkv"])
    if w["kind"] == "random":
        return mask_random(rng, w["B"], w["N1"], QB, KB, w["p"], causal=w["causal"])
    return mask_window_random(rng, w["B"], w["N1"], QB, KB, w["window"], w["n_random"])


def bsa_inputs(cfg):
    """(workload dict, q, k, v, dout, mask, scale) with torch CPU tensors."""
    w = bsa_workload(cfg)
    B, N1, N2, S, D, dt = w["B"], w["N1"], w["N2"], w["S"], w["D"], w["dtype"]
    q = normal((B, N1, S, D), cfg * 10 + 1, dt)
    k = normal((B, N2, S, D), cfg * 10 + 2, dt)
    v = normal((B, N2, S, D), cfg * 10 + 3, dt)
    do = normal((B, N1, S, D), cfg * 10 + 4, dt)
    mask = bsa_mask(w, 1000 + cfg)
    return w, q, k, v, do, mask, 1.0 / math.sqrt(D)


def bsa_tnd_workload():
    return dict(name="bsa_tnd_varlen", seqlens=[2048, 4096, 8192, 2048], N1=16, N2=4, D=128,
                dtype="bf16", bq=128, bkv=128, p=0.25)


def bsa_tnd_inputs(seqlens=None, N1=16, N2=4, bq=128, bkv=128, p=0.25, seed_base=60,
                   dtype="bf16"):
    """(cu_seqlens int32 [B+1], q [T,N1,D], k [T,N2,D], v [T,N2,D], dout, mask).

    Per sequence a causal-shaped block mask: KV block kb <= Q block qb, the
    diagonal kept, every other such block kept i.i.d. with p.  The mask is
    padded to the longest sequence ([B, N1, QB, KB]) and zero past each
    sequence's own blocks."""
    w = bsa_tnd_workload()
    seqlens = w["seqlens"] if seqlens is None else seqlens
    T, D = int(sum(seqlens)), 128
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    q = normal((T, N1, D), seed_base + 1, dtype)
    k = normal((T, N2, D), seed_base + 2, dtype)
    v = normal((T, N2, D), seed_base + 3, dtype)
    do = normal((T, N1, D), seed_base + 4, dtype)
    QB, KB = -(-max(seqlens) // bq), -(-max(seqlens) // bkv)
    mask = mask_random(np.random.default_rng(1000 + seed_base // 10), len(seqlens), N1, QB, KB,
                       p, causal=True)
    for b, L in enumerate(seqlens):
        mask[b, :, -(-L // bq):, :] = 0
        mask[b, :, :, -(-L // bkv):] = 0
    return cu, q, k, v, do, mask


def nsa_workload():
    return dict(name="nsa_varlen", seqlens=[2048, 4096, 8192, 2048], N1=32, N2=2, D=128,
                dtype="bf16", sbs=64, sbc=16, sparse_mode=2)


def nsa_inputs(seqlens=None, N1=32, N2=2, D=128, sbs=64, sbc=16, seed_base=30, dtype="bf16",
               Dv=None):
    """(cu_seqlens int32 [B+1], q [T,N1,D], k [T,N2,D], v [T,N2,Dv], dout [T,N1,Dv], topk);
    Dv defaults to D."""
    w = nsa_workload()
    seqlens = w["seqlens"] if seqlens is None else seqlens
    Dv = D if Dv is None else Dv
    T = int(sum(seqlens))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    q = normal((T, N1, D), seed_base + 1, dtype)
    k = normal((T, N2, D), seed_base + 2, dtype)
    v = normal((T, N2, Dv), seed_base + 3, dtype)
    do = normal((T, N1, Dv), seed_base + 4, dtype)
    topk = nsa_topk_causal(np.random.default_rng(1000 + seed_base // 10), seqlens, N2, sbs, sbc)
    return cu, q, k, v, do, topk


def sfa_workload():
    return dict(name="sfa_decode", B=32, Sq=4, N1=64, N2=1, D=512, Dr=64, dtype="bf16",
                page=128, kv_len=65536, topk=2048)


def sfa_sharedkv_workload():
    return dict(name="sfa_sharedkv_decode", B=32, Sq=4, N1=64, N2=1, D=512, Dr=64, dtype="bf16",
                page=128, kv_len=65536, win_left=127, win_right=0, cmp_ratio=4, cmp_topk=512)


def _paged_table(rng, lens, page, extra=0):
    """block_table int32 [B, max_pages]: entry b's logical pages on a random
    permutation of the physical pages (extra unused pages at the end)."""
    pages = [-(-int(n) // page) for n in lens]
    perm = rng.permutation(sum(pages) + extra)
    bt = np.zeros((len(lens), max(max(pages), 1)), np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, sum(pages) + extra


def sfa_sharedkv_inputs(lens=None, kv_lens=None, N1=64, D=512, Dr=64, page=128, cmp_ratio=4,
                        cmp_topk=512, seed_base=120, dtype="bf16", extra_pages=0):
    """TND decode queries for the two-branch shared-KV decode.

    lens: query tokens per batch entry (default 32 entries of 4); kv_lens: the
    original KV length per entry (default 65536).  The original cache holds
    kv_len rows per entry and the compressed cache kv_len // cmp_ratio, both
    paged on random page permutations.  Each query token selects min(cmp_topk,
    n) distinct sorted compressed ids uniformly from the n = cmp_len - Sq_b + s
    + 1 it may see (rightDownCausal), -1 in the slots left.
    Returns (cu int32 [B+1], q [T, N1, D], q_rope [T, N1, Dr], kv_lens int32
    [B], (ori_kc, ori_krc, ori_bt), (cmp_kc, cmp_krc, cmp_bt, cmp_idx int32
    [T, 1, cmp_topk]))."""
    w = sfa_sharedkv_workload()
    lens = [w["Sq"]] * w["B"] if lens is None else list(lens)
    kv_lens = np.asarray([w["kv_len"]] * len(lens) if kv_lens is None else kv_lens, np.int32)
    rng = np.random.default_rng(1000 + seed_base // 10)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    cmp_lens = kv_lens // cmp_ratio
    ori_bt, P = _paged_table(rng, kv_lens, page, extra_pages)
    cmp_bt, Pc = _paged_table(rng, cmp_lens, page, extra_pages)
    idx = np.full((T, 1, cmp_topk), -1, np.int32)
    for b, n_q in enumerate(lens):
        for s in range(n_q):
            n = int(cmp_lens[b]) - n_q + s + 1
            if n > 0:
                idx[cu[b] + s, 0, :min(cmp_topk, n)] = np.sort(
                    rng.choice(n, size=min(cmp_topk, n), replace=False))
    q = normal((T, N1, D), seed_base + 1, dtype)
    q_rope = normal((T, N1, Dr), seed_base + 2, dtype)
    ori = (normal((P, page, 1, D), seed_base + 3, dtype), normal((P, page, 1, Dr), seed_base + 4, dtype),
           ori_bt)
    cmp = (normal((Pc, page, 1, D), seed_base + 5, dtype),
           normal((Pc, page, 1, Dr), seed_base + 6, dtype), cmp_bt, idx)
    return cu, q, q_rope, kv_lens, ori, cmp


def sfa_inputs(B=32, Sq=4, N1=64, D=512, Dr=64, page=128, kv_len=65536, topk=2048,
               seed_base=40, extra_pages=0, dtype="bf16"):
    """(q, q_rope, key_cache, key_rope_cache, block_table, kv_lens, topk_idx).
    The value cache is the key cache (shared KV)."""
    rng = np.random.default_rng(1000 + seed_base // 10)
    block_table, kv_lens, idx = sfa_paged(rng, B, Sq, kv_len, page, topk)
    P = B * (-(-kv_len // page)) + extra_pages
    q = normal((B, Sq, N1, D), seed_base + 1, dtype)
    q_rope = normal((B, Sq, N1, Dr), seed_base + 2, dtype)
    kc = normal((P, page, 1, D), seed_base + 3, dtype)
    krc = normal((P, page, 1, Dr), seed_base + 4, dtype)
    return q, q_rope, kc, krc, block_table, kv_lens, idx


# ----------------------------------------------------------------------------
# FloydAttention
# ----------------------------------------------------------------------------

def floyd_workload():
    """Pair-representation sized FloydAttention: 256 x 256 query rows per head
    over 256 keys, 8 heads of 64 dims."""
    return dict(name="floyd_256", B=1, H=8, N=256, M=256, K=256, D=64, dtype="bf16")


def floyd_inputs(B=None, H=None, N=None, M=None, K=None, D=None, seed_base=140, dtype=None):
    """(q [B,H,N,M,D], k1 [B,H,N,K,D], v1, k2 [B,H,M,K,D], v2, dout [B,H,N,M,D]):
    standard normals rounded to the working dtype; defaults from floyd_workload()."""
    w = floyd_workload()
    B, H, N, M, K, D = (w[k] if v is None else v for k, v in
                        (("B", B), ("H", H), ("N", N), ("M", M), ("K", K), ("D", D)))
    dtype = w["dtype"] if dtype is None else dtype
    q = normal((B, H, N, M, D), seed_base + 1, dtype)
    k1 = normal((B, H, N, K, D), seed_base + 2, dtype)
    v1 = normal((B, H, N, K, D), seed_base + 3, dtype)
    k2 = normal((B, H, M, K, D), seed_base + 4, dtype)
    v2 = normal((B, H, M, K, D), seed_base + 5, dtype)
    do = normal((B, H, N, M, D), seed_base + 6, dtype)
    return q, k1, v1, k2, v2, do
