"""Checks that pin the fp64 block-sparse oracle to facts other than itself.

Each ``pin_*`` takes ``bref(q, k, v, kb_ptr, kb_idx, block, causal, scale, rows=None)``
(q bf16 bits [B, H_q, N, D], k, v [B, H_kv, N, D]) -> (o, lse) and raises
AssertionError when a result contradicts the (separately pinned) forward or
packed-batch oracles, torch's fp64 SDPA with the expanded boolean mask, a closed
form, or the locality of the mask.  They run on the real oracle
(test_oracle_blocksparse_pins.py) and on copies with planted mistakes
(test_oracle_blocksparse_mutations.py).

What is pinned: attention restricted to listed key blocks per query block
(block-sparse patterns in a compressed storage format: future work on page
"AVO算法优化Transformer注意力机制性能解析", section 6), over the forward's
definition.
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch

import oracle
from synth import lists_to_csr
from tests.oracle_pins import SCALE, bits_to64, close, rnd


def _inputs(seed, B, Hq, Hkv, N, D=16):
    return rnd(seed, (B, Hq, N, D)), rnd(seed + 1, (B, Hkv, N, D)), rnd(seed + 2, (B, Hkv, N, D))


def _expand(lists, mask_heads, n_blocks, block, N, Hq, causal):
    """Boolean [H_q, N, N] mask from the lists (the definition, written out)."""
    m = np.zeros((Hq, N, N), bool)
    for h in range(Hq):
        mh = 0 if mask_heads == 1 else h
        for qb in range(n_blocks):
            for kb in lists[mh * n_blocks + qb]:
                if 0 <= kb < n_blocks:
                    m[h, qb * block:(qb + 1) * block, kb * block:(kb + 1) * block] = True
    if causal:
        m &= np.tril(np.ones((N, N), bool))[None]
    return m


def pin_full_lists_equal_dense(bref):
    """Every key block listed: the (separately pinned) dense forward oracle, in
    both mask modes, with a ragged last block."""
    B, Hq, Hkv, N, blk = 2, 4, 2, 37, 8
    nb = -(-N // blk)
    q, k, v = _inputs(2100, B, Hq, Hkv, N)
    ptr, idx = lists_to_csr([list(range(nb))] * nb)
    for causal in (False, True):
        o, lse = bref(q, k, v, ptr, idx, blk, causal, SCALE)
        eo, el = oracle.attn_ref(q, k, v, causal, SCALE, n_threads=1)
        close(o, eo, tol=1e-13, what=f"full lists O causal={causal}")
        close(lse, el, tol=1e-13, what=f"full lists LSE causal={causal}")


def pin_diagonal_blocks_equal_packed(bref):
    """Each query block listing only its own key block is a packed batch of
    block-long sequences: the (separately pinned) packed-batch oracle with
    cu_seqlens at the block boundaries, in both mask modes."""
    Hq, Hkv, N, blk = 4, 1, 30, 8
    nb = -(-N // blk)
    q, k, v = _inputs(2200, 1, Hq, Hkv, N)
    ptr, idx = lists_to_csr([[qb] for qb in range(nb)])
    cu = np.array(list(range(0, N, blk)) + [N], np.int32)
    for causal in (False, True):
        o, lse = bref(q, k, v, ptr, idx, blk, causal, SCALE)
        eo, el = oracle.attn_varlen_ref(q[0], k[0], v[0], cu, causal, SCALE)
        close(o[0], eo, tol=1e-13, what=f"diagonal blocks O causal={causal}")
        close(lse[0], el, tol=1e-13, what=f"diagonal blocks LSE causal={causal}")


def pin_torch_expanded_mask(bref):
    """Random per-head lists against torch's fp64 SDPA with the expanded boolean
    mask and scipy's logsumexp of the masked scores (GQA, both mask modes, rows
    that see at least one key)."""
    B, Hq, Hkv, N, blk = 1, 4, 2, 40, 8
    nb = N // blk
    rng = np.random.default_rng(7)
    lists = [sorted(set(rng.integers(0, nb, 3).tolist()) | {qb}) for _ in range(Hq) for qb in range(nb)]
    ptr, idx = lists_to_csr(lists)
    q, k, v = _inputs(2300, B, Hq, Hkv, N)
    qt = torch.from_numpy(bits_to64(q))
    kt = torch.from_numpy(bits_to64(k)).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(bits_to64(v)).repeat_interleave(Hq // Hkv, dim=1)
    for causal in (False, True):
        m = _expand(lists, Hq, nb, blk, N, Hq, causal)
        o, lse = bref(q, k, v, ptr, idx, blk, causal, SCALE)
        eo = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(m)[None], scale=SCALE).numpy()
        s = SCALE * torch.matmul(qt, kt.transpose(-1, -2)).numpy()
        s = np.where(m[None], s, -np.inf)
        seen = m.any(-1)[None]
        close(o[seen], eo[seen], tol=1e-12, what=f"torch O causal={causal}")
        close(lse[seen], scipy.special.logsumexp(s, axis=-1)[seen], tol=1e-12,
              what=f"logsumexp causal={causal}")


def pin_empty_rows(bref):
    """A query block with an empty list, and causal rows whose listed blocks
    all lie after them, see no key: O = 0 and LSE = -inf; other rows are
    unaffected by them."""
    B, Hq, Hkv, N, blk = 1, 2, 2, 24, 8
    q, k, v = _inputs(2400, B, Hq, Hkv, N)
    ptr, idx = lists_to_csr([[2], [], [0, 2]])
    for causal in (False, True):
        o, lse = bref(q, k, v, ptr, idx, blk, causal, SCALE)
        empty = np.zeros(N, bool)
        empty[8:16] = True                  # query block 1: empty list
        if causal:
            empty[0:8] = True               # query block 0 lists only block 2
        assert np.all(o[:, :, empty] == 0.0), "empty rows must give O = 0"
        assert np.all(np.isneginf(lse[:, :, empty])), "empty rows must give LSE = -inf"
        assert np.all(np.isfinite(lse[:, :, ~empty])), "non-empty rows must be finite"


def pin_locality(bref):
    """Changing keys and values in blocks a query block does not list leaves its
    rows unchanged (bitwise); changing a listed block changes them."""
    B, Hq, Hkv, N, blk = 1, 2, 1, 32, 8
    q, k, v = _inputs(2500, B, Hq, Hkv, N)
    lists = [[0, 3], [1], [1, 2], [0, 1, 2, 3]]
    ptr, idx = lists_to_csr(lists)
    o, lse = bref(q, k, v, ptr, idx, blk, False, SCALE)
    k2, v2 = k.copy(), v.copy()
    k2[..., 16:24, :] = rnd(2510, k2[..., 16:24, :].shape)   # key block 2
    v2[..., 16:24, :] = rnd(2511, v2[..., 16:24, :].shape)
    o2, lse2 = bref(q, k2, v2, ptr, idx, blk, False, SCALE)
    for qb, ls in enumerate(lists):
        rows = slice(qb * blk, (qb + 1) * blk)
        same = np.array_equal(o[:, :, rows], o2[:, :, rows]) and np.array_equal(lse[:, :, rows], lse2[:, :, rows])
        assert same == (2 not in ls), f"query block {qb}: locality violated"


def pin_list_hygiene_and_sharing(bref):
    """Duplicate and out-of-range entries change nothing; one shared list
    equals the same list repeated for every head; sampled rows equal full rows."""
    B, Hq, Hkv, N, blk = 2, 3, 3, 20, 8
    q, k, v = _inputs(2600, B, Hq, Hkv, N)
    clean = [[0], [0, 1], [2]]
    ptr, idx = lists_to_csr(clean)
    dirty_ptr, dirty_idx = lists_to_csr([[0, 0, -1], [0, 1, 1, 7], [2, 99]])
    per_ptr, per_idx = lists_to_csr(clean * Hq)
    rows = np.array([0, 7, 8, 19, 40, 59, 100, 119], np.int64)
    for causal in (False, True):
        o, lse = bref(q, k, v, ptr, idx, blk, causal, SCALE)
        od, ld = bref(q, k, v, dirty_ptr, dirty_idx, blk, causal, SCALE)
        op, lp = bref(q, k, v, per_ptr, per_idx, blk, causal, SCALE)
        assert np.array_equal(o, od) and np.array_equal(lse, ld), "list hygiene"
        assert np.array_equal(o, op) and np.array_equal(lse, lp), "shared vs per-head lists"
        so, sl = bref(q, k, v, ptr, idx, blk, causal, SCALE, rows=rows)
        assert np.array_equal(so, o.reshape(-1, 16)[rows]) and np.array_equal(sl, lse.reshape(-1)[rows])


def pin_sparse_nonfinite(bref):
    """Non-finite inputs under a block list: a NaN in V of a block a query block
    does not list leaves its rows bitwise unchanged, and reaches every row that
    lists it; a listed key with a -inf score has weight 0 (torch's fp64 SDPA
    over the row's other keys); a row whose listed scores are all -inf is NaN,
    unlike a row with no listed key (O = 0, LSE = -inf)."""
    B, Hq, Hkv, N, blk = 1, 2, 1, 24, 8
    q, k, v = _inputs(2700, B, Hq, Hkv, N)
    lists = [[0], [0, 1], [2], []]
    ptr, idx = lists_to_csr(lists[:3])
    o0, l0 = bref(q, k, v, ptr, idx, blk, False, SCALE)
    v2 = v.copy()
    v2[0, 0, 10, 4] = 0x7FC0        # key block 1: listed by query block 1 only
    o2, l2 = bref(q, k, v2, ptr, idx, blk, False, SCALE)
    assert np.all(np.isnan(o2[0, :, 8:16, 4])), "NaN must reach the rows that list its block"
    keep = np.ones(o0.shape, bool)
    keep[0, :, 8:16, 4] = False
    assert np.array_equal(o2[keep], o0[keep]) and np.array_equal(l2, l0), "NaN spread"
    # -inf score of listed key 3 for row 2 (query block 0 lists block 0 only)
    q3, k3 = q.copy(), k.copy()
    q3[0, 0, 2, 5] = 0x3F80         # +1
    k3[0, 0, 3, 5] = 0xFF80         # -inf
    o3, l3 = bref(q3, k3, v, ptr, idx, blk, False, SCALE)
    keys = [0, 1, 2, 4, 5, 6, 7]
    qi = torch.from_numpy(bits_to64(q3[0, 0, 2:3]))
    ko = torch.from_numpy(bits_to64(k3[0, 0, keys]))
    vo = torch.from_numpy(bits_to64(v[0, 0, keys]))
    eo = torch.nn.functional.scaled_dot_product_attention(qi, ko, vo, scale=SCALE)
    el = scipy.special.logsumexp(SCALE * (qi.numpy() @ ko.numpy().T), axis=-1)
    close(o3[0, 0, 2], eo.numpy()[0], tol=1e-12, what="-inf score drops its key")
    close(l3[0, 0, 2], el[0], tol=1e-12, what="-inf score drops its key (LSE)")
    # all listed scores -inf (row 17 lists block 2: keys 16..23)
    q4, k4 = q.copy(), k.copy()
    k4[0, 0, 16:24, 6] = 0xBF80     # -1
    q4[0, 1, 17, 6] = 0x7F80        # +inf
    for causal in (False, True):
        o4, l4 = bref(q4, k4, v, ptr, idx, blk, causal, SCALE)
        assert np.all(np.isnan(o4[0, 1, 17])) and np.isnan(l4[0, 1, 17]), "all -inf listed scores"


ALL_PINS = [pin_full_lists_equal_dense, pin_diagonal_blocks_equal_packed, pin_torch_expanded_mask,
            pin_empty_rows, pin_locality, pin_list_hygiene_and_sharing, pin_sparse_nonfinite]
