"""Block table of a block-sparse mask (FlexAttention's BlockMask model), from the element
mask.  TEST INFRASTRUCTURE ONLY (see the package docstring).

PyTorch issue 135161 ("Significant Accuracy Difference between Compiled and Eager Flex
Attention", its second repro) builds each mask with ``create_block_mask`` from a predicate
over (q_idx, kv_idx) and runs ``flex_attention(..., block_mask=...)``.  In that model the
(Sq, Sk) plane is cut into 128 x 128 blocks; a block with no visible pair is skipped, a
block whose every pair is visible is computed with no element mask, and any other block
is computed with the predicate applied element by element.  The result is the plain
masked attention of the element mask, which the attention oracle computes directly; this
module states only the classification and the traversal lists.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
EMPTY, FULL, PARTIAL = 0, 1, 2


def block_kinds(mask: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """[..., nqb, nkb] block kind (EMPTY / FULL / PARTIAL) of boolean mask [..., Sq, Sk].

    Only pairs inside the (Sq, Sk) plane count: the last block row and column may be
    partial in extent."""
    mask = np.asarray(mask, dtype=bool)
    sq, sk = mask.shape[-2:]
    nqb, nkb = -(-sq // block), -(-sk // block)
    kinds = np.zeros(mask.shape[:-2] + (nqb, nkb), dtype=np.int32)
    for qb in range(nqb):
        for kb in range(nkb):
            tile = mask[..., qb * block:(qb + 1) * block, kb * block:(kb + 1) * block]
            anyv = tile.any(axis=(-2, -1))
            allv = tile.all(axis=(-2, -1))
            kinds[..., qb, kb] = np.where(allv, FULL, np.where(anyv, PARTIAL, EMPTY))
    return kinds


def block_lists(kinds: np.ndarray):
    """Traversal lists of a kind table [..., nqb, nkb].

    Returns (kv_count [..., nqb], kv_list [..., nqb, nkb], q_count [..., nkb],
    q_list [..., nkb, nqb]).  Row qb of kv_list holds, in increasing kb, 2*kb + 1 for each
    partial block and 2*kb for each full block of that block row; q_list holds the same for
    each block column, in increasing qb.  Entries past the count are -1."""
    kinds = np.asarray(kinds)
    nqb, nkb = kinds.shape[-2:]
    lead = kinds.shape[:-2]
    kv_count = np.zeros(lead + (nqb,), np.int32)
    kv_list = np.full(lead + (nqb, nkb), -1, np.int32)
    q_count = np.zeros(lead + (nkb,), np.int32)
    q_list = np.full(lead + (nkb, nqb), -1, np.int32)
    for idx in np.ndindex(*lead):
        kt = kinds[idx]
        for qb in range(nqb):
            ent = [2 * kb + (kt[qb, kb] == PARTIAL) for kb in range(nkb) if kt[qb, kb] != EMPTY]
            kv_count[idx + (qb,)] = len(ent)
            kv_list[idx + (qb,)][:len(ent)] = ent
        for kb in range(nkb):
            ent = [2 * qb + (kt[qb, kb] == PARTIAL) for qb in range(nqb) if kt[qb, kb] != EMPTY]
            q_count[idx + (kb,)] = len(ent)
            q_list[idx + (kb,)][:len(ent)] = ent
    return kv_count, kv_list, q_count, q_list
