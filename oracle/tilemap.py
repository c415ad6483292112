"""Tile classification of the attention mask (CPU oracle).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.

Block sparsity as the unsloth ``prefix_grouper_kernel.py`` page uses it (module
docstring: masked cross-suffix and cross-group blocks are never computed;
``get_block_mask``: one block mask per layout, built once for every batch index and
head): cut the [T, T] mask into (block_m x block_n) tiles, tile (i, j) covering
rows [i*block_m, (i+1)*block_m) and columns [j*block_n, (j+1)*block_n).  A tile is

* 0 (empty)   when it holds no kept pair,
* 2 (full)    when every one of its block_m*block_n pairs is kept,
* 1 (partial) otherwise.

Positions at or beyond T count as masked, so a tile that crosses T is never full.
The CSR lists, for every q-tile in ascending order, its non-empty kv-tiles in
ascending order with their kinds; the CSC lists, for every kv-tile, its non-empty
q-tiles.  Counts come from the element-wise mask of ``oracle.mask``; tiles whose
rows and columns share no group (or tree) are empty by the same-group conjunct and
are not enumerated.
"""
from __future__ import annotations

import numpy as np


def tile_counts(meta, block_m: int, block_n: int, block_rows: int = 1024) -> np.ndarray:
    """int64 [nq, nk]: number of kept pairs in each tile."""
    T = meta.T
    nq = -(-T // block_m)
    nk = -(-T // block_n)
    counts = np.zeros((nq, nk), dtype=np.int64)
    for comp in meta.components():
        tj = comp // block_n
        cstart = np.concatenate([[0], np.flatnonzero(np.diff(tj)) + 1])
        tj_u = tj[cstart]
        for r0 in range(0, len(comp), block_rows):
            blk = comp[r0:r0 + block_rows]
            m = meta.mask(blk, comp).astype(np.int32)
            per_col_tile = np.add.reduceat(m, cstart, axis=1)
            ti = blk // block_m
            rstart = np.concatenate([[0], np.flatnonzero(np.diff(ti)) + 1])
            per_tile = np.add.reduceat(per_col_tile.astype(np.int64), rstart, axis=0)
            counts[np.ix_(ti[rstart], tj_u)] += per_tile
    return counts


def tile_kinds(counts: np.ndarray, block_m: int, block_n: int) -> np.ndarray:
    kinds = np.where(counts == 0, 0, np.where(counts == block_m * block_n, 2, 1))
    return kinds.astype(np.uint8)


def csr(kinds: np.ndarray):
    """(row_ptr int32 [nq+1], col int32 [nnz], kind uint8 [nnz]) in ascending order."""
    nz = kinds != 0
    row_ptr = np.concatenate([[0], np.cumsum(nz.sum(axis=1))]).astype(np.int32)
    rows, cols = np.nonzero(nz)  # row-major order: rows ascending, then cols
    return row_ptr, cols.astype(np.int32), kinds[rows, cols].astype(np.uint8)


def csc(kinds: np.ndarray):
    """(col_ptr int32 [nk+1], row int32 [nnz], kind uint8 [nnz]) in ascending order."""
    nzt = (kinds != 0).T
    col_ptr = np.concatenate([[0], np.cumsum(nzt.sum(axis=1))]).astype(np.int32)
    cols, rows = np.nonzero(nzt)
    return col_ptr, rows.astype(np.int32), kinds[rows, cols].astype(np.uint8)


def tile_map(meta, block_m: int, block_n: int) -> dict:
    counts = tile_counts(meta, block_m, block_n)
    kinds = tile_kinds(counts, block_m, block_n)
    rp, col, kd = csr(kinds)
    cp, row, kd_c = csc(kinds)
    return {"counts": counts, "kinds": kinds, "row_ptr": rp, "col": col, "kind": kd,
            "col_ptr": cp, "row": row, "kind_csc": kd_c,
            "n_full": int((kinds == 2).sum()), "n_partial": int((kinds == 1).sum())}
