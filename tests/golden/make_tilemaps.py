"""Write the oracle's tile kinds of the two largest workloads (slow to recompute).

Calls only ``oracle/`` (and the seeded layout generator).  Run from the repo root:
    python tests/golden/make_tilemaps.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.mask import meta_from_layout  # noqa: E402
from oracle.tilemap import tile_counts, tile_kinds  # noqa: E402
from shared_prefix_block_amd import workloads as wl  # noqa: E402

for idx in (3, 4):
    lay = wl.layout_for(wl.WORKLOADS[idx])
    counts = tile_counts(meta_from_layout(lay), 128, 128, block_rows=2048)
    kinds = tile_kinds(counts, 128, 128)
    path = os.path.join(HERE, f"tilemap_cfg{idx}_128x128.npz")
    np.savez_compressed(path, kinds=kinds, T=lay.T, kept=counts.sum())
    print(path, kinds.shape, int((kinds == 2).sum()), int((kinds == 1).sum()), int(counts.sum()))
