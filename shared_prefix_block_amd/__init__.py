"""Shared-prefix (prefix-tree) block-sparse attention for MI355X (gfx950).

``shared_prefix_block_amd.psa`` is the Python binding of the C-ABI library
``libpsa.so`` (hand-written HIP kernels); ``shared_prefix_block_amd.workloads``
draws the seeded synthetic inputs.  Importing the package loads nothing: the
library is opened on first use of ``psa`` and its absence raises.
"""
