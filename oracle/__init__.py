"""CPU float64 oracle of shared-prefix / prefix-tree attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything here.
It shares no code with the HIP library and never imports it.

* ``oracle.mask``      - the visibility rule, element by element, from the metadata
* ``oracle.attention`` - dense masked softmax attention and its analytic gradients
* ``oracle.tilemap``   - full / partial / empty tile classification, CSR and CSC
* ``oracle.fold``      - the rollout fold (flat ids, labels, positions, metadata) and unfold
* ``oracle.draft``     - the packed-document draft mask of block-diffusion drafters
"""
from . import attention, draft, fold, mask, tilemap  # noqa: F401
