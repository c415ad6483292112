"""Host-side checks of the C ABI (no GPU needed, no compute call).

The library must load, export every function psa.h declares, and reject bad
arguments before touching the GPU.  Tree layouts are validated on the host, so the
layout rules of the tree builder are tested here too.
"""
import ctypes
import os
import re

import pytest

from shared_prefix_block_amd import psa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(psa.lib_path()):
        pytest.skip("libpsa.so not built")
    return psa.load()


def test_header_declares_binding_exports():
    assert _declared() == sorted(psa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.psa_abi_version() == 6
    for code, name in psa.STATUS.items():
        s = lib.psa_status_string(code).decode()
        assert s and s != "unknown status", name
    assert lib.psa_status_string(99).decode() == "unknown status"


def test_tile_shape(lib):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    assert lib.psa_tile_shape(0, 1, 128, ctypes.byref(bm), ctypes.byref(bn)) == 0
    assert (bm.value, bn.value) == (128, 128)
    assert lib.psa_tile_shape(1, 0, 64, ctypes.byref(bm), ctypes.byref(bn)) == 0
    assert lib.psa_tile_shape(0, 1, 96, ctypes.byref(bm), ctypes.byref(bn)) == 5
    # fp32 and bf16: d in {64, 128, 256}, both passes
    for dt in (0, 1):
        for d in (64, 128, 256):
            for pass_ in (0, 1):
                assert lib.psa_tile_shape(pass_, dt, d, ctypes.byref(bm), ctypes.byref(bn)) == 0
    assert lib.psa_tile_shape(1, 0, 512, ctypes.byref(bm), ctypes.byref(bn)) == 5
    assert lib.psa_tile_shape(0, 7, 128, ctypes.byref(bm), ctypes.byref(bn)) == 4
    # e4m3 inputs: forward only, at the bf16 head sizes
    for d in (64, 128, 256):
        assert lib.psa_tile_shape(0, 2, d, ctypes.byref(bm), ctypes.byref(bn)) == 0
        assert lib.psa_tile_shape(1, 2, d, ctypes.byref(bm), ctypes.byref(bn)) == 5
    assert lib.psa_tile_shape(0, 2, 96, ctypes.byref(bm), ctypes.byref(bn)) == 5
    assert lib.psa_tile_shape(0, 1, 128, None, ctypes.byref(bn)) == 1


def _tree(lib, nl, paths, T=None, bm=128, bn=128):
    import numpy as np
    nl_a = np.asarray(nl, np.int32)
    ptr = np.zeros(len(paths) + 1, np.int32)
    for i, p in enumerate(paths):
        ptr[i + 1] = ptr[i] + len(p)
    nodes = np.asarray([n for p in paths for n in p] or [0], np.int32)
    out = ctypes.c_void_p()
    T = int(nl_a.sum()) if T is None else T
    st = lib.psa_build_tile_map_tree(len(nl), ctypes.c_void_p(nl_a.ctypes.data), len(paths),
                                     ctypes.c_void_p(ptr.ctypes.data),
                                     ctypes.c_void_p(nodes.ctypes.data), T, bm, bn, None,
                                     ctypes.byref(out))
    return st, lib.psa_last_error().decode()


@pytest.mark.parametrize("nl,paths,why", [
    ([4, 4, 4], [[0, 1], [2, 1]], "two different parents"),
    ([4, 4, 4], [[0, 1]], "lies on no path"),
    ([4, 4], [[0, 5]], "out of range"),
    ([4, -1], [[0, 1]], "negative node length"),
    ([4, 4], [[1, 0]], "comes before its parent"),
    ([4, 4, 4], [[0, 2, 1]], "comes before its parent"),  # 1's parent is 2
    ([4], [[]], "empty"),
])
def test_tree_layout_rejected_on_host(lib, nl, paths, why):
    st, msg = _tree(lib, nl, paths)
    assert st == 3, (st, msg)
    assert why in msg


def test_builder_flags_rejected(lib):
    """Only PSA_MAP_NODE_FORM is a known build flag (checked before any device work)."""
    import numpy as np
    out = ctypes.c_void_p()
    assert lib.psa_build_tile_map_tokens_ex(16, None, None, None, 128, 128, 2, None,
                                            ctypes.byref(out)) == 10
    nl = np.asarray([4], np.int32)
    ptr = np.asarray([0, 1], np.int32)
    nodes = np.asarray([0], np.int32)
    assert lib.psa_build_tile_map_tree_ex(1, ctypes.c_void_p(nl.ctypes.data), 1,
                                          ctypes.c_void_p(ptr.ctypes.data),
                                          ctypes.c_void_p(nodes.ctypes.data), 4, 128, 128, 4,
                                          None, ctypes.byref(out)) == 10
    assert b"flag" in lib.psa_last_error()


def test_draft_builder_argument_errors(lib):
    """Checked on the host before any device work."""
    out = ctypes.c_void_p()
    fake = ctypes.c_void_p(256)  # never dereferenced: every check below fails first
    call = lambda S, bs, n, anchors=fake, cdoc=None, adoc=None, flags=0, T=None: \
        lib.psa_build_tile_map_draft(S, bs, n, anchors, None, cdoc, adoc, flags,
                                     S + n * bs if T is None else T, 128, 128, None,
                                     ctypes.byref(out))  # noqa: E731
    assert call(8, 4, 2, flags=2) == 10                  # unknown flag
    assert call(8, 0, 2) == 2                            # block_size < 1
    assert call(8, 4, 2, T=15) == 2                      # T too short
    assert call(1 << 20, 1, 1 << 13) == 2                # (S + 1) * N above 2^32
    assert call(8, 4, 2, anchors=None) == 1              # anchors missing
    assert call(8, 4, 2, cdoc=fake) == 1                 # documents given by halves
    assert call(8, 4, 2, adoc=fake) == 1


def test_tree_shape_errors(lib):
    st, msg = _tree(lib, [4, 4], [[0, 1]], T=7)
    assert st == 2 and "shorter" in msg
    st, _ = _tree(lib, [4, 4], [[0, 1]], bm=0)
    assert st == 2
    st, _ = _tree(lib, [4, 4], [[0, 1]], bn=2048)
    assert st == 2


def test_token_builder_argument_errors(lib):
    out = ctypes.c_void_p()
    assert lib.psa_build_tile_map_tokens(16, None, None, None, 128, 128, None,
                                         ctypes.byref(out)) == 1
    assert lib.psa_build_tile_map_tokens(16, None, None, None, 128, 128, None, None) == 1
    assert lib.psa_build_tile_map_tokens(-1, None, None, None, 128, 128, None,
                                         ctypes.byref(out)) == 2
    assert lib.psa_build_tile_map_tokens(16, None, None, None, 0, 128, None,
                                         ctypes.byref(out)) == 2


def test_attention_argument_errors(lib):
    assert lib.psa_fwd(None, 1, 16, 2, 2, 128, 0.0, None, None, None, None, None, None) == 1
    n = ctypes.c_size_t()
    assert lib.psa_bwd_workspace_size(None, 1, 16, 2, 2, 128, ctypes.byref(n)) == 1
    assert lib.psa_bwd(None, 1, 0, 16, 2, 2, 128, 0.0, *([None] * 9), None, 0, None) == 1
    assert lib.psa_tile_map_info_get(None, None) == 1
    assert lib.psa_tile_map_export(None, *([None] * 8)) == 1
    assert lib.psa_tile_map_export_nodes(None, None, None, None) == 1
    lib.psa_tile_map_destroy(None)  # no-op


def _fold_call(lib, n_groups, prompt_len, comp_ptr, comp_len, T, ws_bytes=1 << 20, outs=True):
    arr = lambda a: (ctypes.c_int32 * len(a))(*a)  # noqa: E731
    fake = ctypes.c_void_p(256)  # never dereferenced: every check below fails first
    o = fake if outs else None
    return lib.psa_fold_rollouts(n_groups, arr(prompt_len), arr(comp_ptr), arr(comp_len or [0]),
                                 fake, fake, T, 0, -100, o, o, o, o, o, None, fake, ws_bytes, None)


def test_fold_rejects_bad_tables(lib):
    assert _fold_call(lib, -1, [1], [0, 1], [1], 8) == 2           # PSA_ERR_SHAPE
    assert _fold_call(lib, 1, [2], [1, 1], [], 8) == 3             # comp_ptr[0] != 0
    assert _fold_call(lib, 2, [2, 2], [0, 2, 1], [1, 1], 8) == 3   # decreasing comp_ptr
    assert _fold_call(lib, 1, [-1], [0, 1], [1], 8) == 3           # negative prompt
    assert _fold_call(lib, 1, [2], [0, 1], [-3], 8) == 3           # negative completion
    assert _fold_call(lib, 1, [4], [0, 1], [5], 8) == 2            # T < folded length
    assert _fold_call(lib, 1, [2], [0, 1], [1], 8, outs=False) == 1  # nothing to write
    assert _fold_call(lib, 1, [2], [0, 1], [1], 8, ws_bytes=4) == 7  # PSA_ERR_WORKSPACE
    assert b"workspace" in lib.psa_last_error()


def test_unfold_rejects_bad_rows(lib):
    arr = lambda a: (ctypes.c_int32 * len(a))(*a)  # noqa: E731
    fake = ctypes.c_void_p(256)
    call = lambda T, rb, ws=1 << 20, dst=1 << 20: lib.psa_unfold_rows(  # noqa: E731
        1, arr([2]), arr([0, 2]), arr([1, 1]), T, rb, fake, fake, dst, fake, ws, None)
    assert call(4, 6) == 2    # row_bytes not a multiple of 4
    assert call(4, 0) == 2
    assert call(3, 8) == 2    # T shorter than the folded length
    assert call(4, 8, ws=8) == 7
    # the two samples [p | c0], [p | c1] take 6 rows of 8 bytes: 47 bytes of dst are short
    assert call(4, 8, dst=47) == 2
    assert b"dst holds 47 bytes" in lib.psa_last_error()
    assert call(4, 8, dst=48, ws=8) == 7  # 48 bytes pass the dst check
    b = ctypes.c_size_t(0)
    assert lib.psa_fold_workspace_size(3, 7, ctypes.byref(b)) == 0 and b.value >= 256
    assert lib.psa_fold_workspace_size(-1, 7, ctypes.byref(b)) == 2
