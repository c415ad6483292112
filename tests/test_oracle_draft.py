"""Pins of the draft-mask oracle (CPU).

The pages fix: the queries are draft blocks, the keys the context followed by the
drafts; a block sees the context before its anchor within the anchor's document and
its own block (all of it, or causally); packing documents must not change what a
block computes (packed == unpacked); generation is the training rule for one block
anchored at the end of the context.
"""
import numpy as np
import pytest

from oracle import attention as oa
from oracle.draft import DraftMeta
from oracle.mask import dense_mask, kept_pairs


def test_worked_example():
    """Context of 6 tokens in two documents [0 0 0 | 1 1 1], blocks of 2 anchored at
    2 (doc 0), 5 (doc 1) and 4 (doc 1, not kept), written out by hand."""
    m = DraftMeta(6, 2, [2, 5, 4], keep=[1, 1, 0], ctx_doc=[0, 0, 0, 1, 1, 1],
                  anchor_doc=[0, 1, 1])
    want = np.zeros((12, 12), dtype=bool)
    for r in (6, 7):            # block 0: context 0, 1 (before anchor 2) + its block
        want[r, [0, 1, 6, 7]] = True
    for r in (8, 9):            # block 1: context 3, 4 (doc 1, before 5) + its block
        want[r, [3, 4, 8, 9]] = True
    np.testing.assert_array_equal(dense_mask(m), want)
    mc = DraftMeta(6, 2, [2, 5, 4], keep=[1, 1, 0], ctx_doc=[0, 0, 0, 1, 1, 1],
                   anchor_doc=[0, 1, 1], causal=True)
    want[6, 7] = want[8, 9] = False  # causal blocks: offset 0 does not see offset 1
    np.testing.assert_array_equal(dense_mask(mc), want)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,bs", [(1, 1), (7, 3), (16, 4), (33, 16)])
def test_generation_block_sees_whole_context(S, bs, causal):
    """One block anchored at ctx_len (the generation layout): the whole context plus
    its own block (causally for the causal variant)."""
    m = DraftMeta(S, bs, [S], causal=causal)
    got = dense_mask(m)
    for j in range(bs):
        row = got[S + j]
        assert row[:S].all()
        want_block = np.arange(bs) <= j if causal else np.ones(bs, bool)
        np.testing.assert_array_equal(row[S:], want_block)
    assert not got[:S].any()  # context tokens are keys only


def _packed_docs(rng, n_docs, max_len, bs, max_blocks):
    lens = [int(rng.integers(1, max_len + 1)) for _ in range(n_docs)]
    ctx_doc = np.concatenate([np.full(n, 10 * d + 3) for d, n in enumerate(lens)])
    starts = np.concatenate([[0], np.cumsum(lens)])
    anchors, adoc, per_doc = [], [], []
    for d, n in enumerate(lens):
        k = int(rng.integers(0, max_blocks + 1))
        local = sorted(int(x) for x in rng.integers(0, n + 1, size=k))
        per_doc.append(local)
        anchors += [int(starts[d]) + a for a in local]
        adoc += [10 * d + 3] * k
    return lens, starts, ctx_doc, anchors, adoc, per_doc


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_unpacked(seed, causal):
    """Packing documents into one context leaves every block's output as it is with
    its own document alone (anchors taken relative to that document)."""
    rng = np.random.default_rng(400 + seed)
    bs = int(rng.integers(1, 5))
    lens, starts, ctx_doc, anchors, adoc, per_doc = _packed_docs(rng, 3, 12, bs, 3)
    S, N = int(sum(lens)), len(anchors)
    hq, hkv, d = 2, 1, 8
    T = S + N * bs
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    packed = DraftMeta(S, bs, anchors, ctx_doc=ctx_doc, anchor_doc=adoc, causal=causal)
    o, lse = oa.forward(packed, q, k, v)
    b0 = 0
    for di, n in enumerate(lens):
        nb = len(per_doc[di])
        ctx = np.arange(starts[di], starts[di] + n)
        drafts = (S + (b0 + np.arange(nb))[:, None] * bs + np.arange(bs)[None, :]).ravel()
        idx = np.concatenate([ctx, drafts]).astype(np.int64)
        alone = DraftMeta(n, bs, per_doc[di], causal=causal)
        o1, lse1 = oa.forward(alone, q[idx], k[idx], v[idx])
        np.testing.assert_allclose(o[drafts], o1[n:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, drafts], lse1[:, n:], rtol=0, atol=1e-12)
        b0 += nb


@pytest.mark.parametrize("seed", range(20))
def test_causal_variant_is_bidirectional_and_flat_causal(seed):
    """The drafts follow the context and blocks are disjoint, so the causal variant is
    the bidirectional mask restricted to kv <= q; a block not kept sees nothing and is
    seen by nothing; context rows see nothing."""
    rng = np.random.default_rng(500 + seed)
    bs = int(rng.integers(1, 6))
    lens, starts, ctx_doc, anchors, adoc, _ = _packed_docs(rng, 2, 9, bs, 3)
    S, N = int(sum(lens)), len(anchors)
    keep = rng.random(N) < 0.7
    extra = int(rng.integers(0, 4))
    bi = DraftMeta(S, bs, anchors, keep, ctx_doc, adoc, causal=False, T=S + N * bs + extra)
    ca = DraftMeta(S, bs, anchors, keep, ctx_doc, adoc, causal=True, T=S + N * bs + extra)
    mb, mc = dense_mask(bi), dense_mask(ca)
    np.testing.assert_array_equal(mc, mb & np.tril(np.ones_like(mb)))
    assert not mb[:S].any() and not mb[S + N * bs:].any() and not mb[:, S + N * bs:].any()
    for b in np.nonzero(~keep)[0]:
        rows = S + b * bs + np.arange(bs)
        assert not mb[rows].any() and not mb[:, rows].any()


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("causal", [False, True])
def test_kept_count_closed_form(seed, causal):
    """Per kept block: block_size x (context tokens of its document before its anchor)
    plus block_size^2 (bidirectional) or block_size (block_size + 1) / 2 (causal)."""
    rng = np.random.default_rng(600 + seed)
    bs = int(rng.integers(1, 9))
    lens, starts, ctx_doc, anchors, adoc, _ = _packed_docs(rng, 3, 20, bs, 4)
    S, N = int(sum(lens)), len(anchors)
    keep = rng.random(N) < 0.8
    m = DraftMeta(S, bs, anchors, keep, ctx_doc, adoc, causal=causal)
    want = 0
    for b in range(N):
        if not keep[b]:
            continue
        ctx = int(((np.arange(S) < anchors[b]) & (ctx_doc == adoc[b])).sum())
        want += bs * ctx + (bs * (bs + 1) // 2 if causal else bs * bs)
    assert kept_pairs(m) == want
