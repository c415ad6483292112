"""Masked softmax attention and its analytic gradients, float64 on the CPU (oracle).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.

What is computed is the plain definition: dense scores over the columns a row may
possibly see, the mask of ``oracle.mask`` applied element by element, a softmax,
and the product with V.  The shared-prefix method (block skipping plus an online
softmax over the prefix run and the own-suffix run) reaches this same result up to
rounding, so the oracle is the definition, not the algorithm.

Sources: unsloth ``prefix_grouper_kernel.py`` page, ``flex_shared_prefix_attention``
docstring (Q/K/V laid out [1, T, heads, head_dim], K/V with the KV head count, GQA
via ``enable_gqa``) and ``_run_flex`` (softmax scale defaults to 1/sqrt(head_dim)).
Readings: the GQA head map is PyTorch's ``enable_gqa`` convention, kv head =
q head // (Hq / Hkv) (A4); LSE is the natural log of the sum of exp(scale * q.k)
over visible keys, and a row with no visible key has O = 0, LSE = -inf and zero
gradients (A2, A3).

Backward (FlashAttention-2 style analytic gradients of the same definition), per
q head h with kv head hk:  P = softmax(S), D = rowsum(dO * O), dP = dO V^T,
dS = P * (dP - D), dQ = scale dS K, dK += scale dS^T Q, dV += P^T dO, with dK and dV
summed over the q heads that share hk.

The computation is split only by row blocks and by groups / trees (tokens of
different groups never see one another), so every kept pair is computed exactly as
in the dense definition.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: upcast its exact values
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)


def _softmax_block(meta, rows, comp, qh, kc, scale):
    """Scores, mask, probabilities and LSE for ``rows`` against columns ``comp``."""
    s = scale * (qh @ kc.T)
    m_ok = meta.mask(rows, comp)
    s = np.where(m_ok, s, NEG_INF)
    mx = s.max(axis=1) if s.shape[1] else np.full(len(rows), NEG_INF)
    has = np.isfinite(mx)
    mx_safe = np.where(has, mx, 0.0)
    e = np.exp(s - mx_safe[:, None])  # exp(-inf) = 0 on masked entries
    l = e.sum(axis=1)
    lse = np.where(has, mx_safe + np.log(np.where(has, l, 1.0)), NEG_INF)
    p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
    return p, lse, m_ok


def forward(meta, q, k, v, scale: Optional[float] = None,
            rows: Optional[Sequence[int]] = None, block_rows: int = 512):
    """O [n, Hq, d] and LSE [Hq, n] for all T rows (``rows`` None) or the listed rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    rep = hq // hkv
    sc = _scale(d, scale)
    sel = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = {int(r): i for i, r in enumerate(sel)}
    o = np.zeros((len(sel), hq, d))
    lse = np.full((hq, len(sel)), NEG_INF)
    for comp in meta.components():
        want = comp if rows is None else np.intersect1d(comp, sel)
        if len(want) == 0:
            continue
        out_idx = np.asarray([pos[int(r)] for r in want], dtype=np.int64)
        for h in range(hq):
            hk = h // rep
            kc, vc = k[comp, hk], v[comp, hk]
            for b0 in range(0, len(want), block_rows):
                blk = want[b0:b0 + block_rows]
                p, lse_b, _ = _softmax_block(meta, blk, comp, q[blk, h], kc, sc)
                o[out_idx[b0:b0 + block_rows], h] = p @ vc
                lse[h, out_idx[b0:b0 + block_rows]] = lse_b
    return o, lse


def backward(meta, q, k, v, do, scale: Optional[float] = None, block_rows: int = 512):
    """Full (O, LSE, dQ, dK, dV) for all T rows."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, hq, d = q.shape
    hkv = k.shape[1]
    rep = hq // hkv
    sc = _scale(d, scale)
    o = np.zeros_like(q)
    lse = np.full((hq, T), NEG_INF)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for comp in meta.components():
        for h in range(hq):
            hk = h // rep
            kc, vc = k[comp, hk], v[comp, hk]
            dkc = np.zeros_like(kc)
            dvc = np.zeros_like(vc)
            for b0 in range(0, len(comp), block_rows):
                blk = comp[b0:b0 + block_rows]
                p, lse_b, _ = _softmax_block(meta, blk, comp, q[blk, h], kc, sc)
                ob = p @ vc
                o[blk, h] = ob
                lse[h, blk] = lse_b
                dob = do[blk, h]
                dd = (dob * ob).sum(axis=1)
                dp = dob @ vc.T
                ds = p * (dp - dd[:, None])
                dq[blk, h] = sc * (ds @ kc)
                dkc += sc * (ds.T @ q[blk, h])
                dvc += p.T @ dob
            dk[comp, hk] += dkc
            dv[comp, hk] += dvc
    return o, lse, dq, dk, dv


def grad_rows(meta, q, k, v, do, rows: Sequence[int], scale: Optional[float] = None,
              block_rows: int = 512):
    """(O, LSE, dQ) of the listed rows only; each needs only its own row of P."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, hq, d = q.shape
    rep = hq // k.shape[1]
    sc = _scale(d, scale)
    sel = np.asarray(rows, dtype=np.int64)
    pos = {int(r): i for i, r in enumerate(sel)}
    o = np.zeros((len(sel), hq, d))
    lse = np.full((hq, len(sel)), NEG_INF)
    dq = np.zeros((len(sel), hq, d))
    for comp in meta.components():
        want = np.intersect1d(comp, sel)
        if len(want) == 0:
            continue
        oi = np.asarray([pos[int(r)] for r in want], dtype=np.int64)
        for h in range(hq):
            hk = h // rep
            kc, vc = k[comp, hk], v[comp, hk]
            for b0 in range(0, len(want), block_rows):
                blk = want[b0:b0 + block_rows]
                ii = oi[b0:b0 + block_rows]
                p, lse_b, _ = _softmax_block(meta, blk, comp, q[blk, h], kc, sc)
                ob = p @ vc
                dob = do[blk, h]
                dd = (dob * ob).sum(axis=1)
                ds = p * (dob @ vc.T - dd[:, None])
                o[ii, h] = ob
                lse[h, ii] = lse_b
                dq[ii, h] = sc * (ds @ kc)
    return o, lse, dq


def grad_cols(meta, q, k, v, do, cols: Sequence[int], scale: Optional[float] = None,
              block_rows: int = 512, kv_heads: Optional[Sequence[int]] = None):
    """(dK, dV) of the listed key/value rows only, [len(cols), hkv, d] each, or
    [len(cols), len(kv_heads), d] for the listed kv heads alone (then only the q heads
    that read those kv heads are computed).

    Each listed column needs, for every row that sees it, that row's full softmax
    (LSE) and D = rowsum(dO * O); those rows are recomputed over their group, and only
    the listed columns of dS and P are reduced.  A block of rows is taken over the
    columns of its group that at least one of its rows sees: every other column is
    masked for the whole block, so its scores are -inf, its probabilities 0, and it
    adds nothing to any sum (the same reason the groups are taken one at a time)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, hq, d = q.shape
    hkv = k.shape[1]
    rep = hq // hkv
    sc = _scale(d, scale)
    heads = list(range(hkv)) if kv_heads is None else [int(x) for x in kv_heads]
    if any(not 0 <= x < hkv for x in heads) or len(set(heads)) != len(heads):
        raise ValueError("kv_heads must be distinct kv head indices")
    slot = {hk: i for i, hk in enumerate(heads)}
    sel = np.asarray(cols, dtype=np.int64)
    pos = {int(c): i for i, c in enumerate(sel)}
    dk = np.zeros((len(sel), len(heads), d))
    dv = np.zeros((len(sel), len(heads), d))
    for comp in meta.components():
        want = np.intersect1d(comp, sel)
        if len(want) == 0:
            continue
        oi = np.asarray([pos[int(c)] for c in want], dtype=np.int64)
        # rows of this component that see at least one listed column
        need = []
        for b0 in range(0, len(comp), 4096):
            blk = comp[b0:b0 + 4096]
            need.append(blk[meta.mask(blk, want).any(axis=1)])
        need = np.concatenate(need) if need else np.zeros(0, np.int64)
        for b0 in range(0, len(need), block_rows):
            blk = need[b0:b0 + block_rows]
            cc = comp[meta.mask(blk, comp).any(axis=0)]  # columns some row of blk sees
            seen = np.isin(want, cc)  # listed columns no row of blk sees get nothing here
            if not seen.any():
                continue
            wpos = np.searchsorted(cc, want[seen])
            ow = oi[seen]
            for h in range(hq):
                hk = h // rep
                if hk not in slot:
                    continue
                kc, vc = k[cc, hk], v[cc, hk]
                p, _, _ = _softmax_block(meta, blk, cc, q[blk, h], kc, sc)
                ob = p @ vc
                dob = do[blk, h]
                dd = (dob * ob).sum(axis=1)
                pw = p[:, wpos]
                dsw = pw * (dob @ vc[wpos].T - dd[:, None])
                dk[ow, slot[hk]] += sc * (dsw.T @ q[blk, h])
                dv[ow, slot[hk]] += pw.T @ dob
    return dk, dv
