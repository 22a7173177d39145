"""fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by the smoke
check and by the benchmark's CPU-baseline leg, never by the library.  It shares
no code with the HIP path; both sides only share the seeded 16-bit inputs from
``synth``.

What is computed (sources are the three pages on the subject):

* Standard attention, ``O = softmax(Q K^T / sqrt(d)) V`` with the softmax over
  keys: page 1, examples 1-3 (the einsum/softmax/einsum formulas), and page 2,
  "Kernel Fusion" (the bmm -> softmax -> bmm baseline).  The method the pages
  describe produces exactly this result (page 2, "Tiling": the online softmax
  agrees with the full-matrix computation), so the oracle is that definition
  written out with the full N x N score matrix, in float64.
* The row log-sum-exp ``LSE_i = log sum_j exp(sigma * q_i . k_j)`` over visible
  keys (natural log, scale included).  The pages do not define it; it is the
  quantity that lets the backward rebuild P blockwise (page 2,
  "Re-computation"), read as ``P_ij = exp(sigma s_ij - LSE_i)``.
* Causal masking: key j is visible to query i iff j <= i (not on the pages; the
  plainest reading with equal query and key lengths).
* The backward: gradients of ``L = <dO, O>`` with respect to Q, K, V, derived
  from the definition (the pages only describe the recompute loop order, page
  2, "Re-computation"; the gradient formulas are pinned by finite differences).

Self-check variants, used only to pin this oracle against the pages' claims:
the key-blocked online softmax of page 2 ("Tiling": local max and exp-sum per
tile, global max update with rescaled normaliser, one final normalisation) and
the query-chunked loop of page 1, example 2.

``scale`` is used as given.  Callers pass the float32 value the GPU receives
(e.g. ``float(np.float32(1/sqrt(d)))``) so both sides use the same scalar.
"""
from __future__ import annotations

import math
from typing import Iterable, Tuple

import numpy as np


def _visible_mask(n_q: int, n_k: int, causal: bool) -> np.ndarray | None:
    if not causal:
        return None
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i


def forward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 causal: bool, bias: np.ndarray | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """One (batch, head): q,k,v float64 [N, d] -> (O [N, d], LSE [N]).

    Materialises S = scale * Q K^T (+ bias [N, N], an additive attention bias
    in the same natural-log units; page 2, "工程落地的关键考量", suggests one
    for masking very long sequences), masks, and takes a max-subtracted
    softmax over each row (page 1 examples 1-3; page 2 "Kernel Fusion"
    baseline).  A row with no visible key or only -inf scores gets O = 0 and
    LSE = -inf.
    """
    s = scale * (q @ k.T)
    if bias is not None:
        s = s + bias
    vis = _visible_mask(q.shape[0], k.shape[0], causal)
    if vis is not None:
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[:, None] > 0, (p @ v) / l[:, None], 0.0)
        lse = np.where(l > 0, m_safe + np.log(l), -np.inf)
    return o, lse


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
            causal: bool, bias: np.ndarray | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """[B, H, N, d] float64 -> (O [B, H, N, d], LSE [B, H, N]), one head at a time.
    ``bias`` (optional) broadcasts to [B, H, N, N]."""
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    bb = None if bias is None else np.broadcast_to(bias, (B, H, N, k.shape[2]))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal,
                                              None if bb is None else bb[b, h])
    return o, lse


def forward_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: Iterable,
                 scale: float, causal: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Selected query rows only.  ``rows`` holds (b, h, i) triples.

    For each row: s = scale * K[visible] q_i, then the same softmax as
    ``forward_head``.  Used at sizes where the full matrix is too large.
    """
    rows = [tuple(int(x) for x in r) for r in rows]
    out_o = np.empty((len(rows), v.shape[-1]), dtype=np.float64)
    out_lse = np.empty(len(rows), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        kk = k[b, h, : i + 1] if causal else k[b, h]
        vv = v[b, h, : i + 1] if causal else v[b, h]
        s = scale * (kk @ q[b, h, i])
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        out_o[n] = (p @ vv) / l
        out_lse[n] = m + math.log(l)
    return out_o, out_lse


def backward_head(q, k, v, do, scale: float, causal: bool, bias=None):
    """Gradients of L = <dO, O> for one head; inputs float64 [N, d].

    With P the normalised softmax of S = scale * Q K^T (+ bias, a constant
    whose gradient dS is not formed here) (masked):
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij            (equals sum_c dO_ic O_ic)
        dS = P * (dP - D 1^T)
        dQ = scale * dS K,   dK = scale * dS^T Q
    """
    s = scale * (q @ k.T)
    if bias is not None:
        s = s + bias
    vis = _visible_mask(q.shape[0], k.shape[0], causal)
    if vis is not None:
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        p = np.where(l > 0, p / l, 0.0)  # a row with every score -inf has O = 0
    dv = p.T @ do
    dp = do @ v.T
    dsum = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward(q, k, v, do, scale: float, causal: bool, bias=None):
    """[B, H, N, d] float64 -> (dQ, dK, dV), one head at a time.
    ``bias`` (optional) broadcasts to [B, H, N, N]."""
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    B, H, N = q.shape[:3]
    bb = None if bias is None else np.broadcast_to(bias, (B, H, N, k.shape[2]))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal,
                None if bb is None else bb[b, h])
    return dq, dk, dv


def backward_dq_rows(q, k, v, do, rows: Iterable, scale: float, causal: bool):
    """dQ for selected query rows only; ``rows`` holds (b, h, i) triples.

    Row i of the backward above depends on row i alone: its softmax over the
    visible keys, O_i, D_i = dO_i . O_i, dP_ij = dO_i . v_j,
    dS_ij = P_ij (dP_ij - D_i) and dQ_i = scale * sum_j dS_ij k_j.  Used at
    sizes where the full matrices are too large (page 2, "Re-computation":
    the row's probabilities are rebuilt from Q and K).
    """
    rows = [tuple(int(x) for x in r) for r in rows]
    out = np.empty((len(rows), k.shape[-1]), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        kk = k[b, h, : i + 1] if causal else k[b, h]
        vv = v[b, h, : i + 1] if causal else v[b, h]
        s = scale * (kk @ q[b, h, i])
        p = np.exp(s - s.max())
        p /= p.sum()
        o_i = p @ vv
        dp = vv @ do[b, h, i]
        ds = p * (dp - do[b, h, i] @ o_i)
        out[n] = scale * (ds @ kk)
    return out


def backward_kv_cols(q, k, v, do, cols: Iterable, scale: float, causal: bool,
                     chunk: int = 1024):
    """dK and dV for selected key rows only; ``cols`` holds (b, h, j) triples.

    Key j's gradients need column j of P and dS over every query row, and
    those need each row's LSE_i and D_i.  Per head touched, a forward over
    query chunks of ``chunk`` rows (the same masked softmax as forward_head,
    one chunk of the N x N matrix at a time) gives LSE and O, hence
    D_i = dO_i . O_i; then for the selected keys
        P_ij = exp(scale q_i . k_j - LSE_i),  dP_ij = dO_i . v_j,
        dS_ij = P_ij (dP_ij - D_i),
        dK_j = scale * sum_i dS_ij q_i,       dV_j = sum_i P_ij dO_i.
    """
    cols = [tuple(int(x) for x in c) for c in cols]
    dk_out = np.empty((len(cols), k.shape[-1]), dtype=np.float64)
    dv_out = np.empty((len(cols), v.shape[-1]), dtype=np.float64)
    heads = sorted({(b, h) for b, h, _ in cols})
    for b, h in heads:
        qh, kh, vh, gh = q[b, h], k[b, h], v[b, h], do[b, h]
        n = qh.shape[0]
        lse = np.empty(n, dtype=np.float64)
        dsum = np.empty(n, dtype=np.float64)
        for i0 in range(0, n, chunk):
            i1 = min(n, i0 + chunk)
            kend = i1 if causal else kh.shape[0]
            s = scale * (qh[i0:i1] @ kh[:kend].T)
            if causal:
                ii = np.arange(i0, i1)[:, None]
                jj = np.arange(kend)[None, :]
                s = np.where(jj <= ii, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            o = (p @ vh[:kend]) / l
            lse[i0:i1] = (m + np.log(l))[:, 0]
            dsum[i0:i1] = (gh[i0:i1] * o).sum(axis=1)
        sel = [(n_, j) for n_, (bb, hh, j) in enumerate(cols) if (bb, hh) == (b, h)]
        idx = np.array([j for _, j in sel])
        s = scale * (qh @ kh[idx].T)                       # [N, m]
        if causal:
            s = np.where(idx[None, :] <= np.arange(n)[:, None], s, -np.inf)
        p = np.exp(s - lse[:, None])
        dp = gh @ vh[idx].T
        ds = p * (dp - dsum[:, None])
        dk_sel = scale * (ds.T @ qh)
        dv_sel = p.T @ gh
        for r, (n_, _) in enumerate(sel):
            dk_out[n_] = dk_sel[r]
            dv_out[n_] = dv_sel[r]
    return dk_out, dv_out


# ----------------------------------------------------------------------------
# Self-check variants (pins for the definition above; never compared to GPU)
# ----------------------------------------------------------------------------
def forward_key_blocked(q, k, v, scale: float, causal: bool, block: int):
    """Online softmax over key blocks, in float64, for one head [N, d].

    Page 2, "Tiling": (1) per tile, the local row max and local exp-sum;
    (2) update the running (global) max and rescale the running normaliser
    and the running weighted sum by exp(old max - new max); (3) divide by the
    normaliser once at the end.
    """
    n_q, n_k = q.shape[0], k.shape[0]
    m = np.full(n_q, -np.inf)
    l = np.zeros(n_q)
    acc = np.zeros((n_q, v.shape[1]))
    rows = np.arange(n_q)[:, None]
    for j0 in range(0, n_k, block):
        j1 = min(j0 + block, n_k)
        s = scale * (q @ k[j0:j1].T)
        if causal:
            s = np.where(np.arange(j0, j1)[None, :] <= rows, s, -np.inf)
        tile_max = s.max(axis=1)
        m_new = np.maximum(m, tile_max)
        m_safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_safe), 0.0)
        p = np.exp(s - m_safe[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
    o = acc / l[:, None]
    lse = m + np.log(l)
    return o, lse


def forward_query_chunked(q, k, v, scale: float, causal: bool, chunk: int):
    """Page 1, example 2: loop over query chunks, full softmax over all keys
    for each chunk, and write each chunk's rows into the output. One head."""
    n_q = q.shape[0]
    o = np.zeros((n_q, v.shape[1]))
    lse = np.zeros(n_q)
    for i0 in range(0, n_q, chunk):
        i1 = min(i0 + chunk, n_q)
        s = scale * (q[i0:i1] @ k.T)
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] <= np.arange(i0, i1)[:, None],
                         s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        o[i0:i1] = (p / l) @ v
        lse[i0:i1] = (m + np.log(l))[:, 0]
    return o, lse


def forward_scalar(q, k, v, scale: float, causal: bool):
    """Brute force with Python floats and explicit loops, for tiny heads
    (a few rows and columns): direct sums, no vectorisation."""
    n_q, d = len(q), len(q[0])
    n_k, dv = len(k), len(v[0])
    o = [[0.0] * dv for _ in range(n_q)]
    lse = [0.0] * n_q
    for i in range(n_q):
        scores = []
        for j in range(n_k):
            if causal and j > i:
                continue
            dot = 0.0
            for c in range(d):
                dot += float(q[i][c]) * float(k[j][c])
            scores.append((j, scale * dot))
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        for j, x in w:
            for c in range(dv):
                o[i][c] += x / tot * float(v[j][c])
        lse[i] = mx + math.log(tot)
    return np.array(o), np.array(lse)
