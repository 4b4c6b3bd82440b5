"""Plain fp64 attention: the definition the HIP path is checked against.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg, never by
the library.

Conventions (the readings are listed with their reasons in the design notes):

* Inputs are taken exactly as stored: bf16 or fp32 values are upcast to
  float64 without rounding, and all arithmetic is float64.
* ``scale`` multiplies the raw dot products: S = scale * Q K^T.  Where the
  scale is applied (pre-scaled Q in the NumPy page's Step 3, scaled scores in
  the worked example and in the FlashAttention-2 page's fused kernel) is the
  same thing in exact arithmetic; the oracle scales S.
* Mask (FlashAttention-2 inference page, Step 3): key j is visible to query
  i iff (not causal or j <= i) and (window < 0 or j >= i - window).  A window
  of W therefore admits W+1 keys including the query's own position.
* Masked scores are set to -inf by selection (FlashAttention-2 page, Step 2),
  so they carry exactly zero weight.
* L is the natural-log logsumexp of the visible scaled scores of a row:
  L = m + ln(l) with m the row max and l the sum of exp(S - m).
* A row with no visible key (cannot happen with the causal mask, which always
  admits the diagonal) has O = 0 and L = -inf.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 (accepts numpy arrays and torch CPU tensors)."""
    if hasattr(x, "detach"):  # torch tensor: bf16 -> fp32 is exact, fp32 -> fp64 exact
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def allowed_mask(rows, n_keys: int, causal: bool, window: int) -> np.ndarray:
    """Visibility of keys 0..n_keys-1 for the query positions in ``rows``.

    FlashAttention-2 inference page, Step 3: a key later than the query is
    hidden by the causal mask, and a key more than ``window`` positions before
    the query is hidden by the sliding ("block-sparse") window.
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], n_keys), dtype=bool)
    if causal:
        ok &= j <= i
    if window >= 0:
        ok &= j >= i - window
    return ok


def _softmax_rows(S: np.ndarray, ok: np.ndarray):
    """Max-subtracted softmax of the visible entries of each row.

    NumPy page, Step 1 (stable softmax: subtract the row max, exponentiate,
    divide by the row sum).  Returns (P, L) with L = m + ln(sum exp(S - m)).
    """
    S = np.where(ok, S, -np.inf)
    empty = ~ok.any(axis=1)
    m = np.where(empty, 0.0, S.max(axis=1, initial=-np.inf))
    E = np.exp(S - m[:, None])  # exp(-inf) == 0 exactly
    ell = E.sum(axis=1)
    ell_safe = np.where(empty, 1.0, ell)
    P = E / ell_safe[:, None]
    L = np.where(empty, -np.inf, m + np.log(ell_safe))
    return P, L


def _head(Q, K, V, scale, rows, causal, window):
    """One (batch, head): scores, mask, softmax, weighted sum of V."""
    S = (Q @ K.T) * scale
    ok = allowed_mask(rows, K.shape[0], causal, window)
    P, L = _softmax_rows(S, ok)
    return P @ V, L, P


def attention_ref(q, k, v, scale: float, causal: bool = False, window: int = -1):
    """O and L of softmax(scale * Q K^T, masked) V for every (batch, head).

    NumPy page, Step 1 (the un-tiled reference used as the oracle there),
    with the scale/mask of the FlashAttention-2 inference page, Steps 2-3.
    q, k, v: [..., N, d] (any leading dims).  Returns (O [..., N, d] float64,
    L [..., N] float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    N = q.shape[-2]
    O = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    L = np.empty(q.shape[:-1], dtype=np.float64)
    rows = np.arange(N)
    for idx in np.ndindex(*lead):
        O[idx], L[idx], _ = _head(q[idx], k[idx], v[idx], scale, rows, causal, window)
    return O, L


def attention_rows_ref(Q, K, V, scale: float, rows, causal: bool = False, window: int = -1):
    """The same definition for a subset of query rows of one head.

    Used to check full-size outputs on sampled rows: row i of O depends only on
    query i and all keys/values, so it can be computed on its own.
    Q, K, V: [N, d].  Returns (O [len(rows), d], L [len(rows)]).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    rows = np.asarray(rows, dtype=np.int64)
    O, L, _ = _head(Q[rows], K, V, scale, rows, causal, window)
    return O, L


def attention_probs_ref(Q, K, scale: float, causal: bool = False, window: int = -1):
    """The normalised attention matrix P of one head ([N, N], float64).

    Exposed for invariant tests (every row of P sums to one, masked entries
    are exactly zero).
    """
    Q, K = _f64(Q), _f64(K)
    S = (Q @ K.T) * scale
    P, _ = _softmax_rows(S, allowed_mask(np.arange(Q.shape[0]), K.shape[0], causal, window))
    return P


def attention_tiled_ref(Q, K, V, scale: float, block_q: int, block_k: int,
                        causal: bool = False, window: int = -1, trace: bool = False):
    """The tiled online-softmax loop, in float64, for one head.

    NumPy page, Architecture Overview and Steps 2-3, and the worked example's
    Steps 1-3: for every query tile keep a running row max m, a running sum
    l and an unnormalised output O; for every key/value tile compute the
    scaled scores, mask them, raise m, rescale l and O by exp(m_old - m_new),
    add exp(S - m_new) and its product with V; divide by l once at the end.

    Differences from the printed listings, each a reading of the pages:
    a ragged last tile is masked rather than zero-padded, the causal and
    window masks of the FlashAttention-2 page are applied by selection to
    -inf, and exp(m_old - m_new) is taken as 0 while m_old is still -inf (a
    row that has seen no visible key yet).

    Returns (O [N, d], L [N], trace) where trace (if requested) is a list,
    per query tile, of per-key-tile dicts {S, m, l, alpha} recorded after each
    update -- the quantities the worked example prints.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    N, d = Q.shape
    Nk = K.shape[0]
    O = np.zeros((N, V.shape[1]))
    L = np.full(N, -np.inf)
    tr = []
    for qs in range(0, N, block_q):
        rows = np.arange(qs, min(qs + block_q, N))
        m = np.full(rows.size, -np.inf)
        ell = np.zeros(rows.size)
        acc = np.zeros((rows.size, V.shape[1]))
        tile_trace = []
        for ks in range(0, Nk, block_k):
            cols = np.arange(ks, min(ks + block_k, Nk))
            S = (Q[rows] @ K[cols].T) * scale
            ok = allowed_mask(rows, Nk, causal, window)[:, cols]
            S = np.where(ok, S, -np.inf)
            m_new = np.maximum(m, S.max(axis=1))
            ref = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - ref))
            P = np.exp(S - ref[:, None])
            ell = alpha * ell + P.sum(axis=1)
            acc = alpha[:, None] * acc + P @ V[cols]
            m = m_new
            if trace:
                tile_trace.append({"S": S.copy(), "m": m.copy(), "l": ell.copy(),
                                   "alpha": alpha.copy()})
        seen = ell > 0
        O[rows] = np.where(seen[:, None], acc / np.where(seen, ell, 1.0)[:, None], 0.0)
        L[rows] = np.where(seen, m + np.log(np.where(seen, ell, 1.0)), -np.inf)
        tr.append(tile_trace)
    return O, L, tr


def decode_ref(q, kcache, vcache, seqlens, scale: float, window: int = -1):
    """Single-token decode over a KV cache, for every (sequence, head).

    KV-cache page, Steps 4-5: the new query attends to every cached key,
    including the key of its own token, which is the last valid cache row.
    Row s of the cache holds seqlens[s] valid tokens; the query sits at
    position seqlens[s]-1, so no causal mask is needed.  With a window W the
    query sees only positions >= seqlens[s]-1-W (the FlashAttention-2 page's
    sliding window, applied at the query's position).

    q: [S, H, d]; kcache, vcache: [S, H, Lmax, d] (rows past seqlens[s] are
    never read); seqlens: [S] ints >= 1.  Returns (o [S, H, d], lse [S, H]).
    """
    Sq, H, d = q.shape
    seqlens = np.asarray(seqlens, dtype=np.int64)
    o = np.empty((Sq, H, vcache.shape[-1]))
    lse = np.empty((Sq, H))
    for s in range(Sq):
        n = int(seqlens[s])
        for h in range(H):
            K = _f64(kcache[s, h, :n])
            V = _f64(vcache[s, h, :n])
            Oh, Lh, _ = _head(_f64(q[s, h])[None, :], K, V, scale, [n - 1], False, window)
            o[s, h] = Oh[0]
            lse[s, h] = Lh[0]
    return o, lse


def _gather(pool, pages, h: int, rows) -> np.ndarray:
    """Rows pool[pages[i], h, rows[i]] as float64 (numpy array or torch tensor)."""
    if hasattr(pool, "detach"):
        import torch
        pages, rows = torch.as_tensor(pages), torch.as_tensor(rows)
    return _f64(pool[pages, h, rows])


def _page_rows(table_row, n: int, P: int, num_pages: int):
    """Where tokens 0..n-1 of one sequence live: (page, row in page, present)."""
    t = np.arange(n)
    page = np.asarray(table_row, dtype=np.int64)[t // P]
    return page, t % P, (page >= 0) & (page < num_pages)


def decode_paged_ref(q, k_pages, v_pages, block_table, seqlens, scale: float, window: int = -1):
    """Single-token decode whose cache rows are held in pages.

    The logical cache is the one of the KV-cache page, Step 2 (one key and one
    value row per token, in token order); the rows are stored in fixed-size
    pages of a shared pool, as in the paged KV cache named among the upgrades
    of the FlashAttention-2 inference page (Extending It).  Token t of
    sequence s is row t % P of page block_table[s, t // P], P the page size.
    A table entry outside [0, num_pages) marks its tokens as absent: they take
    no part in the softmax (a page dropped from a sliding window).  The
    result is then decode_ref's on that logical cache: the query sits at
    position seqlens[s]-1 and, with a window W, sees positions >= seqlens[s]-1-W.

    q: [S, H, d]; k_pages, v_pages: [num_pages, H, P, d]; block_table:
    [S, max_pages] ints; seqlens: [S] ints >= 1.  Returns (o [S, H, d],
    lse [S, H]).
    """
    Sq, H, d = q.shape
    num_pages, _, P, _ = k_pages.shape
    table = np.asarray(block_table, dtype=np.int64)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    o = np.empty((Sq, H, v_pages.shape[-1]))
    lse = np.empty((Sq, H))
    for s in range(Sq):
        n = int(seqlens[s])
        page, row, present = _page_rows(table[s], n, P, num_pages)
        at = np.nonzero(present)[0]
        for h in range(H):
            K = np.zeros((n, k_pages.shape[-1]))
            V = np.zeros((n, v_pages.shape[-1]))
            K[at] = _gather(k_pages, page[at], h, row[at])
            V[at] = _gather(v_pages, page[at], h, row[at])
            S_row = (K @ _f64(q[s, h])) * scale
            ok = allowed_mask([n - 1], n, False, window) & present[None, :]
            P_row, L_row = _softmax_rows(S_row[None, :], ok)
            o[s, h] = (P_row @ V)[0]
            lse[s, h] = L_row[0]
    return o, lse


def attention_bwd_ref(q, k, v, dO, scale: float, causal: bool = False, window: int = -1):
    """Exact gradients of O = attention(Q, K, V) with respect to Q, K and V.

    NumPy page, Step 4: the backward pass recomputes P from the forward
    statistics and uses D = rowsum(dO * O).  The page's own dK and dQ lines
    are declared simplified there; this follows the full chain rule through
    the softmax, which is where the D term enters:

        dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
        dQ = scale * dS K,  dK = scale * dS^T Q.

    L is treated as a by-product of the forward and receives no gradient.
    q, k, v, dO: [..., N, d].  Returns (dQ, dK, dV), float64.
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    dQ = np.empty_like(q)
    dK = np.empty_like(k)
    dV = np.empty_like(v)
    rows = np.arange(q.shape[-2])
    for idx in np.ndindex(*q.shape[:-2]):
        Q, K, V, G = q[idx], k[idx], v[idx], dO[idx]
        O, _, P = _head(Q, K, V, scale, rows, causal, window)
        D = (G * O).sum(axis=1)
        dV[idx] = P.T @ G
        dP = G @ V.T
        dS = P * (dP - D[:, None])
        dQ[idx] = scale * (dS @ K)
        dK[idx] = scale * (dS.T @ Q)
    return dQ, dK, dV
