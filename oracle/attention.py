"""Masked softmax attention in fp64, forward and backward (oracle; test
infrastructure only -- see ``oracle/__init__.py``).

Sources
-------
* "How SepLLM Reorchestrates the Language Model for Speed and Efficiency"
  (beiduofen.top), "SepLLM's Architecture: Composing Efficiency": O = M(A, V, M_b)
  with A the raw attention map, V the values and M_b the binary mask.
* atlas.scime.ai, "Approach": each token attends only to initial tokens,
  preceding separators and its ``n`` neighbours, at inference and in training.
* beiduofen page, "The Mechanics of Compression": in the training-from-scratch
  setting every token is restricted this way, so gradients flow only through
  the kept entries (the backward below is the derivative of the forward).

Readings
--------
* M(.) is read as softmax renormalised over the visible keys (not softmax
  followed by zeroing);
* scale defaults to ``1/sqrt(d)``;
* grouped-query attention maps query head ``h`` to key/value head
  ``h // (Hq // Hkv)``.

Nothing is blocked, fused or reordered beyond processing query rows in blocks
(to bound memory at long sequence lengths); every block materialises its mask
rows against every key up to its last row (later keys are masked by
causality, so they are left out of the products).
"""

import numpy as np

from .sepmask import separator_flags, mask_rows


def _group(Hq, Hkv):
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return Hq // Hkv


def _masked_softmax(Z, M):
    """Row-wise softmax of Z over the entries where M is true.
    Returns (P, lse) with lse the natural-log normaliser."""
    Zm = np.where(M, Z, -np.inf)
    m = Zm.max(axis=1)
    E = np.where(M, np.exp(Zm - m[:, None]), 0.0)
    ssum = E.sum(axis=1)
    lse = m + np.log(ssum)
    P = E / ssum[:, None]
    return P, lse


def attention_forward(q, k, v, tok, sep_ids, a, n, scale=None, row_block=1024):
    """Forward of SepLLM attention.

    q [B,Hq,S,d], k/v [B,Hkv,S,d] (any float, computed in fp64), tok [B,S].
    Returns ``o`` [B,Hq,S,d] and ``lse`` [B,Hq,S] (natural log of the softmax
    normaliser of each row, in the scaled-score domain).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    grp = _group(Hq, Hkv)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        sep = separator_flags(tok[b], sep_ids)
        for r0 in range(0, S, row_block):
            rows = np.arange(r0, min(S, r0 + row_block))
            kc = rows[-1] + 1  # keys beyond the last row are causally masked
            M = mask_rows(sep, a, n, rows)[:, :kc]
            for h in range(Hq):
                g = h // grp
                Z = scale * (q[b, h, rows] @ k[b, g, :kc].T)
                P, l = _masked_softmax(Z, M)
                o[b, h, rows] = P @ v[b, g, :kc]
                lse[b, h, rows] = l
    return o, lse


def attention_backward(q, k, v, do, tok, sep_ids, a, n, scale=None, row_block=1024):
    """Gradients of ``sum(o * do)`` with respect to q, k, v.

    For each query head h with key/value head g:
      P = masked softmax(scale * Q_h K_g^T)
      dV_g += P^T dO_h
      dP    = dO_h V_g^T
      D_i   = sum_j P_ij dP_ij
      dS    = P * (dP - D)
      dQ_h  = scale * dS K_g
      dK_g += scale * dS^T Q_h
    Returns (dq [B,Hq,S,d], dk [B,Hkv,S,d], dv [B,Hkv,S,d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    grp = _group(Hq, Hkv)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        sep = separator_flags(tok[b], sep_ids)
        for r0 in range(0, S, row_block):
            rows = np.arange(r0, min(S, r0 + row_block))
            kc = rows[-1] + 1  # keys beyond the last row are causally masked
            M = mask_rows(sep, a, n, rows)[:, :kc]
            for h in range(Hq):
                g = h // grp
                Z = scale * (q[b, h, rows] @ k[b, g, :kc].T)
                P, _ = _masked_softmax(Z, M)
                dv[b, g, :kc] += P.T @ do[b, h, rows]
                dP = do[b, h, rows] @ v[b, g, :kc].T
                D = (P * dP).sum(axis=1)
                dS = P * (dP - D[:, None])
                dq[b, h, rows] = scale * (dS @ k[b, g, :kc])
                dk[b, g, :kc] += scale * (dS.T @ q[b, h, rows])
    return dq, dk, dv


def attention_rows(q_h, k_g, v_g, sep, a, n, scale, rows):
    """Forward for selected query rows of one (batch, head): returns
    (o [R,d], lse [R]).  ``sep`` is the bool separator flag vector [S]."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_g = np.asarray(k_g, dtype=np.float64)
    v_g = np.asarray(v_g, dtype=np.float64)
    rows = np.asarray(rows)
    M = mask_rows(sep, a, n, rows)
    Z = scale * (q_h[rows] @ k_g.T)
    P, l = _masked_softmax(Z, M)
    return P @ v_g, l


def grad_q_rows(q_h, k_g, v_g, do_h, sep, a, n, scale, rows):
    """dQ for selected query rows of one (batch, head) -- each row's gradient
    needs only that row of P and dP."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_g = np.asarray(k_g, dtype=np.float64)
    v_g = np.asarray(v_g, dtype=np.float64)
    do_h = np.asarray(do_h, dtype=np.float64)
    rows = np.asarray(rows)
    M = mask_rows(sep, a, n, rows)
    Z = scale * (q_h[rows] @ k_g.T)
    P, _ = _masked_softmax(Z, M)
    dP = do_h[rows] @ v_g.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    return scale * (dS @ k_g)


def grad_kv_cols(qs, k_g, v_g, dos, sep, a, n, scale, cols, row_block=1024):
    """dK and dV for selected key rows ``cols`` of one (batch, kv head).

    ``qs`` and ``dos`` are lists of the [S,d] query and output-gradient arrays
    of every query head mapped to this kv head.  Every query row's softmax
    statistics are recomputed over its full mask row, then only the selected
    key columns are accumulated.
    """
    k_g = np.asarray(k_g, dtype=np.float64)
    v_g = np.asarray(v_g, dtype=np.float64)
    cols = np.asarray(cols)
    S, d = k_g.shape
    dk = np.zeros((len(cols), d))
    dv = np.zeros((len(cols), d))
    for q_h, do_h in zip(qs, dos):
        q_h = np.asarray(q_h, dtype=np.float64)
        do_h = np.asarray(do_h, dtype=np.float64)
        first = int(cols.min())
        for r0 in range(first - first % row_block, S, row_block):
            # rows above the first selected key cannot see any of the keys
            rows = np.arange(r0, min(S, r0 + row_block))
            kc = rows[-1] + 1  # keys beyond the last row are causally masked
            M = mask_rows(sep, a, n, rows)[:, :kc]
            Z = scale * (q_h[rows] @ k_g[:kc].T)
            P, _ = _masked_softmax(Z, M)
            dP = do_h[rows] @ v_g[:kc].T
            D = (P * dP).sum(axis=1)
            inb = cols < kc
            Pc = np.zeros((len(rows), len(cols)))
            Pc[:, inb] = P[:, cols[inb]]
            dPc = np.zeros((len(rows), len(cols)))
            dPc[:, inb] = dP[:, cols[inb]]
            dSc = Pc * (dPc - D[:, None])
            dv += Pc.T @ do_h[rows]
            dk += scale * (dSc.T @ q_h[rows])
    return dk, dv
