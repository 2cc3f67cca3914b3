"""The SepLLM attention mask and the tile index derived from it (oracle; test
infrastructure only -- see ``oracle/__init__.py``).

Sources
-------
* SepLLM summary on atlas.scime.ai, "Approach": each token attends only to the
  initial tokens, all preceding separators and a local window of ``n``
  neighbours.
* "How SepLLM Reorchestrates the Language Model for Speed and Efficiency"
  (beiduofen.top), "SepLLM's Architecture: Composing Efficiency": the output is
  O = M(A, V, M_b) with a binary S x S mask M_b (the page's math is garbled;
  the mask is read as {0,1}^(S x S)).
* atlas.scime.ai, "Limitations" and "Measured effects reported in the paper":
  the separator set is a hand-chosen hyper-parameter (nine types by default).

Readings taken where the pages are silent
-----------------------------------------
* window: "``n`` neighbours" counts the query itself, i.e. key ``j`` is in the
  window of query ``i`` iff ``i - j < n``;
* a key is visible if it is initial OR a separator OR in the window (a union;
  only the key's own status matters);
* separator status is membership of the token id in the given id set.

The tile metadata (``build_index``) is not on the pages: it is the bookkeeping
the GPU schedule uses, defined here by direct counting so that the GPU's closed
forms can be checked bit for bit.
"""

import numpy as np


def separator_flags(tok, sep_ids):
    """``sep[j] = tok[j] in SEP`` (atlas.scime.ai, "Limitations": the separator
    set is a fixed, hand-chosen set of token types)."""
    tok = np.asarray(tok)
    sep_ids = np.asarray(sep_ids, dtype=np.int64).reshape(-1)
    out = np.zeros(tok.shape, dtype=bool)
    for s in sep_ids:  # plain membership test, one id at a time
        out |= tok == s
    return out


def interval_flags(S, m):
    """Anchor flags of the fixed-interval baseline (FixLLM): the pages compare
    SepLLM with a variant that keeps tokens at fixed intervals instead of
    separators (beiduofen.top, "Performance in the Spotlight: Experimental
    Results"; atlas.scime.ai, "Measured effects reported in the paper" and
    "Surprising findings").  Neither page gives the interval or its phase;
    the reading taken: position ``j`` is an anchor iff ``j % m == m - 1`` (the
    last token of every ``m``-token segment, as a separator ends its
    segment), for an interval ``m >= 1`` the caller chooses."""
    if m < 1:
        raise ValueError("interval m must be >= 1")
    j = np.arange(S, dtype=np.int64)
    return (j % m) == (m - 1)


def mask_rows(sep, a, n, rows):
    """Rows ``rows`` of the SepLLM mask for one sequence whose separator flags
    are ``sep`` (bool [S]).

    ``M[i, j] = (j <= i) and (j < a or sep[j] or i - j < n)``
    (atlas.scime.ai, "Approach"; reading of the window bound: ``i - j < n``).
    Returns bool [len(rows), S].
    """
    S = sep.shape[0]
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    causal = j <= i
    initial = j < a
    separator = sep[None, :]
    window = (i - j) < n
    return causal & (initial | separator | window)


def sep_mask(tok, sep_ids, a, n):
    """The full S x S boolean mask ``M_b`` of one sequence (beiduofen page,
    "SepLLM's Architecture"; atlas.scime.ai, "Approach")."""
    sep = separator_flags(tok, sep_ids)
    S = sep.shape[0]
    return mask_rows(sep, a, n, np.arange(S))


def row_nnz(sep, a, n, row_block=1024):
    """Number of visible keys of every query row, counted from the mask
    (``mask_rows`` of ``row_block`` rows at a time, to bound memory)."""
    S = sep.shape[0]
    out = np.zeros(S, dtype=np.int64)
    for r0 in range(0, S, row_block):
        rows = np.arange(r0, min(S, r0 + row_block))
        out[rows] = mask_rows(sep, a, n, rows).sum(axis=1)
    return out


def build_index(tok, sep_ids, a, n, tq=128, tk=64):
    """Per-sequence index metadata, defined by direct counting.

    ``tok`` is one sequence [S].  Returns a dict:

    * ``is_sep``      uint8 [S]    -- separator flags;
    * ``sep_prefix``  int32 [S+1]  -- ``#{j : a <= j < x, sep[j]}`` for x in [0, S];
    * ``anchor_pos``  int32 [S]    -- initial tokens ``0..min(a,S)-1`` followed by
      the separators at positions ``>= a`` in ascending order, then ``-1``;
    * ``anchor_count`` int         -- number of anchors;
    * ``qtile``       int32 [QT,6] -- per ``tq``-row query tile ``qi`` with rows
      ``q0 = tq*qi .. q1``: ``lo`` (first key in the window of row ``q0``),
      ``n_anchor`` (anchors strictly below ``lo``), ``kt_begin = lo // tk``,
      ``kt_end = q1 // tk``, ``n_kept = ceil(n_anchor/tk) + kt_end - kt_begin + 1``,
      ``rows = q1 - q0 + 1``;
    * ``tile_class``  uint8 [QT,KT] -- over the original ``tq x tk`` grid, 0 if
      the mask has no visible entry in the tile, 2 if every entry is visible,
      1 otherwise.
    """
    tok = np.asarray(tok).reshape(-1)
    return build_index_from_flags(separator_flags(tok, sep_ids), a, n, tq, tk)


def build_index_from_flags(sep, a, n, tq=128, tk=64):
    """``build_index`` for given anchor flags ``sep`` (bool [S]): the
    separator flags of a token sequence, or the fixed-interval flags of
    ``interval_flags``."""
    sep = np.asarray(sep, dtype=bool).reshape(-1)
    S = sep.shape[0]
    sep_prefix = np.zeros(S + 1, dtype=np.int64)
    running = 0
    for x in range(S + 1):
        sep_prefix[x] = running
        if x < S and x >= a and sep[x]:
            running += 1

    anchors = [j for j in range(min(a, S))] + [j for j in range(a, S) if sep[j]]
    anchor_pos = np.full(S, -1, dtype=np.int64)
    anchor_pos[: len(anchors)] = anchors

    QT = (S + tq - 1) // tq
    KT = (S + tk - 1) // tk
    qtile = np.zeros((QT, 6), dtype=np.int64)
    tile_class = np.zeros((QT, KT), dtype=np.uint8)
    for qi in range(QT):
        q0 = tq * qi
        q1 = min(q0 + tq - 1, S - 1)
        lo = max(0, q0 - n + 1)
        n_anchor = sum(1 for p in anchors if p < lo)
        kt_begin = lo // tk
        kt_end = q1 // tk
        n_kept = -(-n_anchor // tk) + (kt_end - kt_begin + 1)
        qtile[qi] = (lo, n_anchor, kt_begin, kt_end, n_kept, q1 - q0 + 1)

        M = mask_rows(sep, a, n, np.arange(q0, q1 + 1))
        for kj in range(KT):
            c0 = tk * kj
            c1 = min(c0 + tk - 1, S - 1)
            block = M[:, c0 : c1 + 1]
            cnt = int(block.sum())
            if cnt == 0:
                tile_class[qi, kj] = 0
            elif cnt == block.size:
                tile_class[qi, kj] = 2
            else:
                tile_class[qi, kj] = 1

    return {
        "is_sep": sep.astype(np.uint8),
        "sep_prefix": sep_prefix.astype(np.int32),
        "anchor_pos": anchor_pos.astype(np.int32),
        "anchor_count": len(anchors),
        "qtile": qtile.astype(np.int32),
        "tile_class": tile_class,
    }


def kept_entries(qtile, tk=64):
    """Entries of the kept-tile schedule: ``E = sum_q-tiles rows * tk * n_kept``.
    This is the unit the throughput figures count (not a page quantity)."""
    qtile = np.asarray(qtile, dtype=np.int64)
    return int((qtile[:, 5] * tk * qtile[:, 4]).sum())
