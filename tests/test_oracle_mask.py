"""Pins of the oracle's mask and tile index (CPU only).

* the hand-derived worked example in tests/golden/mask_example.txt;
* brute force over every separator pattern of short sequences (a per-element
  loop, independent of the oracle's vectorised form);
* reductions: n >= S or all-separator sequences give the causal mask; no
  separators give sink + sliding window (built with np.tril/np.triu);
* closed forms: per-row visible count, anchor count, anchors below a tile.
"""

import itertools

import numpy as np
import pytest

from oracle import sepmask


def _ints(s):
    return [int(x) for x in s.split()]


def test_golden_mask_example(golden):
    g = golden("mask_example.txt")
    S, a, n = int(g["S"]), int(g["a"]), int(g["n"])
    tq, tk = int(g["tq"]), int(g["tk"])
    seps = _ints(g["separators"])
    sep_ids = [1000 + i for i in range(3)]
    tok = np.full(S, 7, dtype=np.int64)
    for p in seps:
        tok[p] = sep_ids[p % 3]
    M = sepmask.sep_mask(tok, sep_ids, a, n)
    for i in range(S):
        row = g[f"row{i}"]
        assert "".join("1" if x else "." for x in M[i]) == row, i
    assert list(M.sum(1)) == _ints(g["nnz"])
    idx = sepmask.build_index(tok, sep_ids, a, n, tq=tq, tk=tk)
    assert list(idx["is_sep"]) == _ints(g["is_sep"])
    assert list(idx["sep_prefix"]) == _ints(g["sep_prefix"])
    assert list(idx["anchor_pos"]) == _ints(g["anchor_pos"])
    assert idx["anchor_count"] == int(g["anchor_count"])
    for qi in range(idx["qtile"].shape[0]):
        assert list(idx["qtile"][qi]) == _ints(g[f"qtile{qi}"]), qi
        assert list(idx["tile_class"][qi]) == _ints(g[f"class{qi}"]), qi


def _brute_mask(sep, a, n):
    S = len(sep)
    M = np.zeros((S, S), dtype=bool)
    for i in range(S):
        for j in range(S):
            if j > i:
                continue
            if j < a or sep[j] or i - j < n:
                M[i, j] = True
    return M


def _tok_from_flags(flags, sep_ids=(11, 12)):
    tok = np.array([sep_ids[k % 2] if f else 3 + k for k, f in enumerate(flags)])
    return tok, list(sep_ids)


def _check_index_against_mask(tok, sep_ids, a, n, tq, tk):
    S = len(tok)
    sep = np.isin(tok, sep_ids)
    M = _brute_mask(sep, a, n)
    assert np.array_equal(sepmask.sep_mask(tok, sep_ids, a, n), M)
    idx = sepmask.build_index(tok, sep_ids, a, n, tq=tq, tk=tk)
    anchors = [int(p) for p in idx["anchor_pos"] if p >= 0]
    # closed form of the anchor count and of every row's visible count
    assert idx["anchor_count"] == min(a, S) + int(sep[a:].sum())
    sp = idx["sep_prefix"]
    for i in range(S):
        lo_i = max(0, i - n + 1)
        assert M[i].sum() == (i - lo_i + 1) + min(a, lo_i) + sp[lo_i]
    QT = -(-S // tq)
    KT = -(-S // tk)
    for qi in range(QT):
        lo, n_anchor, kb, ke, n_kept, rows = [int(x) for x in idx["qtile"][qi]]
        q0, q1 = tq * qi, min(tq * qi + tq - 1, S - 1)
        assert n_anchor == min(a, lo) + sp[lo]
        # partition identity: visible keys of every row = anchors below lo
        # (disjoint) + the masked band [lo, i]
        for i in range(q0, q1 + 1):
            vis = set(np.nonzero(M[i])[0].tolist())
            below = anchors[:n_anchor]
            assert all(p < lo for p in below)
            band = {j for j in range(lo, i + 1) if M[i, j]}
            assert vis == set(below) | band
            assert not (set(below) & band)
            # the band lies inside key tiles kt_begin..kt_end
            assert all(kb * tk <= j <= ke * tk + tk - 1 for j in band)
        for kj in range(KT):
            blk = M[q0:q1 + 1, tk * kj:min(tk * kj + tk, S)]
            want = 0 if blk.sum() == 0 else (2 if blk.all() else 1)
            assert idx["tile_class"][qi, kj] == want


@pytest.mark.parametrize("S", [1, 2, 5, 8])
def test_brute_force_all_patterns(S):
    for flags in itertools.product([False, True], repeat=S):
        tok, sep_ids = _tok_from_flags(flags)
        for a in range(0, 4):
            for n in range(1, S + 1):
                _check_index_against_mask(tok, sep_ids, a, n, tq=4, tk=2)


def test_brute_force_random_longer():
    r = np.random.default_rng(123)
    for _ in range(60):
        S = int(r.integers(9, 40))
        flags = r.random(S) < r.random()
        tok, sep_ids = _tok_from_flags(flags)
        a = int(r.integers(0, 6))
        n = int(r.integers(1, S + 2))
        tq = int(r.choice([2, 4, 8]))
        tk = int(r.choice([1, 2, 4]))
        _check_index_against_mask(tok, sep_ids, a, n, tq, tk)


def test_dense_reduction():
    """n >= S, or every token a separator: the mask is plain causal."""
    S = 37
    causal = np.tril(np.ones((S, S), dtype=bool))
    tok = np.arange(S) + 100
    assert np.array_equal(sepmask.sep_mask(tok, [5], 2, S), causal)
    assert np.array_equal(sepmask.sep_mask(tok, [5], 0, S + 10), causal)
    allsep = np.full(S, 5)
    assert np.array_equal(sepmask.sep_mask(allsep, [5], 0, 1), causal)


def test_streaming_reduction():
    """No separators: sink tokens + sliding window (StreamingLLM's pattern),
    built here from triangular matrices."""
    S = 50
    tok = np.arange(S) + 100
    for a, n in [(0, 1), (4, 8), (3, 17), (0, 50)]:
        ones = np.ones((S, S), dtype=bool)
        band = np.tril(ones) & np.triu(ones, -(n - 1))
        sink = np.tril(ones) & (np.arange(S)[None, :] < a)
        assert np.array_equal(sepmask.sep_mask(tok, [7], a, n), band | sink)


def _nnz_closed_form(sep, a, n):
    """Visible keys of row i, from the partition of the row (atlas.scime.ai,
    "Approach"): the whole window [lo_i, i] with lo_i = max(0, i - n + 1),
    plus the initial tokens below lo_i and the separators in [a, lo_i).  The
    separator counts are a running sum taken here, not the oracle's index."""
    sep = np.asarray(sep, dtype=bool)
    S = sep.shape[0]
    j = np.arange(S)
    cnt = np.concatenate([[0], np.cumsum(sep & (j >= a))])  # separators in [a, x)
    i = np.arange(S)
    lo = np.maximum(0, i - n + 1)
    return (i - lo + 1) + np.minimum(a, lo) + cnt[lo]


@pytest.mark.parametrize("S", [1, 3, 6, 8])
def test_row_nnz_brute_force_all_patterns(S):
    """row_nnz equals the row sums of the per-element brute-force mask and
    the closed form, for every separator pattern, a and n, with row blocks
    smaller than, equal to and larger than S."""
    for flags in itertools.product([False, True], repeat=S):
        sep = np.array(flags, dtype=bool)
        for a in range(0, 4):
            for n in range(1, S + 2):
                want = _brute_mask(sep, a, n).sum(axis=1)
                assert np.array_equal(want, _nnz_closed_form(sep, a, n))
                for blk in (1, 3, S, S + 5):
                    assert np.array_equal(sepmask.row_nnz(sep, a, n, row_block=blk), want), (flags, a, n, blk)


def test_row_nnz_random_longer_blocked():
    """Longer random sequences (up to 2600 keys, past the default block of
    1024 rows) against the closed form, with blocks that leave a ragged last
    block."""
    r = np.random.default_rng(77)
    for S, blk in [(2600, 1024), (1500, 1024), (700, 97), (129, 64), (64, 64), (300, 299)]:
        sep = r.random(S) < r.random() * 0.3
        a = int(r.integers(0, 8))
        for n in (1, 2, 64, 255, S, S + 3):
            assert np.array_equal(sepmask.row_nnz(sep, a, n, row_block=blk), _nnz_closed_form(sep, a, n)), (S, a, n)


def test_row_nnz_special_cases():
    """No separators and a = 0: min(i + 1, n) keys; every token a separator
    or n >= S: i + 1 keys (causal); n = 1 and no separators: the query and
    the initial tokens below it."""
    S = 300
    i = np.arange(S)
    none = np.zeros(S, dtype=bool)
    assert np.array_equal(sepmask.row_nnz(none, 0, 17, row_block=50), np.minimum(i + 1, 17))
    assert np.array_equal(sepmask.row_nnz(np.ones(S, dtype=bool), 0, 1, row_block=64), i + 1)
    assert np.array_equal(sepmask.row_nnz(none, 3, S, row_block=128), i + 1)
    assert np.array_equal(sepmask.row_nnz(none, 4, 1, row_block=100), np.minimum(i, 4) + 1)


def test_kept_entries_counts_tiles():
    tok = np.arange(300) % 13
    idx = sepmask.build_index(tok, [0, 5], 4, 64)
    E = sepmask.kept_entries(idx["qtile"])
    nnz = sepmask.row_nnz(np.isin(tok, [0, 5]), 4, 64).sum()
    assert nnz <= E  # kept tiles cover every visible entry
    assert E == sum(int(r[5]) * 64 * int(r[4]) for r in idx["qtile"])


# ---- fixed-interval anchors (the FixLLM baseline) ---------------------------

@pytest.mark.parametrize("S,m,a", [(1, 1, 0), (37, 1, 2), (300, 12, 4), (300, 7, 9), (129, 200, 3), (512, 64, 0)])
def test_interval_prefix_closed_form(S, m, a):
    """#{j in [a, x) : j % m == m - 1} = floor(x/m) - floor(a/m) for x >= a."""
    ix = sepmask.build_index_from_flags(sepmask.interval_flags(S, m), a, 64)
    x = np.arange(S + 1)
    expect = np.where(x >= a, x // m - a // m, 0)
    assert np.array_equal(ix["sep_prefix"], expect)
    assert ix["anchor_count"] == min(a, S) + max(0, S // m - a // m) * (S > a)


def test_interval_every_token_is_dense_causal():
    """m = 1 makes every token an anchor: the mask is the causal mask."""
    S = 97
    sep = sepmask.interval_flags(S, 1)
    M = sepmask.mask_rows(sep, 2, 5, np.arange(S))
    assert np.array_equal(M, np.tril(np.ones((S, S), dtype=bool)))


def test_interval_beyond_length_is_sink_plus_window():
    """m > S leaves no interval anchor: initial tokens plus the window only."""
    S, a, n = 150, 3, 20
    sep = sepmask.interval_flags(S, S + 1)
    nnz = sepmask.mask_rows(sep, a, n, np.arange(S)).sum(axis=1)
    i = np.arange(S)
    lo = np.maximum(0, i - n + 1)
    assert np.array_equal(nnz, np.minimum(a, lo) + (i - lo + 1))


@pytest.mark.parametrize("S,m", [(200, 5), (333, 12)])
def test_interval_index_equals_token_index(S, m):
    """The flag path agrees with the token path on a sequence whose separator
    ids sit exactly at the interval positions."""
    sep_id = 7
    tok = np.where(np.arange(S) % m == m - 1, sep_id, 100)
    a, n = 4, 32
    x = sepmask.build_index_from_flags(sepmask.interval_flags(S, m), a, n)
    y = sepmask.build_index(tok, [sep_id], a, n)
    for key in ("is_sep", "sep_prefix", "anchor_pos", "qtile", "tile_class"):
        assert np.array_equal(x[key], y[key]), key
    assert x["anchor_count"] == y["anchor_count"]
