"""GPU parity of the index builder: every field bit-exact against the
oracle's direct-counting definition, on i.i.d. and bursty separator streams,
ragged lengths and degenerate parameters -- in the one-launch form and in
the two-launch form long sequences use (forced here at every length through
SEPATTN_INDEX_TWO_PASS_S)."""

import numpy as np
import pytest
import torch

import synth
from oracle import sepmask
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


def _check(tok, sep, a, n):
    import sparse_attention_sepattn_amd as sa
    B, S = tok.shape
    say(f"index B={B} S={S} a={a} n={n} n_sep={len(sep)}")
    idx = sa.build_index(torch.from_numpy(tok).cuda(), sep, a, n)
    torch.cuda.synchronize()
    for b in range(B):
        ref = sepmask.build_index(tok[b], sep, a, n)
        assert np.array_equal(idx.is_sep[b].cpu().numpy(), ref["is_sep"])
        assert np.array_equal(idx.sep_prefix[b].cpu().numpy(), ref["sep_prefix"])
        assert np.array_equal(idx.anchor_pos[b].cpu().numpy(), ref["anchor_pos"])
        assert int(idx.anchor_count[b]) == ref["anchor_count"]
        qt = idx.qtile[b].cpu().numpy()
        assert np.array_equal(qt[:, :6], ref["qtile"])
        assert np.array_equal(qt[:, 6], 128 * np.arange(qt.shape[0]))
        # field 7: separators of each tile's two 64-position blocks (from the
        # oracle's prefix counts, which start at position a)
        sp = ref["sep_prefix"].astype(np.int64)
        edge = np.minimum(np.arange(0, 2 * qt.shape[0] + 1) * 64, S)
        blk = sp[edge[1:]] - sp[edge[:-1]]
        assert np.array_equal(qt[:, 7].astype(np.int64), blk[0::2] | (blk[1::2] << 16))
        assert np.array_equal(idx.tile_class[b].cpu().numpy(), ref["tile_class"])


@pytest.mark.parametrize("S,a,n,p", [(1, 4, 64, 0.5), (5, 0, 1, 0.5), (127, 4, 64, 0.08), (128, 2, 3, 0.3),
                                     (129, 4, 64, 0.08), (300, 0, 1000, 0.2), (1000, 7, 100, 0.0),
                                     (1000, 4, 64, 1.0), (8193, 4, 256, 0.08), (700, 100, 64, 0.1),
                                     (200, 300, 5, 0.2), (2049, 4, 2049, 0.08), (1500, 70, 130, 0.05),
                                     (777, 64, 63, 0.3), (1025, 1, 1, 0.9), (300, 4, 2**31 - 1, 0.1),
                                     (500, 2**31 - 1, 5, 0.1)])
def test_index_small_and_ragged(S, a, n, p):
    require_gpu()
    r = synth.rng(S + a + n)
    sep = synth.separator_ids(r, 5000)
    tok = synth.token_ids_iid(r, (3, S), 5000, sep, p)
    _check(tok, sep, a, n)


def test_index_no_separator_ids():
    require_gpu()
    tok = synth.token_ids_iid(synth.rng(0), (2, 700), 5000, np.array([1, 2]), 0.1)
    _check(tok, np.zeros(0, dtype=np.int32), 4, 64)


@pytest.mark.parametrize("name", ["pythia160m", "long_context_32k"])
def test_index_full_size(name):
    require_gpu()
    cfg = synth.CONFIGS[name]
    r = synth.rng(cfg["seed"])
    sep = synth.separator_ids(r, cfg["vocab"])
    if cfg["bursty"]:
        tok = synth.token_ids_bursty(r, cfg["B"], cfg["S"], cfg["vocab"], sep)
    else:
        tok = synth.token_ids_iid(r, (cfg["B"], cfg["S"]), cfg["vocab"], sep, cfg["p_sep"])
    if cfg["B"] > 2:
        tok = tok[:2].copy()
    _check(tok, sep, cfg["a"], cfg["n"])


@pytest.fixture
def two_pass(monkeypatch):
    """The two-launch index at every length for the duration of a test."""
    monkeypatch.setenv("SEPATTN_INDEX_TWO_PASS_S", "1")


@pytest.mark.parametrize("S,a,n,p", [(1, 4, 64, 0.5), (5, 0, 1, 0.5), (129, 4, 64, 0.08), (300, 0, 1000, 0.2),
                                     (1000, 4, 64, 1.0), (8193, 4, 256, 0.08), (700, 100, 64, 0.1),
                                     (200, 300, 5, 0.2), (1500, 70, 130, 0.05), (777, 64, 63, 0.3),
                                     (1025, 1, 1, 0.9), (300, 4, 2**31 - 1, 0.1), (500, 2**31 - 1, 5, 0.1)])
def test_index_two_pass_small_and_ragged(two_pass, S, a, n, p):
    require_gpu()
    r = synth.rng(S + a + n + 1)
    sep = synth.separator_ids(r, 5000)
    tok = synth.token_ids_iid(r, (3, S), 5000, sep, p)
    _check(tok, sep, a, n)


def test_index_two_pass_long_context(two_pass):
    """The 32k-token bursty stream through the two-launch form."""
    require_gpu()
    cfg = synth.CONFIGS["long_context_32k"]
    r = synth.rng(cfg["seed"])
    sep = synth.separator_ids(r, cfg["vocab"])
    tok = synth.token_ids_bursty(r, cfg["B"], cfg["S"], cfg["vocab"], sep)
    _check(tok, sep, cfg["a"], cfg["n"])


def test_index_past_two_pass_length():
    """A 70000-token bursty stream: past the length from which the index takes
    two launches by default (no override)."""
    require_gpu()
    r = synth.rng(70000)
    sep = synth.separator_ids(r, 32000)
    tok = synth.token_ids_bursty(r, 1, 70000, 32000, sep)
    _check(tok, sep, 4, 256)


def test_index_forms_agree_at_256k(monkeypatch):
    """262144 tokens, 2 sequences with bursty separators: the one-launch and
    the two-launch forms give the same index bit for bit, and every field of
    the query tiles inside a 16384-token prefix equals the oracle's index of
    that prefix (those fields depend on the prefix alone; the classes of key
    tiles past it are 0)."""
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, S, P, a, n = 2, 262144, 16384, 4, 256
    r = synth.rng(S)
    sep = synth.separator_ids(r, 32000)
    tok = synth.token_ids_bursty(r, B, S, 32000, sep)
    tok_d = torch.from_numpy(tok).cuda()
    got = []
    for form in ("0", "1"):
        monkeypatch.setenv("SEPATTN_INDEX_TWO_PASS_S", form)
        say(f"index B={B} S={S} two_pass_from={form}")
        idx = sa.build_index(tok_d, sep, a, n)
        torch.cuda.synchronize()
        got.append({k: getattr(idx, k).cpu().numpy() for k in
                    ("is_sep", "sep_prefix", "anchor_pos", "anchor_count", "qtile", "tile_class")})
    for k in got[0]:
        assert np.array_equal(got[0][k], got[1][k]), k
    g = got[1]
    for b in range(B):
        ref = sepmask.build_index(tok[b, :P], sep, a, n)
        assert np.array_equal(g["is_sep"][b, :P], ref["is_sep"])
        assert np.array_equal(g["sep_prefix"][b, :P + 1], ref["sep_prefix"])
        m = ref["anchor_count"]
        assert np.array_equal(g["anchor_pos"][b, :m], ref["anchor_pos"][:m])
        assert g["anchor_count"][b] == min(a, S) + g["sep_prefix"][b, S]
        qt = P // 128
        assert np.array_equal(g["qtile"][b, :qt, :6], ref["qtile"])
        kt = P // 64
        assert np.array_equal(g["tile_class"][b, :qt, :kt], ref["tile_class"])
        assert not g["tile_class"][b, :qt, kt:].any()
