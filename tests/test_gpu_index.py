"""GPU parity of the index builder: every field bit-exact against the
oracle's direct-counting definition, on i.i.d. and bursty separator streams,
ragged lengths and degenerate parameters."""

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
