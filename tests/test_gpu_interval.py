"""GPU parity of the fixed-interval (FixLLM) variant: the index bit-exact
against the oracle's flag definition, and forward/backward on that index
against the fp64 oracle.  The attention oracle is driven through token ids
that carry a separator id exactly at the interval positions; the CPU suite
pins that this gives the same index as the interval flags."""

import numpy as np
import pytest
import torch

import synth
from oracle import attention, sepmask
from tests.gpu_util import dev_tensor, host_f64, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("two_pass", [False, True])
@pytest.mark.parametrize("B,S,m,a,n", [(2, 1000, 12, 4, 64), (1, 4097, 1, 0, 5), (3, 333, 400, 2, 30),
                                       (1, 9000, 7, 4, 256), (1, 1, 3, 4, 64), (2, 129, 64, 0, 1)])
def test_interval_index_bit_exact(B, S, m, a, n, two_pass, monkeypatch):
    """Both forms of the index (one launch; two, with the per-tile separator
    counts first, which long sequences use) at every shape."""
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    if two_pass:
        monkeypatch.setenv("SEPATTN_INDEX_TWO_PASS_S", "1")
    say(f"interval index B={B} S={S} m={m} a={a} n={n} two_pass={two_pass}")
    idx = sa.build_index_interval(B, S, m, a, n)
    torch.cuda.synchronize()
    ref = sepmask.build_index_from_flags(sepmask.interval_flags(S, m), a, n)
    for b in range(B):
        assert np.array_equal(idx.is_sep[b].cpu().numpy(), ref["is_sep"])
        assert np.array_equal(idx.sep_prefix[b].cpu().numpy(), ref["sep_prefix"])
        assert np.array_equal(idx.anchor_pos[b].cpu().numpy(), ref["anchor_pos"])
        assert int(idx.anchor_count[b]) == ref["anchor_count"]
        qt = idx.qtile[b].cpu().numpy()
        assert np.array_equal(qt[:, :6], ref["qtile"])
        assert np.array_equal(idx.tile_class[b].cpu().numpy(), ref["tile_class"])


def _interval_tokens(B, S, m):
    sep_id = 7
    tok = np.where(np.arange(S) % m == m - 1, sep_id, 100).astype(np.int32)
    return np.broadcast_to(tok, (B, S)).copy(), np.array([sep_id], dtype=np.int32)


@pytest.mark.parametrize("S,Hq,Hkv,d,dt,m,a,n", [(700, 2, 2, 64, "bf16", 12, 4, 64),
                                                  (530, 4, 1, 128, "bf16", 5, 3, 100),
                                                  (300, 2, 1, 64, "f32", 1, 0, 8)])
def test_interval_fwd_bwd(S, Hq, Hkv, d, dt, m, a, n):
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    say(f"interval fwd/bwd S={S} Hq={Hq} Hkv={Hkv} d={d} {dt} m={m} a={a} n={n}")
    B = 1
    cfg = dict(seed=S + m, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype=dt, vocab=1000, p_sep=0.0, bursty=False,
               a=a, n=n, bwd=True)
    inp = synth.prefill_inputs(cfg)
    tok, sep = _interval_tokens(B, S, m)
    q, k, v, do = (dev_tensor(inp[x], dt) for x in ("q", "k", "v", "do"))
    idx = sa.build_index_interval(B, S, m, a, n)
    o, lse = sa.fwd(q, k, v, idx, inp["scale"])
    dq, dk, dv = sa.bwd(q, k, v, o, lse, do, idx, inp["scale"])
    torch.cuda.synchronize()
    ro, rl = attention.attention_forward(inp["qf"], inp["kf"], inp["vf"], tok, sep, a, n, scale=inp["scale"])
    to, tl = (1e-4, 1e-4) if dt == "f32" else (2e-2, 2e-3)
    assert np.abs(host_f64(o) - ro).max() <= to
    assert np.abs(lse.cpu().numpy() - rl).max() <= tl
    ref = attention.attention_backward(inp["qf"], inp["kf"], inp["vf"], inp["dof"], tok, sep, a, n,
                                       scale=inp["scale"])
    for name, x, y in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        x = host_f64(x)
        rmax = np.abs(x - y).max() / max(np.abs(y).max(), 1e-30)
        rfro = np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-30)
        say(f"  {name}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
        if dt == "f32":
            assert rmax <= 1e-4, name
        else:
            assert rmax <= 3e-2 and rfro <= 1e-2, name
