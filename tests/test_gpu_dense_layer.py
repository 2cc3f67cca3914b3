"""A full-attention layer through the same kernels (the pages' hybrid keeps
the first and last layers dense: atlas.scime.ai, "Measured effects reported
in the paper"): with a window n >= S every key up to the query is visible,
the index has no anchors and every band tile below the diagonal is full.
Forward and backward against the fp64 oracle at that setting."""

import numpy as np
import pytest
import torch

import synth
from oracle import attention
from tests.gpu_util import dev_tensor, host_f64, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,n,d", [(2048, 2048, 64), (1500, 4096, 128)])
def test_dense_layer_fwd_bwd(S, n, d):
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    say(f"dense layer S={S} n={n} d={d}")
    cfg = dict(seed=S + d, B=1, Hq=2, Hkv=2, S=S, d=d, dtype="bf16", vocab=1000, p_sep=0.08, bursty=False,
               a=4, n=n, bwd=True)
    inp = synth.prefill_inputs(cfg)
    q, k, v, do = (dev_tensor(inp[x], "bf16") for x in ("q", "k", "v", "do"))
    idx = sa.build_index(torch.from_numpy(inp["tok"]).cuda(), inp["sep"], 4, n)
    assert int(idx.qtile[0, :, 1].max()) == 0  # no anchor: lo = 0 for every query tile
    o, lse = sa.fwd(q, k, v, idx, inp["scale"])
    dq, dk, dv = sa.bwd(q, k, v, o, lse, do, idx, inp["scale"])
    torch.cuda.synchronize()
    ro, rl = attention.attention_forward(inp["qf"], inp["kf"], inp["vf"], inp["tok"], inp["sep"], 4, n,
                                         scale=inp["scale"])
    assert np.abs(host_f64(o) - ro).max() <= 2e-2
    assert np.abs(lse.cpu().numpy() - rl).max() <= 2e-3
    ref = attention.attention_backward(inp["qf"], inp["kf"], inp["vf"], inp["dof"], inp["tok"], inp["sep"], 4, n,
                                       scale=inp["scale"])
    for name, x, y in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        x = host_f64(x)
        rmax = np.abs(x - y).max() / np.abs(y).max()
        rfro = np.linalg.norm(x - y) / np.linalg.norm(y)
        say(f"  {name}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
        assert rmax <= 3e-2 and rfro <= 1e-2, name
