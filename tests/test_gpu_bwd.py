"""GPU parity of the backward against the fp64 oracle.

Tolerances (per tensor, relative to the tensor's largest reference entry;
a tensor that is zero by construction is held to an absolute bound instead):
  * fp32 inputs: max|diff| / max|ref| <= 1e-4;
  * bf16 inputs: max|diff| / max|ref| <= 3e-2, and the Frobenius-relative
    error <= 1e-2 (P and dS are rounded to bf16 before the second products,
    which bounds the typical error near 2^-9; the Frobenius bound catches a
    missing or doubled contribution that the max bound could hide).  The
    Frobenius bound applies to tensors of at least 64 rows: on a few rows it
    repeats the max error, which D = rowsum(dO*O) from the bf16-rounded O
    can push to ~1 % where a row's dP - D is a small difference.
The forward outputs (o, lse) fed to the backward come from the GPU forward,
as in training.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import attention, sepmask
from tests.gpu_util import dev_tensor, host_f64, require_gpu, say

pytestmark = pytest.mark.gpu


def _gpu_grads(inp):
    import sparse_attention_sepattn_amd as sa
    c = inp["cfg"]
    dt = c["dtype"]
    q, k, v, do = (dev_tensor(inp[x], dt) for x in ("q", "k", "v", "do"))
    idx = sa.build_index(torch.from_numpy(inp["tok"]).cuda(), inp["sep"], c["a"], c["n"])
    o, lse = sa.fwd(q, k, v, idx, inp["scale"])
    dq, dk, dv = sa.bwd(q, k, v, o, lse, do, idx, inp["scale"])
    torch.cuda.synchronize()
    return host_f64(dq), host_f64(dk), host_f64(dv)


def _rel(got, ref):
    m = max(np.abs(ref).max(), 1e-30)
    return np.abs(got - ref).max() / m, np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)


def _check(got, ref, dt, what):
    for name, x, y in zip(("dq", "dk", "dv"), got, ref):
        if np.abs(y).max() <= 1e-9:
            # zero by construction (every row sees one key, so dS = 0): only
            # rounding residue of D = rowsum(dO * O) versus dP may remain
            say(f"  {what} {name}: reference is zero, max|got|={np.abs(x).max():.3g}")
            assert np.abs(x).max() <= (1e-5 if dt == "f32" else 1e-3), name
            continue
        rmax, rfro = _rel(x, y)
        say(f"  {what} {name}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
        if dt == "f32":
            assert rmax <= 1e-4, (name, rmax)
        else:
            assert rmax <= 3e-2 and (rfro <= 1e-2 or y.size // y.shape[-1] < 64), (name, rmax, rfro)


def _inputs(S, B, Hq, Hkv, d, dt, a, n, p, seed, bursty=False):
    cfg = dict(seed=seed, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype=dt, vocab=1000, p_sep=p,
               bursty=bursty, a=a, n=n, bwd=True)
    return synth.prefill_inputs(cfg)


CASES = [
    # S, B, Hq, Hkv, d, dtype, a, n, p_sep
    (1, 1, 1, 1, 64, "f32", 4, 64, 0.1),
    (77, 2, 2, 1, 64, "f32", 0, 1, 0.2),
    (300, 1, 4, 2, 128, "f32", 4, 64, 0.08),
    (600, 1, 2, 2, 64, "f32", 4, 600, 0.0),
    (333, 2, 2, 2, 64, "bf16", 4, 64, 0.08),
    (700, 1, 4, 1, 128, "bf16", 3, 256, 0.15),
    (1000, 1, 2, 2, 64, "bf16", 0, 1, 0.0),
    (640, 1, 2, 1, 128, "bf16", 4, 40, 1.0),
    (2500, 1, 2, 1, 64, "f32", 4, 64, 0.08),
    (300, 1, 2, 1, 64, "bf16", 4, 2**31 - 1, 0.1),  # window beyond S: dense causal, no overflow
    (200, 1, 2, 2, 64, "bf16", 2**31 - 1, 8, 0.1),  # every token initial
]


@pytest.mark.parametrize("case", CASES)
def test_bwd_small(case):
    require_gpu()
    S, B, Hq, Hkv, d, dt, a, n, p = case
    say(f"bwd small {case}")
    inp = _inputs(S, B, Hq, Hkv, d, dt, a, n, p, seed=S + d + 1)
    got = _gpu_grads(inp)
    ref = attention.attention_backward(inp["qf"], inp["kf"], inp["vf"], inp["dof"], inp["tok"], inp["sep"],
                                       a, n, scale=inp["scale"])
    _check(got, ref, dt, f"S={S}")


def test_bwd_multi_chunk_anchors():
    """8192 tokens: 64 query tiles, so every early anchor tile's gradient is
    accumulated over several query-tile chunks; full gradients compared."""
    require_gpu()
    inp = _inputs(8192, 1, 4, 1, 128, "bf16", 4, 256, 0.08, seed=8)
    got = _gpu_grads(inp)
    c = inp["cfg"]
    ref = attention.attention_backward(inp["qf"], inp["kf"], inp["vf"], inp["dof"], inp["tok"], inp["sep"],
                                       c["a"], c["n"], scale=inp["scale"])
    _check(got, ref, "bf16", "S=8192")


def test_bwd_multi_chunk_anchors_fp32():
    require_gpu()
    inp = _inputs(4500, 1, 2, 1, 64, "f32", 4, 64, 0.2, seed=9)
    got = _gpu_grads(inp)
    c = inp["cfg"]
    ref = attention.attention_backward(inp["qf"], inp["kf"], inp["vf"], inp["dof"], inp["tok"], inp["sep"],
                                       c["a"], c["n"], scale=inp["scale"])
    _check(got, ref, "f32", "S=4500 fp32")


def test_bwd_pythia_config_full():
    """Pythia-160m-shaped batch (B8 H12 S2048 d64 bf16): every gradient."""
    require_gpu()
    cfg = synth.CONFIGS["pythia160m"]
    inp = synth.prefill_inputs(cfg)
    got = _gpu_grads(inp)
    ref = attention.attention_backward(inp["qf"], inp["kf"], inp["vf"], inp["dof"], inp["tok"], inp["sep"],
                                       cfg["a"], cfg["n"], scale=inp["scale"])
    _check(got, ref, "bf16", "pythia")


_LONG = {}


def _long_context():
    """Inputs and GPU gradients of the 32k-token configuration, computed once
    for the tests that sample them."""
    if not _LONG:
        cfg = synth.CONFIGS["long_context_32k"]
        inp = synth.prefill_inputs(cfg)
        _LONG.update(cfg=cfg, inp=inp, grads=_gpu_grads(inp))
    return _LONG["cfg"], _LONG["inp"], _LONG["grads"]


def test_bwd_long_context_sampled():
    """32k tokens, 32 q / 8 kv heads, bursty separators: dQ on sampled rows of
    heads 0 and 31; dK/dV on sampled key rows of the last 2048 positions of kv
    heads 0 and 7 (each needs every query row's softmax statistics)."""
    require_gpu()
    cfg, inp, (dq, dk, dv) = _long_context()
    S, grp = cfg["S"], cfg["Hq"] // cfg["Hkv"]
    sepf = sepmask.separator_flags(inp["tok"][0], inp["sep"])
    rows = np.unique(np.concatenate([np.arange(0, S, 331), np.arange(S - 70, S), np.arange(0, 70)]))
    for h in (0, 31):
        g = h // grp
        ref = attention.grad_q_rows(inp["qf"][0, h], inp["kf"][0, g], inp["vf"][0, g], inp["dof"][0, h],
                                    sepf, cfg["a"], cfg["n"], inp["scale"], rows)
        rmax, rfro = _rel(dq[0, h, rows], ref)
        say(f"  32k dq head {h}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
        assert rmax <= 3e-2 and rfro <= 1e-2
    cols = np.unique(np.concatenate([np.arange(S - 2048, S, 37), np.nonzero(sepf[S - 2048:])[0][:40] + S - 2048]))
    for g in (0, 7):
        hs = range(g * grp, (g + 1) * grp)
        rk, rv = attention.grad_kv_cols([inp["qf"][0, h] for h in hs], inp["kf"][0, g], inp["vf"][0, g],
                                        [inp["dof"][0, h] for h in hs], sepf, cfg["a"], cfg["n"],
                                        inp["scale"], cols)
        for name, got, ref in (("dk", dk[0, g, cols], rk), ("dv", dv[0, g, cols], rv)):
            rmax, rfro = _rel(got, ref)
            say(f"  32k {name} kv head {g}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
            assert rmax <= 3e-2 and rfro <= 1e-2


def test_bwd_long_context_early_anchors():
    """32k tokens: dK/dV of kv head 0 on the initial tokens, the first 40
    separators and every 997th key of the whole sequence.  The early anchors
    collect gradient from every later query row; the backward splits that
    sum over anchor chunks of query tiles and a band slot and adds them in
    its last kernel, so these rows pin the multi-chunk path at full size
    (one kv head keeps the fp64 cost bounded)."""
    require_gpu()
    cfg, inp, (dq, dk, dv) = _long_context()
    S, grp = cfg["S"], cfg["Hq"] // cfg["Hkv"]
    sepf = sepmask.separator_flags(inp["tok"][0], inp["sep"])
    seps = np.nonzero(sepf)[0]
    cols = np.unique(np.concatenate([np.arange(0, 70), seps[:40], np.arange(0, S, 997)]))
    g = 0
    hs = range(g * grp, (g + 1) * grp)
    say(f"  32k early anchors: {len(cols)} key rows of kv head {g}")
    rk, rv = attention.grad_kv_cols([inp["qf"][0, h] for h in hs], inp["kf"][0, g], inp["vf"][0, g],
                                    [inp["dof"][0, h] for h in hs], sepf, cfg["a"], cfg["n"],
                                    inp["scale"], cols)
    for name, got, ref in (("dk", dk[0, g, cols], rk), ("dv", dv[0, g, cols], rv)):
        rmax, rfro = _rel(got, ref)
        say(f"  32k early {name} kv head {g}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
        assert rmax <= 3e-2 and rfro <= 1e-2
    _LONG.clear()  # the last test that samples them


def test_bwd_llama_config_sampled():
    """Llama-3-8B-shaped prefill (S 8192, 32 q / 8 kv heads, d128, n 256):
    dQ on sampled rows of heads 0, 13 and 31; dK/dV on key rows sampled over
    the whole sequence -- the initial tokens, the first and last separators
    (anchors whose gradients collect every later query row, over several
    anchor chunks) and every 97th row -- of kv heads 0 and 7."""
    require_gpu()
    cfg = synth.CONFIGS["llama3_8b_prefill"]
    inp = synth.prefill_inputs(cfg, with_grad=True)
    dq, dk, dv = _gpu_grads(inp)
    S, grp = cfg["S"], cfg["Hq"] // cfg["Hkv"]
    sepf = sepmask.separator_flags(inp["tok"][0], inp["sep"])
    rows = np.unique(np.concatenate([np.arange(0, S, 211), np.arange(S - 40, S), np.arange(0, 40)]))
    for h in (0, 13, 31):
        g = h // grp
        ref = attention.grad_q_rows(inp["qf"][0, h], inp["kf"][0, g], inp["vf"][0, g], inp["dof"][0, h],
                                    sepf, cfg["a"], cfg["n"], inp["scale"], rows)
        rmax, rfro = _rel(dq[0, h, rows], ref)
        say(f"  llama dq head {h}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
        assert rmax <= 3e-2 and rfro <= 1e-2
    seps = np.nonzero(sepf)[0]
    cols = np.unique(np.concatenate([np.arange(0, S, 97), np.arange(0, 70), seps[:40], seps[-40:]]))
    for g in (0, 7):
        hs = range(g * grp, (g + 1) * grp)
        rk, rv = attention.grad_kv_cols([inp["qf"][0, h] for h in hs], inp["kf"][0, g], inp["vf"][0, g],
                                        [inp["dof"][0, h] for h in hs], sepf, cfg["a"], cfg["n"],
                                        inp["scale"], cols)
        for name, got, ref in (("dk", dk[0, g, cols], rk), ("dv", dv[0, g, cols], rv)):
            rmax, rfro = _rel(got, ref)
            say(f"  llama {name} kv head {g}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
            assert rmax <= 3e-2 and rfro <= 1e-2


def test_autograd_function_matches_direct_calls():
    """sa.attention under torch.autograd returns the same O and the same
    gradients, bit for bit, as the direct fwd / bwd calls."""
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    inp = _inputs(333, 2, 4, 2, 64, "bf16", 4, 64, 0.08, 11)
    c = inp["cfg"]
    q, k, v, do = (dev_tensor(inp[x], "bf16") for x in ("q", "k", "v", "do"))
    idx = sa.build_index(torch.from_numpy(inp["tok"]).cuda(), inp["sep"], c["a"], c["n"])
    o, lse = sa.fwd(q, k, v, idx, inp["scale"])
    ref = sa.bwd(q, k, v, o, lse, do, idx, inp["scale"])
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    oa = sa.attention(qa, ka, va, idx, inp["scale"])
    oa.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(oa.detach(), o)
    for name, got, want in zip(("dq", "dk", "dv"), (qa.grad, ka.grad, va.grad), ref):
        assert torch.equal(got, want), name


def test_bwd_many_short_anchor_chunks():
    """2304 tokens, one kv head: the split's upper bound of 16 chunks gives 9
    chunks of 2 query tiles, so most anchors sum 9 partial slots; every
    gradient against the oracle."""
    require_gpu()
    inp = _inputs(2304, 1, 2, 1, 128, "bf16", 4, 256, 0.08, seed=2304)
    got = _gpu_grads(inp)
    c = inp["cfg"]
    ref = attention.attention_backward(inp["qf"], inp["kf"], inp["vf"], inp["dof"], inp["tok"], inp["sep"],
                                       c["a"], c["n"], scale=inp["scale"])
    _check(got, ref, "bf16", "S=2304 split")


def test_bwd_split_bounded_at_40_tiles():
    """12288 tokens, 12 heads, d=64: the item target gives 2 chunks of 48
    query tiles, the 40-tile bound 3 of 32; dQ on sampled rows, dK/dV on
    every anchor of the first 2048 positions and sampled keys elsewhere, for
    the first and the last head."""
    require_gpu()
    inp = _inputs(12288, 1, 12, 12, 64, "bf16", 4, 64, 0.08, seed=12288)
    c = inp["cfg"]
    S = c["S"]
    dq, dk, dv = _gpu_grads(inp)
    sepf = sepmask.separator_flags(inp["tok"][0], inp["sep"])
    rows = np.unique(np.concatenate([np.arange(0, S, 211), np.arange(S - 40, S)]))
    early = np.concatenate([np.arange(0, c["a"]), np.nonzero(sepf[:2048])[0]])
    cols = np.unique(np.concatenate([early, np.arange(0, S, 401)]))
    for h in (0, 11):
        ref = attention.grad_q_rows(inp["qf"][0, h], inp["kf"][0, h], inp["vf"][0, h], inp["dof"][0, h],
                                    sepf, c["a"], c["n"], inp["scale"], rows)
        rmax, rfro = _rel(dq[0, h, rows], ref)
        say(f"  12k dq head {h}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
        assert rmax <= 3e-2 and rfro <= 1e-2
        rk, rv = attention.grad_kv_cols([inp["qf"][0, h]], inp["kf"][0, h], inp["vf"][0, h], [inp["dof"][0, h]],
                                        sepf, c["a"], c["n"], inp["scale"], cols)
        for name, got, ref in (("dk", dk[0, h, cols], rk), ("dv", dv[0, h, cols], rv)):
            rmax, rfro = _rel(got, ref)
            say(f"  12k {name} head {h}: max-rel={rmax:.3g} fro-rel={rfro:.3g}")
            assert rmax <= 3e-2 and rfro <= 1e-2
