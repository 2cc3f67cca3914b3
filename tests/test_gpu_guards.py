"""Guard bands around every buffer the library writes (GPU).

Each output, workspace, index buffer and cache slab is carved out of a
larger allocation with 4 KiB on both sides filled with a byte pattern; after
the calls the pattern must be intact, so a store past either end of a
buffer fails here even where it would land in memory no parity test reads.
Shapes are ragged (S = 1, 65, 129, 2049: a partial 64-row tile, a partial
128-row query tile, one row past a multiple of both), the grouped-query
ratio is 1 or 8, the head size 64 or 128, and the cache runs through
compressions with a capacity that leaves a partial 128-slot decode chunk.
The results themselves are checked against the oracle elsewhere; here a
few outputs are compared with the oracle only to show the calls ran.
"""

import ctypes

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_tensor, require_gpu, say

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """Device buffers carved from allocations with pattern-filled guards."""

    def __init__(self):
        self.bufs = []

    def take(self, nbytes, dtype=torch.uint8, shape=None):
        buf = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, nbytes))
        inner = buf[GUARD:GUARD + nbytes]
        t = inner.view(dtype)
        return t.view(shape) if shape is not None else t

    def tensor(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.take(n, dtype, shape)

    def check(self, what):
        torch.cuda.synchronize()
        for i, (buf, n) in enumerate(self.bufs):
            lo = buf[:GUARD]
            hi = buf[GUARD + n:]
            assert bool((lo == PATTERN).all()), f"{what}: buffer {i} ({n} bytes): store below its start"
            assert bool((hi == PATTERN).all()), f"{what}: buffer {i} ({n} bytes): store past its end"


class GuardedIndex:
    """An index whose one device buffer is guarded (same fields as sa.Index)."""

    def __init__(self, g, B, S):
        import sparse_attention_sepattn_amd as sa
        L = sa.load_library()
        n = L.sepattn_index_bytes(B, S)
        self.buf = g.take(n)
        self.st = sa._Index()
        assert L.sepattn_index_bind(ctypes.c_void_p(self.buf.data_ptr()), n, B, S, ctypes.byref(self.st)) == 0


ATTN = [(S, G, d) for S in (1, 65, 129, 2049) for G in (1, 8) for d in (64, 128)]


@pytest.mark.parametrize("S,G,d", ATTN)
def test_attention_outputs_guarded(S, G, d):
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, Hkv = 2, 1
    Hq = G * Hkv
    say(f"guards attention S={S} G={G} d={d}")
    cfg = dict(seed=S + G + d, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype="bf16", vocab=1000, p_sep=0.1,
               bursty=False, a=4, n=64, bwd=True)
    inp = synth.prefill_inputs(cfg)
    q, k, v, do = (dev_tensor(inp[x], "bf16") for x in ("q", "k", "v", "do"))
    g = Guarded()
    idx = GuardedIndex(g, B, S)
    sa.build_index(torch.from_numpy(inp["tok"]).cuda(), inp["sep"], cfg["a"], cfg["n"], index=idx)
    o = g.tensor((B, Hq, S, d), torch.bfloat16)
    lse = g.tensor((B, Hq, S), torch.float32)
    sa.fwd(q, k, v, idx, inp["scale"], o=o, lse=lse)
    g.check("fwd")
    dq = g.tensor((B, Hq, S, d), torch.bfloat16)
    dk = g.tensor((B, Hkv, S, d), torch.bfloat16)
    dv = g.tensor((B, Hkv, S, d), torch.bfloat16)
    ws = g.take(sa.bwd_workspace_bytes(B, Hq, Hkv, S, d))
    sa.bwd(q, k, v, o, lse, do, idx, inp["scale"], dq=dq, dk=dk, dv=dv, ws=ws)
    g.check("bwd")
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(dk.float()).all())


def test_attention_outputs_guarded_fp32():
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, Hq, Hkv, S, d = 1, 4, 2, 129, 128
    cfg = dict(seed=5, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype="f32", vocab=1000, p_sep=0.1,
               bursty=False, a=4, n=64, bwd=True)
    inp = synth.prefill_inputs(cfg)
    q, k, v, do = (dev_tensor(inp[x], "f32") for x in ("q", "k", "v", "do"))
    g = Guarded()
    idx = GuardedIndex(g, B, S)
    sa.build_index(torch.from_numpy(inp["tok"]).cuda(), inp["sep"], cfg["a"], cfg["n"], index=idx)
    o = g.tensor((B, Hq, S, d), torch.float32)
    lse = g.tensor((B, Hq, S), torch.float32)
    sa.fwd(q, k, v, idx, inp["scale"], o=o, lse=lse)
    dq = g.tensor((B, Hq, S, d), torch.float32)
    dk = g.tensor((B, Hkv, S, d), torch.float32)
    dv = g.tensor((B, Hkv, S, d), torch.float32)
    ws = g.take(sa.bwd_workspace_bytes(B, Hq, Hkv, S, d, torch.float32))
    sa.bwd(q, k, v, o, lse, do, idx, inp["scale"], dq=dq, dk=dk, dv=dv, ws=ws)
    g.check("fp32 fwd+bwd")


@pytest.mark.parametrize("G,d", [(1, 64), (8, 128), (4, 128)])
def test_cache_and_decode_guarded(G, d):
    """Cache slabs (k, v, pos, tok, state), the decode output and workspace,
    and a prefill hand-off, all guarded, through compressions; c = 200 gives
    two decode chunks, the second partial."""
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    from oracle import sepcache as osc
    B, Hkv, c, a, s, w = 3, 2, 200, 4, 8, 64
    Hq = G * Hkv
    say(f"guards cache G={G} d={d}")
    g = Guarded()
    cache = sa.SepCache(B, Hkv, d, c, a, s, w)
    cache.k = g.tensor((B, Hkv, c, d), torch.bfloat16)
    cache.v = g.tensor((B, Hkv, c, d), torch.bfloat16)
    cache.pos = g.tensor((B, c), torch.int32)
    cache.tok = g.tensor((B, c), torch.int32)
    cache.state = g.tensor((B, 4), torch.int32)
    cache.st = sa._Cache(B, Hkv, d, c, a, s, w, cache.k.data_ptr(), cache.v.data_ptr(), cache.pos.data_ptr(),
                         cache.tok.data_ptr(), cache.state.data_ptr())
    cache.init()
    stream = synth.DecodeStream(dict(seed=G + d, B=B, Hq=Hq, Hkv=Hkv, d=d, vocab=500, p_sep=0.2))
    cos, sin = sa.rope_table(500000.0, c, d)
    cos, sin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    o = g.tensor((B, Hq, d), torch.bfloat16)
    ws = g.take(cache.workspace_bytes(Hq))
    sims = [osc.SepCacheSim(a, s, w, c, stream.sep) for _ in range(B)]
    comps = 0
    for t in range(420):
        x = stream.step()
        cache.update(dev_tensor(x["k"], "bf16"), dev_tensor(x["v"], "bf16"), torch.from_numpy(x["tok"]).cuda(),
                     stream.sep)
        for b in range(B):
            comps += int(sims[b].append(x["tok"][b], x["k"][b], x["v"][b]))
        if t % 20 == 0 or t == 419:
            cache.decode(dev_tensor(x["q"], "bf16"), cos, sin, o=o, ws=ws)
    g.check("update/decode")
    assert comps >= B
    # the last decode against the oracle (the calls ran and read the right slots)
    out = o.float().cpu().numpy()
    for b in range(B):
        K = np.stack([synth.bf16_to_f64(e.k) for e in sims[b].slots()])
        V = np.stack([synth.bf16_to_f64(e.v) for e in sims[b].slots()])
        ref = osc.decode_attention(x["qf"][b], K, V, d ** -0.5, 500000.0)
        assert np.abs(out[b] - ref).max() <= 2e-2
    # prefill hand-off into the same guarded slabs
    P = 777
    r = synth.rng(9)
    tok = torch.from_numpy(synth.token_ids_iid(r, (B, P), 500, stream.sep, 0.2)).cuda()
    kp = torch.randn((B, Hkv, P, d), device="cuda").to(torch.bfloat16)
    vp = torch.randn((B, Hkv, P, d), device="cuda").to(torch.bfloat16)
    idx = sa.build_index(tok, stream.sep, a, 64)
    cache.prefill(kp, vp, tok, idx)
    cache.decode(dev_tensor(x["q"], "bf16"), cos, sin, o=o, ws=ws)
    g.check("prefill hand-off")
