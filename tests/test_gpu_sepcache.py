"""GPU parity of SepCache update and decode.

* cache contents (K/V rows of the occupied slots, positions, ids, counters)
  are bit-exact against the oracle's list simulation after every step;
* decode output within 2e-2 (max abs) of the fp64 oracle (bf16 inputs, fp32
  rotary table, bf16 output);
* the hand-derived trace of tests/golden/sepcache_trace.txt;
* checkpoint/restore mid-stream equals an uninterrupted run.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import sepcache as osc
from tests.gpu_util import bits_u16, dev_tensor, host_f64, require_gpu, say

pytestmark = pytest.mark.gpu


def _make(B, Hkv, d, c, a, s, w):
    import sparse_attention_sepattn_amd as sa
    return sa.SepCache(B, Hkv, d, c, a, s, w)


def _compare_cache(cache, sims, Hkv, d, c, full_rows=True, where=""):
    st = cache.state.cpu().numpy()
    pos = cache.pos.cpu().numpy()
    tok = cache.tok.cpu().numpy()
    kb = bits_u16(cache.k) if full_rows else None
    vb = bits_u16(cache.v) if full_rows else None
    for b, sim in enumerate(sims):
        k_ref, v_ref, pos_ref, tok_ref, st_ref = osc.cache_arrays(sim, c, Hkv, d)
        assert np.array_equal(st[b], st_ref), (where, b, st[b], st_ref)
        assert np.array_equal(pos[b], pos_ref), (where, b)
        assert np.array_equal(tok[b], tok_ref), (where, b)
        if full_rows:
            L = len(sim.slots())
            assert np.array_equal(kb[b, :, :L], k_ref), (where, b)
            assert np.array_equal(vb[b, :, :L], v_ref), (where, b)


def test_golden_trace_on_gpu(golden):
    require_gpu()
    g = golden("sepcache_trace.txt")
    a, s, w, c = (int(g[x]) for x in ("a", "s", "w", "c"))
    seps = set(int(x) for x in g["separators_at"].split())
    cache = _make(1, 1, 64, c, a, s, w)
    r = synth.rng(0)
    t = 0
    while f"t{t}" in g:
        kb, _ = synth.normal(r, (1, 1, 64), "bf16")
        vb, _ = synth.normal(r, (1, 1, 64), "bf16")
        tok = torch.tensor([1 if t in seps else 2], dtype=torch.int32, device="cuda")
        cache.update(dev_tensor(kb, "bf16"), dev_tensor(vb, "bf16"), tok, [1])
        want = [int(x) for x in g[f"t{t}"].split() if x != "C"]
        pos = cache.pos[0].cpu().numpy()
        assert list(pos[:len(want)]) == want and (pos[len(want):] == -1).all(), t
        t += 1


def _stream_run(B, Hkv, Hq, d, c, a, s, w, steps, p_sep, seed, check_every=1, decode_every=0,
                theta=500000.0, rows_every=None, on_fire=True):
    """Stream `steps` tokens into a GPU cache and the oracle's simulations.
    Positions, ids and counters are compared every `check_every` steps (and
    on every compression if `on_fire`), the K/V rows too every `rows_every`
    steps (default: at every such check); decode every `decode_every`
    steps (and on compressions if `on_fire`) against the oracle."""
    import sparse_attention_sepattn_amd as sa
    cfg = dict(seed=seed, B=B, Hq=Hq, Hkv=Hkv, d=d, vocab=5000, p_sep=p_sep)
    stream = synth.DecodeStream(cfg)
    sep = stream.sep
    cache = _make(B, Hkv, d, c, a, s, w)
    sims = [osc.SepCacheSim(a, s, w, c, sep) for _ in range(B)]
    cos, sin = sa.rope_table(theta, c, d)
    cos_d, sin_d = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    scale = 1.0 / np.sqrt(d)
    worst = 0.0
    compressions = np.zeros(B, dtype=int)
    for t in range(steps):
        x = stream.step()
        cache.update(dev_tensor(x["k"], "bf16"), dev_tensor(x["v"], "bf16"),
                     torch.from_numpy(x["tok"]).cuda(), sep)
        fired = False
        for b in range(B):
            fb = sims[b].append(x["tok"][b], x["k"][b], x["v"][b])
            compressions[b] += int(fb)
            fired |= fb
        fire = fired and on_fire
        if fire or t % check_every == 0 or t == steps - 1:
            rows = rows_every is None or t % rows_every == 0 or t == steps - 1
            _compare_cache(cache, sims, Hkv, d, c, full_rows=rows, where=f"t={t}")
        if decode_every and (t % decode_every == 0 or fire or t == steps - 1):
            o = host_f64(cache.decode(dev_tensor(x["q"], "bf16"), cos_d, sin_d, scale))
            for b in range(B):
                slots = sims[b].slots()
                K = np.stack([synth.bf16_to_f64(e.k) for e in slots])  # [L,Hkv,d]
                V = np.stack([synth.bf16_to_f64(e.v) for e in slots])
                ref = osc.decode_attention(x["qf"][b], K, V, scale, theta)
                worst = max(worst, float(np.abs(o[b] - ref).max()))
    return worst, compressions


@pytest.mark.parametrize("a,s,w,c", [(2, 2, 3, 8), (0, 3, 2, 7), (3, 0, 4, 9), (4, 8, 16, 40), (1, 1, 1, 4)])
def test_update_random_streams_bit_exact(a, s, w, c):
    require_gpu()
    say(f"sepcache stream a={a} s={s} w={w} c={c}")
    worst, nc = _stream_run(B=3, Hkv=2, Hq=4, d=64, c=c, a=a, s=s, w=w, steps=150, p_sep=0.3,
                            seed=c, decode_every=7)
    say(f"  compressions per sequence={nc} decode max err={worst:.3g}")
    assert nc.min() > 3
    assert worst <= 2e-2


def test_update_and_decode_d128_gqa8():
    require_gpu()
    worst, nc = _stream_run(B=2, Hkv=2, Hq=16, d=128, c=60, a=4, s=8, w=16, steps=200, p_sep=0.2,
                            seed=11, decode_every=5)
    say(f"d128 G8: compressions per sequence={nc} decode max err={worst:.3g}")
    assert nc.min() > 3 and worst <= 2e-2


def test_streaming_decode_config_prefix():
    """The streaming-decode configuration (B64, 32 q / 8 kv heads, d128, c=800
    = 4 initial + 64 separator slots + window 256) for 1400 steps: every
    sequence compresses twice (the first time all at step 799, then at steps
    that depend on how many separators each kept); cache bit-exact at every
    compression and every 100 steps, decode checked every 100 steps and at
    each compression."""
    require_gpu()
    cfg = synth.CONFIGS["sepcache_decode"]
    worst, nc = _stream_run(B=cfg["B"], Hkv=cfg["Hkv"], Hq=cfg["Hq"], d=cfg["d"], c=cfg["c"], a=cfg["a"],
                            s=cfg["s"], w=cfg["w"], steps=1400, p_sep=cfg["p_sep"], seed=cfg["seed"],
                            check_every=100, decode_every=100, theta=cfg["theta"])
    say(f"decode config: compressions per sequence min={nc.min()} max={nc.max()} decode max err={worst:.3g}")
    assert nc.min() == 2 and nc.max() == 2
    assert worst <= 2e-2


def test_streaming_decode_config_full_length():
    """The streaming-decode configuration over its whole 4096 steps (every
    sequence compresses 7 to 8 times): positions, ids and counters bit-exact
    every 64 steps, K/V rows every 1024 steps and at the end, decode checked
    every 256 steps against the oracle."""
    require_gpu()
    cfg = synth.CONFIGS["sepcache_decode"]
    worst, nc = _stream_run(B=cfg["B"], Hkv=cfg["Hkv"], Hq=cfg["Hq"], d=cfg["d"], c=cfg["c"], a=cfg["a"],
                            s=cfg["s"], w=cfg["w"], steps=cfg["steps"], p_sep=cfg["p_sep"], seed=cfg["seed"],
                            check_every=64, decode_every=256, theta=cfg["theta"], rows_every=1024, on_fire=False)
    say(f"decode config, 4096 steps: compressions per sequence min={nc.min()} max={nc.max()} "
        f"decode max err={worst:.3g}")
    assert nc.min() >= 6
    assert worst <= 2e-2


def test_checkpoint_restore_bit_exact():
    require_gpu()
    B, Hkv, d, c, a, s, w = 2, 2, 64, 30, 2, 4, 8
    cfg = dict(seed=3, B=B, Hq=4, Hkv=Hkv, d=d, vocab=500, p_sep=0.3)
    st1 = synth.DecodeStream(cfg)
    st2 = synth.DecodeStream(cfg)
    c1 = _make(B, Hkv, d, c, a, s, w)
    c2 = _make(B, Hkv, d, c, a, s, w)

    def feed(cache, x):
        cache.update(dev_tensor(x["k"], "bf16"), dev_tensor(x["v"], "bf16"),
                     torch.from_numpy(x["tok"]).cuda(), st1.sep)

    for _ in range(100):
        feed(c1, st1.step())
        feed(c2, st2.step())
    saved = {n: getattr(c2, n).clone().cpu() for n in ("k", "v", "pos", "tok", "state")}
    c3 = _make(B, Hkv, d, c, a, s, w)
    for n, t in saved.items():
        getattr(c3, n).copy_(t.cuda())
    for _ in range(100):
        x = st1.step()
        feed(c1, x)
        feed(c3, x)
    torch.cuda.synchronize()
    L = int(c1.state[0, :3].sum())
    for n in ("pos", "tok", "state"):
        assert torch.equal(getattr(c1, n), getattr(c3, n))
    assert torch.equal(c1.k[:, :, :L], c3.k[:, :, :L]) and torch.equal(c1.v[:, :, :L], c3.v[:, :, :L])


def test_decode_is_deterministic():
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, Hkv, Hq, d, c = 4, 2, 8, 128, 300
    cache = _make(B, Hkv, d, c, 4, 16, 64)
    g = torch.Generator(device="cuda").manual_seed(0)
    for t in range(250):
        k = torch.randn((B, Hkv, d), device="cuda", generator=g).to(torch.bfloat16)
        tok = torch.full((B,), t % 7, dtype=torch.int32, device="cuda")
        cache.update(k, k, tok, [3])
    cos, sin = sa.rope_table(500000.0, c, d)
    cos, sin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    q = torch.randn((B, Hq, d), device="cuda", generator=g).to(torch.bfloat16)
    o1 = cache.decode(q, cos, sin).clone()
    o2 = cache.decode(q, cos, sin).clone()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("Hq,Hkv,d", [(2, 2, 64), (3, 3, 128), (4, 2, 128), (8, 2, 64), (4, 1, 64), (8, 1, 128)])
def test_decode_every_group_size_and_head_dim(Hq, Hkv, d):
    """Every built decode variant (query heads per kv head G = 1, 2, 4, 8 at
    d = 64 and 128) against the oracle, with a cache long enough (c = 300) to
    split over three 128-slot chunks before the first compression."""
    require_gpu()
    say(f"decode Hq={Hq} Hkv={Hkv} d={d}")
    worst, nc = _stream_run(B=2, Hkv=Hkv, Hq=Hq, d=d, c=300, a=4, s=16, w=64, steps=700, p_sep=0.1,
                            seed=Hq * 10 + Hkv + d, check_every=100, decode_every=37)
    say(f"  compressions per sequence={nc} decode max err={worst:.3g}")
    assert nc.min() >= 2 and worst <= 2e-2
