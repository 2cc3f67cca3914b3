"""Pins of the oracle's SepCache simulation, rotary embedding and decode
attention (CPU only).

* the hand-derived trace in tests/golden/sepcache_trace.txt;
* invariants after every step of random streams;
* a tie to the mask: compressing whenever the window overflows, with an
  unbounded separator cache, leaves exactly the keys the SepLLM mask (with
  n = w) lets the newest token see;
* rotary embedding against a complex-number formulation, its relative-position
  property and norm preservation;
* decode before any compression equals causal attention at original
  positions (torch SDPA on the CPU, fp64);
* checkpoint/restore mid-stream equals an uninterrupted run.
"""

import copy

import numpy as np
import pytest
import torch

from oracle import sepcache, sepmask


def test_golden_trace(golden):
    g = golden("sepcache_trace.txt")
    a, s, w, c = (int(g[x]) for x in ("a", "s", "w", "c"))
    seps = set(int(x) for x in g["separators_at"].split())
    sim = sepcache.SepCacheSim(a, s, w, c, sep_ids=[1])
    t = 0
    while f"t{t}" in g:
        fired = sim.append(1 if t in seps else 2)
        want = g[f"t{t}"].split()
        want_fire = want[0] == "C"
        if want_fire:
            want = want[1:]
        assert fired == want_fire, t
        assert sim.positions() == [int(x) for x in want], t
        t += 1
    assert t == 14


def _payload(pos, Hkv, d, salt):
    """A bf16 bit pattern [Hkv, d] that names its stream position, head and
    element (so a row placed in the wrong slot, head or element is seen)."""
    h = np.arange(Hkv)[:, None]
    j = np.arange(d)[None, :]
    return ((pos * 977 + h * 131 + j * 7 + salt) % 65521).astype(np.uint16)


def test_cache_arrays_golden_trace(golden):
    """cache_arrays lays the cache out as slots I, Sp, W: after every step of
    the hand-derived trace, slot i holds the payload, position and id of the
    trace's i-th position, slots past L hold -1, and the counters are the
    trace's (n_init, n_sep, n_win, tokens seen)."""
    g = golden("sepcache_trace.txt")
    a, s, w, c = (int(g[x]) for x in ("a", "s", "w", "c"))
    seps = set(int(x) for x in g["separators_at"].split())
    Hkv, d = 3, 5
    sim = sepcache.SepCacheSim(a, s, w, c, sep_ids=[1])
    for t in range(14):
        tok = 1 if t in seps else 20 + t
        sim.append(tok, _payload(t, Hkv, d, 0), _payload(t, Hkv, d, 11))
        want = [int(x) for x in g[f"t{t}"].split() if x != "C"]
        L = len(want)
        k, v, pos, tk, st = sepcache.cache_arrays(sim, c, Hkv, d)
        assert k.shape == (Hkv, L, d) and v.shape == (Hkv, L, d), t
        for i, p in enumerate(want):
            assert np.array_equal(k[:, i, :], _payload(p, Hkv, d, 0)), (t, i)
            assert np.array_equal(v[:, i, :], _payload(p, Hkv, d, 11)), (t, i)
        assert list(pos) == want + [-1] * (c - L), t
        assert list(tk) == [1 if p in seps else 20 + p for p in want] + [-1] * (c - L), t
        assert list(st) == [int(x) for x in g[f"state{t}"].split()], t
        assert pos.dtype == np.int32 and tk.dtype == np.int32 and st.dtype == np.int32


def _stream(r, steps, p):
    return np.where(r.random(steps) < p, 1, 2)


@pytest.mark.parametrize("a,s,w,c,p", [(4, 64, 256, 800, 0.08), (2, 2, 3, 8, 0.4), (0, 3, 2, 7, 0.5),
                                       (3, 0, 4, 9, 0.3), (1, 5, 1, 10, 0.9), (4, 8, 16, 40, 0.08)])
def test_invariants(a, s, w, c, p):
    r = np.random.default_rng(a * 100 + c)
    toks = _stream(r, 3000 if c > 100 else 400, p)
    sim = sepcache.SepCacheSim(a, s, w, c, sep_ids=[1])
    compressed_once = False
    for t, x in enumerate(toks):
        fired = sim.append(x)
        compressed_once |= fired
        pos = sim.positions()
        L = len(pos)
        assert L <= c - 1
        assert [e.pos for e in sim.I] == list(range(min(t + 1, a)))
        sp = [e.pos for e in sim.Sp]
        assert sp == sorted(sp) and len(sp) <= s
        assert all(toks[q] == 1 for q in sp)
        wpos = [e.pos for e in sim.W]
        assert wpos == list(range(t - len(wpos) + 1, t + 1))
        if wpos:
            assert all(q < wpos[0] for q in sp)
        assert all(x < y for x, y in zip(pos, pos[1:]))
        if not compressed_once:
            assert pos == list(range(t + 1))
            assert t < c - 1 or fired
        if fired:
            assert len(sim.W) == w
        # every dropped separator is older than every kept one (FIFO)
        kept_sep = set(sp)
        older = [q for q in range(a, t + 1) if toks[q] == 1 and q not in kept_sep and q not in wpos]
        if older and sp:
            assert max(older) < min(sp)
        if s == 0:
            assert sp == []


@pytest.mark.parametrize("a,w,p", [(4, 8, 0.1), (0, 1, 0.5), (2, 5, 0.3), (3, 20, 0.05)])
def test_cache_equals_mask_row_when_compressing_every_overflow(a, w, p):
    r = np.random.default_rng(w)
    toks = _stream(r, 300, p)
    sim = sepcache.SepCacheSim(a, None, w, 10 ** 9, sep_ids=[1], trigger="window")
    M = sepmask.sep_mask(toks, [1], a, w)
    for t, x in enumerate(toks):
        sim.append(x)
        assert sim.positions() == np.nonzero(M[t])[0].tolist(), t


def _rope_complex(x, p, theta):
    """Independent form: pair (x_m, x_{m+d/2}) as the complex number
    x_m + i x_{m+d/2}, multiplied by exp(i p theta^(-2m/d))."""
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    f = np.array([theta ** (-(2.0 * m) / d) for m in range(h)])
    z = z * np.exp(1j * np.asarray(p, dtype=float)[..., None] * f)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_forms_and_properties():
    r = np.random.default_rng(5)
    x = r.standard_normal((7, 16))
    y = r.standard_normal((7, 16))
    p = np.array([0, 1, 5, 77, 799, 1234, 3])
    theta = 500000.0
    xr = sepcache.rope_rotate(x, p, theta)
    assert np.abs(xr - _rope_complex(x, p, theta)).max() < 1e-12
    assert np.array_equal(sepcache.rope_rotate(x, np.zeros(7), theta), x)
    assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    # scores depend only on the position difference
    s1 = (sepcache.rope_rotate(x, p, theta) * sepcache.rope_rotate(y, p + 3, theta)).sum(1)
    s2 = (sepcache.rope_rotate(x, p + 100, theta) * sepcache.rope_rotate(y, p + 103, theta)).sum(1)
    assert np.abs(s1 - s2).max() < 1e-9


def test_decode_before_compression_is_causal_attention():
    """Before the first compression slot k holds position k, so decode of the
    newest token is causal attention at original positions."""
    r = np.random.default_rng(9)
    Hq, Hkv, d, theta = 4, 2, 16, 10000.0
    L = 30
    K = r.standard_normal((L, Hkv, d))
    V = r.standard_normal((L, Hkv, d))
    q = r.standard_normal((Hq, d))
    scale = 1 / np.sqrt(d)
    o = sepcache.decode_attention(q, K, V, scale, theta)
    qr = _rope_complex(q, np.full(Hq, L - 1), theta)
    kr = _rope_complex(K, np.arange(L)[:, None], theta)
    for h in range(Hq):
        g = h // 2
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(qr[h])[None, None, None], torch.tensor(kr[:, g])[None, None],
            torch.tensor(V[:, g])[None, None], scale=scale)
        assert np.abs(o[h] - ref.numpy().reshape(-1)).max() < 1e-12


def test_decode_closed_forms():
    r = np.random.default_rng(10)
    K = r.standard_normal((12, 1, 8))
    V = r.standard_normal((12, 1, 8))
    # zero query -> mean of the values
    o = sepcache.decode_attention(np.zeros((2, 8)), K, V, 0.3, 500000.0)
    assert np.abs(o - V[:, 0].mean(0)).max() < 1e-13
    # one slot -> that slot's value
    o = sepcache.decode_attention(r.standard_normal((3, 8)), K[:1], V[:1], 0.3, 500000.0)
    assert np.abs(o - V[0, 0]).max() < 1e-15


def test_resume_equals_uninterrupted():
    r = np.random.default_rng(3)
    toks = _stream(r, 500, 0.2)
    a_ = sepcache.SepCacheSim(2, 4, 6, 20, sep_ids=[1])
    b_ = sepcache.SepCacheSim(2, 4, 6, 20, sep_ids=[1])
    for x in toks[:250]:
        a_.append(x)
        b_.append(x)
    b_ = copy.deepcopy(b_)
    for x in toks[250:]:
        a_.append(x)
        b_.append(x)
    assert a_.positions() == b_.positions() and a_.state() == b_.state()


def test_capacity_argument_checks():
    with pytest.raises(ValueError):
        sepcache.SepCacheSim(4, 64, 256, 324, sep_ids=[1])
    with pytest.raises(ValueError):
        sepcache.SepCacheSim(4, 64, 0, 800, sep_ids=[1])
