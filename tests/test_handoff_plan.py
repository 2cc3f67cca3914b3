"""Host check of the prefill -> SepCache hand-off plan.

The GPU builds the cache a prompt would leave behind without streaming it
token by token: the Initial block is the first min(a, P) tokens, the Window
is a suffix [ws, P) of the stream and the Separator block holds the last
min(s, #separators in [a, ws)) separators before ws.  ws follows from the
compressions: with Sp separators held, usage reaches c when the Window holds
c - a - Sp tokens, and the compression keeps its w newest.  Once Sp = s the
step is constant.  This test runs that recurrence (the one the kernel
implements) against the oracle's token-by-token simulation."""

import numpy as np
import pytest

from oracle.sepcache import SepCacheSim


def plan(sep, P, a, s, w, c):
    """(n_init, n_sep, n_win, t_seen) and the slot positions, from the
    separator flags ``sep`` [P] by the compression recurrence."""
    pref = np.zeros(P + 1, dtype=np.int64)  # separators in [a, x)
    run = 0
    for x in range(P + 1):
        pref[x] = run
        if a <= x < P and sep[x]:
            run += 1
    if P <= a:
        return (P, 0, 0, P), list(range(P))
    ws, sp = a, 0
    while True:
        if sp == s:  # constant step from here on
            step = c - a - w - s
            first = ws + (c - a - s) - 1  # token whose append fills the cache
            if first <= P - 1:
                ws += ((P - 1 - first) // step + 1) * step
            break
        t = ws + (c - a - sp) - 1
        if t > P - 1:
            break
        ws += c - a - sp - w
        sp = min(s, int(pref[ws]))
    seps = [j for j in range(a, ws) if sep[j]]
    positions = list(range(a)) + seps[len(seps) - sp:] + list(range(ws, P))
    return (a, sp, P - ws, P), positions


@pytest.mark.parametrize("seed", range(40))
def test_plan_matches_streaming(seed):
    r = np.random.default_rng(seed)
    a = int(r.choice([0, 1, 4]))
    s = int(r.choice([0, 1, 3, 8]))
    w = int(r.choice([1, 5, 32]))
    c = a + s + w + int(r.choice([1, 2, 10, 50]))
    P = int(r.integers(1, 3000))
    p_sep = float(r.choice([0.0, 0.05, 0.3, 1.0]))
    tok = np.where(r.random(P) < p_sep, 1, 2)
    sim = SepCacheSim(a, s, w, c, [1])
    for t in range(P):
        sim.append(tok[t])
    st, pos = plan(tok == 1, P, a, s, w, c)
    assert st == sim.state(), (a, s, w, c, P, p_sep)
    assert pos == sim.positions()


def test_plan_decode_config_prompt():
    """The streaming decode configuration (a4 s64 w256 c800) over 5000 tokens."""
    r = np.random.default_rng(5)
    P, a, s, w, c = 5000, 4, 64, 256, 800
    tok = np.where(r.random(P) < 0.08, 1, 2)
    sim = SepCacheSim(a, s, w, c, [1])
    for t in range(P):
        sim.append(tok[t])
    st, pos = plan(tok == 1, P, a, s, w, c)
    assert st == sim.state() and pos == sim.positions()
