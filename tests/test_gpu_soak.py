"""Streaming soak of the SepCache: a long update stream per sequence with the
cache invariants checked on the GPU's own arrays every 1000 steps, full
bit-exact parity with the oracle's list simulation at every check, and at
every check a decode of the newest token over the shifted cache compared with
the oracle's decode attention over the simulated slots (max abs 2e-2).

Invariants (all from pos/tok/state): length <= c - 1; the Initial block holds
positions 0..min(t, a)-1; the Separator block holds at most s separators;
the Window holds the newest n_win positions; positions strictly increase
over the occupied slots (so the Separator block is ascending and older than
the Window); every slot's id is the id streamed at its position; pos/tok are
-1 past the occupied slots.  SEPATTN_SOAK_STEPS sets the length (default
200000; 4000000 reproduces the pages' multi-million-token streaming)."""

import os

import numpy as np
import pytest
import torch

import synth
from oracle import sepcache as osc
from tests.gpu_util import dev_tensor, require_gpu, say
from tests.test_gpu_sepcache import _compare_cache

pytestmark = pytest.mark.gpu


def _invariants(cache, sep, a, s, w, c, t_seen, toks):
    st = cache.state.cpu().numpy()
    pos = cache.pos.cpu().numpy()
    tok = cache.tok.cpu().numpy()
    sep = set(int(x) for x in sep)
    for b in range(st.shape[0]):
        n_init, n_sep, n_win, seen = (int(x) for x in st[b])
        L = n_init + n_sep + n_win
        assert seen == t_seen and L <= c - 1
        assert n_init == min(t_seen, a) and list(pos[b, :n_init]) == list(range(n_init))
        assert n_sep <= s and all(int(x) in sep for x in tok[b, n_init:n_init + n_sep])
        assert list(pos[b, n_init + n_sep:L]) == list(range(t_seen - n_win, t_seen))
        assert np.all(np.diff(pos[b, :L]) > 0)
        assert np.array_equal(tok[b, :L], toks[pos[b, :L], b])
        assert np.all(pos[b, L:] == -1) and np.all(tok[b, L:] == -1)


def test_streaming_soak():
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    steps = int(os.environ.get("SEPATTN_SOAK_STEPS", "200000"))
    B, Hkv, Hq, d, c, a, s, w = 2, 2, 4, 64, 48, 4, 8, 16
    theta, scale = 500000.0, d ** -0.5
    r = synth.rng(77)
    rq = synth.rng(78)  # the decode queries: a stream of their own
    sep = synth.separator_ids(r, 5000)
    cache = sa.SepCache(B, Hkv, d, c, a, s, w)
    cos, sin = sa.rope_table(theta, c, d)
    cos_d, sin_d = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    worst = 0.0
    sims = [osc.SepCacheSim(a, s, w, c, sep) for _ in range(B)]
    toks = np.zeros((steps, B), dtype=np.int32)
    chunk = 1000
    comps = 0
    say(f"soak: {steps} steps, B={B} c={c} a={a} s={s} w={w}")
    for t0 in range(0, steps, chunk):
        n = min(chunk, steps - t0)
        tok = synth.token_ids_iid(r, (n, B), 5000, sep, 0.1)
        kb, _ = synth.normal(r, (n, B, Hkv, d), "bf16")
        vb, _ = synth.normal(r, (n, B, Hkv, d), "bf16")
        toks[t0:t0 + n] = tok
        tok_d = torch.from_numpy(tok).cuda()
        k_d, v_d = dev_tensor(kb, "bf16"), dev_tensor(vb, "bf16")
        for i in range(n):
            cache.update(k_d[i], v_d[i], tok_d[i], sep)
            for b in range(B):
                comps += int(sims[b].append(tok[i, b], kb[i, b], vb[i, b]))
        _invariants(cache, sep, a, s, w, c, t0 + n, toks)
        _compare_cache(cache, sims, Hkv, d, c, where=f"t={t0 + n}")
        qb, qf = synth.normal(rq, (B, Hq, d), "bf16")
        o = cache.decode(dev_tensor(qb, "bf16"), cos_d, sin_d, scale).float().cpu().numpy()
        for b in range(B):
            slots = sims[b].slots()
            K = np.stack([synth.bf16_to_f64(e.k) for e in slots])  # [L, Hkv, d]
            V = np.stack([synth.bf16_to_f64(e.v) for e in slots])
            ref = osc.decode_attention(qf[b], K, V, scale, theta)
            err = float(np.abs(o[b] - ref).max())
            worst = max(worst, err)
            assert err <= 2e-2, (t0 + n, b, err)
        if (t0 // chunk) % 50 == 0:
            say(f"  t={t0 + n} compressions so far={comps} decode max err={worst:.3g}")
    assert comps > steps // 40
